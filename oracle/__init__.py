"""CPU oracle of the SVDQuant W4A4 linear layer (test infrastructure only)."""
