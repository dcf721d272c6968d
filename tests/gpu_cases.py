"""Shared set-up for the GPU parity tests: seeded layers, the oracle's pack of
each (cached per session), the same quantized weights handed to the library
through svdq_quantize_residual, and the comparison helpers with the
tolerances the tests state."""
from __future__ import annotations

import dataclasses
import functools

import numpy as np

import bit_svdquant_diffusion_amd as S
from bit_svdquant_diffusion_amd import synth
from oracle import svdq_oracle as O

# Y tolerance: relative Frobenius error <= 1e-2 and max abs error <= 2e-2 max|Y|
Y_REL_FRO = 1e-2
Y_MAX_ABS = 2e-2


@functools.lru_cache(maxsize=4)
def layer_data(spec: synth.LayerSpec, m_rows: int | None = None):
    lay = synth.make_layer(spec, m_rows=m_rows)
    return lay


def weight_owner(spec: synth.LayerSpec) -> synth.LayerSpec:
    """The layer whose weights and calibration a workload uses: the decode-like
    small-M runs reuse the text stream's packed layers (calibrated on its 1024
    tokens)."""
    for pre in ("m64_", "m256_"):
        if spec.name.startswith(pre):
            return dataclasses.replace(spec, name="txt_" + spec.name[len(pre):], M=1024)
    return spec


def oracle_pack(spec: synth.LayerSpec):
    return _oracle_pack(weight_owner(spec))


@functools.lru_cache(maxsize=4)
def _oracle_pack(spec: synth.LayerSpec):
    """Oracle pack of a layer (calibration max over the layer's full X)."""
    lay = layer_data(spec)
    ax = np.abs(lay.x).max(axis=0)
    return O.pack(lay.w_lin, lay.bias, ax, spec.rank, spec.fmt)


def library_host(spec: synth.LayerSpec):
    return _library_host(weight_owner(spec))


@functools.lru_cache(maxsize=4)
def _library_host(spec: synth.LayerSpec):
    """The oracle's mu/factors quantized by the library (codes bit-exact with the
    oracle's, pinned on the CPU) in the library's device layout."""
    ref = oracle_pack(spec)
    lay = layer_data(spec)
    layer = S.Layer(spec.K, spec.N, spec.rank, spec.fmt)
    host = S.quantize_residual(layer, lay.w_lin, lay.bias, ref["mu"],
                               O.bf16_to_bits(ref["l1"]), O.bf16_to_bits(ref["l2"]))
    return layer, host


def device_layer(spec, device="cuda"):
    layer, host = library_host(spec)
    return layer, S.to_device(layer, host, device)


def x_device(spec, device="cuda"):
    import torch
    lay = layer_data(spec)
    return torch.from_numpy(lay.x_bits.view(np.int16)).to(device).view(torch.bfloat16)


def bf16_tensor_to_f32(t) -> np.ndarray:
    import torch
    u = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return O.bf16_from_bits(u)


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = ""):
    y_ref = np.asarray(y_ref, dtype=np.float64)
    d = y_gpu.astype(np.float64) - y_ref
    fro = np.linalg.norm(d) / max(np.linalg.norm(y_ref), 1e-30)
    mx = np.abs(d).max() / max(np.abs(y_ref).max(), 1e-30)
    print(f"[parity] {what}: rel_fro={fro:.3e} max_abs_rel={mx:.3e}", flush=True)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    assert fro <= Y_REL_FRO, f"{what}: relative Frobenius error {fro:.3e} > {Y_REL_FRO}"
    assert mx <= Y_MAX_ABS, f"{what}: max abs error {mx:.3e} max|Y| > {Y_MAX_ABS}"
    return fro, mx


def sample_rows(M: int, n: int = 96, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    head = np.arange(min(32, M))
    tail = np.arange(max(0, M - 32), M)
    mid = rng.choice(M, size=min(n, M), replace=False)
    return np.unique(np.concatenate([head, mid, tail]))
