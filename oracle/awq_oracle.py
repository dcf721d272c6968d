"""CPU oracle for the AWQ-style W4A16 linear -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package's smoke check and the benchmark's CPU
baseline may import this module. The product never calls it, and it imports
nothing from the product.

The pages keep the precision-sensitive adaptive-normalization and modulation
layers of a diffusion model on an "AWQ style" scheme: 4-bit weights, 16-bit
activations (aiflownews.com, "How Nunchaku four bit quantization actually
works"). They say no more; the plainest reading of activation-aware weight
quantization, written out here step by step:

  pack (offline, with calibration activations X_cal [M_cal][K]):
    1. per input channel the mean magnitude a_k = mean_m |X_cal[m,k]|;
    2. for each alpha on the grid 0, 1/20, ..., 19/20: s_k = max(a_k, 1e-4)^alpha,
       normalized by sqrt(max_k s_k * min_k s_k); the weight W diag(s) is
       quantized (step 3) and the candidate's loss is the squared error
       sum over X_cal of (X diag(1/s) Q(W diag(s))^T - X W^T)^2; the alpha
       with the least loss (the first one on a tie) is kept;
    3. quantization of W' = W diag(s), per output channel per group of 128
       input channels, asymmetric 4-bit, in float32 as the AWQ reference
       does it: scale = max(max - min, 1e-5) / 15, zero = clamp(-rint(min /
       scale), 0, 15), q = clamp(rint(w / scale) + zero, 0, 15); the
       dequantized weight is fl32(scale * (q - zero)).
  forward (runtime): x_hat = fl32(x * inv_s) with the stored inv_s =
    fl32(1 / s); y = x_hat dequant(W')^T + b, summed here in float64.

Every function is pinned by tests/test_awq_oracle.py against brute force,
closed forms and invariants; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

GROUP = 128
ALPHA_GRID = np.arange(20) / 20.0


def quantize_groups(w: np.ndarray, group: int = GROUP):
    """Asymmetric 4-bit per row per group of `group` columns, float32 steps:
    returns (q uint8 [N][K], scale float32 [N][K/group], zero uint8 [N][K/group])."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    g = w.reshape(N, K // group, group)
    mx = g.max(axis=-1)
    mn = g.min(axis=-1)
    scale = (np.maximum(mx - mn, np.float32(1e-5)) / np.float32(15.0)).astype(np.float32)
    zero = np.clip(-np.rint(mn / scale), 0, 15).astype(np.float32)
    q = np.clip(np.rint(g / scale[..., None]) + zero[..., None], 0, 15)
    return q.astype(np.uint8).reshape(N, K), scale, zero.astype(np.uint8)


def dequantize(q: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int = GROUP) -> np.ndarray:
    """fl32(scale * (q - zero)) [N][K] float32."""
    N, K = q.shape
    d = q.reshape(N, K // group, group).astype(np.float32) - zero.astype(np.float32)[..., None]
    return (scale[..., None] * d).astype(np.float32).reshape(N, K)


def channel_scales(act_mean: np.ndarray, alpha: float) -> np.ndarray:
    """s = max(a, 1e-4)^alpha / sqrt(max s * min s), float64."""
    s = np.power(np.maximum(np.asarray(act_mean, np.float64), 1e-4), alpha)
    return s / np.sqrt(s.max() * s.min())


def candidate(w_lin: np.ndarray, act_mean: np.ndarray, alpha: float):
    """(s float64, inv_s float32, q, scale, zero) of one grid point."""
    s = channel_scales(act_mean, alpha)
    ws = (np.asarray(w_lin, np.float64) * s[None, :]).astype(np.float32)
    q, sc, z = quantize_groups(ws)
    inv_s = (1.0 / s).astype(np.float32)
    return s, inv_s, q, sc, z


def loss(x_cal: np.ndarray, w_lin: np.ndarray, inv_s: np.ndarray, q, sc, z) -> float:
    """Squared output error of a candidate on the calibration rows (float64)."""
    x = np.asarray(x_cal, np.float64)
    xh = x * inv_s.astype(np.float64)[None, :]
    y = xh @ dequantize(q, sc, z).astype(np.float64).T
    ref = x @ np.asarray(w_lin, np.float64).T
    return float(np.sum((y - ref) ** 2))


def pack(w_lin: np.ndarray, bias, x_cal: np.ndarray, alpha: float | None = None) -> dict:
    """Offline preparation; with `alpha` given, the search is skipped."""
    w_lin = np.asarray(w_lin, np.float32)
    N, K = w_lin.shape
    a = np.abs(np.asarray(x_cal, np.float32)).astype(np.float64).mean(axis=0)
    losses = None
    if alpha is None:
        losses = np.array([loss(x_cal, w_lin, *candidate(w_lin, a, al)[1:]) for al in ALPHA_GRID])
        alpha = float(ALPHA_GRID[int(np.argmin(losses))])
    s, inv_s, q, sc, z = candidate(w_lin, a, alpha)
    return dict(K=K, N=N, alpha=alpha, losses=losses, act_mean=a, inv_s=inv_s, q=q, scale=sc, zero=z,
                bias=np.zeros(N, np.float32) if bias is None else np.asarray(bias, np.float32))


def forward(packed: dict, x: np.ndarray) -> np.ndarray:
    """y [M][N] float64 for x [M][K] (float32 values of bf16 inputs)."""
    xh = (np.asarray(x, np.float32) * packed["inv_s"][None, :]).astype(np.float64)
    w = dequantize(packed["q"], packed["scale"], packed["zero"]).astype(np.float64)
    return xh @ w.T + packed["bias"].astype(np.float64)[None, :]
