"""Seeded synthetic inputs for the SVDQuant W4A4 linear layer.

This module only draws random numbers and shapes them like the workloads the
pages talk about (FLUX-style DiT linears whose activations carry a few large
outlier channels -- "What SVDQuant actually does", aiflownews.com page). It
holds none of the method's arithmetic: no smoothing, no SVD, no quantization.
Both the CPU oracle and the GPU path take their inputs from here.

Recipe (all draws from NumPy's PCG64; one SeedSequence per layer, spawned
into the streams [outlier channels, X, W, bias, spare]):

* X  [M][K]: N(0,1); a set of round(frac*K) input channels, drawn without
  replacement, is multiplied by ``x_outlier_scale``; the "gelu" variant first
  applies the erf-GELU to the normal draw. Rounded to bf16 (round to nearest
  even) and returned as raw bf16 bits (uint16) plus the exact float32 value.
* W  (math K x N), returned in nn.Linear layout ``w_lin [N][K]`` float32:
  N(0, 1/K) (1/K is a variance); optionally round(w_frac*K) input rows
  multiplied by ``w_outlier_scale``.
* b  [N]: N(0, 0.01) (0.01 is a variance), rounded to a bf16-representable
  float32 so the bf16 bias stored on the device is the same number.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "LayerSpec", "CONFIGS", "config_layers", "make_layer", "bf16_bits",
    "bf16_value", "round_to_bf16", "calibration_rows", "awq_layers",
]


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Input preparation only (the caller hands bf16 tensors to the layer).
    NaNs are not expected in synthetic data.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    return bf16_value(bf16_bits(a))


@dataclass(frozen=True)
class LayerSpec:
    """One linear layer workload: Y[M][N] = layer(X[M][K])."""
    name: str
    M: int
    K: int
    N: int
    rank: int
    fmt: str                    # "int4" (INT4, group 64), "mxfp4" (E2M1 + E8M0 per 32), or "w4a16" (AWQ-style)
    seed: int
    x_kind: str = "normal"      # "normal", "gelu" or "silu"
    x_outlier_frac: float = 0.01
    x_outlier_scale: float = 50.0
    w_outlier_frac: float = 0.02
    w_outlier_scale: float = 10.0
    stream: str = ""            # distinguishes layers that share a seed

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def _layer(name, M, K, N, r, fmt, seed, **kw):
    return LayerSpec(name=name, M=M, K=K, N=N, rank=r, fmt=fmt, seed=seed, **kw)


def config_layers(idx: int, small_m: bool = True) -> list[LayerSpec]:
    """The five workload configurations, as lists of layers.

    0: tiny check layer 256x512->512, r=16, INT4.
    1: FLUX-style attention QKV, 4608 tokens, 3072->9216, r=32, INT4.
    2: FLUX-style MLP up, 4608 tokens, 3072->12288, r=32, MXFP4.
    3: FLUX-style MLP down, 4608 tokens, 12288->3072, r=32, INT4, GELU input
       with 0.5% outlier channels x30 and no weight outlier rows.
    4: a double-stream block's linears at batch 2, 1024^2: image stream
       (8192 tokens) and text stream (1024 tokens), each with QKV, out, MLP up
       and MLP down, r=32, INT4; plus decode-like small-M runs (64, 256).
    """
    if idx == 0:
        return [_layer("tiny", 256, 512, 512, 16, "int4", 0)]
    if idx == 1:
        return [_layer("qkv", 4608, 3072, 9216, 32, "int4", 1)]
    if idx == 2:
        return [_layer("mlp_up_fp4", 4608, 3072, 12288, 32, "mxfp4", 2)]
    if idx == 3:
        return [_layer("mlp_down", 4608, 12288, 3072, 32, "int4", 3, x_kind="gelu",
                       x_outlier_frac=0.005, x_outlier_scale=30.0, w_outlier_frac=0.0)]
    if idx == 4:
        shapes = [("qkv", 3072, 9216, "normal"), ("out", 3072, 3072, "normal"),
                  ("up", 3072, 12288, "normal"), ("down", 12288, 3072, "gelu")]
        out = []
        ms = [("img", 8192), ("txt", 1024)]
        if small_m:
            ms += [("m64", 64), ("m256", 256)]
        for sname, M in ms:
            for lname, K, N, xk in shapes:
                kw = {}
                if xk == "gelu":
                    kw = dict(x_kind="gelu", x_outlier_frac=0.005, x_outlier_scale=30.0)
                # the small-M runs reuse the text stream's weights
                wstream = "txt" if sname.startswith("m") else sname
                out.append(_layer(f"{sname}_{lname}", M, K, N, 32, "int4", 4,
                                  stream=f"{wstream}_{lname}", **kw))
        return out
    raise ValueError(f"unknown config {idx}")


CONFIGS = {i: config_layers(i) for i in range(5)}


def _streams(spec: LayerSpec):
    entropy = [spec.seed]
    if spec.stream:
        entropy.append(int.from_bytes(spec.stream.encode(), "little") % (2**63))
    ss = np.random.SeedSequence(entropy)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5)]


def _gelu(a: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * a * (1.0 + erf(a / math.sqrt(2.0)))


def _silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def _draw_x(spec: LayerSpec, rng, rows: int, xo: np.ndarray) -> np.ndarray:
    xf = rng.standard_normal((rows, spec.K), dtype=np.float64)
    if spec.x_kind == "gelu":
        xf = _gelu(xf)
    elif spec.x_kind == "silu":
        xf = _silu(2.0 * xf)
    xf[:, xo] *= spec.x_outlier_scale
    return xf


@dataclass
class Layer:
    spec: LayerSpec
    x_bits: np.ndarray          # uint16 [M][K] bf16 bits
    x: np.ndarray               # float32 [M][K] exact values of x_bits
    w_lin: np.ndarray           # float32 [N][K]
    bias: np.ndarray            # float32 [N], bf16-representable
    x_outlier_channels: np.ndarray = field(default=None)
    w_outlier_rows: np.ndarray = field(default=None)


def make_layer(spec: LayerSpec, m_rows: int | None = None, with_x: bool = True) -> Layer:
    """Draw one layer's X, W and b. ``m_rows`` draws only the first rows of X
    (the draw is row-major, so the first rows equal those of the full draw)."""
    r_out, r_x, r_w, r_b, _ = _streams(spec)
    M, K, N = spec.M, spec.K, spec.N
    n_xo = int(round(spec.x_outlier_frac * K))
    n_wo = int(round(spec.w_outlier_frac * K))
    xo = np.sort(r_out.choice(K, size=n_xo, replace=False)) if n_xo else np.zeros(0, np.int64)
    wo = np.sort(r_out.choice(K, size=n_wo, replace=False)) if n_wo else np.zeros(0, np.int64)

    x_bits = x = None
    if with_x:
        rows = M if m_rows is None else min(m_rows, M)
        xf = _draw_x(spec, r_x, rows, xo)
        x_bits = bf16_bits(xf.astype(np.float32))
        x = bf16_value(x_bits)

    w = r_w.standard_normal((K, N), dtype=np.float64) * (1.0 / math.sqrt(K))
    if n_wo:
        w[wo, :] *= spec.w_outlier_scale
    w_lin = np.ascontiguousarray(w.T.astype(np.float32))
    bias = round_to_bf16(r_b.standard_normal(N).astype(np.float32) * np.float32(0.1))
    return Layer(spec, x_bits, x, w_lin, bias, xo, wo)


def calibration_rows(spec: LayerSpec, rows: int) -> np.ndarray:
    """`rows` held-out activation rows of the layer's distribution (the same
    outlier channels, drawn from the layer's spare stream), bf16 values as
    float32: calibration data for a layer whose own batch is a few rows."""
    r_out, _, _, _, r_spare = _streams(spec)
    n_xo = int(round(spec.x_outlier_frac * spec.K))
    xo = np.sort(r_out.choice(spec.K, size=n_xo, replace=False)) if n_xo else np.zeros(0, np.int64)
    return bf16_value(bf16_bits(_draw_x(spec, r_spare, rows, xo).astype(np.float32)))


def awq_layers() -> list[LayerSpec]:
    """FLUX-shaped adaptive-normalization and modulation linears (the pages'
    W4A16 layers), batch 2: a double-stream block's per-stream modulation
    3072 -> 6 x 3072, a single-stream block's 3072 -> 3 x 3072, the final
    norm's 3072 -> 2 x 3072, and the double-stream one at 16 rows. Inputs
    are SiLU(2 N(0,1)) (a conditioning vector after its SiLU) with 1% of
    channels x8; weights N(0, 1/K), no outlier rows."""
    kw = dict(x_kind="silu", x_outlier_frac=0.01, x_outlier_scale=8.0, w_outlier_frac=0.0)
    return [_layer("mod_double", 2, 3072, 18432, 0, "w4a16", 5, **kw),
            _layer("mod_single", 2, 3072, 9216, 0, "w4a16", 6, **kw),
            _layer("norm_out", 2, 3072, 6144, 0, "w4a16", 7, **kw),
            _layer("mod_double_m16", 16, 3072, 18432, 0, "w4a16", 5, **kw)]


def ragged_spec(name: str, M: int, K: int, N: int, rank: int, fmt: str, seed: int) -> LayerSpec:
    """Extra (non-config) shapes for edge-case tests, same distributions as config 0."""
    return LayerSpec(name=name, M=M, K=K, N=N, rank=rank, fmt=fmt, seed=seed)
