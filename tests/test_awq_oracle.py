"""Pins of the AWQ-style W4A16 oracle (oracle/awq_oracle.py) against brute
force, closed forms and invariants (no GPU needed)."""
import math

import numpy as np
import pytest

from bit_svdquant_diffusion_amd import synth
from oracle import awq_oracle as A

F32 = np.float32


def _brute_group(vals):
    """One group by scalar float32 steps: (codes, scale, zero)."""
    mx = max(F32(v) for v in vals)
    mn = min(F32(v) for v in vals)
    rng = F32(mx - mn)
    scale = F32(max(rng, F32(1e-5)) / F32(15.0))
    zf = -float(np.rint(F32(mn / scale)))
    zero = min(15.0, max(0.0, zf))
    codes = []
    for v in vals:
        t = float(np.rint(F32(F32(v) / scale))) + zero
        codes.append(int(min(15.0, max(0.0, t))))
    return codes, scale, int(zero)


def test_quantize_groups_brute():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((5, 256)) * np.exp2(rng.integers(-3, 4, (5, 1)))).astype(np.float32)
    w[2, :128] = np.abs(w[2, :128]) + 0.5          # all positive: zero point clipped at 0
    w[3, 128:] = -np.abs(w[3, 128:]) - 0.5         # all negative: zero point clipped at 15
    w[4, :128] = 0.25                              # constant group: range below 1e-5
    q, sc, z = A.quantize_groups(w)
    for n in range(5):
        for g in range(2):
            codes, s, zz = _brute_group(w[n, 128 * g:128 * (g + 1)].tolist())
            assert sc[n, g] == s and z[n, g] == zz
            assert q[n, 128 * g:128 * (g + 1)].tolist() == codes
    assert z[2, 0] == 0 and z[3, 1] == 15
    assert q.min() >= 0 and q.max() <= 15


def test_quantize_exact_grid_reconstructs():
    """A group laid out exactly on a 4-bit grid (min at code 0, max at 15)
    comes back unchanged: q, the zero point and the dequantized values."""
    scale, zero = F32(0.125), 6
    codes = np.arange(128) % 16
    codes[0], codes[1] = 0, 15
    w = (scale * (codes.astype(np.float32) - zero)).astype(np.float32)[None, :]
    q, sc, z = A.quantize_groups(w)
    assert sc[0, 0] == scale and z[0, 0] == zero and np.array_equal(q[0], codes)
    assert np.array_equal(A.dequantize(q, sc, z), w)


def test_rounding_error_bound_and_scale_invariance():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((8, 384)).astype(np.float32)
    q, sc, z = A.quantize_groups(w)
    d = A.dequantize(q, sc, z)
    err = np.abs(d - w).reshape(8, 3, 128)
    assert np.all(err <= sc[..., None] * 0.5 * (1 + 1e-5) + 1e-7)
    # a power-of-two factor scales the scales and keeps codes and zero points
    q2, sc2, z2 = A.quantize_groups(w * F32(4.0))
    assert np.array_equal(q2, q) and np.array_equal(z2, z) and np.array_equal(sc2, sc * F32(4.0))


def test_channel_scales_closed_forms():
    a = np.array([0.5, 2.0, 8.0, 0.0])
    assert np.array_equal(A.channel_scales(a, 0.0), np.ones(4))
    s = A.channel_scales(a, 0.5)
    # s_k = sqrt(max(a_k, 1e-4)) / sqrt(max s min s): geometric middle at 1
    raw = np.sqrt(np.maximum(a, 1e-4))
    np.testing.assert_allclose(s, raw / math.sqrt(raw.max() * raw.min()), rtol=1e-15)
    assert abs(s.max() * s.min() - 1.0) < 1e-12


def _small_layer(seed=3, K=256, N=48):
    spec = synth.LayerSpec("awq_t", 2, K, N, 0, "w4a16", seed, x_kind="silu", x_outlier_frac=0.02,
                           x_outlier_scale=8.0, w_outlier_frac=0.0)
    return spec, synth.make_layer(spec), synth.calibration_rows(spec, 24)


def test_alpha_search_is_the_grid_argmin():
    """The pack's alpha is the first minimum of the loss over the 20-point
    grid, each loss recomputed here by a scalar-free but separate route
    (residual of the dequantized, unscaled weight against W)."""
    spec, lay, xc = _small_layer()
    p = A.pack(lay.w_lin, lay.bias, xc)
    a = np.abs(xc.astype(np.float64)).mean(axis=0)
    mine = []
    for al in A.ALPHA_GRID:
        s, inv_s, q, sc, z = A.candidate(lay.w_lin, a, al)
        w_eff = A.dequantize(q, sc, z).astype(np.float64) * inv_s.astype(np.float64)[None, :]
        e = xc.astype(np.float64) @ (w_eff - lay.w_lin.astype(np.float64)).T
        mine.append(float(np.sum(e * e)))
    mine = np.array(mine)
    np.testing.assert_allclose(p["losses"], mine, rtol=1e-9)
    assert p["alpha"] == A.ALPHA_GRID[int(np.argmin(mine))]
    # the kept quantization is the one of that grid point
    _, inv_s, q, sc, z = A.candidate(lay.w_lin, a, p["alpha"])
    assert np.array_equal(p["q"], q) and np.array_equal(p["scale"], sc) and np.array_equal(p["inv_s"], inv_s)


def test_activation_awareness_helps_on_outliers():
    """On inputs with outlier channels the search does better than plain
    round-to-nearest (alpha = 0, s = 1), which it also considered."""
    spec, lay, xc = _small_layer(seed=4, K=512, N=64)
    p = A.pack(lay.w_lin, lay.bias, xc)
    assert p["losses"][0] > 1.02 * p["losses"].min()
    assert p["alpha"] > 0


def test_forward_brute():
    spec, lay, xc = _small_layer(seed=5, K=128, N=8)
    p = A.pack(lay.w_lin, lay.bias, xc, alpha=0.5)
    y = A.forward(p, lay.x)
    for m in range(lay.x.shape[0]):
        for n in range(8):
            acc = float(lay.bias[n])
            for k in range(128):
                xh = F32(F32(lay.x[m, k]) * p["inv_s"][k])
                w = F32(p["scale"][n, 0] * F32(float(p["q"][n, k]) - float(p["zero"][n, 0])))
                acc += float(xh) * float(w)
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_no_scaling_no_quant_error_limit():
    """With alpha = 0 and weights on the 4-bit grid the layer is exact: y = x W^T + b."""
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 16, (16, 256))
    codes[:, ::128] = 0
    codes[:, 1::128] = 15
    w = (F32(0.03125) * (codes - 7)).astype(np.float32)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    p = A.pack(w, None, x, alpha=0.0)
    np.testing.assert_allclose(A.forward(p, x), x.astype(np.float64) @ w.T.astype(np.float64), rtol=0, atol=1e-12)
