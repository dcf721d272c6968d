"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test ties the oracle to brute force, a closed form, an invariant of the
method or a textbook identity, so that a dropped term, a wrong sign, a wrong
index or a transposed operand anywhere in it fails at least one test.
"""
import math

import numpy as np
import pytest

from oracle import brute
from oracle import svdq_oracle as O
from bit_svdquant_diffusion_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _tiny(M=8, K=64, N=16, seed=5, fmt="int4", outlier=True):
    spec = synth.LayerSpec("t", M, K, N, 0, fmt, seed,
                           x_outlier_frac=0.05 if outlier else 0.0,
                           w_outlier_frac=0.05 if outlier else 0.0)
    return synth.make_layer(spec)


# --------------------------------------------------------------------------
# brute force agreement (independent scalar loops)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
@pytest.mark.parametrize("shape", [(4, 64, 8, 0), (5, 128, 12, 4), (3, 64, 16, 16)])
def test_brute_matches_oracle(fmt, shape):
    M, K, N, r = shape
    lay = _tiny(M, K, N, seed=11 + r, fmt=fmt)
    ax = np.abs(lay.x).max(axis=0)
    p = O.pack(lay.w_lin, lay.bias, ax, r, fmt)
    bp = brute.pack(lay.w_lin.tolist(), lay.bias.tolist(), ax.tolist(),
                    p["l1"].tolist(), p["l2"].tolist(), fmt)
    assert np.array_equal(np.array(bp["mu"], np.float32), p["mu"])
    assert np.array_equal(np.array(bp["R"], np.float32), p["r"])
    assert np.array_equal(np.array(bp["codes"]), p["qw"].astype(np.int64) if fmt == "int4"
                          else p["qw"].astype(np.int64))
    assert np.array_equal(np.array(bp["scales"], dtype=p["sw"].dtype), p["sw"])
    y, parts = O.forward(p, lay.x, return_parts=True)
    by, bxc, bxs, bz = brute.forward(bp, lay.x.tolist())
    assert np.array_equal(np.array(bxc), parts["qx"].astype(np.int64))
    assert np.array_equal(np.array(bxs, dtype=parts["sx"].dtype), parts["sx"])
    np.testing.assert_allclose(np.array(by), y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
    if r:
        np.testing.assert_allclose(np.array(bz), parts["z"], rtol=1e-12, atol=1e-12)


def test_brute_bf16_round_matches():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(2000) * np.exp2(rng.integers(-20, 20, 2000))
    ours = O.to_bf16(v)
    ref = np.array([brute.bf16_round(float(t)) for t in v], dtype=np.float64)
    assert np.array_equal(ours.astype(np.float64), ref)
    # bf16 values keep only the top 16 bits of their float32 pattern
    assert np.all((ours.view(np.uint32) & 0xFFFF) == 0)
    # ties: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert O.to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert O.to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6


def test_bf16_round_bits_every_exponent():
    """to_bf16 of float32 values equals round-to-nearest-even of the float32 bit
    pattern to its top 16 bits (integer arithmetic on the bits, a separate
    formulation that holds for subnormals and at the overflow edge): over every
    bf16 value, the midpoints between neighbours and random patterns, including
    the subnormals below 2^-126, whose spacing is 2^-133."""
    rng = np.random.default_rng(4)
    hi = np.arange(0, 0x7F80, dtype=np.uint32)                # every finite positive bf16
    pats = np.concatenate([hi << 16, (hi << 16) | 0x8000, (hi << 16) | 0x7FFF, (hi << 16) | 0x8001,
                           rng.integers(0, 0x7F800000, 200000, dtype=np.uint32)])
    pats = np.concatenate([pats, pats | 0x80000000])
    u = pats.astype(np.uint64)
    want = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
    got = O.to_bf16(pats.view(np.float32))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # the smallest subnormal, its half (a tie: to zero) and the largest subnormal
    assert O.to_bf16(np.array([2.0 ** -133]))[0] == np.float32(2.0 ** -133)
    assert O.to_bf16(np.array([2.0 ** -134]))[0] == 0.0
    assert O.to_bf16(np.array([3 * 2.0 ** -135]))[0] == np.float32(2.0 ** -133)
    assert O.to_bf16(np.array([127 * 2.0 ** -133]))[0] == np.float32(127 * 2.0 ** -133)
    v = rng.standard_normal(2000) * np.exp2(rng.integers(-140, -120, 2000))
    ref = np.array([brute.bf16_round(float(t)) for t in v], dtype=np.float64)
    assert np.array_equal(O.to_bf16(v).astype(np.float64), ref)


# --------------------------------------------------------------------------
# quantizer definitions: ties, ranges, error bounds, scale invariance
# --------------------------------------------------------------------------
def test_int4_ties_round_half_even():
    g = np.zeros(64, np.float32)
    g[0] = 7.0                      # amax 7 -> s = 1 exactly
    vals = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 4.5, 5.5, 6.5, 0.49999997]
    g[1:1 + len(vals)] = vals
    q, s = O.quant_int4_rows(g[None, :])
    assert s[0, 0] == 1.0
    assert list(q[0, 1:1 + len(vals)]) == [0, 2, 2, 4, 0, -2, -2, -4, 4, 6, 6, 0]
    assert q[0, 0] == 7


def test_int4_exact_quotient_not_float_division():
    # a value whose float32 quotient rounds onto the half-integer while the
    # exact quotient lies just below it: RNE of the exact quotient must win.
    rng = np.random.default_rng(0)
    found = 0
    for _ in range(200000):
        amax = np.float32(rng.uniform(0.5, 2.0))
        s = np.float32(amax / np.float32(7))
        k = rng.integers(0, 7)
        x = np.float32((k + 0.5) * float(s))
        for cand in (x, np.nextafter(x, np.float32(0)), np.nextafter(x, np.float32(10))):
            exact = float(cand) / float(s)
            f32q = float(np.float32(cand) / s)
            if f32q == k + 0.5 and exact != k + 0.5:
                g = np.zeros(64, np.float32)
                g[0], g[1] = amax, cand
                q, _ = O.quant_int4_rows(g[None, :])
                want = k if exact < k + 0.5 else k + 1
                assert q[0, 1] == want
                found += 1
        if found >= 3:
            break
    assert found >= 1


def subnormal_tie_pairs(limit: int = 64):
    """bf16 pairs (amax, v) whose INT4 scale s = fl32(amax / 7) is subnormal and
    for which v - (k + 1/2) s is exactly +-2^-150 (k = floor(v / s)): the
    quotient lies as close to a half-integer as these scales allow. Found by
    walking the bf16 values below 2^-120 with exact rational arithmetic."""
    from fractions import Fraction
    bits = np.arange(1, 0x0780, dtype=np.uint32) << 16           # positive bf16 below 2^-120
    vals = bits.view(np.float32)
    pairs = []
    for amax in vals:
        s = np.float32(amax / np.float32(7.0))
        if s == 0 or s >= np.float32(2.0 ** -125):
            continue
        S = Fraction(float(s))
        for k in range(7):
            mid = (k + Fraction(1, 2)) * S
            b = int(np.array([O.to_bf16(np.array([float(mid)], np.float32))[0]], np.float32).view(np.uint32)[0]) >> 16
            for cb in (max(b - 1, 0), b, b + 1):         # the bf16 values around (k + 1/2) s
                c = np.array([cb << 16], np.uint32).view(np.float32)[0]
                if 0 < c <= amax and abs(Fraction(float(c)) - mid) == Fraction(1, 2 ** 150):
                    pairs.append((np.float32(amax), np.float32(c)))
        if len(pairs) >= limit:
            break
    return sorted(set(pairs))


def test_int4_subnormal_scales_exact():
    # subnormal scales: RNE of the exact quotient, checked with rationals, at
    # the pairs whose quotient is closest to a half-integer
    from fractions import Fraction
    pairs = subnormal_tie_pairs()
    assert len(pairs) >= 16
    ups = downs = 0
    for amax, v in pairs:
        g = np.zeros(64, np.float32)
        g[0], g[1], g[2] = amax, v, -v
        q, s = O.quant_int4_rows(g[None, :])
        assert s[0, 0] == np.float32(amax / np.float32(7.0)) and s[0, 0] < 2.0 ** -126
        e = Fraction(float(v)) / Fraction(float(s[0, 0]))
        k = int(e)
        want = k + 1 if e - k > Fraction(1, 2) else k
        assert q[0, 1] == want and q[0, 2] == -want, (amax, v)
        ups += want == k + 1
        downs += want == k
    assert ups > 0 and downs > 0


def test_int4_ranges_and_error_bound():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((64, 512)) * np.exp2(rng.integers(-8, 8, (64, 1)))).astype(np.float32)
    v[3, 64:128] = 0.0
    q, s = O.quant_int4_rows(v)
    assert q.min() >= -7 and q.max() <= 7
    g = q.reshape(64, 8, 64)
    amax_code = np.abs(g).max(axis=-1)
    assert amax_code[3, 1] == 0 and s[3, 1] == 0
    nz = s > 0
    assert np.all(amax_code[nz] == 7)            # every nonzero group reaches +-7
    err = np.abs(v.reshape(64, 8, 64).astype(np.float64) - g * s[..., None].astype(np.float64))
    assert np.all(err <= 0.5 * s[..., None].astype(np.float64) * (1 + 1e-6) + 0)


def test_int4_scale_invariance():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((16, 256)).astype(np.float32)
    q0, s0 = O.quant_int4_rows(v)
    for j in (-3, 1, 5):
        q1, s1 = O.quant_int4_rows(v * np.float32(2.0 ** j))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, s0 * np.float32(2.0 ** j))


E2M1_TIES = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
             (7.0, 7), (6.0, 7), (100.0, 7), (0.2, 0), (0.3, 1), (2.6, 5), (5.01, 7)]


@pytest.mark.parametrize("v,code", E2M1_TIES)
def test_e2m1_tie_table(v, code):
    assert O.e2m1_encode(np.array([v]))[0] == code
    assert O.e2m1_encode(np.array([-v]))[0] == code | 8
    assert brute.e2m1_code(v) == code


def test_e2m1_decode_grid_and_roundtrip():
    vals = O.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(vals[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.array_equal(O.e2m1_encode(vals[:8]), np.arange(8))


def test_e2m1_nearest_exhaustive_sweep():
    # every float32 in [0, 8) on a fine sweep: the chosen grid point is the nearest
    rng = np.random.default_rng(4)
    v = np.concatenate([np.linspace(0, 8, 200001, dtype=np.float32),
                        rng.uniform(0, 8, 100000).astype(np.float32)])
    codes = O.e2m1_encode(v.astype(np.float64))
    got = O.e2m1_decode(codes)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    best = np.abs(v[:, None].astype(np.float64) - grid).min(axis=1)
    assert np.all(np.abs(got - v) <= best + 0.0)
    assert np.all(np.abs(got - v)[v <= 6] <= 1.0)


def test_mx_exponent_definition():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((32, 256)) * np.exp2(rng.integers(-30, 30, (32, 1)))).astype(np.float32)
    codes, sb = O.quant_mxfp4_rows(v)
    amax = np.abs(v.reshape(32, 8, 32)).max(axis=-1).astype(np.float64)
    scaled_max = amax / np.exp2(sb.astype(np.float64) - 127)
    assert np.all((scaled_max >= 4.0) & (scaled_max < 8.0))     # block max lands in [4, 8)
    mags = np.abs(O.e2m1_decode(codes)).reshape(32, 8, 32).max(axis=-1)
    assert np.all((mags == 4.0) | (mags == 6.0))                 # block max code is 4 or 6
    # powers of two: amax = 2^j -> e = j - 2
    for j in (-10, 0, 3):
        assert O.e8m0_exponent(np.array([2.0 ** j]))[0] == j - 2
        assert O.e8m0_exponent(np.array([np.nextafter(np.float32(2.0 ** j), np.float32(0))]))[0] == j - 3
    assert O.e8m0_exponent(np.array([0.0]))[0] == -127


def test_mx_scale_invariance():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((8, 128)).astype(np.float32)
    c0, s0 = O.quant_mxfp4_rows(v)
    c1, s1 = O.quant_mxfp4_rows(v * np.float32(8.0))
    assert np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + 3)


# --------------------------------------------------------------------------
# smoothing: undone exactly; SVD: Eckart-Young via the Gram eigenvalues
# --------------------------------------------------------------------------
def test_smoothing_is_undone():
    lay = _tiny(16, 128, 24, seed=7)
    ax = np.abs(lay.x).max(axis=0)
    lam, mu = O.smoothing_factors(ax, lay.w_lin)
    # lambda balances the two maxima: max|X_hat_k| == max|W_hat_k| (up to rounding)
    xh = O.smooth_activations(lay.x, mu).astype(np.float64)
    wh = O.smoothed_weight(lay.w_lin, mu)
    np.testing.assert_allclose(np.abs(xh).max(0), np.abs(wh).max(1), rtol=1e-6)
    # x_hat / mu reproduces x within one float32 rounding
    back = xh / mu.astype(np.float64)
    np.testing.assert_allclose(back, lay.x, rtol=2 ** -23, atol=0)
    # X_hat W_hat == X W (float64 rounding only; the float32 x*mu rounding is the only loss)
    ref = lay.x.astype(np.float64) @ lay.w_lin.T.astype(np.float64)
    np.testing.assert_allclose(xh @ wh, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


def test_smoothing_zero_channels():
    w = np.ones((4, 64), np.float32)
    w[:, 5] = 0
    ax = np.ones(64, np.float32) * 4
    ax[7] = 0
    lam, mu = O.smoothing_factors(ax, w)
    assert lam[5] == 1 and lam[7] == 1 and lam[0] == 2.0 and mu[0] == np.float32(0.5)


@pytest.mark.parametrize("r", [1, 4, 16])
def test_eckart_young(r):
    lay = _tiny(8, 128, 96, seed=8)
    ax = np.abs(lay.x).max(axis=0)
    _, mu = O.smoothing_factors(ax, lay.w_lin)
    wh = O.smoothed_weight(lay.w_lin, mu)
    l1, l2 = O.low_rank_factors(wh, r, round_bf16=False)
    err = np.sum((wh - l1 @ l2) ** 2)
    ev = np.sort(np.linalg.eigvalsh(wh.T @ wh))[::-1]      # sigma^2, a different routine
    tail = ev[r:].sum()
    assert abs(err - tail) <= 1e-8 * np.sum(ev)
    # the top-r part is the one kept (a wrong slice would leave more error)
    assert err < np.sum(wh ** 2) - ev[:r].sum() * (1 - 1e-9) + 1e-9


def test_full_rank_no_quant_is_exact_linear():
    lay = _tiny(12, 64, 40, seed=9)
    ax = np.abs(lay.x).max(axis=0)
    p = O.pack(lay.w_lin, lay.bias, ax, 40, "none", round_bf16=False)
    y = O.forward(p, lay.x)
    ref = lay.x.astype(np.float64) @ lay.w_lin.T.astype(np.float64) + lay.bias
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())
    assert np.abs(p["r"]).max() < 1e-10


def test_rank0_reduces_to_plain_w4a4():
    lay = _tiny(10, 128, 24, seed=10)
    ax = np.abs(lay.x).max(axis=0)
    for fmt in ("int4", "mxfp4"):
        p = O.pack(lay.w_lin, lay.bias, ax, 0, fmt)
        _, mu = O.smoothing_factors(ax, lay.w_lin)
        assert np.array_equal(p["r"], O.smoothed_weight(lay.w_lin, mu).T.astype(np.float32))
        y, parts = O.forward(p, lay.x, return_parts=True)
        assert np.all(parts["y_lr"] == 0)
        # written out directly: sum over k of dequantized codes, plus bias
        xh = O.smooth_activations(lay.x, mu)
        if fmt == "int4":
            qx, sx = O.quant_int4_rows(xh)
            qw, sw = O.quant_int4_rows(p["r"])
            P = O.int4_group_sums(qx, qw)
            ref = np.einsum("mg,ng,mng->mn", sx.astype(np.float64), sw.astype(np.float64), P)
        else:
            ref = O.dequant_mxfp4(*O.quant_mxfp4_rows(xh)) @ O.dequant_mxfp4(*O.quant_mxfp4_rows(p["r"])).T
        np.testing.assert_allclose(y - lay.bias, ref, rtol=1e-12, atol=1e-12)


def test_int4_group_sums_brute():
    rng = np.random.default_rng(12)
    qx = rng.integers(-7, 8, (5, 192)).astype(np.int8)
    qw = rng.integers(-7, 8, (7, 192)).astype(np.int8)
    P = O.int4_group_sums(qx, qw)
    for m in range(5):
        for n in range(7):
            for g in range(3):
                assert P[m, n, g] == sum(int(qx[m, k]) * int(qw[n, k]) for k in range(64 * g, 64 * g + 64))
    ext = np.full((1, 64), 7, np.int8)
    assert O.int4_group_sums(ext, -ext)[0, 0, 0] == -3136


def test_residual_order_is_fixed():
    # residual = W_hat - sum_i l1_i l2_i taken term by term in float64
    rng = np.random.default_rng(13)
    wh = rng.standard_normal((64, 32))
    l1 = O.to_bf16(rng.standard_normal((64, 4)))
    l2 = O.to_bf16(rng.standard_normal((4, 32)))
    R = O.residual(wh, l1, l2)
    for k in (0, 17, 63):
        for n in (0, 31):
            acc = 0.0
            for i in range(4):
                acc = acc + float(l1[k, i]) * float(l2[i, n])
            assert R[k, n] == np.float32(wh[k, n] - acc)


def test_method_sanity_lowrank_helps():
    """On outlier-heavy data the rank-32 branch reduces the error against X W + b."""
    spec = synth.LayerSpec("s", 128, 512, 256, 32, "int4", 21)
    lay = synth.make_layer(spec)
    ax = np.abs(lay.x).max(axis=0)
    ref = lay.x.astype(np.float64) @ lay.w_lin.T.astype(np.float64) + lay.bias
    errs = {}
    for r in (0, 32):
        p = O.pack(lay.w_lin, lay.bias, ax, r, "int4")
        errs[r] = np.linalg.norm(O.forward(p, lay.x) - ref) / np.linalg.norm(ref)
    assert errs[32] < errs[0]


def test_dequant_identity_blockwise():
    """Y4 from per-group int sums times scale products equals dequant(X) dequant(W)^T."""
    lay = _tiny(6, 256, 10, seed=14)
    ax = np.abs(lay.x).max(axis=0)
    p = O.pack(lay.w_lin, lay.bias, ax, 4, "int4")
    _, parts = O.forward(p, lay.x, return_parts=True)
    P = O.int4_group_sums(parts["qx"], p["qw"])
    y4 = np.einsum("mg,ng,mng->mn", parts["sx"].astype(np.float64), p["sw"].astype(np.float64), P)
    np.testing.assert_allclose(parts["y_q"], y4, rtol=1e-12, atol=1e-13)


def test_generator_recipe():
    spec = synth.config_layers(0)[0]
    lay = synth.make_layer(spec)
    assert lay.x.shape == (256, 512) and lay.w_lin.shape == (512, 512)
    assert len(lay.x_outlier_channels) == round(0.01 * 512)
    assert len(lay.w_outlier_rows) == round(0.02 * 512)
    # bf16 inputs: low 16 bits of every float32 pattern are zero
    assert np.all((lay.x.view(np.uint32) & 0xFFFF) == 0)
    assert np.all((lay.bias.view(np.uint32) & 0xFFFF) == 0)
    # seeded: same draw twice; first rows of a full draw equal a partial draw
    lay2 = synth.make_layer(spec, m_rows=16)
    assert np.array_equal(lay2.x, lay.x[:16]) and np.array_equal(lay2.w_lin, lay.w_lin)


def test_sigma_goes_into_l1():
    """The singular values ride in L1, not L2: before bf16 rounding the rows of
    L2 are orthonormal and the columns of L1 have the singular values as
    norms (taken here from the Gram matrix's eigenvalues, not from the SVD);
    L1 = W_hat L2^T, the projection of W_hat onto the kept right singular
    vectors. Moving Sigma into L2, splitting it, or transposing a factor
    fails one of these."""
    lay = _tiny(8, 128, 96, seed=31)
    ax = np.abs(lay.x).max(axis=0)
    _, mu = O.smoothing_factors(ax, lay.w_lin)
    wh = O.smoothed_weight(lay.w_lin, mu)
    r = 12
    l1, l2 = O.low_rank_factors(wh, r, round_bf16=False)
    assert l1.shape == (128, r) and l2.shape == (r, 96)
    np.testing.assert_allclose(l2 @ l2.T, np.eye(r), atol=1e-12)
    sig = np.sqrt(np.sort(np.linalg.eigvalsh(wh.T @ wh))[::-1][:r])
    np.testing.assert_allclose(np.linalg.norm(l1, axis=0), sig, rtol=1e-10)
    np.testing.assert_allclose(l1, wh @ l2.T, rtol=0, atol=1e-12 * np.abs(l1).max())
    # the bf16 factors are the roundings of these
    b1, b2 = O.low_rank_factors(wh, r)
    assert np.array_equal(b1, O.to_bf16(l1)) and np.array_equal(b2, O.to_bf16(l2))


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_brute_matches_oracle_config0(fmt):
    """Brute force on the tiny configuration (256 x 512 -> 512, rank 16): the
    whole pack (smoothing factors, residual, weight codes and scales), and the
    forward on a sample of token rows (rows are independent in every step)."""
    spec = synth.config_layers(0)[0]
    lay = synth.make_layer(spec)
    ax = np.abs(lay.x).max(axis=0)
    p = O.pack(lay.w_lin, lay.bias, ax, spec.rank, fmt)
    bp = brute.pack(lay.w_lin.tolist(), lay.bias.tolist(), ax.tolist(),
                    p["l1"].tolist(), p["l2"].tolist(), fmt)
    assert np.array_equal(np.array(bp["mu"], np.float32), p["mu"])
    assert np.array_equal(np.array(bp["R"], np.float32), p["r"])
    assert np.array_equal(np.array(bp["codes"]), p["qw"].astype(np.int64))
    assert np.array_equal(np.array(bp["scales"], dtype=p["sw"].dtype), p["sw"])
    rows = np.array([0, 1, 77, 128, 255])
    y, parts = O.forward(p, lay.x[rows], return_parts=True)
    by, bxc, bxs, bz = brute.forward(bp, lay.x[rows].tolist())
    assert np.array_equal(np.array(bxc), parts["qx"].astype(np.int64))
    assert np.array_equal(np.array(bxs, dtype=parts["sx"].dtype), parts["sx"])
    np.testing.assert_allclose(np.array(bz), parts["z"], rtol=1e-12, atol=1e-12 * np.abs(parts["z"]).max())
    np.testing.assert_allclose(np.array(by), y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


# --------------------------------------------------------------------------
# LoRA without re-quantization
# --------------------------------------------------------------------------
def _pow2_smoothed_layer(K=128, N=48, rank=16, fmt="int4", seed=33):
    """A packed layer whose smoothing factors are exact powers of two (the
    calibration maxima are max|W_k| times 4^j, so lambda_k = 2^j exactly)."""
    lay = _tiny(6, K, N, seed=seed, fmt=fmt)
    aw = np.abs(lay.w_lin).max(axis=0).astype(np.float64)
    j = (np.arange(K) % 5) - 2
    ax = (aw * 4.0 ** j).astype(np.float32)
    assert np.array_equal(ax.astype(np.float64), aw * 4.0 ** j)   # exact in float32
    p = O.pack(lay.w_lin, lay.bias, ax, rank, fmt)
    assert np.array_equal(p["mu"].astype(np.float64), 2.0 ** -j)
    return lay, p


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_lora_extend_adds_scaled_adapter_exactly(fmt):
    """With power-of-two smoothing, bf16 adapter factors and a power-of-two
    scale, every bf16 rounding in the extension is exact, so the extended
    layer's output minus the base layer's is scale * X A B to float64
    rounding, on any input; the residual's codes and scales, mu and the bias
    are untouched. A wrong side of mu (diag(mu) instead of diag(1/mu)), a
    dropped scale or a transposed factor fails this."""
    lay, p = _pow2_smoothed_layer(fmt=fmt)
    rng = np.random.default_rng(4)
    ra = 16
    A = O.to_bf16(rng.standard_normal((128, ra)) * 0.1)
    B = O.to_bf16(rng.standard_normal((ra, 48)) * 0.1)
    ext = O.lora_extend(p, A, B, 0.5)
    assert ext["rank"] == p["rank"] + ra and ext["l1"].shape == (128, p["rank"] + ra)
    assert np.array_equal(ext["l1"][:, :p["rank"]], p["l1"]) and np.array_equal(ext["l2"][:p["rank"]], p["l2"])
    for key in ("qw", "sw", "mu", "bias", "r"):
        assert np.array_equal(ext[key], p[key]), key
    x = rng.standard_normal((9, 128)).astype(np.float32)
    d = O.forward(ext, x) - O.forward(p, x)
    want = 0.5 * (x.astype(np.float64) @ A.astype(np.float64)) @ B.astype(np.float64)
    np.testing.assert_allclose(d, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_lora_extend_general_within_bf16():
    """General smoothing and fp32 adapter factors: the added output is
    scale * X A B up to the bf16 rounding of the two new factors."""
    lay = _tiny(16, 256, 64, seed=35)
    ax = np.abs(lay.x).max(axis=0)
    p = O.pack(lay.w_lin, lay.bias, ax, 16, "int4")
    rng = np.random.default_rng(5)
    A = (rng.standard_normal((256, 32)) / 16).astype(np.float32)
    B = (rng.standard_normal((32, 64)) / 4).astype(np.float32)
    ext = O.lora_extend(p, A, B, 0.75)
    d = O.forward(ext, lay.x) - O.forward(p, lay.x)
    want = 0.75 * (lay.x.astype(np.float64) @ A) @ B
    err = np.linalg.norm(d - want) / np.linalg.norm(want)
    assert err < 2 ** -7, err
    # the appended L1 columns are bf16 of A * scale / mu, row by row
    k = 17
    assert np.array_equal(ext["l1"][k, 16:], O.to_bf16(A[k].astype(np.float64) * 0.75 / float(p["mu"][k])))


# --------------------------------------------------------------------------
# calibrated smoothing strength
# --------------------------------------------------------------------------
def test_smoothing_alpha_closed_forms():
    """alpha = 1/2 is the default rule bit for bit; alpha = 1 moves all of
    each channel's activation range into the weights (max |x_hat| = 1);
    alpha = 0 scales the weights' rows to max 1 (max |W_hat| = 1)."""
    lay = _tiny(16, 128, 24, seed=41)
    ax = np.abs(lay.x).max(axis=0)
    assert np.array_equal(O.smoothing_factors_alpha(ax, lay.w_lin, 0.5)[1], O.smoothing_factors(ax, lay.w_lin)[1])
    _, mu1 = O.smoothing_factors_alpha(ax, lay.w_lin, 1.0)
    xh = O.smooth_activations(lay.x, mu1)
    np.testing.assert_allclose(np.abs(xh).max(axis=0), 1.0, rtol=2 ** -22)
    _, mu0 = O.smoothing_factors_alpha(ax, lay.w_lin, 0.0)
    wh = O.smoothed_weight(lay.w_lin, mu0)
    np.testing.assert_allclose(np.abs(wh).max(axis=1), 1.0, rtol=2 ** -22)
    # the strengths in between lie between, channel by channel (monotone in alpha)
    lam = [O.smoothing_factors_alpha(ax, lay.w_lin, a)[0] for a in (0.0, 0.25, 0.5, 0.75, 1.0)]
    aw = np.abs(lay.w_lin).max(axis=0).astype(np.float64)
    up = ax.astype(np.float64) * aw >= 1.0
    for a, b in zip(lam, lam[1:]):
        assert np.all((b >= a * (1 - 1e-12))[up]) and np.all((b <= a * (1 + 1e-12))[~up])


def test_calibrate_alpha_is_the_argmin():
    """The kept alpha is the grid's first least loss, each loss recomputed
    here from the kept pieces by a separate route: the dequantized weight
    plus the low-rank product, applied to the smoothed rows."""
    spec = synth.LayerSpec("cal", 48, 256, 64, 16, "int4", 44)
    lay = synth.make_layer(spec)
    grid = [0.3, 0.5, 0.7]
    res = O.calibrate_alpha(lay.w_lin, lay.bias, lay.x, 16, "int4", grid)
    assert res["alpha"] == grid[int(np.argmin(res["losses"]))]
    p = res["packed"]
    xh = O.smooth_activations(lay.x, p["mu"]).astype(np.float64)
    qx, sx = O.quant_int4_rows(xh.astype(np.float32))
    w_eff = (O.dequant_int4(p["qw"], p["sw"]).T, p["l1"].astype(np.float64) @ p["l2"].astype(np.float64))
    y = O.dequant_int4(qx, sx) @ w_eff[0] + xh @ w_eff[1] + lay.bias.astype(np.float64)
    ref = lay.x.astype(np.float64) @ lay.w_lin.T.astype(np.float64) + lay.bias
    np.testing.assert_allclose(np.sum((y - ref) ** 2), res["losses"].min(), rtol=1e-9)


# --------------------------------------------------------------------------
# GELU and the two-layer MLP composition
# --------------------------------------------------------------------------
def test_gelu_closed_forms():
    """GELU(v) = v Phi(v): Phi at 1, 2, -3 and -10 (tabulated normal
    distribution values), the odd part v/2 (Phi(v) + Phi(-v) = 1), the even
    part's curvature 1/sqrt(2 pi) at 0, and zero at zero."""
    table = {1.0: 0.8413447460685429486, 2.0: 0.9772498680518207928, -3.0: 0.0013498980316300945267,
             -10.0: 7.6198530241605260660e-24}
    for v, phi in table.items():
        got = float(O.gelu(np.array([v]))[0])
        assert abs(got - v * phi) <= 1e-13 * abs(v * phi), (v, got)
    assert O.gelu(np.array([0.0]))[0] == 0.0
    rng = np.random.default_rng(8)
    v = rng.standard_normal(1000) * 3
    np.testing.assert_allclose(O.gelu(v) - O.gelu(-v), v, rtol=1e-14, atol=1e-15)
    h = 1e-3
    even = (O.gelu(np.array([h])) + O.gelu(np.array([-h])))[0] / 2
    assert abs(even / (h * h) - 1.0 / math.sqrt(2.0 * math.pi)) < 1e-5


def test_gelu_brute():
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.standard_normal(500) * 2, [0.0, 1e-30, -1e-30, 5.0, -5.0]])
    got = O.gelu(v)
    ref = np.array([brute.gelu(float(t)) for t in v])
    # the brute force's 1 + erf loses digits for negative v (about 1e-16 absolute)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_mlp_composition_brute(fmt):
    """The MLP oracle against the scalar brute force: up (64 -> 128, rank 4),
    bf16, GELU, bf16, down (128 -> 32, rank 8), three tokens."""
    up = _tiny(3, 64, 128, seed=61, fmt=fmt)
    down = _tiny(3, 128, 32, seed=62, fmt=fmt)
    pu = O.pack(up.w_lin, up.bias, np.abs(up.x).max(axis=0), 4, fmt)
    pd = O.pack(down.w_lin, down.bias, np.abs(down.x).max(axis=0), 8, fmt)
    y = O.mlp_forward(pu, pd, up.x)
    bu = brute.pack(up.w_lin.tolist(), up.bias.tolist(), np.abs(up.x).max(axis=0).tolist(),
                    pu["l1"].tolist(), pu["l2"].tolist(), fmt)
    bd = brute.pack(down.w_lin.tolist(), down.bias.tolist(), np.abs(down.x).max(axis=0).tolist(),
                    pd["l1"].tolist(), pd["l2"].tolist(), fmt)
    by = np.array(brute.mlp_forward(bu, bd, up.x.tolist()))
    np.testing.assert_allclose(y, by, rtol=1e-12, atol=1e-12 * np.abs(by).max())
    # the hidden activation really goes through the GELU: without it the output differs
    y_lin = O.forward(pd, O.to_bf16(O.forward(pu, up.x)))
    assert np.abs(y_lin - y).max() > 1e-2 * np.abs(y).max()
