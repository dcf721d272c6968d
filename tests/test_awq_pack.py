"""Host pack of the AWQ-style W4A16 layer (svdq_awq_pack, C++, no GPU)
against the AWQ oracle: the same alpha (or one whose loss ties the least
within float64 summation order), the same channel scales to float64 rounding,
and, for those scales, bit-exact codes, scales and zero points."""
import ctypes

import numpy as np
import pytest

import bit_svdquant_diffusion_amd as S
from bit_svdquant_diffusion_amd import synth
from oracle import awq_oracle as A


def _case(K, N, seed, rows=32, outlier=0.02):
    spec = synth.LayerSpec("awq", 2, K, N, 0, "w4a16", seed, x_kind="silu", x_outlier_frac=outlier,
                           x_outlier_scale=8.0, w_outlier_frac=0.0)
    lay = synth.make_layer(spec)
    return lay, synth.calibration_rows(spec, rows)


@pytest.mark.parametrize("K,N,seed", [(256, 48, 1), (512, 64, 2), (1024, 32, 3)])
def test_awq_pack_matches_oracle(K, N, seed):
    lay, xc = _case(K, N, seed)
    host, alpha, s_lib = S.awq_pack(lay.w_lin, lay.bias, xc)
    ref = A.pack(lay.w_lin, lay.bias, xc)
    lmin = ref["losses"].min()
    li = int(round(alpha * 20))
    assert A.ALPHA_GRID[li] == alpha
    assert ref["losses"][li] <= lmin * (1 + 1e-9), (alpha, ref["alpha"])
    s_or = A.channel_scales(ref["act_mean"], alpha)
    np.testing.assert_allclose(s_lib, s_or, rtol=1e-13)
    # the stored parts are the oracle's for the library's scales
    ws = (lay.w_lin.astype(np.float64) * s_lib[None, :]).astype(np.float32)
    q, sc, z = A.quantize_groups(ws)
    u = S.awq_unpack(K, N, host)
    assert np.array_equal(u["codes"], q) and np.array_equal(u["scales"], sc) and np.array_equal(u["zeros"], z)
    assert np.array_equal(u["inv_s"], (1.0 / s_lib).astype(np.float32))
    assert np.array_equal(u["bias"], synth.bf16_bits(lay.bias))


def test_awq_pack_given_alpha_and_errors():
    lay, xc = _case(384, 32, 4)
    host, alpha, s_lib = S.awq_pack(lay.w_lin, None, xc, alpha=0.0)
    assert alpha == 0.0 and np.all(s_lib == 1.0)
    u = S.awq_unpack(384, 32, host)
    q, sc, z = A.quantize_groups(lay.w_lin)
    assert np.array_equal(u["codes"], q) and np.array_equal(u["scales"], sc) and np.array_equal(u["zeros"], z)
    assert not u["bias"].any()
    for bad_k, bad_n in ((200, 32), (384, 40), (8192, 32)):
        with pytest.raises(S.SvdqError) as e:
            S.awq_packed_bytes(bad_k, bad_n)
        assert e.value.status == 2
    xn = xc.copy()
    xn[0, 5] = np.inf
    with pytest.raises(S.SvdqError) as e:
        S.awq_pack(lay.w_lin, None, xn)
    assert e.value.status == 5
    with pytest.raises(S.SvdqError) as e:
        S.awq_pack(lay.w_lin, None, xc, alpha=1.5)
    assert e.value.status == 2
    d = S.AwqDesc(384, 32)
    out = S.AwqPacked()
    assert S.lib().svdq_awq_pack(ctypes.byref(d), lay.w_lin.ctypes.data, None, xc.ctypes.data, 4, -1.0, None,
                                 None, ctypes.byref(out)) == 1


def test_awq_sizes():
    s = S.awq_packed_bytes(3072, 18432)
    assert s == dict(inv_s=3072 * 4, qw=18432 * 3072 // 2, scales=18432 * 24 * 4, zeros=18432 * 24, bias=18432 * 2)
