"""GPU-side pack (svdq_pack_weights_gpu) and the calibrated smoothing
strength (svdq_calibrate_alpha) against the oracle and the host pack
(MI355X only).

Bars: mu bit-exact with the oracle at alpha = 1/2 (within one float32 ulp
elsewhere: pow may round differently); the randomized SVD within 1e-3 of the
exact truncated SVD's residual energy (both bf16-rounded); given the GPU's mu
and bf16 factors, codes, scales and layouts bit-exact with the host pack
(itself bit-exact with the oracle); the calibration's alpha one whose
oracle loss is within 2% of the least."""
import sys

import numpy as np
import pytest

import bit_svdquant_diffusion_amd as S
from bit_svdquant_diffusion_amd import synth
from oracle import svdq_oracle as O
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


CASES = [synth.LayerSpec("gp_int4", 256, 512, 512, 16, "int4", 50),
         synth.LayerSpec("gp_fp4", 256, 768, 544, 32, "mxfp4", 51),
         synth.LayerSpec("gp_int4_pad", 200, 320, 72, 16, "int4", 52),
         synth.LayerSpec("gp_fp4_pad_r48", 128, 384, 200, 48, "mxfp4", 53),
         synth.LayerSpec("gp_qkv", 4608, 3072, 9216, 32, "int4", 1)]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_gpu_pack(spec):
    print(f"[gpu pack] {spec}", file=sys.stderr, flush=True)
    lay = C.layer_data(spec)
    ax = np.abs(lay.x).max(axis=0)
    layer = S.Layer(spec.K, spec.N, spec.rank, spec.fmt)
    dev = S.pack_weights_gpu(layer, _dev(lay.w_lin), _dev(lay.bias), _dev(ax), alpha=0.5, seed=3)
    torch.cuda.synchronize()
    host = S.to_host(dev)
    u = S.unpack_weights(layer, host)
    _, mu = O.smoothing_factors(ax, lay.w_lin)
    assert np.array_equal(u["mu"], mu)
    # the low-rank factors: randomized SVD against the exact truncated SVD
    wh = O.smoothed_weight(lay.w_lin, mu)
    l1 = O.bf16_from_bits(u["l1"]).astype(np.float64)
    l2 = O.bf16_from_bits(u["l2"]).astype(np.float64)
    err = np.sum((wh - l1 @ l2) ** 2)
    if spec.K * spec.N <= 1 << 20:
        ol1, ol2 = O.low_rank_factors(wh, spec.rank)
        err_or = np.sum((wh - ol1.astype(np.float64) @ ol2.astype(np.float64)) ** 2)
        assert err <= err_or * (1 + 1e-3) + 1e-12 * np.sum(wh ** 2)
    else:
        # large layer: against the eigenvalues of W_hat W_hat^T (K x K)
        ev = np.sort(np.linalg.eigvalsh(wh @ wh.T))[::-1]
        assert err <= ev[spec.rank:].sum() * (1 + 2e-2)
    # given these factors the codes, scales and every layout are the host pack's bytes
    ref = S.quantize_residual(layer, lay.w_lin, lay.bias, u["mu"], u["l1"], u["l2"])
    for n in S.PACKED_FIELDS:
        assert np.array_equal(host[n][:ref[n].size], ref[n]), n
    # and the layer runs: Y against the oracle on the same packed values
    x = C.x_device(spec)
    y = S.linear_forward(layer, dev, x)
    torch.cuda.synchronize()
    rows = C.sample_rows(spec.M, n=48)
    orp = O.pack(lay.w_lin, lay.bias, ax, spec.rank, spec.fmt,
                 factors=(u["mu"], O.bf16_from_bits(u["l1"]), O.bf16_from_bits(u["l2"])))
    C.check_y(C.bf16_tensor_to_f32(y)[rows], O.forward(orp, lay.x[rows]), f"gpu pack {spec.name}")


def test_gpu_pack_alpha_and_determinism():
    spec = CASES[0]
    lay = C.layer_data(spec)
    ax = np.abs(lay.x).max(axis=0)
    layer = S.Layer(spec.K, spec.N, spec.rank, spec.fmt)
    args = (_dev(lay.w_lin), _dev(lay.bias), _dev(ax))
    a = S.to_host(S.pack_weights_gpu(layer, *args, alpha=0.3, seed=5))
    b = S.to_host(S.pack_weights_gpu(layer, *args, alpha=0.3, seed=5))
    for n in S.PACKED_FIELDS:
        assert np.array_equal(a[n], b[n]), n
    _, mu = O.smoothing_factors_alpha(ax, lay.w_lin, 0.3)
    got = a["mu"].view(np.float32)[:spec.K]
    assert np.all(np.abs(got.view(np.int32).astype(np.int64) - mu.view(np.int32).astype(np.int64)) <= 1)
    with pytest.raises(S.SvdqError) as e:
        S.pack_weights_gpu(layer, *args, alpha=1.5)
    assert e.value.status == 2


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_calibrate_alpha(fmt):
    print(f"[calibrate] {fmt}", file=sys.stderr, flush=True)
    spec = synth.LayerSpec("cal", 128, 512, 256, 16, fmt, 54)
    lay = synth.make_layer(spec)
    layer = S.Layer(spec.K, spec.N, spec.rank, fmt)
    grid = [0.3, 0.4, 0.5, 0.6, 0.7]
    x = torch.from_numpy(lay.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    dev, alpha, losses = S.calibrate_alpha(layer, _dev(lay.w_lin), _dev(lay.bias), x, grid, seed=2)
    torch.cuda.synchronize()
    ref = O.calibrate_alpha(lay.w_lin, lay.bias, lay.x, spec.rank, fmt, grid)
    i = int(np.argmin(np.abs(np.array(grid) - alpha)))
    assert abs(grid[i] - alpha) < 1e-6
    assert losses[i] == losses.min()
    assert ref["losses"][i] <= ref["losses"].min() * 1.02, (alpha, ref["alpha"], ref["losses"], losses)
    np.testing.assert_allclose(losses, ref["losses"], rtol=0.05)
    # the kept layer is the pack of that alpha
    again = S.to_host(S.pack_weights_gpu(layer, _dev(lay.w_lin), _dev(lay.bias),
                                         _dev(np.abs(lay.x).max(axis=0)), alpha=grid[i], seed=2))
    host = S.to_host(dev)
    for n in S.PACKED_FIELDS:
        assert np.array_equal(host[n], again[n]), n
