"""GPU parity of the AWQ-style W4A16 linear (svdq_awq_forward) against the
AWQ oracle's forward on the same packed layer (MI355X only).

Bar: relative Frobenius error <= 1e-2 and max abs error <= 2e-2 max|y| (the
layer's differences are the bf16 rounding of x_hat for the matrix unit, the
float32 sums and the bf16 output)."""
import sys

import numpy as np
import pytest

import bit_svdquant_diffusion_amd as S
from bit_svdquant_diffusion_amd import synth
from oracle import awq_oracle as A
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _spec(name, M, K, N, seed):
    return synth.LayerSpec(name, M, K, N, 0, "w4a16", seed, x_kind="silu", x_outlier_frac=0.01,
                           x_outlier_scale=8.0, w_outlier_frac=0.0)


CASES = synth.awq_layers() + [
    _spec("awq_m1_k128_n16", 1, 128, 16, 40),          # one n-block, one group
    _spec("awq_m17_k4096_n48", 17, 4096, 48, 41),      # two token chunks, the largest K
    _spec("awq_m33_k1024_n2064", 33, 1024, 2064, 42),  # three chunks, 129 n-blocks
    _spec("awq_m5_k3072_n8208", 5, 3072, 8208, 43),    # two n-blocks a workgroup, a partial last one
    _spec("awq_m16_k3072_n16464", 16, 3072, 16464, 44),  # eight n-blocks a workgroup, a partial last one
]


def _packed(spec, alpha=None):
    lay = synth.make_layer(spec)
    xc = synth.calibration_rows(spec, 32)
    host, al, _ = S.awq_pack(lay.w_lin, lay.bias, xc, alpha=alpha)
    u = S.awq_unpack(spec.K, spec.N, host)
    ref = dict(inv_s=u["inv_s"], q=u["codes"], scale=u["scales"], zero=u["zeros"],
               bias=synth.bf16_value(u["bias"]))
    return lay, host, ref, al


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_awq_forward_matches_oracle(spec):
    print(f"[awq] {spec}", file=sys.stderr, flush=True)
    lay, host, ref, al = _packed(spec)
    dev = S.awq_to_device(host)
    x = torch.from_numpy(lay.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.full((spec.M, spec.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    S.awq_forward(spec.K, spec.N, dev, x, y=y)
    torch.cuda.synchronize()
    C.check_y(C.bf16_tensor_to_f32(y), A.forward(ref, lay.x), f"awq {spec.name} alpha={al}")


@pytest.mark.parametrize("name", ["awq_m16_k3072_n16464", "awq_m17_k4096_n48"])
def test_awq_deterministic_and_m0(name):
    """Repeat calls give the same bits, M = 0 is a no-op, and a row's output
    does not depend on the rows launched with it: one row alone (a one- or
    two-block launch, K in eight or four parts per wave set) against the same
    rows inside 16-row chunks (eight and four blocks a workgroup), bit for
    bit, including the 17th row that forms a chunk of its own."""
    spec = next(s for s in CASES if s.name == name)
    lay, host, ref, _ = _packed(spec, alpha=0.5)
    dev = S.awq_to_device(host)
    x = torch.from_numpy(lay.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y1 = S.awq_forward(spec.K, spec.N, dev, x)
    y2 = S.awq_forward(spec.K, spec.N, dev, x)
    y0 = S.awq_forward(spec.K, spec.N, dev, x[:0])
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)) and y0.shape == (0, spec.N)
    for row in (2, spec.M - 1):
        y3 = S.awq_forward(spec.K, spec.N, dev, x[row:row + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(y3.view(torch.int16), y1[row:row + 1].view(torch.int16)), row
