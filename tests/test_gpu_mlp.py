"""GPU parity of the MLP pair y = down(GELU(up(x))) (svdq_mlp_forward): the
fused path, where the up layer's GEMM epilogue emits the down layer's
kernel-(1) output, against the composition of the two layers, and both
against the oracle's composition (oracle/svdq_oracle.py mlp_forward).

Bars (stated here, applied below):
  - the down layer's activation codes and scales: fused == composition, bit
    for bit, on every row below M (same GELU on the device, same quantizer);
  - its Z = x_hat L1: fused and composition differ only in the fp32
    summation order before the bf16 rounding, so by at most one bf16 step
    (2^-7 relative) plus 1e-6 max|Z|;
  - fused Y against the composition's Y: relative Frobenius <= 2e-3;
  - each half against the oracle at the layer bar (relative Frobenius
    <= 1e-2, max abs <= 2e-2 max): the hidden activation GELU(up(x)) of the
    composition, and the down layer run on the device with the oracle's own
    hidden activation as its input;
  - Y of the whole pair against the oracle's composition: relative Frobenius
    <= 5e-2, max abs <= 1e-1 max|Y|. The device's hidden activation differs
    from the oracle's within the layer bar (mostly one bf16 step, from the
    bf16 Z of the up layer's low-rank branch), and where such a step moves a
    value of the down layer's input across a rounding boundary of its 4-bit
    quantizer, that code moves by a whole step: about 7 eps of the codes for
    a relative input change eps, each adding one quantization step of error
    where quantization noise adds a uniform +-1/2 step. With eps <= 1e-2 that
    is up to a quarter of the down layer's own 4-bit noise (about 1e-1 of
    |Y|), added to the layer bar.
Every input is seeded and synthetic (bit_svdquant_diffusion_amd.synth).
"""
import sys

import numpy as np
import pytest

import bit_svdquant_diffusion_amd as S
from bit_svdquant_diffusion_amd import synth
from oracle import svdq_oracle as O
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    S.lib()
    yield


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _pair(name, M, K, H, N, r_up, r_down, fmt, seed):
    up = synth.LayerSpec(f"{name}_up", M, K, H, r_up, fmt, seed)
    down = synth.LayerSpec(f"{name}_down", M, H, N, r_down, fmt, seed + 1, x_kind="gelu",
                           x_outlier_frac=0.005, x_outlier_scale=30.0, w_outlier_frac=0.0)
    return name, up, down


PAIRS = [
    # 3 row tiles (the last one ragged) by 4 hidden tiles
    _pair("m300", 300, 512, 1024, 512, 32, 32, "int4", 70),
    # the down layer without a low-rank branch (no Z), 769-1024 tokens
    _pair("m1000_down_r0", 1000, 256, 768, 256, 16, 0, "int4", 72),
    # two 32-rank blocks in the fused Z, a padded up K and a padded down N
    _pair("m520_down_r64_padded", 520, 320, 512, 200, 32, 64, "int4", 74),
    # one token past the few-token limit (the last row tile holds one live
    # token: whole wave rows aim every store past the end), a single hidden
    # tile column, three 32-rank blocks in the fused Z, the smallest up K
    _pair("m257_h256_down_r96", 257, 64, 256, 128, 16, 96, "int4", 80),
    # MXFP4 pairs (384-channel tile columns; the hidden width also whole
    # 256-channel steps): two row tiles (the last one ragged) by two hidden
    # tile columns; a rank-0 down layer over four columns and three row
    # tiles; two 32-rank blocks with a padded up K and down N
    _pair("m300_h768_fp4", 300, 512, 768, 256, 32, 32, "mxfp4", 82),
    _pair("m500_h1536_down_r0_fp4", 500, 256, 1536, 128, 16, 0, "mxfp4", 84),
    _pair("m260_h768_down_r64_fp4", 260, 384, 768, 200, 32, 64, "mxfp4", 86),
]


def _run(up_spec, down_spec, mode):
    lu, du = C.device_layer(up_spec)
    ld, dd = C.device_layer(down_spec)
    M = up_spec.M
    x = C.x_device(up_spec)
    total, off = S.mlp_workspace_bytes(lu, ld, M)
    ws = torch.full((total,), 0xFF, dtype=torch.uint8, device="cuda")
    y = torch.full((M, ld.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    S.mlp_forward(lu, du, ld, dd, x, y=y, workspace=ws, mode=mode)
    torch.cuda.synchronize()
    wsh = ws.cpu().numpy()
    wd = S.workspace_bytes(ld, M)
    down_ws = S.unpack_workspace(ld, M, wsh[off:off + wd])
    return C.bf16_tensor_to_f32(y), down_ws, wsh, off + (wd + 255) // 256 * 256


def _oracle_hidden(up_spec, rows):
    pu = C.oracle_pack(up_spec)
    lay = C.layer_data(up_spec)
    return O.to_bf16(O.gelu(O.to_bf16(O.forward(pu, lay.x[rows]))))


def _check_pair_y(y_gpu, y_ref, what):
    """The whole pair's bar (see the module docstring)."""
    d = y_gpu.astype(np.float64) - y_ref
    fro = np.linalg.norm(d) / np.linalg.norm(y_ref)
    mx = np.abs(d).max() / np.abs(y_ref).max()
    _say(f"  pair {what}: rel_fro={fro:.3e} max_abs_rel={mx:.3e}")
    assert np.all(np.isfinite(y_gpu)), what
    assert fro <= 5e-2 and mx <= 1e-1, (what, fro, mx)


def _check_pair(up_spec, down_spec, rows=None):
    M = up_spec.M
    lu, _ = C.library_host(up_spec)
    ld, _ = C.library_host(down_spec)
    assert S.mlp_fused(lu, ld, M)
    yf, wf, _, _ = _run(up_spec, down_spec, S.MLP_AUTO)
    yu, wu, wsh_u, hid_off = _run(up_spec, down_spec, S.MLP_UNFUSED)
    assert np.array_equal(wf["codes"], wu["codes"]), "down codes: fused != composition"
    assert np.array_equal(wf["scales"], wu["scales"]), "down scales: fused != composition"
    if down_spec.rank:
        zf, zu = wf["z"].astype(np.float64), wu["z"].astype(np.float64)
        assert np.all(np.abs(zf - zu) <= 2.0 ** -7 * np.abs(zu) + 1e-6 * np.abs(zu).max()), "down Z"
    d = np.linalg.norm(yf.astype(np.float64) - yu) / np.linalg.norm(yu.astype(np.float64))
    _say(f"  fused vs composition rel_fro={d:.2e}")
    assert d <= 2e-3
    # against the oracle's composition (all rows, or sampled ones at full size)
    rows = np.arange(M) if rows is None else rows
    h_gpu = O.bf16_from_bits(wsh_u[hid_off:hid_off + M * lu.N * 2].view(np.uint16).reshape(M, lu.N))
    h_ref = _oracle_hidden(up_spec, rows)
    C.check_y(h_gpu[rows], h_ref, f"{up_spec.name} hidden")
    pd = C.oracle_pack(down_spec)
    y_ref = O.forward(pd, h_ref)
    # the down half alone, on the oracle's hidden activation
    ld, dd = C.device_layer(down_spec)
    hx = torch.from_numpy(O.bf16_to_bits(h_ref).view(np.int16)).cuda().view(torch.bfloat16)
    yd = C.bf16_tensor_to_f32(S.linear_forward(ld, dd, hx))
    C.check_y(yd, y_ref, f"{down_spec.name} on the oracle's hidden")
    # the whole pair
    qg = wu["codes"][rows]
    qr = O.quantize_activations(O.smooth_activations(h_ref, pd["mu"]), down_spec.fmt)[0]
    _say(f"  down codes that differ from the oracle's: {np.mean(qg != qr):.2%}")
    _check_pair_y(yf[rows], y_ref, "fused")
    _check_pair_y(yu[rows], y_ref, "composition")


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: p[0])
def test_mlp_fused_matches_composition_and_oracle(pair):
    name, up, down = pair
    _say(f"[mlp] {name}: {up} -> {down}")
    _check_pair(up, down)


def test_mlp_few_tokens_and_partial_columns_take_the_composition():
    """With 256 tokens or fewer (weight-streaming GEMM), and with a hidden
    width that is not whole tile columns (384 channels for MXFP4) or whole
    256-channel steps (1152), the automatic mode runs the composition: the
    same bits as mode UNFUSED."""
    for name, up, down in (_pair("m256", 256, 512, 512, 256, 32, 32, "int4", 76),
                           _pair("m300_h512_fp4", 300, 512, 512, 256, 32, 32, "mxfp4", 78),
                           _pair("m300_h1152_fp4", 300, 256, 1152, 128, 16, 16, "mxfp4", 79)):
        _say(f"[mlp composition] {name}")
        lu, _ = C.library_host(up)
        ld, _ = C.library_host(down)
        assert not S.mlp_fused(lu, ld, up.M)
        ya, _, _, _ = _run(up, down, S.MLP_AUTO)
        yu, _, _, _ = _run(up, down, S.MLP_UNFUSED)
        assert np.array_equal(ya.view(np.uint32), yu.view(np.uint32))
        pu, pd = C.oracle_pack(up), C.oracle_pack(down)
        _check_pair_y(yu, O.mlp_forward(pu, pd, C.layer_data(up).x), name)


def test_mlp_fused_is_deterministic_and_rejects_bad_shapes():
    name, up, down = PAIRS[0]
    y1, _, _, _ = _run(up, down, S.MLP_AUTO)
    y2, _, _, _ = _run(up, down, S.MLP_AUTO)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    lu, du = C.device_layer(up)
    ld, dd = C.device_layer(down)
    x = C.x_device(up)
    with pytest.raises(S.SvdqError) as e:   # unknown mode
        S.mlp_forward(lu, du, ld, dd, x, mode=7)
    assert e.value.status == 2
    with pytest.raises(S.SvdqError) as e:   # workspace one byte short
        ws = torch.empty(S.mlp_workspace_bytes(lu, ld, up.M)[0] - 1, dtype=torch.uint8, device="cuda")
        S.mlp_forward(lu, du, ld, dd, x, workspace=ws)
    assert e.value.status == 4
    other = S.Layer(lu.N + 256, ld.N, ld.rank, ld.fmt)   # down K != up N
    with pytest.raises(S.SvdqError) as e:
        S.mlp_workspace_bytes(lu, other, up.M)
    assert e.value.status == 2


# the image stream's MLP of a FLUX-style double-stream block at batch 2
# (8192 tokens, 3072 -> 12288 -> 3072, rank 32, INT4): the pair the benchmark
# times fused, sampled rows against the oracle
FULL_UP = next(s for s in synth.config_layers(4, small_m=False) if s.name == "img_up")
FULL_DOWN = next(s for s in synth.config_layers(4, small_m=False) if s.name == "img_down")


@pytest.mark.slow
def test_mlp_full_size_sampled():
    _say(f"[mlp full] {FULL_UP} -> {FULL_DOWN}")
    _check_pair(FULL_UP, FULL_DOWN, rows=C.sample_rows(FULL_UP.M))


# the MXFP4 pair of the same block at one image with its text (4608 tokens):
# the headline layer (MLP up, 3072 -> 12288) followed by its down layer
FP4_UP = synth.config_layers(2)[0]
FP4_DOWN = synth.LayerSpec("mlp_down_fp4", 4608, 12288, 3072, 32, "mxfp4", 3, x_kind="gelu",
                           x_outlier_frac=0.005, x_outlier_scale=30.0, w_outlier_frac=0.0)


@pytest.mark.slow
def test_mlp_full_size_mxfp4_sampled():
    _say(f"[mlp full fp4] {FP4_UP} -> {FP4_DOWN}")
    _check_pair(FP4_UP, FP4_DOWN, rows=C.sample_rows(FP4_UP.M))
