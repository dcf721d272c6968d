"""GPU parity of libsvdq's HIP path against the CPU oracle (MI355X only).

Bars (stated here, applied below):
  - activation codes, scales and INT4 int32 group sums: bit-exact;
  - Z = x_hat L1 (bf16 on the device): relative Frobenius <= 1e-2, max abs <= 2e-2 max|Z|;
  - Y: relative Frobenius <= 1e-2 and max abs <= 2e-2 max|Y|.
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


def _spec(name, M, K, N, r, fmt, seed, **kw):
    return synth.LayerSpec(name, M, K, N, r, fmt, seed, **kw)


SMALL = [
    _spec("c0", 256, 512, 512, 16, "int4", 0),
    _spec("c0_fp4", 256, 512, 512, 16, "mxfp4", 0),
    _spec("ragged_m300", 300, 768, 544, 32, "int4", 11),
    _spec("ragged_m300_fp4", 300, 768, 544, 32, "mxfp4", 11),
    _spec("m1", 1, 512, 256, 16, "int4", 12),
    _spec("m1_fp4", 1, 512, 256, 16, "mxfp4", 12),
    _spec("m17_r0", 17, 256, 96, 0, "int4", 13),
    _spec("m17_r0_fp4", 17, 256, 96, 0, "mxfp4", 13),
    _spec("r128", 200, 256, 160, 128, "int4", 14),
    _spec("r128_fp4", 200, 256, 160, 128, "mxfp4", 14),
    _spec("wide_k", 96, 2048, 64, 48, "int4", 15),
    # 32-token stage-1 workgroups (MXFP4 from M = 2048, INT4 from M = 8192
    # with K >= 6144): the last workgroup's second half holds 2 tokens
    # (M = 2066, 8194) or 4 (M = 2100, rank32 = 64). INT4 with a short K
    # keeps 16-token workgroups at M = 8194, the last one holding 2 tokens.
    _spec("two_halves_m8194", 8194, 6144, 64, 32, "int4", 16),
    _spec("one_half_m8194_short_k", 8194, 256, 64, 32, "int4", 16),
    _spec("two_halves_m2066_fp4", 2066, 512, 256, 32, "mxfp4", 16),
    _spec("two_halves_m2100_r48_fp4", 2100, 256, 96, 48, "mxfp4", 17),
    # INT4 GEMM split: 6 tiles of 24 K stages on 6 XCDs, each cut into four
    # runs of 6 stages (one owner adding three partials)
    _spec("split_k_4_pieces", 384, 3072, 512, 16, "int4", 18),
    # INT4 with few tokens (weight-streaming kernel). 3 token blocks over
    # eight K parts, K cut into two shares whose partials a second kernel
    # adds; 7 token blocks in four token parts by two K parts, three shares;
    # more channel blocks than half the CUs: four-wave workgroups, K parts
    # (2 token blocks) or token parts (8 token blocks, the last one ragged)
    _spec("small_m70_shares", 70, 8192, 512, 32, "int4", 20),
    _spec("small_m200_shares", 200, 3072, 256, 32, "int4", 21),
    _spec("small_m40_four_waves", 40, 512, 4160, 16, "int4", 22),
    _spec("small_m250_four_waves", 250, 256, 8224, 32, "int4", 23),
    # MXFP4 with few tokens, the same kernel on block-scaled MFMA: two K
    # shares over eight K parts, three shares over token parts, four-wave
    # workgroups, and a decode-like QKV projection
    _spec("small_m70_shares_fp4", 70, 8192, 512, 32, "mxfp4", 20),
    _spec("small_m200_shares_fp4", 200, 3072, 256, 32, "mxfp4", 21),
    _spec("small_m250_four_waves_fp4", 250, 256, 8224, 32, "mxfp4", 23),
    _spec("small_m64_qkv_fp4", 64, 3072, 9216, 32, "mxfp4", 29),
    # 769 to 1024 tokens: eight token parts of four blocks (M = 1000: the
    # last block ragged, K cut into two shares; M = 800: 25 blocks, the
    # surplus parts repeating the last block)
    _spec("small_m1000_shares", 1000, 1024, 512, 32, "int4", 27),
    _spec("small_m800", 800, 512, 4160, 16, "int4", 28),
    # MXFP4 GEMM: 9 x 32 = 288 tiles, so 32 workgroups run two tiles of three
    # ring steps; the next tile's bias transfer is issued before the first
    # tile's epilogue reads its own
    _spec("two_tiles_k256_fp4", 1728, 256, 12288, 32, "mxfp4", 19),
    # K and N that are not whole 256-channel steps or 32-row blocks (K % 64
    # for INT4, K % 128 for MXFP4, N % 8): the tiled kernels (with the INT4
    # split and both stage-1 modes), the few-token kernel with K shares and
    # its 769-1024 token shape
    _spec("k320_n40", 300, 320, 40, 16, "int4", 30),
    _spec("k192_n72", 600, 192, 72, 16, "int4", 31),
    _spec("k1088_n4104_split", 4200, 1088, 4104, 32, "int4", 32),
    _spec("k384_n72_fp4", 300, 384, 72, 32, "mxfp4", 33),
    _spec("k640_n1544_fp4", 2100, 640, 1544, 32, "mxfp4", 34),
    _spec("k320_n40_few", 70, 320, 40, 16, "int4", 35),
    _spec("k4160_n200_few_shares", 100, 4160, 200, 32, "int4", 36),
    _spec("k384_n40_few_fp4", 50, 384, 40, 16, "mxfp4", 37),
    _spec("k576_n1000_m1000", 1000, 576, 1000, 32, "int4", 38),
]


def _run_stage1(spec):
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    ws = torch.full((S.workspace_bytes(layer, spec.M),), 0xFF, dtype=torch.uint8, device="cuda")
    S.stage1(layer, dev, x, ws)
    torch.cuda.synchronize()
    return layer, dev, x, ws


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_stage1_codes_scales_z(spec):
    _say(f"[stage1] {spec}")
    layer, dev, x, ws = _run_stage1(spec)
    got = S.unpack_workspace(layer, spec.M, ws.cpu().numpy())
    ref = C.oracle_pack(spec)
    lay = C.layer_data(spec)
    y, parts = O.forward(ref, lay.x, return_parts=True)
    assert np.array_equal(got["codes"], parts["qx"].astype(np.int8)), "activation codes"
    assert np.array_equal(got["scales"], parts["sx"]), "activation scales"
    if spec.rank:
        zr = parts["z"]
        d = got["z"] - zr
        assert np.linalg.norm(d) <= 1e-2 * np.linalg.norm(zr)
        assert np.abs(d).max() <= 2e-2 * np.abs(zr).max()


LOGICAL = [s for s in SMALL if s.name in ("c0", "c0_fp4", "ragged_m300", "ragged_m300_fp4", "m17_r0", "m17_r0_fp4",
                                          "r128_fp4", "wide_k", "two_halves_m2100_r48_fp4", "small_m70_shares")]


@pytest.mark.parametrize("spec", LOGICAL, ids=lambda s: s.name)
def test_stage1_outputs_logical(spec):
    """svdq_stage1_outputs: the device-side logical views equal the host
    unpack of the same workspace bit for bit, and the codes and scales equal
    the oracle's (Z within the layer's bar, being bf16 on the device). The
    views start filled with 0x7f codes, NaN or 0xff scales and NaN Z, none of
    which a correct view holds, so every element must have been written."""
    _say(f"[stage1 outputs] {spec}")
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    ws = torch.full((S.workspace_bytes(layer, spec.M),), 0xFF, dtype=torch.uint8, device="cuda")
    g = 64 if spec.fmt == "int4" else 32
    out = S.stage1_outputs(
        layer, dev, x, workspace=ws,
        codes=torch.full((spec.M, spec.K), 0x7F, dtype=torch.int8, device="cuda"),
        scales=(torch.full((spec.M, spec.K // g), float("nan"), device="cuda") if spec.fmt == "int4"
                else torch.full((spec.M, spec.K // g), 0xFF, dtype=torch.uint8, device="cuda")),
        z=torch.full((spec.M, spec.rank), float("nan"), device="cuda"))
    torch.cuda.synchronize()
    host = S.unpack_workspace(layer, spec.M, ws.cpu().numpy())
    codes = out["codes"].cpu().numpy()
    scales = out["scales"].cpu().numpy()
    assert np.array_equal(codes, host["codes"]), "codes: device view != host unpack"
    assert np.array_equal(scales.view(np.uint8), host["scales"].view(np.uint8)), "scales: device view != host unpack"
    ref = C.oracle_pack(spec)
    lay = C.layer_data(spec)
    _, parts = O.forward(ref, lay.x, return_parts=True)
    assert np.array_equal(codes, parts["qx"].astype(np.int8)), "activation codes"
    assert np.array_equal(scales, parts["sx"]), "activation scales"
    if spec.rank:
        z = out["z"].cpu().numpy()
        assert np.array_equal(z.view(np.uint32), host["z"].astype(np.float32).view(np.uint32)), "z: view != unpack"
        zr = parts["z"]
        d = z - zr
        assert np.linalg.norm(d) <= 1e-2 * np.linalg.norm(zr)
        assert np.abs(d).max() <= 2e-2 * np.abs(zr).max()


def _e2m3(f: np.ndarray) -> np.ndarray:
    """Values of 6-bit FP6 E2M3 fields: sign bit 5, exponent bits 4..3 (bias
    1, zero = subnormal), mantissa bits 2..0."""
    f = f.astype(np.int64)
    e, m = (f >> 3) & 3, f & 7
    v = np.where(e == 0, m / 8.0, (1.0 + m / 8.0) * np.exp2(e - 1.0))
    return np.where(f & 32, -v, v)


def _fp6_copy_values(buf: np.ndarray, rows32: int, kp: int) -> np.ndarray:
    """[rows32][kp] values of an FP6 copy of 4-bit codes, as the tiled INT4
    GEMM's operand layout states it: per 32-row block and 128-channel stage
    3 KiB, the 64 lanes' 16-byte heads of group 0, then of group 1, then the
    8-byte tails of group 0 and of group 1; lane 32h + r's 24 bytes are 32
    six-bit fields, field i at bit 6i holding channel 32h + i of row r."""
    nb, nst = rows32 // 32, kp // 128
    a = buf[: nb * nst * 3072].reshape(nb, nst, 3, 1024)
    heads = a[:, :, :2, :].reshape(nb, nst, 2, 64, 16)
    tails = a[:, :, 2, :].reshape(nb, nst, 2, 64, 8)
    lane = np.concatenate([heads, tails], axis=-1)
    bits = np.unpackbits(lane, axis=-1, bitorder="little").reshape(nb, nst, 2, 64, 32, 6)
    f = (bits.astype(np.int64) << np.arange(6)).sum(-1)
    v = _e2m3(f).reshape(nb, nst, 2, 2, 32, 32)   # [block][stage][group][h][r][i]
    return v.transpose(0, 4, 1, 2, 3, 5).reshape(nb * 32, nst * 128)


@pytest.mark.parametrize("name", ["ragged_m300", "k1088_n4104_split", "k320_n40", "two_halves_m8194"])
def test_int4_fp6_copies_hold_the_codes(name):
    """The tiled INT4 GEMM's FP6 copies (the last two workspace areas after a
    GEMM): decoded on the host they equal the oracle's activation codes and
    weight codes exactly, with zeros in the padded channels and rows."""
    spec = next(s for s in SMALL if s.name == name)
    _say(f"[fp6 copies] {spec}")
    layer, dev, x, ws = _run_stage1(spec)
    y = torch.empty((spec.M, spec.N), dtype=torch.bfloat16, device="cuda")
    S.gemm(layer, dev, ws, spec.M, y)
    torch.cuda.synchronize()
    kp, rows, np_ = (spec.K + 255) // 256 * 256, (spec.M + 31) // 32 * 32, (spec.N + 31) // 32 * 32
    a256 = lambda v: (v + 255) // 256 * 256
    buf = ws.cpu().numpy()
    w6 = buf.size - a256(np_ * kp * 3 // 4)
    x6 = w6 - a256(rows * kp * 3 // 4)
    ref = C.oracle_pack(spec)
    _, parts = O.forward(ref, C.layer_data(spec).x, return_parts=True)
    xv = _fp6_copy_values(buf[x6:w6], rows, kp)
    wv = _fp6_copy_values(buf[w6:], np_, kp)
    assert np.array_equal(xv[:spec.M, :spec.K], parts["qx"].astype(np.float64)), "activation codes"
    assert not np.any(xv[:spec.M, spec.K:]), "activation padding"
    assert np.array_equal(wv[:spec.N, :spec.K], ref["qw"].astype(np.float64)), "weight codes"
    assert not np.any(wv[:, spec.K:]) and not np.any(wv[spec.N:, :]), "weight padding"


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_forward_matches_oracle(spec):
    _say(f"[forward] {spec}")
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    ws = torch.full((S.workspace_bytes(layer, spec.M),), 0xFF, dtype=torch.uint8, device="cuda")
    y = torch.full((spec.M, spec.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    S.linear_forward(layer, dev, x, y=y, workspace=ws)
    torch.cuda.synchronize()
    yg = C.bf16_tensor_to_f32(y)
    ref = C.oracle_pack(spec)
    yr = O.forward(ref, C.layer_data(spec).x)
    fro, mx = C.check_y(yg, yr, spec.name)
    _say(f"  rel_fro={fro:.2e} max_rel={mx:.2e}")


SENTINEL = -(2 ** 31)


def _group_sums(layer, dev, ws, M, m0, mc, n0, nc):
    """The hook's int32 sums into a buffer pre-filled with a value no sum can
    take, so a group the kernel skipped shows up as a mismatch."""
    out = torch.full((mc, nc, layer.K // 64), SENTINEL, dtype=torch.int32, device="cuda")
    S.debug_int4_group_sums(layer, dev, ws, M, m0, mc, n0, nc, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("spec", [s for s in SMALL if s.fmt == "int4"], ids=lambda s: s.name)
def test_int4_group_sums_bit_exact(spec):
    """Every INT4 launch shape, through the same dispatch as the forward (the
    tiled kernel, or the few-token kernel for M <= 256 and 769..1024 with its
    K shares, K parts and token parts)."""
    _say(f"[group sums] {spec}")
    layer, dev, x, ws = _run_stage1(spec)
    p = _group_sums(layer, dev, ws, spec.M, 0, spec.M, 0, spec.N)
    ref = C.oracle_pack(spec)
    xh = O.smooth_activations(C.layer_data(spec).x, ref["mu"])
    qx, _ = O.quant_int4_rows(xh)
    want = O.int4_group_sums(qx, ref["qw"])
    assert np.array_equal(p, want)


@pytest.mark.parametrize("name,win", [("ragged_m300", (131, 150, 67, 200)),
                                      ("small_m200_shares", (37, 150, 67, 120)),
                                      ("small_m1000_shares", (500, 333, 200, 77))])
def test_group_sums_window(name, win):
    spec = next(s for s in SMALL if s.name == name)
    m0, mc, n0, nc = win
    layer, dev, x, ws = _run_stage1(spec)
    p = _group_sums(layer, dev, ws, spec.M, m0, mc, n0, nc)
    ref = C.oracle_pack(spec)
    qx, _ = O.quant_int4_rows(O.smooth_activations(C.layer_data(spec).x, ref["mu"]))
    want = O.int4_group_sums(qx[m0:m0 + mc], ref["qw"][n0:n0 + nc])
    assert np.array_equal(p, want)


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_deterministic_and_m0(fmt):
    spec = _spec("det", 300, 768, 544, 32, fmt, 11)
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    y1 = S.linear_forward(layer, dev, x)
    y2 = S.linear_forward(layer, dev, x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # M == 0: no-op
    y0 = S.linear_forward(layer, dev, x[:0])
    assert y0.shape == (0, spec.N)


def test_split_tiles_deterministic():
    """The last piece of a cut INT4 tile adds the tile's partials in piece
    order, whichever piece it is, so repeated calls give identical bits
    (four-piece split case)."""
    spec = next(s for s in SMALL if s.name == "split_k_4_pieces")
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    ys = [S.linear_forward(layer, dev, x) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0].view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("name,M,K,N", [("split_k_4_pieces", 384, 3072, 512),
                                        ("split_two_pieces_per_tile", 1024, 1536, 4096),
                                        ("split_after_rounds", 2304, 1024, 9216)])
def test_split_tiles_beside_a_concurrent_kernel(name, M, K, N):
    """The INT4 GEMM's split needs no workgroups to run at the same time:
    pieces publish partials and the last one finishes the tile, nobody waits.
    With a long bf16 GEMM on another stream holding CUs, the layer gives the
    bits it gives alone, and both match the oracle."""
    _say(f"[split concurrent] {name}")
    spec = _spec(name, M, K, N, 32, "int4", 18)
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    alone = S.linear_forward(layer, dev, x)
    torch.cuda.synchronize()
    big = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")
    other = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(other):
            for _ in range(2):
                big = (big @ big) * (1.0 / 128)
        outs.append(S.linear_forward(layer, dev, x))
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(y.view(torch.int16), alone.view(torch.int16))
    rows = C.sample_rows(M, n=48)
    C.check_y(C.bf16_tensor_to_f32(alone)[rows], O.forward(C.oracle_pack(spec), C.layer_data(spec).x[rows]), name)


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_rows_are_independent(fmt):
    """Rows past M in a ragged last tile or token block do not leak into the
    real rows: dropping trailing rows leaves the others' bits unchanged, for
    the tiled GEMMs (M = 300 vs 299 and 290) and the INT4 few-token kernel
    (M = 60 vs 43)."""
    spec = _spec("indep", 300, 768, 544, 32, fmt, 11)
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    full = S.linear_forward(layer, dev, x)
    for m, n in ((300, 299), (300, 290), (60, 43)):
        a = full if m == 300 else S.linear_forward(layer, dev, x[:m].contiguous())
        b = S.linear_forward(layer, dev, x[:n].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(a[:n].view(torch.int16), b.view(torch.int16)), (m, n)


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_stage1_z_same_in_both_modes(fmt):
    """Z = X_hat L1 of a token does not depend on the batch: 100 tokens (their
    K pieces dealt over the CUs, partials added by a second kernel) and 4200
    tokens (one workgroup walks a token group's whole K) give the same bits
    for the shared rows, as do the codes and scales."""
    spec = _spec("zmodes", 4200, 3072, 64, 32, fmt, 25)
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    got = {}
    for m in (100, 4200):
        _say(f"[z modes] {fmt} M={m}")
        ws = torch.full((S.workspace_bytes(layer, m),), 0xFF, dtype=torch.uint8, device="cuda")
        S.stage1(layer, dev, x[:m].contiguous(), ws)
        torch.cuda.synchronize()
        got[m] = S.unpack_workspace(layer, m, ws.cpu().numpy())
    for key in ("z", "codes", "scales"):
        a, b = np.asarray(got[100][key]), np.asarray(got[4200][key])
        assert np.array_equal(a, b[:a.shape[0]]), key


@pytest.mark.parametrize("fmt,M", [("int4", 70), ("int4", 300), ("mxfp4", 300)])
def test_graph_replays_match_eager(fmt, M):
    """svdq_linear_forward captured in a HIP graph: each replay, with eager
    work and synchronizations between replays and the workspace refilled with
    0xFF each time, gives the eager result's bits. The forward records kernel
    nodes only (stage 1 clears the INT4 split flags in a kernel)."""
    _say(f"[graph] {fmt} M={M}")
    spec = _spec("graph", M, 768, 544, 32, fmt, 24)
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    want = S.linear_forward(layer, dev, x)
    ws = torch.empty(S.workspace_bytes(layer, M), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, spec.N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.linear_forward(layer, dev, x, y=y, workspace=ws)
    for i in range(4):
        y.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want.view(torch.int16)), f"replay {i}"


def test_library_pack_end_to_end():
    """svdq_pack_weights (randomized SVD) + forward stays within the Y bar of the oracle."""
    spec = SMALL[0]
    lay = C.layer_data(spec)
    ax = np.abs(lay.x).max(axis=0)
    layer = S.Layer(spec.K, spec.N, spec.rank, spec.fmt)
    lin = S.SVDQLinear(layer, S.pack_weights(layer, lay.w_lin, lay.bias, ax, seed=3))
    y = lin(C.x_device(spec))
    torch.cuda.synchronize()
    ref = C.oracle_pack(spec)
    C.check_y(C.bf16_tensor_to_f32(y), O.forward(ref, lay.x), "library pack")


def test_bad_device_args_rejected():
    spec = SMALL[0]
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(S.SvdqError) as e:
        S.linear_forward(layer, dev, x, workspace=ws)
    assert e.value.status == 4
    xm = torch.empty(spec.M * spec.K + 1, dtype=torch.bfloat16, device="cuda")[1:].view(spec.M, spec.K)
    with pytest.raises(S.SvdqError) as e:
        S.linear_forward(layer, dev, xm)
    assert e.value.status == 2


# ----------------------------------------------------------------------------
# full-size workloads (the configurations the benchmark times), sampled rows
# ----------------------------------------------------------------------------
FULL = [synth.config_layers(i)[0] for i in (1, 2, 3)] + synth.config_layers(4)


@pytest.mark.slow
@pytest.mark.parametrize("spec", FULL, ids=lambda s: s.name)
def test_full_size_sampled(spec):
    _say(f"[full] {spec}")
    layer, dev = C.device_layer(spec)
    x = C.x_device(spec)
    ws = torch.full((S.workspace_bytes(layer, spec.M),), 0xFF, dtype=torch.uint8, device="cuda")
    y = torch.full((spec.M, spec.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    S.linear_forward(layer, dev, x, y=y, workspace=ws)
    torch.cuda.synchronize()
    lay = C.layer_data(spec)
    ref = C.oracle_pack(spec)
    # codes and scales of every row, bit-exact
    got = S.unpack_workspace(layer, spec.M, ws.cpu().numpy())
    xh = O.smooth_activations(lay.x, ref["mu"])
    qx, sx = O.quantize_activations(xh, spec.fmt)
    assert np.array_equal(got["codes"], qx.astype(np.int8))
    assert np.array_equal(got["scales"], sx)
    # Y on sampled rows (rows are independent in every step)
    rows = C.sample_rows(spec.M)
    yr = O.forward(ref, lay.x[rows])
    yg = C.bf16_tensor_to_f32(y)[rows]
    fro, mx = C.check_y(yg, yr, spec.name)
    _say(f"  rows={len(rows)} rel_fro={fro:.2e} max_rel={mx:.2e}")
    if spec.fmt == "int4":
        # int32 group sums bit-exact, from the kernel this M's forward runs:
        # with at most 1024 tokens every row (the few-token kernel's token
        # parts), else a 64-row window; the first 128 and last 96 channels
        if spec.M <= 1024:
            m0, mc = 0, spec.M
        else:
            m0 = int(rows[len(rows) // 2])
            mc = min(64, spec.M - m0)
        for n0, nc in ((0, 128), (spec.N - 96, 96)):
            p = _group_sums(layer, dev, ws, spec.M, m0, mc, n0, nc)
            want = O.int4_group_sums(qx[m0:m0 + mc], ref["qw"][n0:n0 + nc])
            assert np.array_equal(p, want), (n0, nc)


def _tie_rows(fmt: str, K: int, M: int) -> np.ndarray:
    """bf16-representable rows that put the quantizer's decision points in front
    of the device code with mu = 1: every E2M1 tie (0.25 0.75 1.25 1.75 2.5 3.5
    5, block max 6 so the MX exponent is 0) or every INT4 half-integer (group
    max 7 so s = 1), their bf16 neighbours, zeros of both signs, values past
    saturation, and an all-zero group; each row scaled by its own power of two
    (the codes are scale invariant, the scales are not)."""
    rng = np.random.default_rng(123)
    if fmt == "mxfp4":
        ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        top, blk = 6.0, 32
    else:
        ties = np.arange(7) + 0.5
        top, blk = 7.0, 64
    up = ties * (1 + 2.0 ** -7)          # next bf16 above each tie (one ulp at 8 mantissa bits)
    dn = ties * (1 - 2.0 ** -8)          # next bf16 below
    base = np.concatenate([ties, up, dn, [0.0, 0.1, top * 0.999]])
    rows = np.zeros((M, K))
    for m in range(M):
        for g in range(K // blk):
            vals = np.resize(rng.permutation(np.concatenate([base, -base])), blk)
            vals[g % blk] = top if (m + g) % 2 else -top
            if (m * 7 + g) % 11 == 0:
                vals[:] = 0.0                            # all-zero group
            if (m + 3 * g) % 13 == 0:
                vals[(g + 1) % blk] = -0.0
            rows[m, g * blk:(g + 1) * blk] = vals
        rows[m] *= 2.0 ** ((m % 21) - 10)
    return O.to_bf16(rows.astype(np.float32))


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_stage1_quantizer_tie_points(fmt):
    """Codes and scales bit-exact with the oracle on every rounding decision point."""
    _say(f"[stage1 ties] {fmt}")
    K, N, r, M = 512, 64, 16, 48
    layer = S.Layer(K, N, r, fmt)
    rng = np.random.default_rng(7)
    l1 = O.bf16_to_bits(O.to_bf16(rng.standard_normal((K, r)).astype(np.float32)))
    l2 = O.bf16_to_bits(O.to_bf16(rng.standard_normal((r, N)).astype(np.float32)))
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    host = S.quantize_residual(layer, w, None, np.ones(K, np.float32), l1, l2)
    dev = S.to_device(layer, host, "cuda")
    xr = _tie_rows(fmt, K, M)
    x = torch.from_numpy(O.bf16_to_bits(xr).view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.full((S.workspace_bytes(layer, M),), 0xFF, dtype=torch.uint8, device="cuda")
    S.stage1(layer, dev, x, ws)
    torch.cuda.synchronize()
    got = S.unpack_workspace(layer, M, ws.cpu().numpy())
    qx, sx = O.quantize_activations(xr.astype(np.float32), fmt)
    assert np.array_equal(got["codes"], qx.astype(np.int8)), "activation codes at tie points"
    assert np.array_equal(got["scales"], sx), "activation scales at tie points"


@pytest.mark.parametrize("fmt,regime", [("int4", "tiny"), ("mxfp4", "tiny"), ("int4", "huge"), ("mxfp4", "huge")])
def test_stage1_extreme_blocks(fmt, regime):
    """Codes and scales bit-exact with the oracle for groups (blocks) at the
    ends of the bf16 range. tiny: maxima between the smallest bf16 subnormal
    and 2^-90; INT4 scales below 2^-100 take the per-level comparison
    (subnormal scales included), MXFP4 blocks whose shared exponent clamps at
    -127 take the software E2M1 encoder, and those at -126 the converter with
    the smallest normal scale. huge: maxima up to about 2^121 (INT4 scales
    up to about 2^118, MXFP4 exponents up to 118)."""
    _say(f"[stage1 extreme] {fmt} {regime}")
    K, N, r, M = 512, 64, 16, 48
    layer = S.Layer(K, N, r, fmt)
    rng = np.random.default_rng(11)
    l1 = O.bf16_to_bits(O.to_bf16(rng.standard_normal((K, r)).astype(np.float32)))
    l2 = O.bf16_to_bits(O.to_bf16(rng.standard_normal((r, N)).astype(np.float32)))
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    host = S.quantize_residual(layer, w, None, np.ones(K, np.float32), l1, l2)
    dev = S.to_device(layer, host, "cuda")
    base = _tie_rows(fmt, K, M).astype(np.float64)   # ties, neighbours, saturation, zeros
    if regime == "tiny":
        shift = -(100 + 3 * (np.arange(M) % 12))      # rows at 2^-90 down to below 2^-133
    else:
        shift = 100 + (np.arange(M) % 12)             # block maxima up to about 2^121
    xr = O.to_bf16((base * np.exp2(shift)[:, None]).astype(np.float32))
    assert np.all(np.isfinite(xr))
    if regime == "tiny" and fmt == "int4":
        # groups whose quotient lies 2^-150 / s from a half-integer
        from tests.test_oracle import subnormal_tie_pairs
        for i, (amax, v) in enumerate(subnormal_tie_pairs()):
            rr, g = i % M, 3 + i // M
            xr[rr, 64 * g:64 * (g + 1)] = 0.0
            xr[rr, 64 * g:64 * g + 4] = [amax, v, -v, -amax]
    qx, sx = O.quantize_activations(xr.astype(np.float32), fmt)
    if regime == "huge":
        big = sx.astype(np.float64).max() if fmt == "int4" else int(sx.max()) - 127
        assert big > (2.0 ** 110 if fmt == "int4" else 110)
    elif fmt == "int4":
        tiny = (sx > 0) & (sx < 2.0 ** -100)
        assert tiny.sum() > 100 and ((sx > 0) & (sx < 2.0 ** -126)).sum() > 20, "subnormal scales covered"
    else:
        assert (sx == 0).sum() > 100 and (sx == 1).sum() > 10, "exponents -127 and -126 covered"
    x = torch.from_numpy(O.bf16_to_bits(xr).view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.full((S.workspace_bytes(layer, M),), 0xFF, dtype=torch.uint8, device="cuda")
    S.stage1(layer, dev, x, ws)
    torch.cuda.synchronize()
    got = S.unpack_workspace(layer, M, ws.cpu().numpy())
    assert np.array_equal(got["codes"], qx.astype(np.int8)), f"activation codes of {regime} groups"
    assert np.array_equal(got["scales"], sx), f"activation scales of {regime} groups"


# ----------------------------------------------------------------------------
# LoRA adapter without re-quantization
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name,M,K,N,fmt", [("qkv", 4608, 3072, 9216, "int4"),
                                            ("lora_m64", 64, 3072, 3072, "int4"),
                                            ("lora_fp4", 700, 1536, 2048, "mxfp4"),
                                            ("lora_m40_fp4", 40, 1024, 2048, "mxfp4")])
def test_lora_extended_forward(name, M, K, N, fmt):
    """A rank-16 adapter on a rank-32 layer (rank 48 in all): only L1 and L2
    are re-laid and uploaded, the device buffers of mu, the 4-bit codes and
    scales and the bias are the base layer's. Y matches the oracle's
    extended layer (sampled rows at full size) to the Y bar."""
    _say(f"[lora] {name}")
    if name == "qkv":
        spec = synth.config_layers(1)[0]
    else:
        spec = _spec(name, M, K, N, 32, fmt, 43)
    layer, host = C.library_host(spec)
    _, dev = C.device_layer(spec)
    rng = np.random.default_rng(77)
    A = (rng.standard_normal((K, 16)) / np.sqrt(K)).astype(np.float32)
    B = (rng.standard_normal((16, N)) * 0.5).astype(np.float32)
    ext_layer, ext_host = S.lora_extend(layer, host, A, B, 2.0, share_base=True)
    ext_dev = dict(dev)
    for n in ("l1", "l2"):
        ext_dev[n] = torch.from_numpy(ext_host[n].copy()).cuda()
    x = C.x_device(spec)
    y = torch.full((spec.M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    S.linear_forward(ext_layer, ext_dev, x, y=y)
    torch.cuda.synchronize()
    ref = O.lora_extend(C.oracle_pack(spec), A, B, 2.0)
    rows = C.sample_rows(spec.M, n=64)
    lay = C.layer_data(spec)
    C.check_y(C.bf16_tensor_to_f32(y)[rows], O.forward(ref, lay.x[rows]), f"lora {name}")
    # the adapter's share of the output is really there: the base layer differs
    yb = S.linear_forward(layer, dev, x)
    torch.cuda.synchronize()
    d = C.bf16_tensor_to_f32(y)[rows].astype(np.float64) - C.bf16_tensor_to_f32(yb)[rows]
    want = 2.0 * (lay.x[rows].astype(np.float64) @ A) @ B
    assert np.linalg.norm(d - want) <= 0.05 * np.linalg.norm(want)
