"""Host pack of libsvdq (C++, no GPU) against the CPU oracle.

mu is bit-exact; given the oracle's smoothing and bf16 factors the library's
residual codes and scales are bit-exact; the library's own randomized SVD
lands within the Eckart-Young bound of the oracle's exact truncated SVD."""
import numpy as np
import pytest

import bit_svdquant_diffusion_amd as S
from bit_svdquant_diffusion_amd import synth
from oracle import svdq_oracle as O


def _layer(spec_idx=0, fmt=None, K=None, N=None, r=None, M=None, seed=None):
    spec = synth.config_layers(spec_idx)[0]
    if any(v is not None for v in (fmt, K, N, r, M, seed)):
        spec = synth.LayerSpec("t", M or spec.M, K or spec.K, N or spec.N,
                               spec.rank if r is None else r, fmt or spec.fmt,
                               spec.seed if seed is None else seed)
    return spec, synth.make_layer(spec)


CASES = [
    dict(),                                  # config 0: 256x512->512 r16 INT4
    dict(fmt="mxfp4"),                       # same shapes, MXFP4
    dict(K=256, N=96, r=0, M=40, seed=3),    # no low-rank branch
    dict(K=256, N=128, r=128, M=40, seed=4), # rank == min(K, N) limit of the ABI
    dict(K=768, N=224, r=48, M=64, seed=5, fmt="mxfp4"),
    dict(K=320, N=40, r=16, M=32, seed=6),                  # K % 64, N % 8: padded inside
    dict(K=384, N=72, r=32, M=32, seed=6, fmt="mxfp4"),     # K % 128
]


@pytest.mark.parametrize("case", CASES)
def test_quantize_residual_bit_exact(case):
    spec, lay = _layer(**case)
    ax = np.abs(lay.x).max(axis=0)
    ref = O.pack(lay.w_lin, lay.bias, ax, spec.rank, spec.fmt)
    layer = S.Layer(spec.K, spec.N, spec.rank, spec.fmt)
    host = S.quantize_residual(layer, lay.w_lin, lay.bias, ref["mu"],
                               O.bf16_to_bits(ref["l1"]), O.bf16_to_bits(ref["l2"]))
    u = S.unpack_weights(layer, host)
    assert np.array_equal(u["mu"], ref["mu"])
    want_codes = ref["qw"].astype(np.int8)
    assert np.array_equal(u["codes"], want_codes)
    assert np.array_equal(u["scales"], ref["sw"])
    assert np.array_equal(u["l1"], O.bf16_to_bits(ref["l1"]))
    assert np.array_equal(u["l2"], O.bf16_to_bits(ref["l2"]))
    assert np.array_equal(u["bias"], O.bf16_to_bits(lay.bias))


@pytest.mark.parametrize("case", CASES)
def test_pack_weights_smoothing_and_svd(case):
    spec, lay = _layer(**case)
    ax = np.abs(lay.x).max(axis=0)
    layer = S.Layer(spec.K, spec.N, spec.rank, spec.fmt)
    host = S.pack_weights(layer, lay.w_lin, lay.bias, ax, seed=7)
    u = S.unpack_weights(layer, host)
    _, mu = O.smoothing_factors(ax, lay.w_lin)
    assert np.array_equal(u["mu"], mu)                                   # bit-exact
    wh = O.smoothed_weight(lay.w_lin, mu)
    l1 = O.bf16_from_bits(u["l1"]).astype(np.float64)
    l2 = O.bf16_from_bits(u["l2"]).astype(np.float64)
    err_lib = np.sum((wh - l1 @ l2) ** 2)
    ol1, ol2 = O.low_rank_factors(wh, spec.rank, round_bf16=True)
    err_or = np.sum((wh - ol1.astype(np.float64) @ ol2.astype(np.float64)) ** 2)
    sv = np.linalg.svd(wh, compute_uv=False)
    tail = np.sum(sv[spec.rank:] ** 2)
    # randomized SVD within 1e-3 of the exact truncated SVD (both bf16-rounded)
    assert err_lib <= err_or * (1 + 1e-3) + 1e-12 * np.sum(sv ** 2)
    assert err_lib >= tail * (1 - 1e-9)
    # the codes are the oracle's quantization of the residual against these factors
    ref = O.pack(lay.w_lin, lay.bias, ax, spec.rank, spec.fmt,
                 factors=(u["mu"], O.bf16_from_bits(u["l1"]), O.bf16_from_bits(u["l2"])))
    assert np.array_equal(u["codes"], ref["qw"].astype(np.int8))
    assert np.array_equal(u["scales"], ref["sw"])


def test_pack_deterministic_and_seeded():
    spec, lay = _layer()
    ax = np.abs(lay.x).max(axis=0)
    layer = S.Layer(spec.K, spec.N, spec.rank, spec.fmt)
    a = S.pack_weights(layer, lay.w_lin, lay.bias, ax, seed=1)
    b = S.pack_weights(layer, lay.w_lin, lay.bias, ax, seed=1)
    for n in S.PACKED_FIELDS:
        assert np.array_equal(a[n], b[n])


def test_pack_null_bias_is_zero():
    spec, lay = _layer(K=256, N=64, r=16, M=8, seed=9)
    ax = np.abs(lay.x).max(axis=0)
    layer = S.Layer(spec.K, spec.N, spec.rank, spec.fmt)
    u = S.unpack_weights(layer, S.pack_weights(layer, lay.w_lin, None, ax))
    assert np.all(u["bias"] == 0)


def test_device_layout_of_l1_matches_stage1_order():
    """L1 is stored so that lane 16j+c of MFMA t of wave w in step s holds
    L1[256s+64w+16j+8t+e][16cb+c]."""
    K, N, r = 512, 64, 48
    layer = S.Layer(K, N, r, "int4")
    rng = np.random.default_rng(2)
    l1 = O.bf16_to_bits(O.to_bf16(rng.standard_normal((K, r))))
    l2 = O.bf16_to_bits(O.to_bf16(rng.standard_normal((r, N))))
    host = S.quantize_residual(layer, rng.standard_normal((N, K)).astype(np.float32), None,
                               np.ones(K, np.float32), l1, l2)
    dev_l1 = host["l1"].view(np.uint16).reshape(K // 256, 4, 4, 2, 64, 8)   # r32 = 64: 4 blocks of 16
    for (k, c) in [(0, 0), (5, 47), (200, 33), (255, 16), (300, 1), (511, 40), (77, 20)]:
        s, kk = divmod(k, 256)
        w, kk = divmod(kk, 64)
        j, kk = divmod(kk, 16)
        t, e = divmod(kk, 8)
        assert dev_l1[s, w, c // 16, t, 16 * j + c % 16, e] == l1[k, c]
    assert np.all(dev_l1[:, :, 3] == 0)   # columns 48..63 are padding
    # L2^T in 16-column fragment order: [N/32][r32/16][lane 32h + row%32][8]
    dev_l2 = host["l2"].view(np.uint16).reshape(N // 32, 4, 2, 32, 8)
    lin = dev_l2.transpose(0, 3, 1, 2, 4).reshape(N, 64)   # [n][16c + 8h + e]
    assert np.array_equal(lin[:, :r], l2.T) and np.all(lin[:, r:] == 0)


@pytest.mark.parametrize("fmt,r0,ra", [("int4", 16, 16), ("mxfp4", 32, 16), ("int4", 0, 32), ("mxfp4", 96, 32)])
def test_lora_extend_matches_oracle(fmt, r0, ra):
    """svdq_lora_extend: the extended L1 and L2 are bit-exact with the
    oracle's (base factors kept, adapter columns bf16(A scale / mu) and rows
    bf16(B)); codes, scales, mu and bias are the base layer's bytes."""
    spec, lay = _layer(K=512, N=256, r=r0, M=64, seed=7, fmt=fmt)
    ax = np.abs(lay.x).max(axis=0)
    ref = O.pack(lay.w_lin, lay.bias, ax, r0, fmt)
    layer = S.Layer(512, 256, r0, fmt)
    host = S.quantize_residual(layer, lay.w_lin, lay.bias, ref["mu"],
                               O.bf16_to_bits(ref["l1"]), O.bf16_to_bits(ref["l2"]))
    rng = np.random.default_rng(9)
    A = (rng.standard_normal((512, ra)) / 20).astype(np.float32)
    B = (rng.standard_normal((ra, 256)) / 5).astype(np.float32)
    ext_layer, ext = S.lora_extend(layer, host, A, B, 0.625)
    assert ext_layer.rank == r0 + ra
    want = O.lora_extend(ref, A, B, 0.625)
    u = S.unpack_weights(ext_layer, ext)
    assert np.array_equal(u["l1"], O.bf16_to_bits(want["l1"]))
    assert np.array_equal(u["l2"], O.bf16_to_bits(want["l2"]))
    for n in ("qw", "sw", "mu", "bias"):
        assert np.array_equal(ext[n], host[n]), n
    # sharing the base's buffers: only l1 and l2 are written
    _, shared = S.lora_extend(layer, host, A, B, 0.625, share_base=True)
    assert np.array_equal(shared["l1"], ext["l1"]) and np.array_equal(shared["l2"], ext["l2"])
    assert shared["qw"] is host["qw"]


def test_lora_extend_errors():
    import ctypes
    spec, lay = _layer(K=256, N=128, r=112, M=16, seed=8)
    ax = np.abs(lay.x).max(axis=0)
    ref = O.pack(lay.w_lin, lay.bias, ax, 112, "int4")
    layer = S.Layer(256, 128, 112, "int4")
    host = S.quantize_residual(layer, lay.w_lin, lay.bias, ref["mu"],
                               O.bf16_to_bits(ref["l1"]), O.bf16_to_bits(ref["l2"]))
    A = np.ones((256, 32), np.float32)
    B = np.ones((32, 128), np.float32)
    with pytest.raises(S.SvdqError) as e:          # 112 + 32 > 128
        S.lora_extend(layer, host, A, B, 1.0)
    assert e.value.status == 2
    with pytest.raises(S.SvdqError) as e:          # rank not a multiple of 16
        S.lora_extend(layer, host, A[:, :8], B[:8], 1.0)
    assert e.value.status == 2
    A16, B16 = A[:, :16].copy(), B[:16].copy()
    A16[3, 2] = np.nan
    with pytest.raises(S.SvdqError) as e:
        S.lora_extend(layer, host, A16, B16, 1.0)
    assert e.value.status == 5
    L = S.lib()
    p = S._packed_struct(layer, host)
    out = S.Packed()
    assert L.svdq_lora_extend(ctypes.byref(layer.desc), ctypes.byref(p), 0, A.ctypes.data, B.ctypes.data,
                              1.0, ctypes.byref(out)) == 2
    assert L.svdq_lora_extend(ctypes.byref(layer.desc), ctypes.byref(p), 16, A.ctypes.data, B.ctypes.data,
                              1.0, ctypes.byref(out)) == 1


@pytest.mark.parametrize("fmt,K,N", [("int4", 320, 40), ("mxfp4", 384, 72)])
def test_padding_is_zero(fmt, K, N):
    """Channels K..Kp and rows N..Np of the device layout are zero (codes,
    scales, L1 rows, L2 columns, bias), so they add nothing to the GEMM."""
    spec, lay = _layer(K=K, N=N, r=16, M=32, seed=9, fmt=fmt)
    ax = np.abs(lay.x).max(axis=0)
    layer = S.Layer(K, N, 16, fmt)
    host = S.pack_weights(layer, lay.w_lin, lay.bias, ax, seed=1)
    Kp, Np = 512, (N + 31) // 32 * 32
    qw = host["qw"].reshape(Np // 32, Kp // 64, 64, 16)
    # rows past N: lanes 32h + r with 32 b + r >= N
    for b in range(Np // 32):
        for lane in range(64):
            if 32 * b + lane % 32 >= N:
                assert not qw[b, :, lane].any()
    # channels past K: whole 64-channel steps past K // 64
    assert not qw[:, K // 64:].any()
    bias = host["bias"].view(np.uint16)
    assert not bias[N:Np].any()
    if fmt == "int4":
        sw = host["sw"].view(np.float32).reshape(Kp // 64, Np)
        assert not sw[K // 64:].any() and not sw[:, N:].any()
