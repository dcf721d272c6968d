"""The C-ABI library loads without a GPU, exports every symbol its header
declares, and its host-side validation returns the documented status codes.
No GPU kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_svdquant_diffusion_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    hdr = open(os.path.join(ROOT, "include", "svdq.h")).read()
    return sorted(set(re.findall(r"SVDQ_API\s+[\w\s\*]+?\b(svdq_\w+)\s*\(", hdr)))


def test_header_symbols_exported():
    L = S.lib()
    decl = _declared()
    assert len(decl) >= 11
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(S.EXPORTED_SYMBOLS) == decl


def test_status_strings():
    for s in range(7):
        assert S.status_string(s).startswith("SVDQ_")
    assert "UNKNOWN" in S.status_string(99)
    assert S.lib().svdq_version() >= 100


@pytest.mark.parametrize("K,N,r,fmt,status", [
    (512, 512, 16, 0, 0), (3072, 12288, 32, 1, 0),
    (320, 40, 16, 0, 0),       # INT4 takes K % 64, N % 8 (padded inside)
    (384, 72, 32, 1, 0),       # MXFP4 takes K % 128
    (500, 512, 16, 0, 2),      # K % 64
    (320, 64, 16, 1, 2),       # MXFP4 K % 128
    (512, 500, 16, 0, 2),      # N % 8
    (512, 36, 16, 0, 2),       # N % 8
    (512, 512, 17, 0, 2),      # rank % 16
    (512, 512, 144, 0, 2),     # rank > 128
    (256, 32, 48, 0, 2),       # rank > N
    (512, 512, 16, 7, 3),      # format
    (0, 512, 0, 0, 2), (131072, 32, 0, 0, 2),
])
def test_desc_validation(K, N, r, fmt, status):
    d = S.LayerDesc(K, N, r, fmt)
    out = S.PackedSizes()
    assert S.lib().svdq_packed_bytes(ctypes.byref(d), ctypes.byref(out)) == status
    if status == 0:
        r32 = (r + 31) // 32 * 32
        Kp, Np = (K + 255) // 256 * 256, (N + 31) // 32 * 32
        assert out.mu == 4 * K and out.qw == Np * Kp // 2
        assert out.l1 == Kp * r32 * 2 and out.l2 == Np * r32 * 2 and out.bias == 2 * Np
        assert out.sw == (Np * Kp // 64 * 4 if fmt == 0 else Np * Kp // 32)


def test_null_pointers():
    L = S.lib()
    d = S.LayerDesc(512, 512, 16, 0)
    assert L.svdq_packed_bytes(None, None) == 1
    assert L.svdq_packed_bytes(ctypes.byref(d), None) == 1
    sz = ctypes.c_size_t()
    assert L.svdq_workspace_bytes(ctypes.byref(d), -1, ctypes.byref(sz)) == 2
    assert L.svdq_workspace_bytes(ctypes.byref(d), 256, ctypes.byref(sz)) == 0 and sz.value > 0
    p = S.Packed()
    assert L.svdq_pack_weights(ctypes.byref(d), None, None, None, 0, ctypes.byref(p)) == 1
    # forward/stage1 validate before touching the device: null packed buffers -> NULL
    assert L.svdq_linear_forward(ctypes.byref(d), ctypes.byref(p), None, 4, None, None, 0, None) == 1
    assert L.svdq_stage1(ctypes.byref(d), None, None, 4, None, 0, None) == 1
    assert L.svdq_stage1_outputs(ctypes.byref(d), None, None, 4, None, None, None, None, 0, None) == 1
    # a misaligned fp32 output is refused before anything else
    assert L.svdq_stage1_outputs(ctypes.byref(d), ctypes.byref(p), None, 4, None, None, ctypes.c_void_p(2), None,
                                 0, None) == 2


def test_forward_validation_before_device():
    """Shape/workspace errors come back before any HIP call (host pointers are fine here)."""
    L = S.lib()
    layer = S.Layer(512, 512, 16, "int4")
    d = layer.desc
    bufs = {n: np.zeros(64, np.uint8) for n in S.PACKED_FIELDS}
    p = S.Packed(*[b.ctypes.data for b in bufs.values()])
    x = np.zeros(16, np.uint16)
    ws = np.zeros(64, np.uint8)
    y = np.zeros(16, np.uint16)
    # M == 0 is a no-op
    assert L.svdq_linear_forward(ctypes.byref(d), ctypes.byref(p), None, 0, None, None, 0, None) == 0
    # workspace too small
    st = L.svdq_linear_forward(ctypes.byref(d), ctypes.byref(p), x.ctypes.data, 4, y.ctypes.data,
                               ws.ctypes.data, ws.nbytes, None)
    assert st == 4
    # M too large
    st = L.svdq_linear_forward(ctypes.byref(d), ctypes.byref(p), x.ctypes.data, 1 << 25,
                               y.ctypes.data, ws.ctypes.data, ws.nbytes, None)
    assert st == 2
    # MXFP4 activation scales use 32-bit stage offsets: (K + 128) * ceil(M / 32) < 2^31
    big = S.LayerDesc(65536, 512, 16, 1)
    for M, want in ((32704 * 32, 4), (32705 * 32, 2), (1 << 20, 2)):
        st = L.svdq_linear_forward(ctypes.byref(big), ctypes.byref(p), x.ctypes.data, M, y.ctypes.data,
                                   ws.ctypes.data, ws.nbytes, None)
        assert st == want, (M, st)
    # the tiled INT4 GEMM's FP6 activation codes use 32-bit byte offsets:
    # round32(M) * K * 3 / 4 < 2^32 (below 4 GiB; 87360 * 65536 * 3 / 4 is
    # the largest multiple of 32 rows under it)
    big4 = S.LayerDesc(65536, 512, 16, 0)
    for M, want in ((87360, 4), (87361, 2), (1 << 17, 2), (1 << 20, 2)):
        st = L.svdq_linear_forward(ctypes.byref(big4), ctypes.byref(p), x.ctypes.data, M, y.ctypes.data,
                                   ws.ctypes.data, ws.nbytes, None)
        assert st == want, (M, st)
        st = L.svdq_debug_int4_group_sums(ctypes.byref(big4), ctypes.byref(p), ws.ctypes.data, ws.nbytes, M,
                                          0, 1, 0, 1, ws.ctypes.data, None)
        assert st == want, ("group sums", M, st)
    # debug hook: format and window checks
    d4 = S.LayerDesc(512, 512, 16, 1)
    pp = ctypes.byref(p)
    assert L.svdq_debug_int4_group_sums(ctypes.byref(d4), pp, ws.ctypes.data, ws.nbytes, 4, 0, 1, 0, 1,
                                        ws.ctypes.data, None) == 3


def test_workspace_layout_monotone():
    layer = S.Layer(3072, 9216, 32, "int4")
    a, b = S.workspace_bytes(layer, 100), S.workspace_bytes(layer, 4608)
    assert a < b
    assert b >= 4608 * 3072 // 2 + 4608 * 48 * 4 + 4608 * 32 * 2


def test_pack_rejects_nonfinite():
    layer = S.Layer(256, 32, 16, "int4")
    rng = np.random.default_rng(0)
    w = rng.standard_normal((32, 256)).astype(np.float32)
    ax = np.ones(256, np.float32)
    w[3, 7] = np.nan
    with pytest.raises(S.SvdqError) as e:
        S.pack_weights(layer, w, None, ax)
    assert e.value.status == 5
    w[3, 7] = 0
    ax[5] = np.inf
    with pytest.raises(S.SvdqError) as e:
        S.pack_weights(layer, w, None, ax)
    assert e.value.status == 5


def test_pack_svd_nonconvergence_reported(monkeypatch):
    layer = S.Layer(256, 64, 16, "int4")
    rng = np.random.default_rng(1)
    w = rng.standard_normal((64, 256)).astype(np.float32)
    ax = np.ones(256, np.float32)
    monkeypatch.setenv("SVDQ_JACOBI_MAX_SWEEPS", "0")
    with pytest.raises(S.SvdqError) as e:
        S.pack_weights(layer, w, None, ax)
    assert e.value.status == 5
    monkeypatch.delenv("SVDQ_JACOBI_MAX_SWEEPS")
    S.pack_weights(layer, w, None, ax)


def test_noalloc_host_checks():
    """svdq_linear_forward_noalloc refuses, on the host and before touching a
    device, an M whose workspace exceeds the library's array, and treats
    M == 0 as a no-op."""
    L = S.lib()
    assert S.NOALLOC_SCRATCH_BYTES == 256 << 20
    buf = np.zeros(1 << 16, np.uint8)
    p = S.Packed(*([buf.ctypes.data] * 6))
    x = np.zeros(16, np.uint16)
    for K, N, fmt in ((3072, 9216, 0), (12288, 3072, 0), (3072, 12288, 1)):
        d = S.LayerDesc(K, N, 32, fmt)
        # 4608 tokens fit (the documented bound); far more do not
        assert S.workspace_bytes(S.Layer(K, N, 32, "int4" if fmt == 0 else "mxfp4"), 4608) <= S.NOALLOC_SCRATCH_BYTES
        big = 1 << 18   # its workspace exceeds the array in every format
        assert S.workspace_bytes(S.Layer(K, N, 32, "int4" if fmt == 0 else "mxfp4"), big) > S.NOALLOC_SCRATCH_BYTES
        assert L.svdq_linear_forward_noalloc(ctypes.byref(d), ctypes.byref(p), x.ctypes.data, big,
                                             x.ctypes.data, None) == 4
        assert L.svdq_linear_forward_noalloc(ctypes.byref(d), ctypes.byref(p), x.ctypes.data, 0,
                                             x.ctypes.data, None) == 0
        assert L.svdq_linear_forward_noalloc(ctypes.byref(d), ctypes.byref(p), x.ctypes.data, -1,
                                             x.ctypes.data, None) == 2


def test_mlp_host_logic():
    """svdq_mlp_workspace_bytes / svdq_mlp_fused / svdq_mlp_forward host
    checks: the layout holds both layers' workspaces and the larger of the
    hidden activation and the fused partial Z; the fused path needs one
    format for both layers, whole tile columns of hidden channels and more
    than 256 tokens."""
    up = S.Layer(3072, 12288, 32, "int4")
    down = S.Layer(12288, 3072, 32, "int4")
    M = 4608
    total, off = S.mlp_workspace_bytes(up, down, M)
    wu, wd = S.workspace_bytes(up, M), S.workspace_bytes(down, M)
    assert off >= wu and off % 256 == 0
    assert total >= off + wd + M * 12288 * 2
    assert S.mlp_fused(up, down, M) and S.mlp_fused(up, down, 257)
    assert not S.mlp_fused(up, down, 256)
    assert S.mlp_fused(S.Layer(3072, 12288, 32, "mxfp4"), S.Layer(12288, 3072, 32, "mxfp4"), M)
    # mixed formats, and hidden widths that are not whole tile columns (256 INT4, 384 MXFP4)
    assert not S.mlp_fused(S.Layer(3072, 12288, 32, "mxfp4"), S.Layer(12288, 3072, 32, "int4"), M)
    assert not S.mlp_fused(S.Layer(3072, 12160, 32, "int4"), S.Layer(12160, 3072, 32, "int4"), M)
    assert not S.mlp_fused(S.Layer(3072, 12544, 32, "mxfp4"), S.Layer(12544, 3072, 32, "mxfp4"), M)
    assert not S.mlp_fused(S.Layer(3072, 1152, 32, "mxfp4"), S.Layer(1152, 3072, 32, "mxfp4"), M)
    assert S.mlp_fused(S.Layer(3072, 1536, 32, "mxfp4"), S.Layer(1536, 3072, 32, "mxfp4"), M)
    with pytest.raises(S.SvdqError) as e:   # down K != up N
        S.mlp_workspace_bytes(up, S.Layer(3072, 3072, 32, "int4"), M)
    assert e.value.status == 2
    L = S.lib()
    bufs = {n: np.zeros(64, np.uint8) for n in S.PACKED_FIELDS}
    p = S.Packed(*[b.ctypes.data for b in bufs.values()])
    du, dd = up.desc, down.desc
    x = np.zeros(16, np.uint16)
    ws = np.zeros(64, np.uint8)
    # M == 0: no-op; unknown mode; short workspace (all before any HIP call)
    assert L.svdq_mlp_forward(ctypes.byref(du), ctypes.byref(p), ctypes.byref(dd), ctypes.byref(p), None, 0,
                              None, None, 0, 0, None) == 0
    assert L.svdq_mlp_forward(ctypes.byref(du), ctypes.byref(p), ctypes.byref(dd), ctypes.byref(p),
                              x.ctypes.data, 4, x.ctypes.data, ws.ctypes.data, ws.nbytes, 5, None) == 2
    assert L.svdq_mlp_forward(ctypes.byref(du), ctypes.byref(p), ctypes.byref(dd), ctypes.byref(p),
                              x.ctypes.data, 4, x.ctypes.data, ws.ctypes.data, ws.nbytes, 0, None) == 4
    assert L.svdq_mlp_forward(None, ctypes.byref(p), ctypes.byref(dd), ctypes.byref(p),
                              x.ctypes.data, 4, x.ctypes.data, ws.ctypes.data, ws.nbytes, 0, None) == 1


def test_missing_library_fails_loudly(monkeypatch):
    """Without libsvdq.so the binding raises: there is no CPU fallback."""
    monkeypatch.setattr(S, "_lib", None)
    monkeypatch.setattr(S, "lib_path", lambda: "/nonexistent/libsvdq.so")
    with pytest.raises(RuntimeError, match="missing"):
        S.lib()
    layer = S.Layer(512, 512, 16, "int4")
    with pytest.raises(RuntimeError, match="missing"):
        S.workspace_bytes(layer, 64)
