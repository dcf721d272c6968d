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
    (500, 512, 16, 0, 2),      # K % 256
    (512, 500, 16, 0, 2),      # N % 32
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
        assert out.mu == 4 * K and out.qw == N * K // 2
        assert out.l1 == K * r32 * 2 and out.l2 == N * r32 * 2 and out.bias == 2 * N
        assert out.sw == (N * K // 64 * 4 if fmt == 0 else N * K // 32)


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
    # INT4 activation codes use 32-bit byte offsets: round32(M) * K <= 2^33
    big4 = S.LayerDesc(65536, 512, 16, 0)
    for M, want in ((1 << 17, 4), ((1 << 17) + 1, 2), (1 << 20, 2)):
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
