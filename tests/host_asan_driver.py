"""Runs the library's host entry points (pack, residual quantization, LoRA
extension, unpack, sizes, workspace queries, argument checks) from a library
built with AddressSanitizer and UndefinedBehaviorSanitizer, and checks that
they give the bytes the regular build gives. Started by
tests/test_host_sanitizers.py in a process with libasan preloaded; any
sanitizer finding aborts it.

usage: python tests/host_asan_driver.py <sanitized lib> <regular lib>"""
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from bit_svdquant_diffusion_amd import LayerDesc, Packed, PackedSizes, PACKED_FIELDS  # noqa: E402


def load(path):
    L = ctypes.CDLL(path)
    vp, D, P = ctypes.c_void_p, ctypes.POINTER(LayerDesc), ctypes.POINTER
    sigs = {
        "svdq_packed_bytes": [D, P(PackedSizes)],
        "svdq_pack_weights": [D, vp, vp, vp, ctypes.c_uint64, P(Packed)],
        "svdq_quantize_residual": [D, vp, vp, vp, vp, vp, P(Packed)],
        "svdq_unpack_weights": [D, P(Packed), vp, vp, vp, vp, vp],
        "svdq_lora_extend": [D, P(Packed), ctypes.c_int32, vp, vp, ctypes.c_float, P(Packed)],
        "svdq_workspace_bytes": [D, ctypes.c_int64, P(ctypes.c_size_t)],
        "svdq_unpack_workspace": [D, ctypes.c_int64, vp, ctypes.c_size_t, vp, vp, vp],
    }
    for n, a in sigs.items():
        getattr(L, n).argtypes = a
        getattr(L, n).restype = ctypes.c_int
    L.svdq_status_string.restype = ctypes.c_char_p
    return L


def alloc(L, d):
    s = PackedSizes()
    assert L.svdq_packed_bytes(ctypes.byref(d), ctypes.byref(s)) == 0
    bufs = {n: np.zeros(max(getattr(s, n), 1), np.uint8) for n in PACKED_FIELDS}
    return bufs, Packed(*[bufs[n].ctypes.data for n in PACKED_FIELDS])


def run(L, K, N, r, fmt, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32) * 0.1
    ax = np.abs(rng.standard_normal((8, K))).max(0).astype(np.float32)
    d = LayerDesc(K, N, r, fmt)
    out = {}
    bufs, p = alloc(L, d)
    assert L.svdq_pack_weights(ctypes.byref(d), w.ctypes.data, b.ctypes.data, ax.ctypes.data, 7, ctypes.byref(p)) == 0
    out["pack"] = bufs
    g = 64 if fmt == 0 else 32
    codes = np.zeros((N, K), np.int8)
    scales = np.zeros((N, K // g), np.float32 if fmt == 0 else np.uint8)
    l1 = np.zeros((K, max(r, 1)), np.uint16)
    l2 = np.zeros((max(r, 1), N), np.uint16)
    bias = np.zeros(N, np.uint16)
    assert L.svdq_unpack_weights(ctypes.byref(d), ctypes.byref(p), codes.ctypes.data, scales.ctypes.data,
                                 l1.ctypes.data if r else None, l2.ctypes.data if r else None, bias.ctypes.data) == 0
    out["unpack"] = (codes, scales, l1, l2, bias)
    mu = bufs["mu"].view(np.float32)[:K].copy()
    bufs2, p2 = alloc(L, d)
    assert L.svdq_quantize_residual(ctypes.byref(d), w.ctypes.data, b.ctypes.data, mu.ctypes.data,
                                    l1.ctypes.data if r else None, l2.ctypes.data if r else None,
                                    ctypes.byref(p2)) == 0
    out["resid"] = bufs2
    if r + 16 <= min(K, N, 128):
        A = rng.standard_normal((K, 16)).astype(np.float32)
        B = rng.standard_normal((16, N)).astype(np.float32)
        de = LayerDesc(K, N, r + 16, fmt)
        bufs3, p3 = alloc(L, de)
        assert L.svdq_lora_extend(ctypes.byref(d), ctypes.byref(p), 16, A.ctypes.data, B.ctypes.data, 0.5,
                                  ctypes.byref(p3)) == 0
        out["lora"] = bufs3
    for M in (1, 33, 300):
        ws = ctypes.c_size_t()
        assert L.svdq_workspace_bytes(ctypes.byref(d), M, ctypes.byref(ws)) == 0
        wsb = np.zeros(ws.value, np.uint8)
        qx = np.zeros((M, K), np.int8)
        sx = np.zeros((M, K // g), np.float32 if fmt == 0 else np.uint8)
        z = np.zeros((M, max(r, 1)), np.float32)
        assert L.svdq_unpack_workspace(ctypes.byref(d), M, wsb.ctypes.data, wsb.nbytes, qx.ctypes.data,
                                       sx.ctypes.data, z.ctypes.data if r else None) == 0
    # argument checks: errors, no crash
    bad = LayerDesc(K + 8, N, r, fmt)
    assert L.svdq_pack_weights(ctypes.byref(bad), w.ctypes.data, None, ax.ctypes.data, 1, ctypes.byref(p)) == 2
    assert L.svdq_pack_weights(ctypes.byref(d), None, None, ax.ctypes.data, 1, ctypes.byref(p)) == 1
    for s in range(-1, 9):
        L.svdq_status_string(s)
    return out


def main():
    san, reg = load(sys.argv[1]), load(sys.argv[2])
    cases = [(256, 64, 16, 0, 1), (320, 40, 16, 0, 2), (384, 72, 32, 1, 3), (512, 96, 0, 1, 4),
             (192, 128, 112, 0, 5)]
    for c in cases:
        a, b = run(san, *c), run(reg, *c)
        for key in a:
            va, vb = a[key], b[key]
            if isinstance(va, dict):
                for n in va:
                    assert np.array_equal(va[n], vb[n]), (c, key, n)
            else:
                for x, y in zip(va, vb):
                    assert np.array_equal(x, y), (c, key)
        print("ok", c, flush=True)
    print("HOST_SANITIZED_OK")


if __name__ == "__main__":
    main()
