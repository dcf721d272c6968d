"""MI355X (gfx950) SVDQuant W4A4 linear layer.

A thin ctypes binding over libsvdq.so (C ABI in include/svdq.h): argument
marshalling only. Every step of the runtime path runs in the library's HIP
kernels; PyTorch is used for device memory and streams. The library must be
built (``python -m bit_svdquant_diffusion_amd.build``); without it every call
raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

__all__ = [
    "SvdqError", "FMT_INT4", "FMT_MXFP4", "LayerDesc", "lib", "lib_path", "status_string",
    "packed_bytes", "pack_weights", "quantize_residual", "unpack_weights", "workspace_bytes",
    "to_device", "linear_forward", "stage1", "gemm", "unpack_workspace", "debug_int4_group_sums",
    "SVDQLinear", "EXPORTED_SYMBOLS", "Layer",
]

FMT_INT4 = 0
FMT_MXFP4 = 1
FORMATS = {"int4": FMT_INT4, "mxfp4": FMT_MXFP4}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libsvdq.so"

EXPORTED_SYMBOLS = [
    "svdq_status_string", "svdq_version", "svdq_packed_bytes", "svdq_pack_weights",
    "svdq_quantize_residual", "svdq_unpack_weights", "svdq_workspace_bytes",
    "svdq_linear_forward", "svdq_stage1", "svdq_unpack_workspace",
    "svdq_debug_int4_group_sums", "svdq_gemm",
]


class SvdqError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}")


class LayerDesc(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("N", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("format", ctypes.c_int32)]


class PackedSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("mu", "l1", "l2", "qw", "sw", "bias")]


class Packed(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("mu", "l1", "l2", "qw", "sw", "bias")]


PACKED_FIELDS = ("mu", "l1", "l2", "qw", "sw", "bias")

_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """Load libsvdq.so (built in-tree). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m bit_svdquant_diffusion_amd.build`")
    L = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    D = P(LayerDesc)
    L.svdq_status_string.restype = ctypes.c_char_p
    L.svdq_status_string.argtypes = [ctypes.c_int]
    L.svdq_version.restype = ctypes.c_int32
    L.svdq_version.argtypes = []
    sigs = {
        "svdq_packed_bytes": [D, P(PackedSizes)],
        "svdq_pack_weights": [D, vp, vp, vp, ctypes.c_uint64, P(Packed)],
        "svdq_quantize_residual": [D, vp, vp, vp, vp, vp, P(Packed)],
        "svdq_unpack_weights": [D, P(Packed), vp, vp, vp, vp, vp],
        "svdq_workspace_bytes": [D, i64, P(sz)],
        "svdq_linear_forward": [D, P(Packed), vp, i64, vp, vp, sz, vp],
        "svdq_stage1": [D, P(Packed), vp, i64, vp, sz, vp],
        "svdq_gemm": [D, P(Packed), vp, sz, i64, vp, vp],
        "svdq_unpack_workspace": [D, i64, vp, sz, vp, vp, vp],
        "svdq_debug_int4_group_sums": [D, P(Packed), vp, sz, i64, i64, i64, i64, i64, vp, vp],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().svdq_status_string(int(status)).decode()


def _check(status: int, fn: str):
    if status != 0:
        raise SvdqError(status, fn)


def _desc(K: int, N: int, rank: int, fmt) -> LayerDesc:
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    return LayerDesc(int(K), int(N), int(rank), f)


def _ptr(a) -> int | None:
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"]
        return a.ctypes.data
    return a.data_ptr()   # torch tensor


@dataclass
class Layer:
    """Shape and format of one SVDQuant linear."""
    K: int
    N: int
    rank: int
    fmt: str

    @property
    def desc(self) -> LayerDesc:
        return _desc(self.K, self.N, self.rank, self.fmt)


def packed_bytes(layer: Layer) -> dict:
    s = PackedSizes()
    d = layer.desc
    _check(lib().svdq_packed_bytes(ctypes.byref(d), ctypes.byref(s)), "svdq_packed_bytes")
    return {n: getattr(s, n) for n in PACKED_FIELDS}


def _alloc_host(layer: Layer) -> tuple[dict, Packed]:
    sizes = packed_bytes(layer)
    bufs = {n: np.zeros(max(sizes[n], 1), dtype=np.uint8) for n in PACKED_FIELDS}
    p = Packed(*[bufs[n].ctypes.data if sizes[n] else None for n in PACKED_FIELDS])
    return bufs, p


def pack_weights(layer: Layer, w_lin: np.ndarray, bias: np.ndarray | None,
                 act_absmax: np.ndarray, seed: int = 0) -> dict:
    """svdq_pack_weights on host numpy arrays; returns host buffers (uint8 arrays)."""
    w = np.ascontiguousarray(w_lin, dtype=np.float32)
    ax = np.ascontiguousarray(act_absmax, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    bufs, p = _alloc_host(layer)
    d = layer.desc
    _check(lib().svdq_pack_weights(ctypes.byref(d), _ptr(w), _ptr(b), _ptr(ax), int(seed),
                                   ctypes.byref(p)), "svdq_pack_weights")
    return bufs


def quantize_residual(layer: Layer, w_lin, bias, mu, l1_bits, l2_bits) -> dict:
    """svdq_quantize_residual: host buffers from given mu (fp32 [K]) and bf16 factors."""
    w = np.ascontiguousarray(w_lin, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    mu = np.ascontiguousarray(mu, dtype=np.float32)
    l1 = np.ascontiguousarray(l1_bits, dtype=np.uint16)
    l2 = np.ascontiguousarray(l2_bits, dtype=np.uint16)
    bufs, p = _alloc_host(layer)
    d = layer.desc
    _check(lib().svdq_quantize_residual(ctypes.byref(d), _ptr(w), _ptr(b), _ptr(mu),
                                        _ptr(l1) if layer.rank else None,
                                        _ptr(l2) if layer.rank else None, ctypes.byref(p)),
           "svdq_quantize_residual")
    return bufs


def _packed_struct(layer: Layer, bufs: dict) -> Packed:
    sizes = packed_bytes(layer)
    return Packed(*[_ptr(bufs[n]) if sizes[n] else None for n in PACKED_FIELDS])


def unpack_weights(layer: Layer, host: dict) -> dict:
    """Logical codes [N][K], scales [N][K/g], l1 [K][r] / l2 [r][N] / bias bf16 bits."""
    K, N, r = layer.K, layer.N, layer.rank
    g = 64 if layer.fmt == "int4" else 32
    codes = np.zeros((N, K), np.int8)
    scales = np.zeros((N, K // g), np.float32 if layer.fmt == "int4" else np.uint8)
    l1 = np.zeros((K, r), np.uint16)
    l2 = np.zeros((r, N), np.uint16)
    bias = np.zeros(N, np.uint16)
    p = _packed_struct(layer, host)
    d = layer.desc
    _check(lib().svdq_unpack_weights(ctypes.byref(d), ctypes.byref(p), _ptr(codes), _ptr(scales),
                                     _ptr(l1) if r else None, _ptr(l2) if r else None, _ptr(bias)),
           "svdq_unpack_weights")
    mu = host["mu"].view(np.float32)[:K].copy()
    return dict(codes=codes, scales=scales, l1=l1, l2=l2, bias=bias, mu=mu)


def workspace_bytes(layer: Layer, M: int) -> int:
    out = ctypes.c_size_t()
    d = layer.desc
    _check(lib().svdq_workspace_bytes(ctypes.byref(d), int(M), ctypes.byref(out)),
           "svdq_workspace_bytes")
    return out.value


def to_device(layer: Layer, host: dict, device="cuda"):
    """Copy host buffers into torch device tensors (byte for byte)."""
    import torch
    sizes = packed_bytes(layer)
    return {n: torch.from_numpy(host[n][:max(sizes[n], 1)].copy()).to(device) for n in PACKED_FIELDS}


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def linear_forward(layer: Layer, dev: dict, x, y=None, workspace=None, stream=None):
    """y[M][N] (bf16 tensor) = layer(x[M][K] bf16 tensor) via svdq_linear_forward."""
    import torch
    assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape[-1] == layer.K
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, layer.N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(layer, M), 1), dtype=torch.uint8, device=x.device)
    p = _packed_struct(layer, dev)
    d = layer.desc
    _check(lib().svdq_linear_forward(ctypes.byref(d), ctypes.byref(p), _ptr(x), M, _ptr(y),
                                     _ptr(workspace), workspace.numel(), _stream(stream)),
           "svdq_linear_forward")
    return y


def stage1(layer: Layer, dev: dict, x, workspace=None, stream=None):
    import torch
    M = x.shape[0]
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(layer, M), 1), dtype=torch.uint8, device=x.device)
    p = _packed_struct(layer, dev)
    d = layer.desc
    _check(lib().svdq_stage1(ctypes.byref(d), ctypes.byref(p), _ptr(x), M, _ptr(workspace),
                             workspace.numel(), _stream(stream)), "svdq_stage1")
    return workspace


def gemm(layer: Layer, dev: dict, workspace, M: int, y, stream=None):
    """Kernel (2) alone on a workspace filled by stage1() for the same M."""
    p = _packed_struct(layer, dev)
    d = layer.desc
    _check(lib().svdq_gemm(ctypes.byref(d), ctypes.byref(p), _ptr(workspace), workspace.numel(),
                           int(M), _ptr(y), _stream(stream)), "svdq_gemm")
    return y


def unpack_workspace(layer: Layer, M: int, ws_host: np.ndarray) -> dict:
    K, r = layer.K, layer.rank
    g = 64 if layer.fmt == "int4" else 32
    codes = np.zeros((M, K), np.int8)
    scales = np.zeros((M, K // g), np.float32 if layer.fmt == "int4" else np.uint8)
    z = np.zeros((M, r), np.float32)
    ws = np.ascontiguousarray(ws_host, dtype=np.uint8)
    d = layer.desc
    _check(lib().svdq_unpack_workspace(ctypes.byref(d), int(M), _ptr(ws), ws.nbytes, _ptr(codes),
                                       _ptr(scales), _ptr(z) if r else None),
           "svdq_unpack_workspace")
    return dict(codes=codes, scales=scales, z=z)


def debug_int4_group_sums(layer: Layer, dev: dict, workspace, M: int, m0: int, mc: int,
                          n0: int, nc: int, stream=None):
    import torch
    p_out = torch.empty((mc, nc, layer.K // 64), dtype=torch.int32, device=workspace.device)
    p = _packed_struct(layer, dev)
    d = layer.desc
    _check(lib().svdq_debug_int4_group_sums(ctypes.byref(d), ctypes.byref(p), _ptr(workspace),
                                            workspace.numel(), int(M), int(m0), int(mc), int(n0),
                                            int(nc), _ptr(p_out), _stream(stream)),
           "svdq_debug_int4_group_sums")
    return p_out


class SVDQLinear:
    """A packed SVDQuant W4A4 linear held in device memory; call it on bf16 input."""

    def __init__(self, layer: Layer, host: dict, device="cuda"):
        self.layer = layer
        self.dev = to_device(layer, host, device)
        self._ws = None

    @classmethod
    def from_float(cls, w_lin, bias, act_absmax, rank: int, fmt: str, seed: int = 0, device="cuda"):
        N, K = w_lin.shape
        layer = Layer(K, N, rank, fmt)
        return cls(layer, pack_weights(layer, w_lin, bias, act_absmax, seed), device)

    def __call__(self, x, y=None, stream=None):
        import torch
        need = max(workspace_bytes(self.layer, x.shape[0]), 1)
        if self._ws is None or self._ws.numel() < need or self._ws.device != x.device:
            self._ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        return linear_forward(self.layer, self.dev, x, y=y, workspace=self._ws, stream=stream)
