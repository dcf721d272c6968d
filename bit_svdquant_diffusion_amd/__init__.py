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
    "packed_bytes", "pack_weights", "quantize_residual", "lora_extend", "unpack_weights", "workspace_bytes",
    "to_device", "linear_forward", "linear_forward_noalloc", "stage1", "gemm", "unpack_workspace", "debug_int4_group_sums",
    "SVDQLinear", "EXPORTED_SYMBOLS", "Layer", "measure_mfma_peak", "measure_copy",
    "awq_packed_bytes", "awq_pack", "awq_unpack", "awq_to_device", "awq_forward",
    "pack_weights_gpu", "calibrate_alpha", "to_host", "mlp_workspace_bytes", "mlp_fused", "mlp_forward",
    "MLP_AUTO", "MLP_UNFUSED", "stage1_outputs",
]

FMT_INT4 = 0
FMT_MXFP4 = 1
FORMATS = {"int4": FMT_INT4, "mxfp4": FMT_MXFP4}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libsvdq.so"

EXPORTED_SYMBOLS = [
    "svdq_status_string", "svdq_version", "svdq_packed_bytes", "svdq_pack_weights",
    "svdq_quantize_residual", "svdq_unpack_weights", "svdq_workspace_bytes",
    "svdq_linear_forward", "svdq_stage1", "svdq_stage1_outputs", "svdq_unpack_workspace",
    "svdq_debug_int4_group_sums", "svdq_gemm", "svdq_linear_forward_noalloc", "svdq_lora_extend",
    "svdq_measure_mfma_peak", "svdq_measure_copy",
    "svdq_awq_packed_bytes", "svdq_awq_pack", "svdq_awq_unpack", "svdq_awq_forward",
    "svdq_pack_gpu_workspace_bytes", "svdq_pack_weights_gpu", "svdq_calibrate_workspace_bytes",
    "svdq_calibrate_alpha", "svdq_mlp_workspace_bytes", "svdq_mlp_fused", "svdq_mlp_forward",
]

# svdq_mlp_forward modes
MLP_AUTO = 0
MLP_UNFUSED = 1

# bytes of the library-owned device workspace of svdq_linear_forward_noalloc
NOALLOC_SCRATCH_BYTES = 256 << 20


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


class AwqDesc(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("N", ctypes.c_int32)]


AWQ_FIELDS = ("inv_s", "qw", "scales", "zeros", "bias")


class AwqSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in AWQ_FIELDS]


class AwqPacked(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in AWQ_FIELDS]

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
        "svdq_lora_extend": [D, P(Packed), ctypes.c_int32, vp, vp, ctypes.c_float, P(Packed)],
        "svdq_measure_mfma_peak": [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(ctypes.c_double), vp],
        "svdq_measure_copy": [vp, vp, sz, vp],
        "svdq_awq_packed_bytes": [P(AwqDesc), P(AwqSizes)],
        "svdq_awq_pack": [P(AwqDesc), vp, vp, vp, i64, ctypes.c_float, P(ctypes.c_double), vp, P(AwqPacked)],
        "svdq_awq_unpack": [P(AwqDesc), P(AwqPacked), vp, vp, vp],
        "svdq_awq_forward": [P(AwqDesc), P(AwqPacked), vp, i64, vp, vp],
        "svdq_pack_gpu_workspace_bytes": [D, P(sz)],
        "svdq_pack_weights_gpu": [D, vp, vp, vp, ctypes.c_float, ctypes.c_uint64, P(Packed), vp, sz, vp],
        "svdq_calibrate_workspace_bytes": [D, i64, P(sz)],
        "svdq_calibrate_alpha": [D, vp, vp, vp, i64, vp, ctypes.c_int32, ctypes.c_uint64, P(ctypes.c_float),
                                 vp, P(Packed), vp, sz, vp],
        "svdq_workspace_bytes": [D, i64, P(sz)],
        "svdq_linear_forward": [D, P(Packed), vp, i64, vp, vp, sz, vp],
        "svdq_linear_forward_noalloc": [D, P(Packed), vp, i64, vp, vp],
        "svdq_stage1": [D, P(Packed), vp, i64, vp, sz, vp],
        "svdq_stage1_outputs": [D, P(Packed), vp, i64, vp, vp, vp, vp, sz, vp],
        "svdq_gemm": [D, P(Packed), vp, sz, i64, vp, vp],
        "svdq_unpack_workspace": [D, i64, vp, sz, vp, vp, vp],
        "svdq_debug_int4_group_sums": [D, P(Packed), vp, sz, i64, i64, i64, i64, i64, vp, vp],
        "svdq_mlp_workspace_bytes": [D, D, i64, P(sz), P(sz)],
        "svdq_mlp_fused": [D, D, i64, P(ctypes.c_int32)],
        "svdq_mlp_forward": [D, P(Packed), D, P(Packed), vp, i64, vp, vp, sz, ctypes.c_int32, vp],
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


def lora_extend(layer: Layer, host: dict, lora_a, lora_b, scale: float, share_base: bool = False):
    """svdq_lora_extend: (extended Layer, host buffers) of `layer` with the LoRA
    adapter scale * X A B (A fp32 [K][r_a], B fp32 [r_a][N]) in its 16-bit
    branch. With share_base, only l1 and l2 are returned (the rest of the base
    layer's buffers are used as they are)."""
    a = np.ascontiguousarray(lora_a, dtype=np.float32)
    b = np.ascontiguousarray(lora_b, dtype=np.float32)
    ra = a.shape[1]
    assert a.shape == (layer.K, ra) and b.shape == (ra, layer.N)
    ext = Layer(layer.K, layer.N, layer.rank + ra, layer.fmt)
    bufs, p = _alloc_host(ext)
    if share_base:
        for n in ("mu", "qw", "sw", "bias"):
            setattr(p, n, None)
    base = _packed_struct(layer, host)
    _check(lib().svdq_lora_extend(ctypes.byref(layer.desc), ctypes.byref(base), int(ra), _ptr(a), _ptr(b),
                                  float(scale), ctypes.byref(p)), "svdq_lora_extend")
    if share_base:
        bufs = {n: (bufs[n] if n in ("l1", "l2") else host[n]) for n in PACKED_FIELDS}
    return ext, bufs


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


def linear_forward_noalloc(layer: Layer, dev: dict, x, y, stream=None):
    """svdq_linear_forward_noalloc: y (caller's bf16 tensor [M][N]) = layer(x),
    with the library's own device workspace (no allocation by the call)."""
    import torch
    assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape[-1] == layer.K
    assert y.dtype == torch.bfloat16 and y.is_contiguous() and tuple(y.shape) == (x.shape[0], layer.N)
    p = _packed_struct(layer, dev)
    d = layer.desc
    _check(lib().svdq_linear_forward_noalloc(ctypes.byref(d), ctypes.byref(p), _ptr(x), x.shape[0],
                                             _ptr(y), _stream(stream)),
           "svdq_linear_forward_noalloc")
    return y


def mlp_workspace_bytes(up: Layer, down: Layer, M: int):
    """(total bytes, offset of the down layer's part) of svdq_mlp_forward's workspace."""
    out, off = ctypes.c_size_t(), ctypes.c_size_t()
    du, dd = up.desc, down.desc
    _check(lib().svdq_mlp_workspace_bytes(ctypes.byref(du), ctypes.byref(dd), int(M), ctypes.byref(out),
                                          ctypes.byref(off)), "svdq_mlp_workspace_bytes")
    return out.value, off.value


def mlp_fused(up: Layer, down: Layer, M: int) -> bool:
    """Whether svdq_mlp_forward in MLP_AUTO mode takes the fused path for M tokens."""
    f = ctypes.c_int32()
    du, dd = up.desc, down.desc
    _check(lib().svdq_mlp_fused(ctypes.byref(du), ctypes.byref(dd), int(M), ctypes.byref(f)), "svdq_mlp_fused")
    return bool(f.value)


def mlp_forward(up: Layer, dev_up: dict, down: Layer, dev_down: dict, x, y=None, workspace=None,
                mode: int = MLP_AUTO, stream=None):
    """y[M][down N] = down(GELU(up(x))) via svdq_mlp_forward (bf16 tensors)."""
    import torch
    assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape[-1] == up.K
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, down.N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(mlp_workspace_bytes(up, down, M)[0], 1), dtype=torch.uint8, device=x.device)
    pu, pd = _packed_struct(up, dev_up), _packed_struct(down, dev_down)
    du, dd = up.desc, down.desc
    _check(lib().svdq_mlp_forward(ctypes.byref(du), ctypes.byref(pu), ctypes.byref(dd), ctypes.byref(pd), _ptr(x), M, _ptr(y), _ptr(workspace), workspace.numel(),
                                  int(mode), _stream(stream)), "svdq_mlp_forward")
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


def stage1_outputs(layer: Layer, dev: dict, x, workspace=None, codes=None, scales=None, z=None,
                   stream=None) -> dict:
    """Kernel (1) with its outputs in logical layouts as device tensors:
    codes int8 [M][K], scales float32 [M][K/64] (INT4) or uint8 [M][K/32]
    (MXFP4), z float32 [M][rank]; allocated here unless given."""
    import torch
    M = x.shape[0]
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(layer, M), 1), dtype=torch.uint8, device=x.device)
    g = 64 if layer.fmt == "int4" else 32
    if codes is None:
        codes = torch.empty((M, layer.K), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((M, layer.K // g), dtype=torch.float32 if layer.fmt == "int4" else torch.uint8,
                             device=x.device)
    if z is None:
        z = torch.empty((M, layer.rank), dtype=torch.float32, device=x.device)
    assert codes.shape == (M, layer.K) and codes.dtype == torch.int8 and codes.is_contiguous()
    assert scales.shape == (M, layer.K // g) and scales.is_contiguous()
    assert scales.dtype == (torch.float32 if layer.fmt == "int4" else torch.uint8)
    assert z.shape == (M, layer.rank) and z.dtype == torch.float32 and z.is_contiguous()
    p = _packed_struct(layer, dev)
    d = layer.desc
    _check(lib().svdq_stage1_outputs(ctypes.byref(d), ctypes.byref(p), _ptr(x), M, _ptr(codes), _ptr(scales),
                                     _ptr(z) if layer.rank else None, _ptr(workspace), workspace.numel(),
                                     _stream(stream)), "svdq_stage1_outputs")
    return {"codes": codes, "scales": scales, "z": z, "workspace": workspace}


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
                          n0: int, nc: int, stream=None, out=None):
    """int32 group sums P [mc][nc][K/64] of the window, from the GEMM kernel the
    forward runs for this M. ``out`` (int32 device tensor of that shape) is
    written in place when given."""
    import torch
    p_out = out if out is not None else torch.empty((mc, nc, layer.K // 64), dtype=torch.int32,
                                                    device=workspace.device)
    assert p_out.dtype == torch.int32 and p_out.is_contiguous() and p_out.numel() == mc * nc * (layer.K // 64)
    p = _packed_struct(layer, dev)
    d = layer.desc
    _check(lib().svdq_debug_int4_group_sums(ctypes.byref(d), ctypes.byref(p), _ptr(workspace),
                                            workspace.numel(), int(M), int(m0), int(mc), int(n0),
                                            int(nc), _ptr(p_out), _stream(stream)),
           "svdq_debug_int4_group_sums")
    return p_out


MFMA_KINDS = {"mxfp4": 0, "int8": 1, "bf16": 2}


def measure_mfma_peak(kind: str, iters: int, constant: bool = False, stream=None) -> float:
    """Enqueue the MFMA-only loop of `kind` on the current stream; returns its
    flop count (time it with events on the same stream)."""
    f = ctypes.c_double()
    _check(lib().svdq_measure_mfma_peak(MFMA_KINDS[kind], 1 if constant else 0, int(iters), ctypes.byref(f),
                                        _stream(stream)), "svdq_measure_mfma_peak")
    return f.value


def measure_copy(src, dst, stream=None):
    """Enqueue dst = src (device tensors of the same byte size) on the stream."""
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nbytes
    _check(lib().svdq_measure_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "svdq_measure_copy")


# ----------------------------------------------------------------------------
# GPU-side pack and the calibrated smoothing strength
# ----------------------------------------------------------------------------
def _alloc_device(layer: Layer, device="cuda") -> dict:
    import torch
    sizes = packed_bytes(layer)
    return {n: torch.zeros(max(sizes[n], 1), dtype=torch.uint8, device=device) for n in PACKED_FIELDS}


def pack_weights_gpu(layer: Layer, w_lin, bias, act_absmax, alpha: float = 0.5, seed: int = 0, stream=None):
    """svdq_pack_weights_gpu: device tensors in (fp32 w_lin [N][K], bias [N] or
    None, act_absmax [K]); returns the packed layer as device uint8 tensors."""
    import torch
    dev = _alloc_device(layer, w_lin.device)
    d = layer.desc
    n = ctypes.c_size_t()
    _check(lib().svdq_pack_gpu_workspace_bytes(ctypes.byref(d), ctypes.byref(n)), "svdq_pack_gpu_workspace_bytes")
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=w_lin.device)
    p = _packed_struct(layer, dev)
    _check(lib().svdq_pack_weights_gpu(ctypes.byref(d), _ptr(w_lin), _ptr(bias), _ptr(act_absmax), float(alpha),
                                       int(seed), ctypes.byref(p), _ptr(ws), ws.numel(), _stream(stream)),
           "svdq_pack_weights_gpu")
    return dev


def calibrate_alpha(layer: Layer, w_lin, bias, x_cal, alphas, seed: int = 0, stream=None):
    """svdq_calibrate_alpha: (packed device layer of the best alpha, alpha, losses)."""
    import torch
    dev = _alloc_device(layer, w_lin.device)
    d = layer.desc
    M = x_cal.shape[0]
    n = ctypes.c_size_t()
    _check(lib().svdq_calibrate_workspace_bytes(ctypes.byref(d), M, ctypes.byref(n)),
           "svdq_calibrate_workspace_bytes")
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=w_lin.device)
    al = np.ascontiguousarray(alphas, dtype=np.float32)
    losses = np.zeros(len(al), np.float64)
    a_out = ctypes.c_float()
    p = _packed_struct(layer, dev)
    _check(lib().svdq_calibrate_alpha(ctypes.byref(d), _ptr(w_lin), _ptr(bias), _ptr(x_cal), M, _ptr(al), len(al),
                                      int(seed), ctypes.byref(a_out), _ptr(losses), ctypes.byref(p), _ptr(ws),
                                      ws.numel(), _stream(stream)), "svdq_calibrate_alpha")
    return dev, a_out.value, losses


def to_host(dev: dict) -> dict:
    """Device packed buffers back to host uint8 arrays (byte for byte)."""
    return {n: t.cpu().numpy() for n, t in dev.items()}


# ----------------------------------------------------------------------------
# AWQ-style W4A16 linear (adaptive-normalization and modulation layers)
# ----------------------------------------------------------------------------
def awq_packed_bytes(K: int, N: int) -> dict:
    s = AwqSizes()
    d = AwqDesc(int(K), int(N))
    _check(lib().svdq_awq_packed_bytes(ctypes.byref(d), ctypes.byref(s)), "svdq_awq_packed_bytes")
    return {n: getattr(s, n) for n in AWQ_FIELDS}


def awq_pack(w_lin: np.ndarray, bias, x_cal: np.ndarray, alpha: float | None = None):
    """svdq_awq_pack on host arrays: (host buffers, chosen alpha, s float64 [K])."""
    w = np.ascontiguousarray(w_lin, dtype=np.float32)
    N, K = w.shape
    xc = np.ascontiguousarray(x_cal, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    sizes = awq_packed_bytes(K, N)
    bufs = {n: np.zeros(max(sizes[n], 1), np.uint8) for n in AWQ_FIELDS}
    p = AwqPacked(*[bufs[n].ctypes.data for n in AWQ_FIELDS])
    a_out = ctypes.c_double()
    s_out = np.zeros(K, np.float64)
    d = AwqDesc(K, N)
    _check(lib().svdq_awq_pack(ctypes.byref(d), _ptr(w), _ptr(b), _ptr(xc), xc.shape[0],
                               -1.0 if alpha is None else float(alpha), ctypes.byref(a_out), _ptr(s_out),
                               ctypes.byref(p)), "svdq_awq_pack")
    return bufs, a_out.value, s_out


def _awq_struct(bufs: dict) -> AwqPacked:
    return AwqPacked(*[_ptr(bufs[n]) for n in AWQ_FIELDS])


def awq_unpack(K: int, N: int, host: dict) -> dict:
    codes = np.zeros((N, K), np.uint8)
    scales = np.zeros((N, K // 128), np.float32)
    zeros = np.zeros((N, K // 128), np.uint8)
    d = AwqDesc(int(K), int(N))
    p = _awq_struct(host)
    _check(lib().svdq_awq_unpack(ctypes.byref(d), ctypes.byref(p), _ptr(codes), _ptr(scales), _ptr(zeros)),
           "svdq_awq_unpack")
    return dict(codes=codes, scales=scales, zeros=zeros, inv_s=host["inv_s"].view(np.float32)[:K].copy(),
                bias=host["bias"].view(np.uint16)[:N].copy())


def awq_to_device(host: dict, device="cuda") -> dict:
    import torch
    return {n: torch.from_numpy(host[n].copy()).to(device) for n in AWQ_FIELDS}


def awq_forward(K: int, N: int, dev: dict, x, y=None, stream=None):
    """y[M][N] bf16 = AWQ layer(x[M][K] bf16) via svdq_awq_forward."""
    import torch
    assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape[-1] == K
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    d = AwqDesc(int(K), int(N))
    p = _awq_struct(dev)
    _check(lib().svdq_awq_forward(ctypes.byref(d), ctypes.byref(p), _ptr(x), M, _ptr(y), _stream(stream)),
           "svdq_awq_forward")
    return y


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
