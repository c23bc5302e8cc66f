"""Python binding of librfx (the C ABI in include/rfx.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of librfx.so. PyTorch is used for device memory and streams; device
arguments are torch tensors (their data_ptr() is passed through) and the
stream defaults to torch's current stream.

The library must be built first (``python -m bit_block_quantized_amd.build``
or ``__graft_entry__.build()``); importing this package without it raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

FP2, FP3, FP4 = 2, 3, 4
FORMATS = (FP2, FP3, FP4)
# Variant: fp16 scale and fp16 minimum per block (weight = s * c + m),
# GEMV entry points only.
FP2M = 12
# A tier above FP4: 32 int8 codes + an fp16 scale (34 B), GEMV entry points only.
Q8 = 8
# Variant: FP2 codes with two fp16 sub-scales, one per 16-weight half (12 B),
# GEMV entry points only.
FP2S = 16
# A 3-bit tier at about 3.3 bits per weight: FP3 codes + an e8m0 byte (13 B),
# GEMV entry points only.
FP3E = 13
VARIANT_FORMATS = (FP2M, Q8, FP2S, FP3E)

RFX_OK = 0
RFX_E_TIMEOUT = -7
_STATUS = {-1: "RFX_E_INVAL", -2: "RFX_E_ALIGN", -3: "RFX_E_RANGE", -4: "RFX_E_UNSUPPORTED",
           -5: "RFX_E_WORKSPACE", -6: "RFX_E_HIP", -7: "RFX_E_TIMEOUT"}

HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(HERE, "librfx.so")


class RfxError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class QMat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("count", ctypes.c_int32), ("data", ctypes.c_void_p)]


class GemvJob(ctypes.Structure):
    _fields_ = [("W", QMat), ("q", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("xq", ctypes.c_void_p), ("xs", ctypes.c_void_p), ("xsum", ctypes.c_void_p),
                ("y", ctypes.c_void_p)]


MAX_GEMV_JOBS = 16


class MoeLayerC(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("gate", QMat), ("up", QMat), ("down", QMat),
                ("sh_gate", QMat), ("sh_up", QMat), ("sh_down", QMat),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("expert_data", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGS = {
    "rfx_status_str": ([_I], ctypes.c_char_p),
    "rfx_last_error": ([], ctypes.c_char_p),
    "rfx_version": ([], ctypes.c_char_p),
    "rfx_block_bytes": ([_I], _I),
    "rfx_code_bytes": ([_I], _I),
    "rfx_scale_bytes": ([_I], _I),
    "rfx_quantize_block": ([_I, _P, _P], _I),
    "rfx_dequantize_block": ([_I, _P, _P], _I),
    "rfx_qmat_bytes": ([_I, _I64, _I64], _I64),
    "rfx_quantize_matrix": ([_I, _P, _I64, _I64, _P, _I], _I),
    "rfx_export_blocks": ([_I, _P, _I64, _I64, _P], _I),
    "rfx_import_blocks": ([_I, _P, _I64, _I64, _P], _I),
    "rfx_quantize_act": ([_P, _I, _I, _P, _P, _P, _P], _I),
    "rfx_gemv_workspace_bytes": ([_P, _I], _SZ),
    "rfx_gemv": ([_P, _P, _P, _P, _I, _P, _P, _SZ, _P], _I),
    "rfx_gemv_noalloc": ([_P, _P, _P, _P, _I, _P, _P], _I),
    "rfx_gemv_q1": ([_P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "rfx_gemv_q4": ([_P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "rfx_gemv_grouped_workspace_bytes": ([_P, _I], _SZ),
    "rfx_gemv_grouped": ([_P, _I, _P, _SZ, _P], _I),
    "rfx_debug_block_dots": ([_P, _P, _P, _I, _P, _P], _I),
    "rfx_read_reference": ([_P, _SZ, _P, _I, _P], _I),
    "rfx_moe_workspace_bytes": ([_P, _I, _I], _SZ),
    "rfx_moe_route_topk": ([_P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "rfx_moe_ffn": ([_P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "rfx_moe_forward": ([_P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, ctypes.c_uint, _P], _I),
    "rfx_moe_forward_single_launch": ([_P, _I, _I], _I),
    "rfx_moe_forward_status": ([_P, _I, _I, _P, _SZ, _P], _I),
    "rfx_moe_debug_hidden": ([_P, _I, _I, _P, _SZ, _P, _P, _P, _P], _I),
    "rfx_moe_debug_prefill": ([_P, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _I, _I, _P, _P, _P, _P, _P], _I),
}

EXPORTED = tuple(_SIGS)

_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBPATH):
        raise ImportError(f"{LIBPATH} is missing: build it with "
                          "`python -m bit_block_quantized_amd.build`")
    L = ctypes.CDLL(LIBPATH)
    for name, (args, res) in _SIGS.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(st: int):
    if st != RFX_OK:
        raise RfxError(st, lib().rfx_last_error().decode())
    return st


def _check_nonneg(v: int):
    if v < 0:
        raise RfxError(v, lib().rfx_last_error().decode())
    return v


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dptr(t):
    """Device pointer of a torch tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ host

def block_bytes(fmt):
    return lib().rfx_block_bytes(fmt)


def code_bytes(fmt):
    return lib().rfx_code_bytes(fmt)


def scale_bytes(fmt):
    return lib().rfx_scale_bytes(fmt)


def qmat_bytes(fmt, rows, cols) -> int:
    n = lib().rfx_qmat_bytes(fmt, rows, cols)
    if n < 0:
        _check(int(n))
    return int(n)


def quantize_block(fmt, w) -> np.ndarray:
    w = np.ascontiguousarray(w, np.float32)
    if w.shape != (32,):
        raise ValueError("a block is 32 weights")
    out = np.zeros(max(block_bytes(fmt), 1), np.uint8)
    _check(lib().rfx_quantize_block(fmt, _np_ptr(w), _np_ptr(out)))
    return out


def dequantize_block(fmt, blk) -> np.ndarray:
    blk = np.ascontiguousarray(blk, np.uint8)
    out = np.zeros(32, np.float32)
    _check(lib().rfx_dequantize_block(fmt, _np_ptr(blk), _np_ptr(out)))
    return out


def quantize_matrix(fmt, W, threads: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """fp32 [rows][cols] -> tiled device layout (host uint8 array)."""
    W = np.ascontiguousarray(W, np.float32)
    rows, cols = W.shape
    n = qmat_bytes(fmt, rows, cols)
    if out is None:
        out = np.empty(n, np.uint8)
    elif out.nbytes < n or not out.flags.c_contiguous:
        raise ValueError("output buffer too small or not contiguous")
    _check(lib().rfx_quantize_matrix(fmt, _np_ptr(W), rows, cols, _np_ptr(out), threads))
    return out


def export_blocks(fmt, tiled, rows, cols) -> np.ndarray:
    tiled = np.ascontiguousarray(tiled, np.uint8)
    out = np.zeros((rows, cols // 32, block_bytes(fmt)), np.uint8)
    _check(lib().rfx_export_blocks(fmt, _np_ptr(tiled), rows, cols, _np_ptr(out)))
    return out


def import_blocks(fmt, blocks) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, np.uint8)
    rows, nb, bb = blocks.shape
    out = np.empty(qmat_bytes(fmt, rows, nb * 32), np.uint8)
    _check(lib().rfx_import_blocks(fmt, _np_ptr(blocks), rows, nb * 32, _np_ptr(out)))
    return out


# ---------------------------------------------------------------- device

class DeviceQMat:
    """A tiled matrix (or a stack of `count` matrices) in device memory."""

    def __init__(self, fmt, rows, cols, data, count=1):
        self.fmt, self.rows, self.cols, self.count = fmt, rows, cols, count
        self.data = data  # torch uint8 tensor on the GPU (kept alive here)
        self.c = QMat(fmt, rows, cols, count, _dptr(data))

    @classmethod
    def from_host(cls, fmt, rows, cols, tiled: np.ndarray, count=1, device="cuda"):
        import torch
        t = torch.from_numpy(np.ascontiguousarray(tiled)).to(device)
        return cls(fmt, rows, cols, t, count)

    def expert(self, e: int) -> "DeviceQMat":
        nb = qmat_bytes(self.fmt, self.rows, self.cols)
        return DeviceQMat(self.fmt, self.rows, self.cols, self.data[e * nb:(e + 1) * nb], 1)

    def ref(self):
        return ctypes.byref(self.c)


def quantize_act(x, xq, xs, xsum, stream=None):
    q, K = x.shape
    _check(lib().rfx_quantize_act(_dptr(x), q, K, _dptr(xq), _dptr(xs), _dptr(xsum),
                                  _stream(stream)))


def gemv_workspace_bytes(W: DeviceQMat, q: int) -> int:
    return int(lib().rfx_gemv_workspace_bytes(W.ref(), q))


def gemv(W: DeviceQMat, xq, xs, xsum, q, y, ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().rfx_gemv(W.ref(), _dptr(xq), _dptr(xs), _dptr(xsum), q, _dptr(y), _dptr(ws),
                          ws_bytes, _stream(stream)))


def gemv_noalloc(W: DeviceQMat, xq, xs, xsum, q, y, stream=None):
    """rfx_gemv with the library's own per-GPU scratch (no workspace)."""
    _check(lib().rfx_gemv_noalloc(W.ref(), _dptr(xq), _dptr(xs), _dptr(xsum), q, _dptr(y), _stream(stream)))


def gemv_q1(W: DeviceQMat, xq, xs, xsum, y, ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().rfx_gemv_q1(W.ref(), _dptr(xq), _dptr(xs), _dptr(xsum), _dptr(y), _dptr(ws),
                             ws_bytes, _stream(stream)))


def gemv_q4(W: DeviceQMat, xq, xs, xsum, y, ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().rfx_gemv_q4(W.ref(), _dptr(xq), _dptr(xs), _dptr(xsum), _dptr(y), _dptr(ws),
                             ws_bytes, _stream(stream)))


def gemv_jobs(jobs):
    """[(W: DeviceQMat, q, xq, xs, xsum, y), ...] -> ctypes array of rfx_gemv_job."""
    arr = (GemvJob * len(jobs))()
    for i, (W, q, xq, xs, xsum, y) in enumerate(jobs):
        arr[i] = GemvJob(W.c, q, 0, _dptr(xq), _dptr(xs), _dptr(xsum), _dptr(y))
    return arr


def gemv_grouped_workspace_bytes(jobs) -> int:
    arr = jobs if isinstance(jobs, ctypes.Array) else gemv_jobs(jobs)
    return int(lib().rfx_gemv_grouped_workspace_bytes(arr, len(arr)))


def gemv_grouped(jobs, ws=None, stream=None):
    """Several independent GEMVs in one launch; jobs as for gemv_jobs (or
    its result, reusable across calls)."""
    arr = jobs if isinstance(jobs, ctypes.Array) else gemv_jobs(jobs)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().rfx_gemv_grouped(arr, len(arr), _dptr(ws), ws_bytes, _stream(stream)))


def debug_block_dots(W: DeviceQMat, xq, xsum, q, dots, stream=None):
    _check(lib().rfx_debug_block_dots(W.ref(), _dptr(xq), _dptr(xsum), q, _dptr(dots),
                                      _stream(stream)))


def read_reference(buf, out, stream=None):
    """Measurement aid: stream `buf` (a device tensor) once; out (int32 or
    uint32 device tensor) gets one XOR fold per workgroup."""
    _check(lib().rfx_read_reference(_dptr(buf), buf.numel() * buf.element_size(), _dptr(out), out.numel(),
                                    _stream(stream)))


# ------------------------------------------------------------------ MoE

def moe_workspace_bytes(layer, q: int, k: int) -> int:
    return int(lib().rfx_moe_workspace_bytes(layer.ref(), q, k))


def moe_route_topk(layer, x, q, k, topk_idx, topk_w, pairs_sorted, expert_off, xq, xs, xsum, ws,
                   stream=None):
    _check(lib().rfx_moe_route_topk(layer.ref(), _dptr(x), q, k, _dptr(topk_idx), _dptr(topk_w),
                                    _dptr(pairs_sorted), _dptr(expert_off), _dptr(xq), _dptr(xs),
                                    _dptr(xsum), _dptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def moe_ffn(layer, q, k, xq, xs, xsum, topk_idx, topk_w, pairs_sorted, expert_off, y, ws,
            resid=None, stream=None):
    _check(lib().rfx_moe_ffn(layer.ref(), q, k, _dptr(xq), _dptr(xs), _dptr(xsum), _dptr(topk_idx),
                             _dptr(topk_w), _dptr(pairs_sorted), _dptr(expert_off), _dptr(resid),
                             _dptr(y), _dptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


FORWARD_ONE_LAUNCH = 1


def moe_forward(layer, x, q, k, y, topk_idx, topk_w, pairs_sorted, expert_off, xq, xs, xsum, ws,
                resid=None, one_launch=False, stream=None):
    """moe_route_topk then moe_ffn in one call; one_launch: the single-launch
    layer kernel where moe_forward_single_launch says it can take the call."""
    _check(lib().rfx_moe_forward(layer.ref(), _dptr(x), q, k, _dptr(resid), _dptr(y), _dptr(topk_idx),
                                 _dptr(topk_w), _dptr(pairs_sorted), _dptr(expert_off), _dptr(xq), _dptr(xs),
                                 _dptr(xsum), _dptr(ws), ws.numel() * ws.element_size(),
                                 FORWARD_ONE_LAUNCH if one_launch else 0, _stream(stream)))


def moe_forward_single_launch(layer, q: int, k: int) -> bool:
    return bool(_check_nonneg(lib().rfx_moe_forward_single_launch(layer.ref(), q, k)))


def moe_forward_status(layer, q, k, ws, stream=None):
    """Raises RfxError(RFX_E_TIMEOUT) if a bounded wait of the one-launch
    layer kernel ran out since the last check (synchronizes the stream)."""
    _check(lib().rfx_moe_forward_status(layer.ref(), q, k, _dptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream)))


def moe_debug_hidden(layer, q, k, ws, h=None, hq=None, hs=None, stream=None):
    _check(lib().rfx_moe_debug_hidden(layer.ref(), q, k, _dptr(ws), ws.numel() * ws.element_size(), _dptr(h),
                                      _dptr(hq), _dptr(hs), _stream(stream)))


def moe_debug_prefill(layer, q, k, xq, xs, topk_w, pairs_sorted, expert_off, ws, probe_expert, probe_first,
                      h=None, dots_gate=None, dots_up=None, dots_down=None, stream=None):
    """Test hook of the prefill path: reruns gate/up and down with the fp32 h
    and one work item's block dots stored (see include/rfx.h)."""
    _check(lib().rfx_moe_debug_prefill(layer.ref(), q, k, _dptr(xq), _dptr(xs), _dptr(topk_w), _dptr(pairs_sorted),
                                       _dptr(expert_off), _dptr(ws), ws.numel() * ws.element_size(), probe_expert,
                                       probe_first, _dptr(h), _dptr(dots_gate), _dptr(dots_up), _dptr(dots_down),
                                       _stream(stream)))


from .layer import DeviceMoeLayer, MoeBuffers, PlacedMoeLayer, hot_experts_by_frequency  # noqa: E402,F401
from . import layer  # noqa: E402,F401
