"""CPU oracle for the block-quantized decode path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg import this package. It shares no code with
the GPU library and never imports it; the GPU library never imports this.

The scalar arithmetic (block encoder, decoder, activation quantizer, exact
per-block integer dots with fp64 accumulation) is plain C in ``oracle.c``.
This module wraps it with ctypes and composes the MoE layer from it in
numpy fp64: router logits, softmax, top-k by a full stable sort, stable
bucketing of (token, slot) pairs by expert, SwiGLU, requantization of the
intermediate activation, down projection and the weighted combine.

Pages cited (title, site):
  [HM]  "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
        (hellomarvisaitoday.com), paragraphs numbered from the top.
  [AIN] "Token Freedom via APU: AMD Ryzen AI MAX+ 395 Runs DeepSeek V4
        Flash at 32 tok/s on a 284B Model" (ainomam.com), by section.
  [KK]  the kaikai365.com post on DeepSeek V4 Flash on Strix Halo, by
        section heading.

Parity status: every function here is pinned by the not-gpu tests
(hand-worked blocks, brute force, closed forms, invariants, library
identities) except where a docstring says "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

FP2, FP3, FP4 = 2, 3, 4
FORMATS = (FP2, FP3, FP4)
# Variant with a scale and a minimum per block (weight = s * c + m, 12 B):
# the pages let a block carry a second small value; this one is a reading.
FP2M = 12
# A tier above FP4 (the same paragraph keeps dense and sensitive
# projections at FP4 or higher): 32 int8 codes + an fp16 scale, 34 B.
Q8 = 8
# Variant with two 16-weight sub-scales (each half an FP2 block of its own,
# 12 B): the second of the two small values a block may carry is a second
# scale; a reading.
FP2S = 16
# A 3-bit tier at about 3.3 bits per weight (the figure another system on
# the pages gives for its 3-bit experts): FP3 codes + an e8m0 byte, 13 B.
FP3E = 13
VARIANT_FORMATS = (FP2M, Q8, FP2S, FP3E)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i8p = ctypes.POINTER(ctypes.c_int8)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_intp = ctypes.POINTER(ctypes.c_int)


def lib():
    """Load liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIBPATH):
        from . import build as _b
        _b.build()
    L = ctypes.CDLL(_LIBPATH)
    L.orc_block_bytes.argtypes = [ctypes.c_int]
    L.orc_code_bytes.argtypes = [ctypes.c_int]
    L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_f16_to_f64.restype = ctypes.c_double
    L.orc_f32_to_f16.argtypes = [ctypes.c_float]
    L.orc_f32_to_f16.restype = ctypes.c_uint16
    L.orc_codebook.argtypes = [ctypes.c_int, ctypes.c_int]
    L.orc_nearest_code.argtypes = [ctypes.c_int, ctypes.c_double]
    L.orc_unpack_codes.argtypes = [ctypes.c_int, _u8p, _intp]
    L.orc_unpack_codes.restype = None
    L.orc_pack_codes.argtypes = [ctypes.c_int, _intp, _u8p]
    L.orc_pack_codes.restype = None
    L.orc_block_scale.argtypes = [ctypes.c_int, _u8p]
    L.orc_block_scale.restype = ctypes.c_double
    L.orc_block_min.argtypes = [ctypes.c_int, _u8p]
    L.orc_block_min.restype = ctypes.c_double
    L.orc_weight_scale.argtypes = [ctypes.c_int, _u8p, ctypes.c_int]
    L.orc_weight_scale.restype = ctypes.c_double
    L.orc_dequantize_block.argtypes = [ctypes.c_int, _u8p, _f64p]
    L.orc_dequantize_block.restype = None
    L.orc_dequantize_matrix.argtypes = [ctypes.c_int, _u8p, ctypes.c_int64, ctypes.c_int64, _f64p]
    L.orc_dequantize_matrix.restype = None
    L.orc_quantize_block.argtypes = [ctypes.c_int, _f32p, _u8p]
    L.orc_quantize_matrix.argtypes = [ctypes.c_int, _f32p, ctypes.c_int64, ctypes.c_int64, _u8p]
    L.orc_quantize_act.argtypes = [_f32p, ctypes.c_int64, _i8p, _f32p]
    L.orc_gemv.argtypes = [ctypes.c_int, _u8p, ctypes.c_int64, ctypes.c_int64, _i8p, _f32p,
                           ctypes.c_int, _f64p, _i32p]
    _lib = L
    return L


def _p(a, t):
    return a.ctypes.data_as(t)


class OracleError(RuntimeError):
    pass


def _check(st):
    if st != 0:
        raise OracleError(f"oracle status {st}")


# ---------------------------------------------------------------- format

def block_bytes(fmt: int) -> int:
    """Bytes per 32-weight block: 10 / 14 / 17 ([HM] para 2)."""
    return lib().orc_block_bytes(fmt)


def code_bytes(fmt: int) -> int:
    return lib().orc_code_bytes(fmt)


def codebook(fmt: int, code: int) -> int:
    return lib().orc_codebook(fmt, code)


def nearest_code(fmt: int, t: float) -> int:
    return lib().orc_nearest_code(fmt, float(t))


def f32_to_f16(x: float) -> int:
    return int(lib().orc_f32_to_f16(float(np.float32(x))))


def f16_to_f64(h: int) -> float:
    return float(lib().orc_f16_to_f64(int(h)))


def quantize_block(fmt: int, w) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.shape == (32,)
    out = np.zeros(block_bytes(fmt), np.uint8)
    _check(lib().orc_quantize_block(fmt, _p(w, _f32p), _p(out, _u8p)))
    return out


def unpack_codes(fmt: int, blk) -> np.ndarray:
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    codes = np.zeros(32, np.intc)
    lib().orc_unpack_codes(fmt, _p(blk, _u8p), _p(codes, _intp))
    return codes.astype(np.int64)


def pack_codes(fmt: int, codes) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.intc)
    out = np.zeros(block_bytes(fmt), np.uint8)
    lib().orc_pack_codes(fmt, _p(codes, _intp), _p(out, _u8p))
    return out[: code_bytes(fmt)]


def block_scale(fmt: int, blk) -> float:
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    return float(lib().orc_block_scale(fmt, _p(blk, _u8p)))


def weight_scale(fmt: int, blk, t: int) -> float:
    """Scale of weight t of a block: FP2S's scale of the half holding t,
    the block scale otherwise."""
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    return float(lib().orc_weight_scale(fmt, _p(blk, _u8p), t))


def block_min(fmt: int, blk) -> float:
    """FP2M's fp16 minimum (0 for the symmetric formats)."""
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    return float(lib().orc_block_min(fmt, _p(blk, _u8p)))


def dequantize_block(fmt: int, blk) -> np.ndarray:
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    out = np.zeros(32, np.float64)
    lib().orc_dequantize_block(fmt, _p(blk, _u8p), _p(out, _f64p))
    return out


def quantize_matrix(fmt: int, W) -> np.ndarray:
    """fp32 [N][K] -> canonical blocks uint8 [N][K/32][block_bytes]."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    out = np.zeros((N, K // 32, block_bytes(fmt)), np.uint8)
    _check(lib().orc_quantize_matrix(fmt, _p(W, _f32p), N, K, _p(out, _u8p)))
    return out


def dequantize_matrix(fmt: int, blocks) -> np.ndarray:
    """Canonical blocks [N][K/32][bb] -> fp64 [N][K]: dequantize_block on
    every block (one C loop)."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    N, nb, bb = blocks.shape
    assert bb == block_bytes(fmt)
    out = np.zeros((N, nb * 32), np.float64)
    lib().orc_dequantize_matrix(fmt, _p(blocks, _u8p), N, nb, _p(out, _f64p))
    return out


# ----------------------------------------------------------- activations

def quantize_act(x):
    """fp32 [q][K] (or [K]) -> (int8 [q][K], fp32 scales [q][K/32]).

    Per 32-block: s = amax/127 in fp32, q = clamp(rne(x/s), +-127)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    squeeze = x.ndim == 1
    x2 = x.reshape(-1, x.shape[-1])
    q = np.zeros(x2.shape, np.int8)
    s = np.zeros((x2.shape[0], x2.shape[1] // 32), np.float32)
    _check(lib().orc_quantize_act(_p(x2, _f32p), x2.size, _p(q, _i8p), _p(s, _f32p)))
    if squeeze:
        return q[0], s[0]
    return q, s


def act_sums(xq) -> np.ndarray:
    """Per-32-block integer sums of quantized activations, int32 [q][K/32]."""
    xq = np.asarray(xq)
    return xq.reshape(*xq.shape[:-1], -1, 32).astype(np.int64).sum(-1).astype(np.int32)


# ----------------------------------------------------------------- gemv

def gemv(fmt: int, blocks, xq, xs, want_dots: bool = False):
    """y[j][n] = sum_b S[n,b] * s[j,b] * D[j,n,b] in fp64 (exact int dots);
    FP2M adds s[j,b] * M[n,b] * X[j,b] (X the activation block sum); FP2S
    takes s[j,b] * (S0 D0 + S1 D1) over the two halves (the dots returned
    are D = D0 + D1).

    blocks: uint8 [N][K/32][bb]; xq int8 [Q][K]; xs fp32 [Q][K/32].
    Returns fp64 [Q][N] (and int32 dots [Q][N][K/32] when asked)."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    xq = np.ascontiguousarray(np.atleast_2d(xq), dtype=np.int8)
    xs = np.ascontiguousarray(np.atleast_2d(xs), dtype=np.float32)
    N, nb, bb = blocks.shape
    assert bb == block_bytes(fmt)
    Q, K = xq.shape
    assert K == nb * 32 and xs.shape == (Q, nb)
    y = np.zeros((Q, N), np.float64)
    dots = np.zeros((Q, N, nb), np.int32) if want_dots else None
    _check(lib().orc_gemv(fmt, _p(blocks, _u8p), N, K, _p(xq, _i8p), _p(xs, _f32p), Q,
                          _p(y, _f64p), _p(dots, _i32p) if want_dots else None))
    return (y, dots) if want_dots else y


# ---------------------------------------------------------------- router

def route(x, Wr, bias, k: int):
    """Router: logits l = x.Wr^T (+ bias) in fp64; experts ranked by a full
    stable sort on (-l, e) so equal logits go to the lower expert id; the
    first k are picked; weights are the softmax over all experts of the
    picked ones, not renormalised. ([HM] para 3 and [KK] DSpark section name
    the TOP_K and ARGSORT routing step; the arithmetic is a reading.)

    x fp32 [T][H]; Wr fp32 [E][H]; bias fp32 [E] or None."""
    x64 = np.asarray(x, np.float64)
    l = x64 @ np.asarray(Wr, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    T, E = l.shape
    idx = np.zeros((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -l[t]))  # primary -l, then e
        idx[t] = order[:k]
    m = l.max(axis=1, keepdims=True)
    p = np.exp(l - m)
    p /= p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return {"logits": l, "probs": p, "idx": idx, "w": w}


def bucket(idx, n_experts: int):
    """Stable grouping of (token, slot) pairs by expert. Pair p = t*k + j.
    pairs_sorted = stable argsort of the pairs' expert ids; expert_off is
    the exclusive prefix sum of per-expert counts (length E + 1)."""
    e_of_pair = np.asarray(idx).reshape(-1)
    pairs_sorted = np.argsort(e_of_pair, kind="stable").astype(np.int32)
    counts = np.bincount(e_of_pair, minlength=n_experts)
    off = np.zeros(n_experts + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return pairs_sorted, off


# ------------------------------------------------------------- expert FFN

def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def ffn(gate_fmt, gate_blk, up_fmt, up_blk, down_fmt, down_blk, xq, xs, hq_override=None):
    """One expert's SwiGLU FFN over a few tokens.

    g = G.x~, u = U.x~ (fp64); h = silu(g) * u; h~ = activation quantizer
    applied to fp32(h); o = D.h~. xq int8 [n][H], xs [n][H/32].
    hq_override = (hq, hs) feeds given quantized h instead (stage-wise
    checks). Returns dict with g, u, h (fp64), hq, hs, o (fp64 [n][H_out])."""
    g = gemv(gate_fmt, gate_blk, xq, xs)
    u = gemv(up_fmt, up_blk, xq, xs)
    h = silu(g) * u
    if hq_override is None:
        hq, hs = quantize_act(h.astype(np.float32))
    else:
        hq, hs = hq_override
    o = gemv(down_fmt, down_blk, hq, hs)
    return {"g": g, "u": u, "h": h, "hq": hq, "hs": hs, "o": o}


def combine(o_shared, o_pairs, w):
    """y[t] = o_shared[t] + sum_j w[t][j] * o_pairs[t][j], fp64, j ascending.
    o_shared [T][H]; o_pairs [T][k][H]; w [T][k]."""
    y = np.array(o_shared, np.float64, copy=True)
    T, k = np.asarray(w).shape
    for t in range(T):
        for j in range(k):
            y[t] += float(w[t][j]) * np.asarray(o_pairs[t][j], np.float64)
    return y
