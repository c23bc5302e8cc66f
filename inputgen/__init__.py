"""Seeded synthetic inputs for the block-quantized decode path.

This module only draws numbers. It holds none of the method's arithmetic
(no quantization, no codebooks, no products): both the CPU oracle and the
GPU library receive the arrays made here, so the two sides see the same
fp32 inputs bit for bit.

Every stream is a counter-based Philox4x32-10 generator (numpy's
``np.random.Philox``) keyed by what the numbers are for, so any single
matrix (one expert of one layer, say) can be regenerated on its own without
drawing the others first. Normals come from numpy's float32 ziggurat.

Workload shapes and distributions follow the dense-GEMV and MoE-decode
workloads: weights N(0, 0.02) with an optional 1% outlier mask scaled by
10, activations N(0, 1), router weights N(0, 0.02), and a Zipf(1.1) router
bias that skews which experts get picked.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Domain tags keep the key spaces of different purposes apart.
_DOM_DENSE_W = 1
_DOM_DENSE_X = 2
_DOM_OUTLIER = 3
_DOM_EXPERT = 4
_DOM_ROUTER = 5
_DOM_PERM = 6
_DOM_TOKENS = 7
_DOM_RAW = 8

MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2
MAT_SH_GATE, MAT_SH_UP, MAT_SH_DOWN = 3, 4, 5

WEIGHT_SIGMA = np.float32(0.02)


def _gen(domain: int, *ids: int) -> np.random.Generator:
    """A Philox stream keyed by (domain, ids...) packed into 128 bits."""
    lo = 0
    for i in ids:
        if not 0 <= i < (1 << 20):
            raise ValueError("stream id out of range")
        lo = (lo << 20) | int(i)
    if lo >= (1 << 64):
        raise ValueError("too many stream ids")
    key = (int(domain) << 64) | lo
    return np.random.Generator(np.random.Philox(key=key))


def normal(gen: np.random.Generator, shape, sigma=1.0) -> np.ndarray:
    z = gen.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        z *= np.float32(sigma)
    return z


def dense_weight(rows: int, cols: int, seed: int, outliers: bool = False) -> np.ndarray:
    """fp32 [rows][cols] ~ N(0, 0.02); with ``outliers`` a Bernoulli(0.01)
    mask (its own stream) multiplies the chosen entries by 10."""
    w = normal(_gen(_DOM_DENSE_W, seed), (rows, cols), WEIGHT_SIGMA)
    if outliers:
        m = _gen(_DOM_OUTLIER, seed).random((rows, cols), dtype=np.float32) < np.float32(0.01)
        w[m] *= np.float32(10.0)
    return w


def activations(q: int, cols: int, seed: int) -> np.ndarray:
    """fp32 [q][cols] ~ N(0, 1); column j uses stream (seed + j)."""
    return np.stack([normal(_gen(_DOM_DENSE_X, seed + j), cols) for j in range(q)])


def expert_weight(layer: int, expert: int, mat: int, rows: int, cols: int) -> np.ndarray:
    """fp32 [rows][cols] ~ N(0, 0.02) for one matrix of one expert.

    ``expert`` = n_experts names the shared expert (use MAT_SH_*)."""
    return normal(_gen(_DOM_EXPERT, layer, expert, mat), (rows, cols), WEIGHT_SIGMA)


def router_weight(layer: int, n_experts: int, hidden: int) -> np.ndarray:
    """fp32 [n_experts][hidden] ~ N(0, 0.02)."""
    return normal(_gen(_DOM_ROUTER, layer), (n_experts, hidden), WEIGHT_SIGMA)


def zipf_router_bias(layer: int, n_experts: int, s: float = 1.1) -> np.ndarray:
    """fp32 [n_experts]: b_e = ln(r_e^-s / H) with r_e = pi(e) + 1 the rank
    of expert e under a seeded permutation pi, H the generalised harmonic
    number. Adding it to the logits makes the top-k pick roughly a Zipf(s)
    draw without replacement (the realised histogram is what tests report)."""
    perm = _gen(_DOM_PERM, layer).permutation(n_experts)
    r = perm.astype(np.float64) + 1.0
    h = float(np.sum(np.arange(1, n_experts + 1, dtype=np.float64) ** -s))
    return (np.log(r ** -s / h)).astype(np.float32)


def tokens(layer: int, step: int, q: int, hidden: int) -> np.ndarray:
    """fp32 [q][hidden] ~ N(0, 1) hidden states for one decode step."""
    return normal(_gen(_DOM_TOKENS, layer, step), (q, hidden))


def raw_normal(seed: int, shape, sigma=1.0) -> np.ndarray:
    """A generic seeded fp32 normal array for small test cases."""
    return normal(_gen(_DOM_RAW, seed), shape, sigma)


def raw_uniform_int(seed: int, shape, lo: int, hi: int) -> np.ndarray:
    """Seeded integers in [lo, hi) (int64)."""
    return _gen(_DOM_RAW, seed).integers(lo, hi, size=shape)


def parallel_map(fn, items, workers: int | None = None):
    """Run ``fn`` over ``items`` on a thread pool (numpy's generators and
    ctypes calls release the GIL). Results keep the order of ``items``."""
    if workers is None:
        workers = min(16, max(1, _cpu_count()))
    if workers <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


def _cpu_count() -> int:
    try:
        import os
        return len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        import os
        return os.cpu_count() or 1


def expected_distinct(n_experts: int, k: int, q: int) -> float:
    """Expected number of distinct experts hit by q independent uniform
    top-k picks (each pick is k distinct experts)."""
    return n_experts * (1.0 - ((n_experts - k) / n_experts) ** q)
