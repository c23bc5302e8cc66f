"""Pins for the oracle's activation quantizer and block GEMV: brute force on
tiny inputs, constructed rounding ties, numpy fp64 matmul identity, the
decode-once q-column invariant and closed-form special cases."""

import numpy as np
import pytest

import inputgen
import oracle as O

FMTS = (2, 3, 4)


def _e2m1_int(c):
    m = c & 7
    e, man = (m >> 1) & 3, m & 1
    v = 0.5 * man if e == 0 else (1.0 + 0.5 * man) * 2.0 ** (e - 1)
    return int(-2 * v if c & 8 else 2 * v)


def _cb(fmt, c):
    """Codebooks from their closed forms (independent of the oracle)."""
    return 2 * c - 3 if fmt == 2 else 2 * c - 7 if fmt == 3 else _e2m1_int(c)


# ---------------------------------------------------------------- act quant

def test_act_quant_brute_force():
    rng = np.random.default_rng(1)
    for trial in range(200):
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-4, 3)).astype(np.float32)
        if trial % 5 == 0:
            x[rng.integers(0, 32, 4)] = 0
        q, s = O.quantize_act(x)
        amax = np.max(np.abs(x))
        assert s[0] == amax / np.float32(127)  # fp32 IEEE division
        for t in range(32):
            r = float(np.float32(x[t]) / s[0])  # the fp32 quotient
            cands = np.arange(-127, 128)
            d = np.abs(r - cands)
            best = cands[d == d.min()]
            want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert q[t] == want
        # |x - q s| <= s/2 (no clamping happens: |x/s| <= 127 up to rounding)
        assert np.all(np.abs(x.astype(np.float64) - q * np.float64(s[0])) <= s[0] * 0.5000001)
        assert np.max(np.abs(q)) == 127


def test_act_quant_constructed_ties():
    # amax 127 -> s = 1 exactly; x = k + 1/2 must round to the even neighbour
    ks = np.arange(-127, 127)
    for start in range(0, len(ks), 31):
        x = np.zeros(32, np.float32)
        x[0] = 127.0
        sel = ks[start:start + 31]
        x[1:1 + len(sel)] = sel + 0.5
        q, s = O.quantize_act(x)
        assert s[0] == 1.0
        for i, k in enumerate(sel):
            lo, hi = k, k + 1
            assert q[1 + i] == (lo if lo % 2 == 0 else hi)


def test_act_quant_zero_block_and_shape():
    x = np.zeros((2, 64), np.float32)
    x[1, 40] = -3.0
    q, s = O.quantize_act(x)
    assert np.all(q[0] == 0) and np.all(s[0] == 0)
    assert s[1, 0] == 0 and q[1, 40] == -127 and s[1, 1] == np.float32(3.0) / np.float32(127)
    assert np.array_equal(O.act_sums(q)[1], [0, -127])


# --------------------------------------------------------------------- gemv

@pytest.mark.parametrize("fmt", FMTS)
def test_block_dots_brute_force_from_codes(fmt):
    """Codes and scales drawn directly (not by the encoder); D and y are
    recomputed with Python integers from the closed-form codebooks."""
    rng = np.random.default_rng(100 + fmt)
    N, nb, Q = 5, 3, 3
    ncode = 4 if fmt == 2 else 8 if fmt == 3 else 16
    bb = O.block_bytes(fmt)
    codes = rng.integers(0, ncode, (N, nb, 32))
    blocks = np.zeros((N, nb, bb), np.uint8)
    scale = np.zeros((N, nb))
    for n in range(N):
        for b in range(nb):
            blocks[n, b, :O.code_bytes(fmt)] = O.pack_codes(fmt, codes[n, b])
            if fmt == 4:
                E = int(rng.integers(100, 140))
                blocks[n, b, 16] = E
                scale[n, b] = 2.0 ** (E - 128)
            else:
                h = np.float16(rng.uniform(0.01, 2.0))
                blocks[n, b, -2:] = np.frombuffer(h.tobytes(), np.uint8)
                scale[n, b] = float(h)
    xq = rng.integers(-127, 128, (Q, nb * 32)).astype(np.int8)
    xs = rng.uniform(0.001, 0.1, (Q, nb)).astype(np.float32)
    y, dots = O.gemv(fmt, blocks, xq, xs, want_dots=True)
    for j in range(Q):
        for n in range(N):
            acc = 0.0
            for b in range(nb):
                D = sum(_cb(fmt, int(codes[n, b, t])) * int(xq[j, 32 * b + t]) for t in range(32))
                assert dots[j, n, b] == D
                acc += scale[n, b] * float(xs[j, b]) * D
            assert y[j, n] == pytest.approx(acc, rel=1e-15, abs=1e-300)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_equals_numpy_fp64_matmul(fmt):
    N, K, Q = 40, 256, 4
    W = inputgen.dense_weight(N, K, seed=7, outliers=True)
    x = inputgen.activations(Q, K, seed=8)
    blocks = O.quantize_matrix(fmt, W)
    xq, xs = O.quantize_act(x)
    y = O.gemv(fmt, blocks, xq, xs)
    Wd = O.dequantize_matrix(fmt, blocks)
    xd = xq.astype(np.float64) * np.repeat(xs.astype(np.float64), 32, axis=1)
    ref = xd @ Wd.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("fmt", FMTS)
def test_q4_equals_four_q1(fmt):
    """Decoding once for four columns equals four one-column products."""
    W = inputgen.dense_weight(33, 320, seed=9)
    x = inputgen.activations(4, 320, seed=10)
    blocks = O.quantize_matrix(fmt, W)
    xq, xs = O.quantize_act(x)
    y4, d4 = O.gemv(fmt, blocks, xq, xs, want_dots=True)
    for j in range(4):
        y1, d1 = O.gemv(fmt, blocks, xq[j:j + 1], xs[j:j + 1], want_dots=True)
        assert np.array_equal(y1[0], y4[j]) and np.array_equal(d1[0], d4[j])


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_extracts_a_column(fmt):
    N, K = 24, 128
    W = inputgen.dense_weight(N, K, seed=11)
    blocks = O.quantize_matrix(fmt, W)
    Wd = O.dequantize_matrix(fmt, blocks)
    for t in (0, 31, 77, 127):
        x = np.zeros((1, K), np.float32)
        x[0, t] = 2.5
        xq, xs = O.quantize_act(x)
        assert xq[0, t] == 127
        y = O.gemv(fmt, blocks, xq, xs)
        assert np.allclose(y[0], Wd[:, t] * 127 * np.float64(xs[0, t // 32]), rtol=1e-14, atol=0)


@pytest.mark.parametrize("fmt", FMTS)
def test_constant_x_gives_row_sums(fmt):
    N, K = 16, 96
    W = inputgen.dense_weight(N, K, seed=12)
    blocks = O.quantize_matrix(fmt, W)
    Wd = O.dequantize_matrix(fmt, blocks)
    x = np.full((1, K), 0.75, np.float32)
    xq, xs = O.quantize_act(x)
    assert np.all(xq == 127)
    y = O.gemv(fmt, blocks, xq, xs)
    assert np.allclose(y[0], Wd.sum(1) * 127 * np.float64(xs[0, 0]), rtol=1e-13, atol=1e-15)


def test_fp2_fp3_affine_codebook_identity():
    """D = 2 * sum(c x) - (2^bits - 1) * sum(x): the codebooks are affine in
    the code, so a decoder may skip the table (closed form)."""
    rng = np.random.default_rng(3)
    for fmt, off in ((2, 3), (3, 7)):
        ncode = 4 if fmt == 2 else 8
        c = rng.integers(0, ncode, (200, 32))
        x = rng.integers(-127, 128, (200, 32))
        D = np.array([[O.codebook(fmt, int(v)) for v in row] for row in c])
        assert np.array_equal((D * x).sum(1), 2 * (c * x).sum(1) - off * x.sum(1))
