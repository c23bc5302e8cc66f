"""Pins for the oracle's block format: page-given sizes, hand-worked
blocks, IEEE binary16 against numpy, codebooks against the E2M1 definition,
the nearest-code rule, the bit layout and encoder invariants."""

import math

import numpy as np
import pytest

import inputgen
import oracle as O
from conftest import expand_list, load_golden

FMTS = (2, 3, 4)


def test_block_sizes_from_pages():
    recs = load_golden("format_sizes.txt")
    wpb = [r for r in recs if "weights_per_block" in r][0]
    assert int(wpb["weights_per_block"]) == 32
    rows = [r for r in recs if "fmt" in r]
    assert len(rows) == 3
    for r in rows:
        parts = r["fmt"].split()
        fmt, bpw, nbytes = int(parts[0]), float(parts[2]), int(parts[4])
        assert nbytes == 32 * bpw / 8
        assert O.block_bytes(fmt) == nbytes


@pytest.mark.parametrize("rec", [r for r in load_golden("hand_blocks.txt") if "fmt" in r],
                         ids=lambda r: r["name"])
def test_hand_worked_blocks(rec):
    fmt = int(rec["fmt"])
    w = np.array(expand_list(rec["w"]), np.float32)
    blk = O.quantize_block(fmt, w)
    want = bytes(int(b, 16) for b in rec["bytes"].split())
    assert bytes(blk) == want
    vals = O.dequantize_block(fmt, blk)
    assert list(vals[:8]) == expand_list(rec["values"])
    xq = np.ones((1, 32), np.int8)
    xs = np.ones((1, 1), np.float32)
    y, d = O.gemv(fmt, blk[None, None, :], xq, xs, want_dots=True)
    assert d[0, 0, 0] == int(rec["dot1"])


def test_hand_worked_activation_and_product():
    recs = {r["name"]: r for r in load_golden("hand_blocks.txt")}
    act = recs["ACT-D"]
    x = np.array(expand_list(act["x"]), np.float32)
    q, s = O.quantize_act(x)
    assert list(q) == expand_list(act["xq"], int)
    assert float(s[0]) == float(act["xs"])
    fp4 = recs["FP4-A"]
    blk = O.quantize_block(4, np.array(expand_list(fp4["w"]), np.float32))
    y, d = O.gemv(4, blk[None, None, :], q[None], s[None], want_dots=True)
    assert d[0, 0, 0] == int(act["dot_with"].split()[1])
    assert y[0, 0] == float(act["y_with"].split()[1])


def test_f16_decode_every_pattern_matches_numpy():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([O.f16_to_f64(int(h)) for h in pats])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    # signed zeros keep their sign
    assert math.copysign(1.0, O.f16_to_f64(0x8000)) == -1.0


def _f16_cases():
    rng = np.random.default_rng(5)
    xs = [0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 70000.0, 5.96e-8, 2.98e-8, 2.99e-8,
          6.1035e-5, 6.1e-5, 1e-10, -3.3333333, 1.0 / 3.0]
    # exact halfway points between binary16 neighbours (ties to even)
    for h in list(range(1, 40)) + list(range(1020, 1030)) + list(range(0x3bf0, 0x3c10)) + [0x7bfe]:
        a = np.uint16(h).view(np.float16).astype(np.float64)
        b = np.uint16(h + 1).view(np.float16).astype(np.float64)
        mid = (a + b) / 2
        xs += [mid, -mid, np.nextafter(np.float32(mid), np.float32(0)),
               np.nextafter(np.float32(mid), np.float32(1e9))]
    xs += list(rng.standard_normal(3000) * 10.0 ** rng.uniform(-9, 5, 3000))
    return np.array(xs, np.float32)


def test_f32_to_f16_matches_numpy_rne():
    xs = _f16_cases()
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([O.f32_to_f16(float(x)) for x in xs], np.uint16)
    assert np.array_equal(ref, got)


def _e2m1_value(m):
    """OCP E2M1 (1 sign bit dropped): 2 exponent bits, 1 mantissa bit,
    exponent bias 1; e = 0 is subnormal (mantissa * 0.5)."""
    e, man = (m >> 1) & 3, m & 1
    if e == 0:
        return 0.5 * man
    return (1.0 + 0.5 * man) * 2.0 ** (e - 1)


def test_codebooks_closed_forms():
    assert [O.codebook(2, c) for c in range(4)] == [-3, -1, 1, 3]
    assert [O.codebook(3, c) for c in range(8)] == [-7, -5, -3, -1, 1, 3, 5, 7]
    for c in range(16):
        mag = 2.0 * _e2m1_value(c & 7)
        want = -mag if c & 8 else mag
        assert O.codebook(4, c) == want
    # FP4 with one e8m0 scale is MX: max |E2M1| is 6, times 2 = 12
    assert max(abs(O.codebook(4, c)) for c in range(16)) == 12


def _values(fmt):
    return {c: O.codebook(fmt, c) for c in range(4 if fmt == 2 else 8 if fmt == 3 else 16)
            if not (fmt == 4 and c == 8)}


@pytest.mark.parametrize("fmt", FMTS)
def test_nearest_code_is_an_argmin(fmt):
    vals = _values(fmt)
    rng = np.random.default_rng(fmt)
    for t in rng.uniform(-16, 16, 4000):
        c = O.nearest_code(fmt, float(t))
        d = abs(t - vals[c])
        assert all(d <= abs(t - v) for v in vals.values())


@pytest.mark.parametrize("fmt,t,want", [
    (2, 2.0, 3), (2, -2.0, -3), (2, 0.0, 1), (2, -0.0, 1), (2, 1e-30, 1), (2, -1e-30, -1),
    (2, 99.0, 3), (2, -99.0, -3),
    (3, 2.0, 3), (3, 4.0, 5), (3, 6.0, 7), (3, -2.0, -3), (3, -4.0, -5), (3, -6.0, -7),
    (3, 0.0, 1), (3, -0.0, 1), (3, 8.0, 7),
    # FP4: E2M1 round half to even, in int8 units (2x E2M1)
    (4, 0.5, 0), (4, 1.5, 2), (4, 2.5, 2), (4, 3.5, 4), (4, 5.0, 4), (4, 7.0, 8), (4, 10.0, 8),
    (4, -0.5, 0), (4, -1.5, -2), (4, -2.5, -2), (4, -3.5, -4), (4, -5.0, -4), (4, -7.0, -8),
    (4, -10.0, -8), (4, 11.0, 12), (4, 15.9, 12), (4, -15.9, -12), (4, 0.0, 0), (4, -0.0, 0),
])
def test_nearest_code_ties_and_saturation(fmt, t, want):
    c = O.nearest_code(fmt, t)
    assert O.codebook(fmt, c) == want
    if fmt == 4 and want == 0:
        assert c == 0  # -0 is never emitted


@pytest.mark.parametrize("fmt", FMTS)
def test_pack_unpack_bijection(fmt):
    rng = np.random.default_rng(10 + fmt)
    ncode = 4 if fmt == 2 else 8 if fmt == 3 else 16
    seen = set()
    for _ in range(500):
        codes = rng.integers(0, ncode, 32)
        blk = O.pack_codes(fmt, codes)
        assert len(blk) == O.code_bytes(fmt)
        full = np.concatenate([blk, np.zeros(O.block_bytes(fmt) - len(blk), np.uint8)])
        assert np.array_equal(O.unpack_codes(fmt, full), codes)
        seen.add(bytes(blk))
    assert len(seen) == 500


def test_bit_positions_single_code():
    """Each code lands in the documented bits and nowhere else."""
    for t in range(32):
        c = np.zeros(32, np.int64)
        c[t] = 3
        word = np.frombuffer(O.pack_codes(2, c).tobytes(), "<u4")
        m, r = divmod(t, 16)
        i, j = divmod(r, 4)
        want = np.zeros(2, np.uint32)
        want[m] = 3 << (8 * j + 2 * i)
        assert np.array_equal(word, want)
        c[t] = 4  # FP3 high bit only
        word = np.frombuffer(O.pack_codes(3, c).tobytes(), "<u4")
        want = np.zeros(3, np.uint32)
        ih, jh = divmod(t, 4)
        want[2] = 1 << (8 * jh + ih)
        assert np.array_equal(word, want)
        c[t] = 15
        word = np.frombuffer(O.pack_codes(4, c).tobytes(), "<u4")
        m, r = divmod(t, 8)
        i, j = divmod(r, 4)
        want = np.zeros(4, np.uint32)
        want[m] = 15 << (8 * j + 4 * i)
        assert np.array_equal(word, want)


def _random_blocks(seed, n=300):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        w = (rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 2)).astype(np.float32)
        if k % 7 == 0:
            w[rng.integers(0, 32, 3)] *= 10  # outliers
        if k % 11 == 0:
            w[rng.integers(0, 32, 8)] = 0
        out.append(w)
    return out


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_idempotent(fmt):
    for w in _random_blocks(20 + fmt):
        b1 = O.quantize_block(fmt, w)
        w2 = O.dequantize_block(fmt, b1).astype(np.float32)
        assert np.array_equal(O.dequantize_block(fmt, b1), w2.astype(np.float64))  # exact in fp32
        b2 = O.quantize_block(fmt, w2)
        assert np.array_equal(O.dequantize_block(fmt, b2), O.dequantize_block(fmt, b1))
        assert bytes(b1) == bytes(b2)


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_scale_equivariance(fmt):
    for w in _random_blocks(30 + fmt, 100):
        b = O.quantize_block(fmt, w)
        for k in (-3, 1, 4):
            if fmt in (2, 3):
                s = O.block_scale(fmt, b) * 2.0 ** k
                if not (6.2e-5 < s < 6.0e4):  # binary16 normal range only
                    continue
            bk = O.quantize_block(fmt, (w * np.float32(2.0 ** k)).astype(np.float32))
            assert np.array_equal(O.unpack_codes(fmt, bk), O.unpack_codes(fmt, b))
            assert O.block_scale(fmt, bk) == O.block_scale(fmt, b) * 2.0 ** k


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_sign_symmetry(fmt):
    for w in _random_blocks(40 + fmt, 150):
        d = O.dequantize_block(fmt, O.quantize_block(fmt, w))
        dn = O.dequantize_block(fmt, O.quantize_block(fmt, -w))
        nz = w != 0
        assert np.array_equal(dn[nz], -d[nz])
        if fmt == 4:
            assert np.array_equal(dn, -d + 0.0)


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_error_bound(fmt):
    for w in _random_blocks(50 + fmt):
        blk = O.quantize_block(fmt, w)
        S = O.block_scale(fmt, blk)
        d = O.dequantize_block(fmt, blk)
        err = np.abs(w.astype(np.float64) - d)
        amax = float(np.max(np.abs(w)))
        if fmt in (2, 3):
            cmax = 3 if fmt == 2 else 7
            # interior: half the spacing 2S; top clip: amax/S may exceed cmax
            # by fp16 rounding of the scale (relative 2^-11)
            bound = S * (1 + 1e-6) + amax * 2.0 ** -10
            assert np.all(err <= bound)
            assert S == pytest.approx(amax / cmax, rel=2 ** -10)
        else:
            t = np.abs(w.astype(np.float64)) / S
            assert np.all(t < 16)  # floor rule keeps amax in [8, 16) * S
            spacing = np.where(t <= 4, 1.0, np.where(t <= 8, 2.0, 4.0))
            inside = t <= 12
            assert np.all(err[inside] <= spacing[inside] / 2 * S * (1 + 1e-12))
            assert np.all(err[~inside] <= (t[~inside] - 12) * S * (1 + 1e-12))


@pytest.mark.parametrize("fmt", (2, 3))
def test_fp16_scale_matches_numpy(fmt):
    cmax = np.float32(3 if fmt == 2 else 7)
    for w in _random_blocks(60 + fmt):
        amax = np.max(np.abs(w))
        want = (amax / cmax).astype(np.float16).view(np.uint16)
        blk = O.quantize_block(fmt, w)
        got = int(blk[-2]) | (int(blk[-1]) << 8)
        assert got == int(want)


@pytest.mark.parametrize("amax,E", [(6.0, 127), (1.0, 125), (0.999, 124), (8.0, 128), (7.99, 127),
                                    (2.0 ** -130, 0), (2.0 ** -125, 0), (2.0 ** -124, 1),
                                    (3.0e38, 252), (0.0, 0)])
def test_fp4_exponent_hand_values(amax, E):
    w = np.zeros(32, np.float32)
    w[5] = np.float32(amax)
    blk = O.quantize_block(4, w)
    assert blk[16] == E


def test_zero_and_tiny_blocks():
    z = np.zeros(32, np.float32)
    b2 = O.quantize_block(2, z)
    assert list(O.unpack_codes(2, b2)) == [2] * 32 and O.block_scale(2, b2) == 0.0
    b3 = O.quantize_block(3, z)
    assert list(O.unpack_codes(3, b3)) == [4] * 32 and O.block_scale(3, b3) == 0.0
    b4 = O.quantize_block(4, z)
    assert list(O.unpack_codes(4, b4)) == [0] * 32 and b4[16] == 0
    # fp16 scale underflows to 0 -> every weight decodes to 0
    tiny = np.full(32, 1e-9, np.float32)
    assert np.all(O.dequantize_block(2, O.quantize_block(2, tiny)) == 0.0)
    # subnormal fp16 scale is kept
    small = inputgen.raw_normal(1, 32, 1e-5)
    b = O.quantize_block(2, small)
    s = O.block_scale(2, b)
    assert 0 < s < 6.1e-5


def test_nonfinite_rejected():
    for bad in (np.inf, -np.inf, np.nan):
        w = np.zeros(32, np.float32)
        w[3] = bad
        for fmt in FMTS:
            with pytest.raises(O.OracleError):
                O.quantize_block(fmt, w)
    big = np.full(32, 3.0e5, np.float32)  # 3e5/3 overflows binary16
    with pytest.raises(O.OracleError):
        O.quantize_block(2, big)
    O.quantize_block(4, big)  # e8m0 has the range


def test_matrix_is_rowwise_blocks():
    W = inputgen.dense_weight(5, 96, seed=3, outliers=True)
    for fmt in FMTS:
        M = O.quantize_matrix(fmt, W)
        assert M.shape == (5, 3, O.block_bytes(fmt))
        for r in range(5):
            for b in range(3):
                assert bytes(M[r, b]) == bytes(O.quantize_block(fmt, W[r, 32 * b:32 * b + 32]))


# ------------------------------------------------- FP2M (scale + minimum)
# The variant with two small values per block: weight = s * c + m, c 0..3.

FP2M = O.FP2M


def test_fp2m_sizes_and_codebook():
    assert O.block_bytes(FP2M) == 12 and O.code_bytes(FP2M) == 8
    assert [O.codebook(FP2M, c) for c in range(4)] == [0, 1, 2, 3]


def test_fp2m_nearest_code_argmin_and_ties():
    rng = np.random.default_rng(7)
    for t in rng.uniform(-3, 6, 4000):
        c = O.nearest_code(FP2M, float(t))
        assert all(abs(t - c) <= abs(t - v) for v in range(4))
    for t, want in ((0.5, 1), (1.5, 2), (2.5, 3), (-0.7, 0), (9.0, 3), (0.0, 0), (-0.0, 0)):
        assert O.nearest_code(FP2M, t) == want


def test_fp2m_bit_layout_is_fp2s():
    rng = np.random.default_rng(8)
    for _ in range(50):
        codes = rng.integers(0, 4, 32)
        assert bytes(O.pack_codes(FP2M, codes)) == bytes(O.pack_codes(2, codes))
        blk = np.zeros(12, np.uint8)
        blk[:8] = O.pack_codes(FP2M, codes)
        assert np.array_equal(O.unpack_codes(FP2M, blk), codes)


def test_fp2m_scale_and_min_from_the_block_extremes():
    """m = fp16(min w) and s = fp16(max(max w - m, 0) / 3), recomputed here
    with numpy's binary16 rounding; every code is the nearest to the fp32
    t = (w - m) / s (ties up); reconstruction stays within half a step plus
    the fp16 roundings of m and s."""
    for w in _random_blocks(70) + [np.full(32, 0.7, np.float32), np.arange(32, dtype=np.float32) - 40]:
        blk = O.quantize_block(FP2M, w)
        lo, hi = np.float32(w.min()), np.float32(w.max())
        m16 = np.float16(lo)
        m = np.float32(m16)
        span = np.float32(max(np.float32(hi - m), np.float32(0.0)))
        s = np.float32(np.float16(span / np.float32(3.0)))
        assert O.block_min(FP2M, blk) == float(m)
        assert O.block_scale(FP2M, blk) == float(s)
        codes = O.unpack_codes(FP2M, blk)
        if s == 0:
            assert np.all(codes == 0)
            continue
        t = (w - m) / s  # fp32, as the format fixes
        want = np.clip(np.floor(t.astype(np.float64) + 0.5), 0, 3)
        assert np.array_equal(codes, want)
        d = O.dequantize_block(FP2M, blk)
        err = np.abs(w.astype(np.float64) - d)
        bound = 0.5 * float(s) + max(float(m) - float(lo), 0.0) + 3 * abs(float(span) / 3 - float(s)) \
            + 1e-6 * float(np.max(np.abs(w)))
        assert np.all(err <= bound)


def test_fp2m_power_of_two_equivariance():
    for w in _random_blocks(71, 100):
        b = O.quantize_block(FP2M, w)
        s, m = O.block_scale(FP2M, b), O.block_min(FP2M, b)
        for k in (-2, 3):
            if not all(v == 0 or 6.2e-5 < abs(v) * 2.0 ** k < 6.0e4 for v in (s, m)):
                continue
            if s != 0 and s < 6.2e-5:
                continue
            bk = O.quantize_block(FP2M, (w * np.float32(2.0 ** k)).astype(np.float32))
            assert np.array_equal(O.unpack_codes(FP2M, bk), O.unpack_codes(FP2M, b))
            assert O.block_scale(FP2M, bk) == s * 2.0 ** k and O.block_min(FP2M, bk) == m * 2.0 ** k


def test_fp2m_gemv_is_the_dequantized_product():
    """The oracle's per-block s * (S D + M X) against the plain fp64 sum of
    dequantized weights times dequantized activations (a different order of
    the same exact terms; a dropped or mis-signed minimum term fails)."""
    rng = np.random.default_rng(72)
    N, K, Q = 5, 96, 3
    W = (rng.standard_normal((N, K)) * 0.3 + rng.uniform(-1, 1, (N, 1))).astype(np.float32)
    blocks = O.quantize_matrix(FP2M, W)
    x = rng.standard_normal((Q, K)).astype(np.float32)
    xq, xs = O.quantize_act(x)
    y, dots = O.gemv(FP2M, blocks, xq, xs, want_dots=True)
    Wd = O.dequantize_matrix(FP2M, blocks)
    xd = xq.astype(np.float64) * np.repeat(xs.astype(np.float64), 32, axis=1)
    assert np.allclose(y, xd @ Wd.T, rtol=1e-12, atol=1e-12)
    codes = np.array([[O.unpack_codes(FP2M, blocks[n, b]) for b in range(K // 32)] for n in range(N)])
    for j in range(Q):
        want = (codes * xq[j].reshape(1, K // 32, 32)).sum(-1)
        assert np.array_equal(dots[j], want)


def test_fp2m_range_errors():
    w = np.zeros(32, np.float32)
    w[0] = np.float32(-70000.0)  # the fp16 minimum overflows
    with pytest.raises(O.OracleError):
        O.quantize_block(FP2M, w)
    w = np.zeros(32, np.float32)
    w[0] = np.float32(3.0e5)  # the fp16 scale overflows
    with pytest.raises(O.OracleError):
        O.quantize_block(FP2M, w)
    w[0] = np.nan
    with pytest.raises(O.OracleError):
        O.quantize_block(FP2M, w)


# ------------------------------------------------------ Q8 (the int8 tier)
# 32 int8 codes + an fp16 scale; weight = s * c.

Q8 = O.Q8


def test_q8_sizes_and_codebook():
    assert O.block_bytes(Q8) == 34 and O.code_bytes(Q8) == 32
    assert [O.codebook(Q8, c) for c in (0, 1, 127, 0x81, 0xFF, 0x80)] == [0, 1, 127, -127, -1, -128]


def test_q8_nearest_code_is_clamped_round_half_even():
    """The brute-force argmin over the 255 codes (never -128) equals the
    plain definition the encoder writes out: clamp(rint(t), -127, 127)."""
    rng = np.random.default_rng(9)
    ts = list(rng.uniform(-140, 140, 3000)) + [k + 0.5 for k in range(-130, 130)] + [127.6, -127.6, 300.0, -0.0]
    for t in ts:
        c = O.nearest_code(Q8, float(t))
        assert c != 0x80
        want = int(np.clip(np.rint(t), -127, 127))
        assert O.codebook(Q8, c) == want, t


def test_q8_scale_codes_and_error_bound():
    for w in _random_blocks(80) + [np.zeros(32, np.float32), np.full(32, -3e-7, np.float32)]:
        blk = O.quantize_block(Q8, w)
        amax = np.float32(np.max(np.abs(w)))
        s = np.float32(np.float16(amax / np.float32(127.0)))
        assert O.block_scale(Q8, blk) == float(s)
        codes = np.array([O.codebook(Q8, c) for c in O.unpack_codes(Q8, blk)])
        if s == 0:
            assert np.all(codes == 0)
            continue
        want = np.clip(np.rint((w / s).astype(np.float64)), -127, 127)  # w / s in fp32
        assert np.array_equal(codes, want)
        d = O.dequantize_block(Q8, blk)
        err = np.abs(w.astype(np.float64) - d)
        assert np.all(err <= 0.5 * float(s) + abs(float(amax) - 127 * float(s)) + 1e-7 * float(amax))


def test_q8_power_of_two_equivariance():
    for w in _random_blocks(81, 100):
        b = O.quantize_block(Q8, w)
        s = O.block_scale(Q8, b)
        for k in (-3, 2):
            # both scales normal fp16 (a subnormal one has fewer bits)
            if not (s == 0 or (6.2e-5 < s < 6.0e4 and 6.2e-5 < s * 2.0 ** k < 6.0e4)):
                continue
            bk = O.quantize_block(Q8, (w * np.float32(2.0 ** k)).astype(np.float32))
            assert np.array_equal(O.unpack_codes(Q8, bk), O.unpack_codes(Q8, b))
            assert O.block_scale(Q8, bk) == s * 2.0 ** k


def test_q8_gemv_is_the_dequantized_product():
    rng = np.random.default_rng(82)
    N, K, Q = 6, 128, 3
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    blocks = O.quantize_matrix(Q8, W)
    x = rng.standard_normal((Q, K)).astype(np.float32)
    xq, xs = O.quantize_act(x)
    y, dots = O.gemv(Q8, blocks, xq, xs, want_dots=True)
    Wd = O.dequantize_matrix(Q8, blocks)
    xd = xq.astype(np.float64) * np.repeat(xs.astype(np.float64), 32, axis=1)
    assert np.allclose(y, xd @ Wd.T, rtol=1e-12, atol=1e-12)
    vals = np.array([[[O.codebook(Q8, c) for c in O.unpack_codes(Q8, blocks[n, b])] for b in range(K // 32)]
                     for n in range(N)])
    for j in range(Q):
        assert np.array_equal(dots[j], (vals * xq[j].reshape(1, K // 32, 32)).sum(-1))


def test_q8_range_errors():
    w = np.zeros(32, np.float32)
    w[3] = np.float32(1e7)  # fp16 scale overflow
    with pytest.raises(O.OracleError):
        O.quantize_block(Q8, w)
    w[3] = np.inf
    with pytest.raises(O.OracleError):
        O.quantize_block(Q8, w)


# ---------------------------------------------- FP2S (two 16-weight scales)
# The FP2 codes and codebook; weights 0..15 take the fp16 scale s0, weights
# 16..31 the fp16 scale s1, each half encoded as an FP2 block of its own.

FP2S = O.FP2S


def test_fp2s_sizes_codebook_and_layout():
    assert O.block_bytes(FP2S) == 12 and O.code_bytes(FP2S) == 8
    assert [O.codebook(FP2S, c) for c in range(4)] == [O.codebook(2, c) for c in range(4)]
    rng = np.random.default_rng(90)
    for _ in range(20):
        codes = rng.integers(0, 4, 32)
        assert bytes(O.pack_codes(FP2S, codes)) == bytes(O.pack_codes(2, codes))


def test_fp2s_each_half_is_an_fp2_block():
    """Half h of an FP2S block equals the first half of the FP2 encoding of
    the block [w_h, w_h] (same amax, so the same scale and codes): the FP2
    encoder, pinned on its own, pins the per-half scale and codes."""
    for w in _random_blocks(91) + [np.r_[np.zeros(16), np.full(16, 0.7)].astype(np.float32)]:
        blk = O.quantize_block(FP2S, w)
        codes = O.unpack_codes(FP2S, blk)
        for h in range(2):
            half = w[16 * h:16 * h + 16]
            ref = O.quantize_block(2, np.r_[half, half].astype(np.float32))
            assert O.weight_scale(FP2S, blk, 16 * h) == O.block_scale(2, ref)
            assert all(O.weight_scale(FP2S, blk, t) == O.weight_scale(FP2S, blk, 16 * h)
                       for t in range(16 * h, 16 * h + 16))
            assert np.array_equal(codes[16 * h:16 * h + 16], O.unpack_codes(2, ref)[:16])
            d = O.dequantize_block(FP2S, blk)[16 * h:16 * h + 16]
            assert np.array_equal(d, O.dequantize_block(2, ref)[:16])


def test_fp2s_equal_halves_reduce_to_fp2():
    """With the same amax in both halves the two scales equal FP2's one
    scale and the block decodes to the FP2 block exactly."""
    rng = np.random.default_rng(92)
    for _ in range(40):
        w = (rng.standard_normal(32) * 0.02).astype(np.float32)
        w[rng.integers(0, 16)] = np.float32(0.09)
        w[16 + rng.integers(0, 16)] = np.float32(-0.09)
        b2, bs = O.quantize_block(2, w), O.quantize_block(FP2S, w)
        assert O.weight_scale(FP2S, bs, 0) == O.weight_scale(FP2S, bs, 31) == O.block_scale(2, b2)
        assert np.array_equal(O.dequantize_block(FP2S, bs), O.dequantize_block(2, b2))


def test_fp2s_power_of_two_equivariance():
    for w in _random_blocks(93, 100):
        b = O.quantize_block(FP2S, w)
        s0, s1 = O.weight_scale(FP2S, b, 0), O.weight_scale(FP2S, b, 16)
        for k in (-3, 2):
            # every scale normal fp16 before and after (a subnormal one has
            # fewer bits)
            ok = all(s == 0 or (6.2e-5 < s < 6.0e4 and 6.2e-5 < s * 2.0 ** k < 6.0e4) for s in (s0, s1))
            if not ok:
                continue
            bk = O.quantize_block(FP2S, (w * np.float32(2.0 ** k)).astype(np.float32))
            assert np.array_equal(O.unpack_codes(FP2S, bk), O.unpack_codes(FP2S, b))
            assert O.weight_scale(FP2S, bk, 0) == s0 * 2.0 ** k
            assert O.weight_scale(FP2S, bk, 16) == s1 * 2.0 ** k


def test_fp2s_gemv_is_the_dequantized_product():
    """The oracle's per-block s * (S0 D0 + S1 D1) against the plain fp64 sum
    of dequantized weights times dequantized activations (swapped or shared
    half scales, or a half dot over the wrong weights, fail); the dots are
    the unit-scale block dots D0 + D1."""
    rng = np.random.default_rng(94)
    N, K, Q = 5, 128, 3
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    W[:, 16:32] *= 8.0  # the second half of block 0 on a different scale
    blocks = O.quantize_matrix(FP2S, W)
    x = rng.standard_normal((Q, K)).astype(np.float32)
    xq, xs = O.quantize_act(x)
    y, dots = O.gemv(FP2S, blocks, xq, xs, want_dots=True)
    Wd = O.dequantize_matrix(FP2S, blocks)
    xd = xq.astype(np.float64) * np.repeat(xs.astype(np.float64), 32, axis=1)
    assert np.allclose(y, xd @ Wd.T, rtol=1e-12, atol=1e-12)
    vals = np.array([[[O.codebook(FP2S, c) for c in O.unpack_codes(FP2S, blocks[n, b])] for b in range(K // 32)]
                     for n in range(N)])
    for j in range(Q):
        assert np.array_equal(dots[j], (vals * xq[j].reshape(1, K // 32, 32)).sum(-1))


def test_fp2s_range_errors():
    w = np.zeros(32, np.float32)
    w[20] = np.float32(3.0e5)  # the second half's fp16 scale overflows
    with pytest.raises(O.OracleError):
        O.quantize_block(FP2S, w)
    w[20] = 0.0
    w[3] = np.nan
    with pytest.raises(O.OracleError):
        O.quantize_block(FP2S, w)


# ------------------------------------------- FP3E (3-bit, e8m0 scale byte)
# FP3's codes and codebook with a power-of-two scale 2^(E - 127): 13 bytes.

FP3E = O.FP3E


def test_fp3e_sizes_codebook_and_layout():
    assert O.block_bytes(FP3E) == 13 and O.code_bytes(FP3E) == 12
    assert [O.codebook(FP3E, c) for c in range(8)] == [O.codebook(3, c) for c in range(8)]
    rng = np.random.default_rng(100)
    for _ in range(20):
        codes = rng.integers(0, 8, 32)
        assert bytes(O.pack_codes(FP3E, codes)) == bytes(O.pack_codes(3, codes))


@pytest.mark.parametrize("amax,E", [(1.0, 125), (7.9, 127), (8.0, 128), (3.9, 126), (2.0 ** -126, 0),
                                    (2.0 ** -100 * 1.5, 25), (3.0e38, 252), (0.0, 0)])
def test_fp3e_exponent_hand_values(amax, E):
    """E = floor(log2 amax) - 2 + 127, clamped at 0 (2 = floor(log2 7))."""
    w = np.zeros(32, np.float32)
    w[5] = np.float32(amax)
    assert O.quantize_block(FP3E, w)[12] == E


def _fp3e_code(t):
    """The nearest of -7, -5, ..., 7 to t with ties to the larger magnitude
    (0 to +1), as a code c = (v + 7) / 2: a closed form, not a search."""
    u = (t + 7.0) / 2.0
    c = np.floor(u + 0.5) if t >= 0 else np.ceil(u - 0.5)
    return int(np.clip(c, 0, 7))


def test_fp3e_codes_closed_form_and_error_bound():
    for w in _random_blocks(101) + [np.zeros(32, np.float32)]:
        blk = O.quantize_block(FP3E, w)
        E = int(blk[12])
        S = 2.0 ** (E - 127)
        assert O.block_scale(FP3E, blk) == S
        codes = O.unpack_codes(FP3E, blk)
        for t in range(32):
            assert codes[t] == _fp3e_code(float(w[t]) / S), (t, w[t], S)
        d = O.dequantize_block(FP3E, blk)
        # half a step inside the codebook's range; amax / S < 8 saturates by < 1
        assert np.all(np.abs(w.astype(np.float64) - d) <= S)


def test_fp3e_equals_fp3_when_its_scale_is_a_power_of_two():
    """amax = 7 * 2^j: FP3's fp16 scale is exactly 2^j, FP3E's 2^(E-127)
    is the same, so both decode every weight alike."""
    rng = np.random.default_rng(102)
    for j in (-10, -3, 0, 2, 5):
        for _ in range(10):
            w = (rng.uniform(-1, 1, 32) * 7 * 2.0 ** j).astype(np.float32)
            w[rng.integers(0, 32)] = np.float32(7 * 2.0 ** j)
            b3, be = O.quantize_block(3, w), O.quantize_block(FP3E, w)
            assert O.block_scale(3, b3) == O.block_scale(FP3E, be) == 2.0 ** j
            assert np.array_equal(O.dequantize_block(3, b3), O.dequantize_block(FP3E, be))


def test_fp3e_power_of_two_equivariance():
    for w in _random_blocks(103, 100):
        b = O.quantize_block(FP3E, w)
        for k in (-3, 2):
            if not 0 < int(b[12]) + k < 254:
                continue
            bk = O.quantize_block(FP3E, (w * np.float32(2.0 ** k)).astype(np.float32))
            assert np.array_equal(O.unpack_codes(FP3E, bk), O.unpack_codes(FP3E, b))
            assert int(bk[12]) == int(b[12]) + k


def test_fp3e_gemv_is_the_dequantized_product():
    rng = np.random.default_rng(104)
    N, K, Q = 5, 128, 3
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    blocks = O.quantize_matrix(FP3E, W)
    x = rng.standard_normal((Q, K)).astype(np.float32)
    xq, xs = O.quantize_act(x)
    y, dots = O.gemv(FP3E, blocks, xq, xs, want_dots=True)
    Wd = O.dequantize_matrix(FP3E, blocks)
    xd = xq.astype(np.float64) * np.repeat(xs.astype(np.float64), 32, axis=1)
    assert np.allclose(y, xd @ Wd.T, rtol=1e-12, atol=1e-12)
    vals = np.array([[[O.codebook(FP3E, c) for c in O.unpack_codes(FP3E, blocks[n, b])] for b in range(K // 32)]
                     for n in range(N)])
    for j in range(Q):
        assert np.array_equal(dots[j], (vals * xq[j].reshape(1, K // 32, 32)).sum(-1))


def test_fp3e_nonfinite_rejected():
    w = np.zeros(32, np.float32)
    w[9] = np.inf
    with pytest.raises(O.OracleError):
        O.quantize_block(FP3E, w)


@pytest.mark.parametrize("fmt", (2, 3, 4, 12, 8, 16, 13))
def test_dequantize_matrix_is_the_block_decoder_on_every_block(fmt):
    """The matrix dequantizer is dequantize_block applied block by block, in
    row-major block order (a swapped index or stride would misplace them)."""
    W = inputgen.dense_weight(7, 96, seed=31, outliers=True)
    blocks = O.quantize_matrix(fmt, W)
    Wd = O.dequantize_matrix(fmt, blocks)
    for n in range(7):
        for b in range(3):
            assert np.array_equal(Wd[n, 32 * b:32 * b + 32], O.dequantize_block(fmt, blocks[n, b]))
