/*
 * CPU oracle for ROCmFPX-style 32-weight block quantization.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library under test links,
 * imports or calls this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do. It shares no code, header or table with
 * the GPU library.
 *
 * Plain scalar C, written to be checked by eye: every operation is the
 * definition itself, with no blocking, fusion or reordering. Floating-point
 * steps that decide an integer (a scale, a code) are done in IEEE fp32 with
 * the same operations the format fixes; products are exact integers summed
 * in fp64.
 *
 * Pages cited (title, site):
 *   [HM]  "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
 *         (hellomarvisaitoday.com), paragraphs numbered from the top.
 *   [AIN] "Token Freedom via APU: AMD Ryzen AI MAX+ 395 Runs DeepSeek V4
 *         Flash at 32 tok/s on a 284B Model" (ainomam.com), by section.
 *   [KK]  the kaikai365.com post on DeepSeek V4 Flash on Strix Halo, by
 *         section heading.
 *
 * What the pages fix: a block holds 32 weights as packed codes of a few bits
 * each, with a single small scale or a pair of them; FP2 takes 10 bytes per block (2.50 bits per
 * weight), FP3 3.50 bits per weight, FP4 4.25 bits per weight ([HM] para 2;
 * [KK] section on the mixed-precision assignment). Decoding expands a small
 * codebook and feeds integer dot products ([HM] para 3).
 *
 * What the pages leave open is fixed here by a stated reading (each marked
 * "Reading"): one scale per block; the codebook values; scale rules;
 * rounding and tie rules; the bit order inside a block; how activations are
 * quantized. Byte counts per block follow from the pages: 32 x 2.5 / 8 = 10,
 * 32 x 3.5 / 8 = 14, 32 x 4.25 / 8 = 17.
 *
 * Canonical block (all formats): code bytes, then the scale.
 *   FP2: 8 code bytes + fp16 scale (little-endian)       = 10 bytes
 *   FP3: 12 code bytes + fp16 scale                       = 14 bytes
 *   FP4: 16 code bytes + one e8m0 exponent byte           = 17 bytes
 *
 * Variant with two small values per block (the page's format overview lets a
 * block carry a second small value beside its scale; this variant is a
 * reading, not one of the three named formats):
 *   FP2M: the FP2 code bytes + fp16 scale s + fp16 minimum m = 12 bytes
 *         (3.0 bits per weight); weight = s * c + m, c in 0..3.
 *
 * Variant with two small scales per block (the same overview; a reading):
 *   FP2S: the FP2 code bytes + fp16 scale s0 of weights 0..15 + fp16 scale
 *         s1 of weights 16..31 = 12 bytes (3.0 bits per weight);
 *         weight t = s_(t/16) * (2c - 3), each half encoded as FP2 is.
 *
 * A 3-bit tier at about 3.3 bits per weight including scales (the figure
 * another system on the pages gives for its 3-bit experts, without a
 * layout; this one is a reading):
 *   FP3E: the FP3 code bytes + one e8m0 exponent byte E = 13 bytes
 *         (3.25 bits per weight); weight = 2^(E - 127) * (2c - 7).
 *
 * A tier above FP4 for the dense and sensitive projections (the same
 * paragraph keeps those at FP4 or a wider format without naming one; this
 * tier is a reading):
 *   Q8:   32 int8 codes in weight order + fp16 scale = 34 bytes
 *         (8.5 bits per weight); weight = s * c, c in -127..127.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FP2 2
#define ORC_FP3 3
#define ORC_FP4 4
#define ORC_FP2M 12
#define ORC_Q8 8
#define ORC_FP2S 16
#define ORC_FP3E 13

#define ORC_OK 0
#define ORC_E_INVAL (-1)
#define ORC_E_RANGE (-3)

int orc_block_bytes(int fmt)
{
    /* [HM] para 2: 2.50 / 3.50 / 4.25 bits per weight, 32 weights. */
    switch (fmt) {
    case ORC_FP2: return 10;
    case ORC_FP3: return 14;
    case ORC_FP4: return 17;
    case ORC_FP2M: return 12; /* Reading: 8 code bytes + two fp16 values */
    case ORC_Q8: return 34;   /* Reading: 32 int8 codes + an fp16 scale */
    case ORC_FP2S: return 12; /* Reading: 8 code bytes + two fp16 scales */
    case ORC_FP3E: return 13; /* Reading: 12 code bytes + an e8m0 byte */
    }
    return ORC_E_INVAL;
}

int orc_code_bytes(int fmt)
{
    switch (fmt) {
    case ORC_FP2: return 8;
    case ORC_FP3: return 12;
    case ORC_FP4: return 16;
    case ORC_FP2M: return 8;
    case ORC_Q8: return 32;
    case ORC_FP2S: return 8;
    case ORC_FP3E: return 12;
    }
    return ORC_E_INVAL;
}

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16, written out from its definition.                */
/* ------------------------------------------------------------------ */

/* Value of a binary16 bit pattern, exactly, as a double. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* fp32 -> binary16, round to nearest, ties to even. Non-negative binary16
 * patterns are ordered like their values, so the nearest value is found by
 * a binary search over the patterns and a comparison of the two
 * neighbours: slow, but plainly the definition. */
uint16_t orc_f32_to_f16(float f)
{
    double a = fabs((double)f);
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f))
        return 0x7e00;
    /* Largest finite binary16 is 65504; halfway to the next binade step
     * (65520) and beyond rounds to infinity. */
    if (a >= 65520.0)
        return sign | 0x7c00;
    /* Binary search over the 0x7c00 monotone non-negative finite patterns
     * for the last pattern whose value is <= a. */
    int lo = 0, hi = 0x7bff;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (orc_f16_to_f64((uint16_t)mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int below = lo;
    if (below == 0x7bff)
        return sign | 0x7bff; /* a in [65504, 65520) */
    double vb = orc_f16_to_f64((uint16_t)below);
    double va = orc_f16_to_f64((uint16_t)(below + 1));
    double db = a - vb, da = va - a; /* both exact in double */
    int pick;
    if (db < da)
        pick = below;
    else if (da < db)
        pick = below + 1;
    else
        pick = (below & 1) ? below + 1 : below; /* tie: even mantissa */
    return sign | (uint16_t)pick;
}

/* ------------------------------------------------------------------ */
/* Codebooks (Reading: the pages say "codebooks" without values).     */
/* ------------------------------------------------------------------ */

/* FP2: codes 0..3 -> -3, -1, +1, +3 (odd, symmetric).
 * FP3: codes 0..7 -> -7, -5, ..., +7.
 * FP4: code = sign<<3 | m, m the OCP E2M1 magnitude pattern; value =
 *      2 x E2M1 so it is an integer: m -> 0,1,2,3,4,6,8,12. Code 8 (-0)
 *      decodes to 0 and the encoder never emits it.
 * FP2M: the integer part is the code itself, 0..3; the block's minimum is
 *      added after the scale (weight = s * c + m).
 * FP2S: FP2's codebook; the scale depends on the half of the block.
 * FP3E: FP3's codebook; the scale is a power of two. */
int orc_codebook(int fmt, int code)
{
    static const int fp4_mag[8] = {0, 1, 2, 3, 4, 6, 8, 12};
    switch (fmt) {
    case ORC_FP2:
    case ORC_FP2S: return 2 * code - 3;
    case ORC_FP3:
    case ORC_FP3E: return 2 * code - 7;
    case ORC_FP4: return (code & 8) ? -fp4_mag[code & 7] : fp4_mag[code & 7];
    case ORC_FP2M: return code;
    case ORC_Q8: return (int)(int8_t)(uint8_t)code; /* the byte as two's complement */
    }
    return 0;
}

static int n_codes(int fmt)
{
    return fmt == ORC_FP2 || fmt == ORC_FP2M || fmt == ORC_FP2S ? 4 : fmt == ORC_FP3 || fmt == ORC_FP3E ? 8 : fmt == ORC_Q8 ? 256 : 16;
}

/* Nearest codebook value to t, by brute force over every code.
 * Two candidates a != b are compared exactly: t is nearer to a than to b
 * when it lies on a's side of their midpoint (a + b) / 2, which is exact in
 * double; t equal to the midpoint is a tie. (Subtracting t - v in floating
 * point would round for tiny t and turn near-ties into false ties.)
 * Reading (ties): FP2/FP3 prefer the larger magnitude, and between equal
 * magnitudes (t = 0) the positive one; FP4 prefers the even E2M1 mantissa
 * (round-half-even on the E2M1 grid), saturating at +-12 by distance;
 * FP2M (values 0..3, all non-negative) prefers the larger value. */
int orc_nearest_code(int fmt, double t)
{
    int best = -1;
    for (int c = 0; c < n_codes(fmt); c++) {
        if (fmt == ORC_FP4 && c == 8)
            continue; /* -0 is never emitted */
        if (fmt == ORC_Q8 && c == 0x80)
            continue; /* -128 is never emitted: the codes are symmetric */
        if (best < 0) {
            best = c;
            continue;
        }
        int v = orc_codebook(fmt, c), vb = orc_codebook(fmt, best);
        double mid = ((double)v + (double)vb) / 2.0;
        int nearer = (v < vb) ? (t < mid) : (t > mid);
        if (nearer) {
            best = c;
        } else if (t == mid) { /* exact tie between c and best */
            if (fmt == ORC_FP4) {
                if (((c & 7) % 2) == 0)
                    best = c;
            } else if (fmt == ORC_Q8) {
                if ((v & 1) == 0) /* half to even, as the activations */
                    best = c;
            } else if (abs(v) > abs(vb) || (abs(v) == abs(vb) && v > vb)) {
                best = c;
            }
        }
    }
    return best;
}

/* ------------------------------------------------------------------ */
/* Bit layout inside a block (Reading: the pages do not give one).    */
/* ------------------------------------------------------------------ */
/* Code words are little-endian 32-bit words.
 * FP2 (and FP2M, FP2S): word m (0..1) holds weights 16m..16m+15; weight
 *      16m + 4i + j (i, j in 0..3) occupies bits [8j + 2i, 8j + 2i + 2).
 * FP3 (and FP3E): words 0..1 hold the low two bits of every code exactly as FP2;
 *      word 2 holds the high bit, weight 4i + j (i in 0..7, j in 0..3) at
 *      bit 8j + i.
 * FP4: word m (0..3) holds weights 8m..8m+7; weight 8m + 4i + j (i in 0..1)
 *      occupies bits [8j + 4i, 8j + 4i + 4). */

static uint32_t rd32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

static void wr32(uint8_t *p, uint32_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
    p[2] = (uint8_t)(v >> 16);
    p[3] = (uint8_t)(v >> 24);
}

void orc_unpack_codes(int fmt, const uint8_t *blk, int *codes)
{
    for (int t = 0; t < 32; t++) {
        if (fmt == ORC_FP2 || fmt == ORC_FP2M || fmt == ORC_FP2S) {
            int m = t / 16, r = t % 16, i = r / 4, j = r % 4;
            codes[t] = (int)((rd32(blk + 4 * m) >> (8 * j + 2 * i)) & 3u);
        } else if (fmt == ORC_FP3 || fmt == ORC_FP3E) {
            int m = t / 16, r = t % 16, i = r / 4, j = r % 4;
            int lo = (int)((rd32(blk + 4 * m) >> (8 * j + 2 * i)) & 3u);
            int ih = t / 4, jh = t % 4;
            int hi = (int)((rd32(blk + 8) >> (8 * jh + ih)) & 1u);
            codes[t] = lo | (hi << 2);
        } else if (fmt == ORC_Q8) {
            codes[t] = blk[t]; /* byte t is weight t */
        } else {
            int m = t / 8, r = t % 8, i = r / 4, j = r % 4;
            codes[t] = (int)((rd32(blk + 4 * m) >> (8 * j + 4 * i)) & 15u);
        }
    }
}

void orc_pack_codes(int fmt, const int *codes, uint8_t *blk)
{
    if (fmt == ORC_Q8) {
        for (int t = 0; t < 32; t++)
            blk[t] = (uint8_t)codes[t];
        return;
    }
    uint32_t w[4] = {0, 0, 0, 0};
    for (int t = 0; t < 32; t++) {
        if (fmt == ORC_FP2 || fmt == ORC_FP2M || fmt == ORC_FP2S) {
            int m = t / 16, r = t % 16, i = r / 4, j = r % 4;
            w[m] |= (uint32_t)(codes[t] & 3) << (8 * j + 2 * i);
        } else if (fmt == ORC_FP3 || fmt == ORC_FP3E) {
            int m = t / 16, r = t % 16, i = r / 4, j = r % 4;
            w[m] |= (uint32_t)(codes[t] & 3) << (8 * j + 2 * i);
            int ih = t / 4, jh = t % 4;
            w[2] |= (uint32_t)((codes[t] >> 2) & 1) << (8 * jh + ih);
        } else {
            int m = t / 8, r = t % 8, i = r / 4, j = r % 4;
            w[m] |= (uint32_t)(codes[t] & 15) << (8 * j + 4 * i);
        }
    }
    for (int m = 0; m < orc_code_bytes(fmt) / 4; m++)
        wr32(blk + 4 * m, w[m]);
}

/* Dequantization scale S of a block, in int8-codebook units: a weight's
 * value is S * codebook(code).
 * FP2/FP3: S = the fp16 scale. FP4: S = 2^(E - 128) (E the e8m0 byte;
 * the MX scale 2^(E - 127) halved because the codebook is 2 x E2M1).
 * FP3E: S = 2^(E - 127). */
double orc_block_scale(int fmt, const uint8_t *blk)
{
    int cb = orc_code_bytes(fmt);
    if (fmt == ORC_FP4)
        return ldexp(1.0, (int)blk[cb] - 128);
    if (fmt == ORC_FP3E)
        return ldexp(1.0, (int)blk[cb] - 127);
    return orc_f16_to_f64((uint16_t)(blk[cb] | (blk[cb + 1] << 8)));
}

/* Scale of weight t of a block: FP2S's fp16 scale of the half holding t
 * (bytes cb..cb+1 for weights 0..15, cb+2..cb+3 for 16..31); the block
 * scale for every other format. */
double orc_weight_scale(int fmt, const uint8_t *blk, int t)
{
    int cb = orc_code_bytes(fmt);
    if (fmt != ORC_FP2S)
        return orc_block_scale(fmt, blk);
    int o = cb + 2 * (t / 16);
    return orc_f16_to_f64((uint16_t)(blk[o] | (blk[o + 1] << 8)));
}

/* The value added after the scale: FP2M's fp16 minimum (after the fp16
 * scale), zero for the symmetric formats. */
double orc_block_min(int fmt, const uint8_t *blk)
{
    int cb = orc_code_bytes(fmt);
    if (fmt != ORC_FP2M)
        return 0.0;
    return orc_f16_to_f64((uint16_t)(blk[cb + 2] | (blk[cb + 3] << 8)));
}

void orc_dequantize_block(int fmt, const uint8_t *blk, double *w)
{
    int codes[32];
    orc_unpack_codes(fmt, blk, codes);
    double m = orc_block_min(fmt, blk);
    for (int t = 0; t < 32; t++)
        w[t] = orc_weight_scale(fmt, blk, t) * (double)orc_codebook(fmt, codes[t]) + m;
}

/* Canonical blocks [rows][nb][block bytes] -> fp64 [rows][32 nb]: the
 * block decoder above applied to every block in turn. */
void orc_dequantize_matrix(int fmt, const uint8_t *blocks, int64_t rows, int64_t nb, double *w)
{
    const int bb = orc_block_bytes(fmt);
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++)
            orc_dequantize_block(fmt, blocks + (r * nb + b) * bb, w + (r * nb + b) * 32);
}

/* ------------------------------------------------------------------ */
/* Encoder (Reading: absmax scaling; the real model used an importance  */
/* matrix [KK, mixed-precision section], which needs calibration data). */
/* ------------------------------------------------------------------ */
int orc_quantize_block(int fmt, const float *w, uint8_t *blk)
{
    int codes[32];
    int cb = orc_code_bytes(fmt);
    if (cb < 0)
        return ORC_E_INVAL;
    float amax = 0.0f;
    for (int t = 0; t < 32; t++) {
        if (!isfinite(w[t]))
            return ORC_E_RANGE;
        float a = fabsf(w[t]);
        if (a > amax)
            amax = a;
    }
    memset(blk, 0, (size_t)orc_block_bytes(fmt));
    if (fmt == ORC_FP2M) {
        /* Reading (asymmetric variant): m = fp16(min w) (round to nearest
         * even); s = fp16((max w - m) / 3) with the subtraction and the
         * division in fp32 (a negative span, when m rounded above every
         * weight, counts as 0); code = the value of 0..3 nearest to
         * (w - m) / s in fp32, ties to the larger; s = 0 gives code 0. */
        float lo = w[0], hi = w[0];
        for (int t = 1; t < 32; t++) {
            if (w[t] < lo)
                lo = w[t];
            if (w[t] > hi)
                hi = w[t];
        }
        uint16_t m16 = orc_f32_to_f16(lo);
        if ((m16 & 0x7fff) == 0x7c00)
            return ORC_E_RANGE;
        float m = (float)orc_f16_to_f64(m16);
        float span = hi - m;
        if (span < 0.0f)
            span = 0.0f;
        uint16_t s16 = orc_f32_to_f16(span / 3.0f);
        if ((s16 & 0x7fff) == 0x7c00)
            return ORC_E_RANGE;
        float s = (float)orc_f16_to_f64(s16);
        for (int t = 0; t < 32; t++)
            codes[t] = s == 0.0f ? 0 : orc_nearest_code(fmt, (double)((w[t] - m) / s));
        orc_pack_codes(fmt, codes, blk);
        blk[cb] = (uint8_t)(s16 & 0xff);
        blk[cb + 1] = (uint8_t)(s16 >> 8);
        blk[cb + 2] = (uint8_t)(m16 & 0xff);
        blk[cb + 3] = (uint8_t)(m16 >> 8);
        return ORC_OK;
    }
    if (fmt == ORC_FP4) {
        /* OCP MX shared exponent: floor(log2 amax) - emax(E2M1 = 2), biased
         * by 127, clamped to [0, 254]; amax = 0 gives E = 0. */
        int E = 0;
        if (amax > 0.0f) {
            int ex;
            frexp((double)amax, &ex); /* amax = f * 2^ex, f in [0.5, 1) */
            int fl = ex - 1;          /* floor(log2 amax), exact */
            E = fl - 2 + 127;
            if (E < 0)
                E = 0;
            if (E > 254)
                E = 254;
        }
        for (int t = 0; t < 32; t++) {
            double tt = ldexp((double)w[t], 128 - E); /* exact */
            codes[t] = orc_nearest_code(fmt, tt);
        }
        orc_pack_codes(fmt, codes, blk);
        blk[cb] = (uint8_t)E;
        return ORC_OK;
    }
    if (fmt == ORC_FP3E) {
        /* Reading: the OCP MX shared-exponent rule with FP3's largest value
         * 7 (floor(log2 7) = 2): E = floor(log2 amax) - 2 + 127, clamped
         * to [0, 254], amax = 0 gives E = 0; t = w * 2^(127 - E) (exact);
         * code = FP3's nearest value, ties to the larger magnitude, 0 to
         * +1; |t| in [7, 8) saturates at 7. */
        int E = 0;
        if (amax > 0.0f) {
            int ex;
            frexp((double)amax, &ex);
            E = (ex - 1) - 2 + 127;
            if (E < 0)
                E = 0;
            if (E > 254)
                E = 254;
        }
        for (int t = 0; t < 32; t++)
            codes[t] = orc_nearest_code(fmt, ldexp((double)w[t], 127 - E));
        orc_pack_codes(fmt, codes, blk);
        blk[cb] = (uint8_t)E;
        return ORC_OK;
    }
    if (fmt == ORC_Q8) {
        /* Reading: s = fp16(amax / 127), the division in fp32; code = the
         * int8 value nearest to w / s in fp32, ties to even, within
         * -127..127; s = 0 gives code 0. */
        uint16_t q16 = orc_f32_to_f16(amax / 127.0f);
        if ((q16 & 0x7fff) == 0x7c00)
            return ORC_E_RANGE;
        float qs = (float)orc_f16_to_f64(q16);
        for (int t = 0; t < 32; t++) {
            double r = qs == 0.0f ? 0.0 : rint((double)(w[t] / qs)); /* half to even */
            r = r > 127.0 ? 127.0 : r < -127.0 ? -127.0 : r;
            codes[t] = (int)(uint8_t)(int8_t)(int)r; /* stored as the byte */
        }
        orc_pack_codes(fmt, codes, blk);
        blk[cb] = (uint8_t)(q16 & 0xff);
        blk[cb + 1] = (uint8_t)(q16 >> 8);
        return ORC_OK;
    }
    if (fmt == ORC_FP2S) {
        /* Reading: each 16-weight half h is encoded exactly as an FP2
         * block would be with its own amax: s_h = fp16(amax_h / 3), the
         * division in fp32; code = the FP2 value nearest to w / s_h in
         * fp32; s_h = 0 gives every weight of the half the code of +1. */
        for (int h = 0; h < 2; h++) {
            float ah = 0.0f;
            for (int t = 16 * h; t < 16 * h + 16; t++)
                if (fabsf(w[t]) > ah)
                    ah = fabsf(w[t]);
            uint16_t h16 = orc_f32_to_f16(ah / 3.0f);
            if ((h16 & 0x7fff) == 0x7c00)
                return ORC_E_RANGE;
            float hs = (float)orc_f16_to_f64(h16);
            for (int t = 16 * h; t < 16 * h + 16; t++)
                codes[t] = hs == 0.0f ? 2 : orc_nearest_code(fmt, (double)(w[t] / hs));
            blk[cb + 2 * h] = (uint8_t)(h16 & 0xff);
            blk[cb + 2 * h + 1] = (uint8_t)(h16 >> 8);
        }
        orc_pack_codes(fmt, codes, blk);
        return ORC_OK;
    }
    float cmax = (fmt == ORC_FP2) ? 3.0f : 7.0f;
    float s32 = amax / cmax; /* IEEE fp32 division */
    uint16_t s16 = orc_f32_to_f16(s32);
    if ((s16 & 0x7fff) == 0x7c00)
        return ORC_E_RANGE;
    float s = (float)orc_f16_to_f64(s16);
    for (int t = 0; t < 32; t++) {
        if (s == 0.0f) {
            codes[t] = (fmt == ORC_FP2) ? 2 : 4; /* every weight -> +1 */
        } else {
            float tt = w[t] / s; /* IEEE fp32 division */
            codes[t] = orc_nearest_code(fmt, (double)tt);
        }
    }
    orc_pack_codes(fmt, codes, blk);
    blk[cb] = (uint8_t)(s16 & 0xff);
    blk[cb + 1] = (uint8_t)(s16 >> 8);
    return ORC_OK;
}

/* Row-major fp32 [rows][cols] -> canonical blocks [rows][cols/32][bytes]. */
int orc_quantize_matrix(int fmt, const float *W, int64_t rows, int64_t cols, uint8_t *out)
{
    int bb = orc_block_bytes(fmt);
    if (bb < 0 || cols % 32 != 0 || rows < 0)
        return ORC_E_INVAL;
    int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            int st = orc_quantize_block(fmt, W + r * cols + b * 32, out + (r * nb + b) * bb);
            if (st != ORC_OK)
                return st;
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Activation quantization (Reading: int8 per 32-block, fp32 scale).   */
/* ------------------------------------------------------------------ */
/* s = amax / 127 (fp32); q = clamp(round-half-even(x / s), -127, 127);
 * an all-zero block gets s = 0 and q = 0. Integer dots need integer
 * activations ([HM] para 3). n must be a multiple of 32. */
int orc_quantize_act(const float *x, int64_t n, int8_t *q, float *s)
{
    if (n % 32 != 0)
        return ORC_E_INVAL;
    for (int64_t b = 0; b < n / 32; b++) {
        const float *xb = x + 32 * b;
        float amax = 0.0f;
        for (int t = 0; t < 32; t++) {
            if (!isfinite(xb[t]))
                return ORC_E_RANGE;
            if (fabsf(xb[t]) > amax)
                amax = fabsf(xb[t]);
        }
        float sc = amax / 127.0f;
        s[b] = sc;
        for (int t = 0; t < 32; t++) {
            if (sc == 0.0f) {
                q[32 * b + t] = 0;
                continue;
            }
            float r = nearbyintf(xb[t] / sc); /* default mode: ties to even */
            if (r > 127.0f)
                r = 127.0f;
            if (r < -127.0f)
                r = -127.0f;
            q[32 * b + t] = (int8_t)r;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Product: y = W_hat . x_hat (the plain result the method reaches).   */
/* ------------------------------------------------------------------ */
/* Per block: D = sum_t codebook(c_t) * q_t, an exact integer; then
 * y[j][n] = sum_b S[n][b] * s[j][b] * D[j][n][b] in fp64, b ascending.
 * FP2M adds its minimum: sum_t (S c_t + M) s q_t = s (S D + M X) with X the
 * block's activation sum, also an exact integer.
 * FP2S scales its halves apart: s (S0 D0 + S1 D1), D0 and D1 the exact
 * dots over weights 0..15 and 16..31 (D = D0 + D1 is the block dot).
 * Each decoded weight serves every one of the Q columns ([AIN] section on
 * the optimization trio: decode once, apply to all verification columns);
 * the result is the same as Q separate one-column products.
 * W: canonical blocks [N][K/32]; xq [Q][K]; xs [Q][K/32]; y [Q][N];
 * dots (optional) [Q][N][K/32]. */
int orc_gemv(int fmt, const uint8_t *W, int64_t N, int64_t K, const int8_t *xq, const float *xs,
             int Q, double *y, int32_t *dots)
{
    int bb = orc_block_bytes(fmt);
    if (bb < 0 || K % 32 != 0 || N < 0 || Q < 1)
        return ORC_E_INVAL;
    int64_t nb = K / 32;
    for (int64_t n = 0; n < N; n++) {
        for (int j = 0; j < Q; j++)
            y[(int64_t)j * N + n] = 0.0;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = W + (n * nb + b) * bb;
            int codes[32];
            orc_unpack_codes(fmt, blk, codes);
            double S = orc_block_scale(fmt, blk), M = orc_block_min(fmt, blk);
            double S0 = orc_weight_scale(fmt, blk, 0), S1 = orc_weight_scale(fmt, blk, 16);
            for (int j = 0; j < Q; j++) {
                const int8_t *xb = xq + (int64_t)j * K + 32 * b;
                int64_t D = 0, X = 0, Dh[2] = {0, 0};
                for (int t = 0; t < 32; t++) {
                    D += (int64_t)orc_codebook(fmt, codes[t]) * (int64_t)xb[t];
                    Dh[t / 16] += (int64_t)orc_codebook(fmt, codes[t]) * (int64_t)xb[t];
                    X += (int64_t)xb[t];
                }
                if (dots)
                    dots[((int64_t)j * N + n) * nb + b] = (int32_t)D;
                if (fmt == ORC_FP2S)
                    y[(int64_t)j * N + n] += (double)xs[(int64_t)j * nb + b] * (S0 * (double)Dh[0] + S1 * (double)Dh[1]);
                else if (fmt == ORC_FP2M)
                    y[(int64_t)j * N + n] += (double)xs[(int64_t)j * nb + b] * (S * (double)D + M * (double)X);
                else
                    y[(int64_t)j * N + n] += S * (double)xs[(int64_t)j * nb + b] * (double)D;
            }
        }
    }
    return ORC_OK;
}
