// Host side of librfx: status strings, argument validation, the block
// encoder/decoder and the packer for the tiled device layout.
//
// Pages cited (title, site):
//   [HM] "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
//        (hellomarvisaitoday.com), paragraphs numbered from the top.
//   [KK] the kaikai365.com post on DeepSeek V4 Flash on Strix Halo, by
//        section heading.
//
// A block is 32 weights of one row, packed codes plus one scale; FP2/FP3/FP4
// take 10/14/17 bytes ([HM] para 2; [KK] mixed-precision section). The
// pages leave codebooks, scale and rounding rules and the bit order open;
// the choices made here are documented in include/rfx.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "rfx_internal.h"

namespace rfx {

static thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int check_ptr(const void *p, size_t align, const char *what)
{
    if (!p)
        return fail(RFX_E_INVAL, "%s is NULL", what);
    if (reinterpret_cast<uintptr_t>(p) % align)
        return fail(RFX_E_ALIGN, "%s is not %zu-byte aligned", what, align);
    return RFX_OK;
}

int check_qmat(const rfx_qmat *W, const char *what, bool allow_stack, bool data_optional)
{
    if (!W)
        return fail(RFX_E_INVAL, "%s descriptor is NULL", what);
    if (!fmt_ok(W->fmt))
        return fail(RFX_E_INVAL, "%s: unknown format %d", what, W->fmt);
    if (W->rows < 1 || W->cols < 32 || W->cols % 32)
        return fail(RFX_E_INVAL, "%s: bad shape %d x %d (cols must be a positive multiple of 32)",
                    what, W->rows, W->cols);
    if (W->count < 1 || (!allow_stack && W->count != 1))
        return fail(RFX_E_INVAL, "%s: bad count %d", what, W->count);
    if (data_optional && !W->data)
        return RFX_OK;
    return check_ptr(W->data, 256, what);
}

} // namespace rfx

using namespace rfx;

extern "C" {

const char *rfx_status_str(int st)
{
    switch (st) {
    case RFX_OK: return "ok";
    case RFX_E_INVAL: return "invalid argument";
    case RFX_E_ALIGN: return "misaligned pointer";
    case RFX_E_RANGE: return "value out of range";
    case RFX_E_UNSUPPORTED: return "unsupported";
    case RFX_E_WORKSPACE: return "workspace missing or too small";
    case RFX_E_HIP: return "HIP runtime error";
    case RFX_E_TIMEOUT: return "a bounded device-side wait ran out";
    }
    return "unknown status";
}

const char *rfx_last_error(void) { return g_last_error.c_str(); }

const char *rfx_version(void) { return "rfx 0.1 gfx950"; }

int rfx_block_bytes(int fmt)
{
    return fmt == RFX_FP2 ? 10 : fmt == RFX_FP3 ? 14 : fmt == RFX_FP4 ? 17 : fmt == RFX_FP2M || fmt == RFX_FP2S ? 12
         : fmt == RFX_Q8 ? 34 : fmt == RFX_FP3E ? 13 : RFX_E_INVAL;
}

int rfx_code_bytes(int fmt)
{
    return fmt == RFX_FP2 || fmt == RFX_FP2M || fmt == RFX_FP2S ? 8 : fmt == RFX_FP3 || fmt == RFX_FP3E ? 12
         : fmt == RFX_FP4 ? 16
         : fmt == RFX_Q8 ? 32 : RFX_E_INVAL;
}

int rfx_scale_bytes(int fmt)
{
    return fmt == RFX_FP2 || fmt == RFX_FP3 || fmt == RFX_Q8 ? 2 : fmt == RFX_FP4 || fmt == RFX_FP3E ? 1
         : fmt == RFX_FP2M || fmt == RFX_FP2S ? 4
         : RFX_E_INVAL;
}

} // extern "C"

namespace {

// Nearest codebook value, as threshold comparisons on |t| (the codebooks
// are symmetric). Ties: FP2/FP3 to the larger magnitude, FP4 to the even
// E2M1 mantissa. Returns the code.
inline int code_fp2(float t)
{
    float a = std::fabs(t);
    int m = a >= 2.0f ? 3 : 1;               // magnitude
    int v = std::signbit(t) && t != 0.0f ? -m : m; // +-0 -> +1
    return (v + 3) / 2;
}

inline int code_fp3(float t)
{
    float a = std::fabs(t);
    int m = a >= 6.0f ? 7 : a >= 4.0f ? 5 : a >= 2.0f ? 3 : 1;
    int v = std::signbit(t) && t != 0.0f ? -m : m;
    return (v + 7) / 2;
}

inline int code_fp4(float t)
{
    // E2M1 magnitudes in int8 units 0,1,2,3,4,6,8,12 at indices 0..7;
    // round half to even on the E2M1 grid (even index), saturate at 12.
    float a = std::fabs(t);
    int idx = a <= 0.5f ? 0 : a < 1.5f ? 1 : a <= 2.5f ? 2 : a < 3.5f ? 3
            : a <= 5.0f ? 4 : a < 7.0f ? 5 : a <= 10.0f ? 6 : 7;
    if (idx != 0 && std::signbit(t))
        idx |= 8;
    return idx;
}

inline void put_code(int fmt, uint8_t *codes, int t, int c)
{
    if (fmt == RFX_Q8) {
        codes[t] = (uint8_t)c;
    } else if (fmt == RFX_FP2 || fmt == RFX_FP3 || fmt == RFX_FP2M || fmt == RFX_FP2S || fmt == RFX_FP3E) {
        int m = t >> 4, i = (t >> 2) & 3, j = t & 3;
        codes[4 * m + j] |= (uint8_t)((c & 3) << (2 * i));
        if (fmt == RFX_FP3 || fmt == RFX_FP3E)
            codes[8 + j] |= (uint8_t)(((c >> 2) & 1) << (t >> 2));
    } else {
        int m = t >> 3, i = (t >> 2) & 1, j = t & 3;
        codes[4 * m + j] |= (uint8_t)((c & 15) << (4 * i));
    }
}

inline int get_code(int fmt, const uint8_t *codes, int t)
{
    if (fmt == RFX_Q8)
        return codes[t];
    if (fmt == RFX_FP2 || fmt == RFX_FP3 || fmt == RFX_FP2M || fmt == RFX_FP2S || fmt == RFX_FP3E) {
        int m = t >> 4, i = (t >> 2) & 3, j = t & 3;
        int c = (codes[4 * m + j] >> (2 * i)) & 3;
        if (fmt == RFX_FP3 || fmt == RFX_FP3E)
            c |= ((codes[8 + j] >> (t >> 2)) & 1) << 2;
        return c;
    }
    int m = t >> 3, i = (t >> 2) & 1, j = t & 3;
    return (codes[4 * m + j] >> (4 * i)) & 15;
}

inline int code_value(int fmt, int c)
{
    static const int mag[8] = {0, 1, 2, 3, 4, 6, 8, 12};
    if (fmt == RFX_FP2 || fmt == RFX_FP2S)
        return 2 * c - 3;
    if (fmt == RFX_FP3 || fmt == RFX_FP3E)
        return 2 * c - 7;
    if (fmt == RFX_FP2M)
        return c;
    if (fmt == RFX_Q8)
        return (int)(int8_t)(uint8_t)c;
    return (c & 8) ? -mag[c & 7] : mag[c & 7];
}

inline void put_half(uint8_t *p, _Float16 h)
{
    uint16_t bits;
    std::memcpy(&bits, &h, 2);
    p[0] = (uint8_t)(bits & 0xff);
    p[1] = (uint8_t)(bits >> 8);
}

inline float get_half(const uint8_t *p)
{
    const uint16_t bits = (uint16_t)(p[0] | (p[1] << 8));
    _Float16 h;
    std::memcpy(&h, &bits, 2);
    return (float)h;
}

// FP2M: the minimum and the span over three, both rounded to fp16; codes
// by threshold on t = (w - m) / s (fp32), ties to the larger code.
int encode_fp2m(const float *w, uint8_t *blk)
{
    // strict comparisons: among equal values (+0 and -0) the first one
    // stays, so the signs of zero are fixed by the block's order
    float lo = w[0], hi = w[0];
    for (int t = 1; t < 32; t++) {
        if (w[t] < lo)
            lo = w[t];
        if (w[t] > hi)
            hi = w[t];
    }
    const _Float16 mh = (_Float16)lo;
    const float m = (float)mh;
    if (std::isinf(m))
        return fail(RFX_E_RANGE, "fp16 minimum overflow (min %g)", (double)lo);
    float span = hi - m;
    if (span < 0.0f)
        span = 0.0f;
    const _Float16 sh = (_Float16)(span / 3.0f);
    const float s = (float)sh;
    if (std::isinf(s))
        return fail(RFX_E_RANGE, "fp16 scale overflow (span %g)", (double)span);
    for (int t = 0; t < 32; t++) {
        int c = 0;
        if (s != 0.0f) {
            const float q = (w[t] - m) / s;
            c = q >= 2.5f ? 3 : q >= 1.5f ? 2 : q >= 0.5f ? 1 : 0;
        }
        put_code(RFX_FP2M, blk, t, c);
    }
    put_half(blk + 8, sh);
    put_half(blk + 10, mh);
    return RFX_OK;
}

// FP2S: each 16-weight half is an FP2 block of its own: its scale is the
// half's amax over three rounded to fp16, its codes are FP2's.
int encode_fp2s(const float *w, uint8_t *blk)
{
    for (int h = 0; h < 2; h++) {
        float amax = 0.0f;
        for (int t = 16 * h; t < 16 * h + 16; t++)
            amax = std::fmax(amax, std::fabs(w[t]));
        const _Float16 sh = (_Float16)(amax / 3.0f); // fp32 division, then RNE to binary16
        const float s = (float)sh;
        if (std::isinf(s))
            return fail(RFX_E_RANGE, "fp16 scale overflow (half %d, amax %g)", h, (double)amax);
        for (int t = 16 * h; t < 16 * h + 16; t++)
            put_code(RFX_FP2S, blk, t, s == 0.0f ? 2 : code_fp2(w[t] / s));
        put_half(blk + 8 + 2 * h, sh);
    }
    return RFX_OK;
}

int encode_block(int fmt, const float *w, uint8_t *blk)
{
    const int cb = rfx_code_bytes(fmt);
    float amax = 0.0f;
    for (int t = 0; t < 32; t++) {
        if (!std::isfinite(w[t]))
            return fail(RFX_E_RANGE, "non-finite weight");
        amax = std::fmax(amax, std::fabs(w[t]));
    }
    std::memset(blk, 0, (size_t)rfx_block_bytes(fmt));
    if (fmt == RFX_FP2M)
        return encode_fp2m(w, blk);
    if (fmt == RFX_FP2S)
        return encode_fp2s(w, blk);
    if (fmt == RFX_Q8) {
        const _Float16 h = (_Float16)(amax / 127.0f); // fp32 division, then RNE to binary16
        const float s = (float)h;
        if (std::isinf(s))
            return fail(RFX_E_RANGE, "fp16 scale overflow (amax %g)", (double)amax);
        for (int t = 0; t < 32; t++) {
            float r = s == 0.0f ? 0.0f : std::nearbyint(w[t] / s); // half to even
            r = std::fmin(std::fmax(r, -127.0f), 127.0f);
            put_code(fmt, blk, t, (int)r);
        }
        put_half(blk + cb, h);
        return RFX_OK;
    }
    if (fmt == RFX_FP3E) {
        // the OCP MX rule with FP3's largest value 7 (floor(log2 7) = 2);
        // the scale 2^(E - 127) applied exactly by ldexp
        int E = 0;
        if (amax > 0.0f) {
            E = std::ilogb(amax) - 2 + 127;
            E = E < 0 ? 0 : E > 254 ? 254 : E;
        }
        for (int t = 0; t < 32; t++)
            put_code(fmt, blk, t, code_fp3(std::ldexp(w[t], 127 - E)));
        blk[cb] = (uint8_t)E;
        return RFX_OK;
    }
    if (fmt == RFX_FP4) {
        // OCP MX: E = floor(log2 amax) - 2 + 127, clamped; ilogb is exact,
        // subnormals included.
        int E = 0;
        if (amax > 0.0f) {
            E = std::ilogb(amax) - 2 + 127;
            E = E < 0 ? 0 : E > 254 ? 254 : E;
        }
        for (int t = 0; t < 32; t++)
            put_code(fmt, blk, t, code_fp4(std::ldexp(w[t], 128 - E)));
        blk[cb] = (uint8_t)E;
        return RFX_OK;
    }
    const float cmax = fmt == RFX_FP2 ? 3.0f : 7.0f;
    const _Float16 h = (_Float16)(amax / cmax); // fp32 division, then RNE to binary16
    const float s = (float)h;
    if (std::isinf(s))
        return fail(RFX_E_RANGE, "fp16 scale overflow (amax %g)", (double)amax);
    for (int t = 0; t < 32; t++) {
        int c = s == 0.0f ? (fmt == RFX_FP2 ? 2 : 4) : (fmt == RFX_FP2 ? code_fp2(w[t] / s)
                                                                      : code_fp3(w[t] / s));
        put_code(fmt, blk, t, c);
    }
    uint16_t bits;
    std::memcpy(&bits, &h, 2);
    blk[cb] = (uint8_t)(bits & 0xff);
    blk[cb + 1] = (uint8_t)(bits >> 8);
    return RFX_OK;
}

// Byte positions of block (row r, block b) in the tiled layout.
struct TilePos {
    size_t code0;  // first 8 or 16 code bytes
    size_t code1;  // FP3: the 4 high-bit bytes
    size_t scale;  // scale byte(s)
    size_t second; // FP2M: the fp16 minimum; FP2S: the second half's fp16 scale
};

inline TilePos tile_pos(int fmt, int64_t cols, int64_t r, int64_t b)
{
    const int64_t S = ceil_div(cols, kTileCols);
    const int64_t g = r / kTileRows, lane = r % kTileRows;
    const int64_t s = b / kTileBlocks, bi = b % kTileBlocks;
    const size_t tile = (size_t)(g * S + s) * (size_t)tile_bytes(fmt);
    TilePos p{};
    if (fmt == RFX_FP4) {
        p.code0 = tile + bi * kChunk + lane * 16;
        p.scale = tile + 8 * kChunk + lane * 8 + bi;
    } else if (fmt == RFX_FP3E) { // FP3's code chunks, then FP4's scale area
        p.code0 = tile + (bi / 2) * kChunk + lane * 16 + (bi % 2) * 8;
        p.code1 = tile + (4 + bi / 4) * kChunk + lane * 16 + (bi % 4) * 4;
        p.scale = tile + 6 * kChunk + lane * 8 + bi;
    } else if (fmt == RFX_Q8) {
        p.code0 = tile + (2 * bi) * kChunk + lane * 16;
        p.code1 = tile + (2 * bi + 1) * kChunk + lane * 16;
        p.scale = tile + 16 * kChunk + lane * 16 + bi * 2;
    } else {
        p.code0 = tile + (bi / 2) * kChunk + lane * 16 + (bi % 2) * 8;
        if (fmt == RFX_FP3) {
            p.code1 = tile + (4 + bi / 4) * kChunk + lane * 16 + (bi % 4) * 4;
            p.scale = tile + 6 * kChunk + lane * 16 + bi * 2;
        } else {
            p.scale = tile + 4 * kChunk + lane * 16 + bi * 2;
            p.second = tile + 5 * kChunk + lane * 16 + bi * 2;
        }
    }
    return p;
}

void place_block(int fmt, int64_t cols, int64_t r, int64_t b, const uint8_t *blk, uint8_t *tiled)
{
    TilePos p = tile_pos(fmt, cols, r, b);
    const int cb = rfx_code_bytes(fmt);
    if (fmt == RFX_FP4) {
        std::memcpy(tiled + p.code0, blk, 16);
        tiled[p.scale] = blk[16];
    } else if (fmt == RFX_FP3E) {
        std::memcpy(tiled + p.code0, blk, 8);
        std::memcpy(tiled + p.code1, blk + 8, 4);
        tiled[p.scale] = blk[12];
    } else if (fmt == RFX_Q8) {
        std::memcpy(tiled + p.code0, blk, 16);
        std::memcpy(tiled + p.code1, blk + 16, 16);
        std::memcpy(tiled + p.scale, blk + cb, 2);
    } else {
        std::memcpy(tiled + p.code0, blk, 8);
        if (fmt == RFX_FP3)
            std::memcpy(tiled + p.code1, blk + 8, 4);
        std::memcpy(tiled + p.scale, blk + cb, 2);
        if (fmt == RFX_FP2M || fmt == RFX_FP2S)
            std::memcpy(tiled + p.second, blk + cb + 2, 2);
    }
}

void fetch_block(int fmt, int64_t cols, int64_t r, int64_t b, const uint8_t *tiled, uint8_t *blk)
{
    TilePos p = tile_pos(fmt, cols, r, b);
    const int cb = rfx_code_bytes(fmt);
    if (fmt == RFX_FP4) {
        std::memcpy(blk, tiled + p.code0, 16);
        blk[16] = tiled[p.scale];
    } else if (fmt == RFX_FP3E) {
        std::memcpy(blk, tiled + p.code0, 8);
        std::memcpy(blk + 8, tiled + p.code1, 4);
        blk[12] = tiled[p.scale];
    } else if (fmt == RFX_Q8) {
        std::memcpy(blk, tiled + p.code0, 16);
        std::memcpy(blk + 16, tiled + p.code1, 16);
        std::memcpy(blk + cb, tiled + p.scale, 2);
    } else {
        std::memcpy(blk, tiled + p.code0, 8);
        if (fmt == RFX_FP3)
            std::memcpy(blk + 8, tiled + p.code1, 4);
        std::memcpy(blk + cb, tiled + p.scale, 2);
        if (fmt == RFX_FP2M || fmt == RFX_FP2S)
            std::memcpy(blk + cb + 2, tiled + p.second, 2);
    }
}

int check_matrix_args(int fmt, const void *a, int64_t rows, int64_t cols, const void *b)
{
    if (!fmt_ok(fmt))
        return fail(RFX_E_INVAL, "unknown format %d", fmt);
    if (rows < 1 || cols < 32 || cols % 32 || rows > (1ll << 31) || cols > (1ll << 31))
        return fail(RFX_E_INVAL, "bad shape %lld x %lld", (long long)rows, (long long)cols);
    if (!a || !b)
        return fail(RFX_E_INVAL, "NULL buffer");
    return RFX_OK;
}

// Runs fn(row_group) over all 64-row groups on `threads` host threads.
template <class F>
int for_row_groups(int64_t rows, int threads, F fn)
{
    const int64_t G = ceil_div(rows, kTileRows);
    if (threads <= 0)
        threads = (int)std::thread::hardware_concurrency();
    threads = (int)std::max<int64_t>(1, std::min<int64_t>(threads, G));
    std::vector<int> status(threads, RFX_OK);
    std::vector<std::string> errs(threads);
    auto work = [&](int tid) {
        for (int64_t g = tid; g < G; g += threads) {
            int st = fn(g);
            if (st != RFX_OK) {
                status[tid] = st;
                errs[tid] = g_last_error;
                return;
            }
        }
    };
    if (threads == 1) {
        work(0);
    } else {
        std::vector<std::thread> pool;
        for (int t = 0; t < threads; t++)
            pool.emplace_back(work, t);
        for (auto &th : pool)
            th.join();
    }
    for (int t = 0; t < threads; t++)
        if (status[t] != RFX_OK) {
            g_last_error = errs[t];
            return status[t];
        }
    return RFX_OK;
}

} // namespace

extern "C" {

int rfx_quantize_block(int fmt, const float *w32, uint8_t *blk)
{
    if (!fmt_ok(fmt))
        return fail(RFX_E_INVAL, "unknown format %d", fmt);
    if (!w32 || !blk)
        return fail(RFX_E_INVAL, "NULL buffer");
    return encode_block(fmt, w32, blk);
}

int rfx_dequantize_block(int fmt, const uint8_t *blk, float *w32)
{
    if (!fmt_ok(fmt))
        return fail(RFX_E_INVAL, "unknown format %d", fmt);
    if (!w32 || !blk)
        return fail(RFX_E_INVAL, "NULL buffer");
    const int cb = rfx_code_bytes(fmt);
    const float s = fmt == RFX_FP4    ? std::ldexp(1.0f, (int)blk[cb] - 128)
                  : fmt == RFX_FP3E ? std::ldexp(1.0f, (int)blk[cb] - 127)
                                    : get_half(blk + cb);
    const float m = fmt == RFX_FP2M ? get_half(blk + cb + 2) : 0.0f;
    const float s1 = fmt == RFX_FP2S ? get_half(blk + cb + 2) : s; // FP2S: weights 16..31
    for (int t = 0; t < 32; t++)
        w32[t] = (t < 16 ? s : s1) * (float)code_value(fmt, get_code(fmt, blk, t)) + m;
    return RFX_OK;
}

int64_t rfx_qmat_bytes(int fmt, int64_t rows, int64_t cols)
{
    if (!fmt_ok(fmt) || rows < 1 || cols < 32 || cols % 32)
        return fail(RFX_E_INVAL, "bad matrix %d %lld x %lld", fmt, (long long)rows, (long long)cols);
    return ceil_div(rows, kTileRows) * ceil_div(cols, kTileCols) * (int64_t)tile_bytes(fmt);
}

int rfx_quantize_matrix(int fmt, const float *W, int64_t rows, int64_t cols, void *tiled,
                        int threads)
{
    int st = check_matrix_args(fmt, W, rows, cols, tiled);
    if (st)
        return st;
    uint8_t *out = static_cast<uint8_t *>(tiled);
    const int64_t S = ceil_div(cols, kTileCols), nb = cols / 32;
    const size_t group_bytes = (size_t)S * tile_bytes(fmt);
    return for_row_groups(rows, threads, [&](int64_t g) -> int {
        std::memset(out + g * group_bytes, 0, group_bytes);
        uint8_t blk[kMaxBlockBytes];
        for (int64_t r = g * kTileRows; r < std::min<int64_t>(rows, (g + 1) * kTileRows); r++)
            for (int64_t b = 0; b < nb; b++) {
                int s2 = encode_block(fmt, W + r * cols + b * 32, blk);
                if (s2)
                    return s2;
                place_block(fmt, cols, r, b, blk, out);
            }
        return RFX_OK;
    });
}

int rfx_export_blocks(int fmt, const void *tiled, int64_t rows, int64_t cols, uint8_t *blocks)
{
    int st = check_matrix_args(fmt, tiled, rows, cols, blocks);
    if (st)
        return st;
    const int bb = rfx_block_bytes(fmt);
    const int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++)
            fetch_block(fmt, cols, r, b, static_cast<const uint8_t *>(tiled), blocks + (r * nb + b) * bb);
    return RFX_OK;
}

int rfx_import_blocks(int fmt, const uint8_t *blocks, int64_t rows, int64_t cols, void *tiled)
{
    int st = check_matrix_args(fmt, blocks, rows, cols, tiled);
    if (st)
        return st;
    const int bb = rfx_block_bytes(fmt);
    const int64_t nb = cols / 32;
    std::memset(tiled, 0, (size_t)rfx_qmat_bytes(fmt, rows, cols));
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++)
            place_block(fmt, cols, r, b, blocks + (r * nb + b) * bb, static_cast<uint8_t *>(tiled));
    return RFX_OK;
}

} // extern "C"
