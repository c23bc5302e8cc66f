// Activation quantizer and fused dequantize-and-multiply (GEMV) kernels for
// gfx950 (CDNA4, wave64).
//
// Pages cited (title, site):
//   [HM]  "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
//         (hellomarvisaitoday.com), paragraphs numbered from the top.
//   [AIN] "Token Freedom via APU: AMD Ryzen AI MAX+ 395 Runs DeepSeek V4
//         Flash at 32 tok/s on a 284B Model" (ainomam.com), by section.
//
// What the pages describe ([HM] para 3): decode at batch one is bound by
// weight traffic; the kernels read packed blocks straight from memory,
// expand the codebook with byte-permute instructions in registers and feed
// integer dot products; at q = 4 each packed weight is decoded once and
// used for all four verification columns ([AIN] optimization-trio section).
//
// Mapping on gfx950:
//   - one lane = one output row; a wave covers 64 rows of a 64 x 256 tile
//     and every 128-bit load of a wave reads 1 KiB of contiguous memory;
//   - the activation block is the same for all 64 lanes, so it is read with
//     scalar loads into SGPRs and used directly as the SGPR operand of
//     v_dot4_i32_i8: no LDS traffic and no cross-lane reduction per row;
//   - FP2/FP3 codebooks are affine in the code (v = 2c - 3, v = 2c - 7), so
//     the selector bytes go straight into v_dot4 and the offset is folded in
//     once per block with the precomputed activation block sum; FP4 (E2M1,
//     not affine) expands through two v_perm_b32 table lookups and a v_perm
//     merge on the sign bit;
//   - the 256-column tiles of a row group are split into contiguous runs over
//     the W waves of a workgroup (fixed-order LDS reduce) and, when the row
//     groups alone cannot fill 256 CUs, over P = 2^k workgroups; their
//     partials meet pairwise up a binary tree of exchange slots, each node
//     one two-term fp32 sum, so the result does not depend on arrival order
//     (deterministic, no float atomics, no counters, no L2 write-back);
//   - each wave keeps the next tile's loads in flight while it decodes the
//     current one.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rfx_internal.h"

namespace rfx {

int hip_status(const char *where)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(RFX_E_HIP, "%s: %s", where, hipGetErrorString(e));
    return RFX_OK;
}

} // namespace rfx

using namespace rfx;

namespace {


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef const int32_t __attribute__((address_space(4))) *sptr_i32;
typedef const float __attribute__((address_space(4))) *sptr_f32;

// Uniform pointer -> constant address space, so the compiler reads it with
// scalar loads (s_load_dwordxN) into SGPRs.
__device__ __forceinline__ sptr_i32 as_scalar_i32(const void *p)
{
    return (sptr_i32)(uintptr_t)p;
}
__device__ __forceinline__ sptr_f32 as_scalar_f32(const void *p)
{
    return (sptr_f32)(uintptr_t)p;
}

// ------------------------------------------------------------------
// Activation quantization: one lane per element, two 32-element blocks
// per wave. s = amax/127 (IEEE division), code = clamp(rne(x/s)).
// ------------------------------------------------------------------
__global__ __launch_bounds__(256) void act_quant_kernel(const float *__restrict__ x, int64_t n,
                                                        int8_t *__restrict__ xq,
                                                        float *__restrict__ xs,
                                                        int32_t *__restrict__ xsum)
{
#pragma clang fp contract(off)
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool valid = i < n;
    const float v = valid ? x[i] : 0.0f;
    float a = fabsf(v);
    for (int o = 16; o > 0; o >>= 1)
        a = fmaxf(a, __shfl_xor(a, o, 32));
    const float s = a / 127.0f;
    int qv = 0;
    if (s != 0.0f) {
        float r = rintf(v / s);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        qv = (int)r;
    }
    int sum = qv;
    for (int o = 16; o > 0; o >>= 1)
        sum += __shfl_xor(sum, o, 32);
    if (valid) {
        xq[i] = (int8_t)qv;
        if ((threadIdx.x & 31) == 0) {
            xs[i >> 5] = s;
            xsum[i >> 5] = sum;
        }
    }
}

// ------------------------------------------------------------------
// Per-block decode + integer dots.
// ------------------------------------------------------------------

// Selector bytes of one block, computed once and shared by every column.
struct Sel8 {
    int v[8];
};

__device__ __forceinline__ Sel8 sel_fp2(uint32_t w0, uint32_t w1)
{
    Sel8 s;
    s.v[0] = (int)(w0 & 0x03030303u);
    s.v[1] = (int)((w0 >> 2) & 0x03030303u);
    s.v[2] = (int)((w0 >> 4) & 0x03030303u);
    s.v[3] = (int)((w0 >> 6) & 0x03030303u);
    s.v[4] = (int)(w1 & 0x03030303u);
    s.v[5] = (int)((w1 >> 2) & 0x03030303u);
    s.v[6] = (int)((w1 >> 4) & 0x03030303u);
    s.v[7] = (int)((w1 >> 6) & 0x03030303u);
    return s;
}

// FP3: low two bits as FP2, high bit of weight 4i+j at bit 8j+i of h;
// selector byte = lo | hi << 2 = the 3-bit code.
__device__ __forceinline__ Sel8 sel_fp3(uint32_t w0, uint32_t w1, uint32_t h)
{
    Sel8 s = sel_fp2(w0, w1);
    s.v[0] |= (int)((h << 2) & 0x04040404u);
    s.v[1] |= (int)((h << 1) & 0x04040404u);
    s.v[2] |= (int)(h & 0x04040404u);
    s.v[3] |= (int)((h >> 1) & 0x04040404u);
    s.v[4] |= (int)((h >> 2) & 0x04040404u);
    s.v[5] |= (int)((h >> 3) & 0x04040404u);
    s.v[6] |= (int)((h >> 4) & 0x04040404u);
    s.v[7] |= (int)((h >> 5) & 0x04040404u);
    return s;
}

// FP4: nibble codes sign<<3 | m (m = E2M1 magnitude pattern). Two v_perm
// lookups give the positive and negative value of each byte lane; a third
// v_perm picks per byte on the sign bit. Values: 2 x E2M1 as int8.
constexpr uint32_t kPosLo = 0x03020100u; // 0 1 2 3
constexpr uint32_t kPosHi = 0x0C080604u; // 4 6 8 12
constexpr uint32_t kNegLo = 0xFDFEFF00u; // 0 -1 -2 -3
constexpr uint32_t kNegHi = 0xF4F8FAFCu; // -4 -6 -8 -12

__device__ __forceinline__ int fp4_expand(uint32_t nib_shifted_word, uint32_t sign_shifted_word)
{
    const uint32_t idx = nib_shifted_word & 0x07070707u;
    const uint32_t pos = __builtin_amdgcn_perm(kPosHi, kPosLo, idx);
    const uint32_t neg = __builtin_amdgcn_perm(kNegHi, kNegLo, idx);
    const uint32_t msel = (sign_shifted_word & 0x04040404u) | 0x03020100u;
    return (int)__builtin_amdgcn_perm(neg, pos, msel);
}

__device__ __forceinline__ Sel8 sel_fp4(u32x4 c)
{
    Sel8 s;
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int m = 0; m < 4; m++) {
        s.v[2 * m] = fp4_expand(w[m], w[m] >> 1);
        s.v[2 * m + 1] = fp4_expand(w[m] >> 4, w[m] >> 5);
    }
    return s;
}

__device__ __forceinline__ int dot8(const Sel8 &s, sptr_i32 xp)
{
    int d = 0;
#pragma unroll
    for (int i = 0; i < 8; i++)
        d = __builtin_amdgcn_sdot4(s.v[i], xp[i], d, false);
    return d;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)bits16);
}

struct GemvArgs {
    const uint8_t *W;
    int N, K, S, nb, P;
    const int8_t *xq;
    const float *xs;
    const int32_t *xsum;
    float *y;
    int32_t *dots;
    unsigned *slots; // split-K exchange slots (workspace)
};

template <int FMT>
struct TileFmt {
    static constexpr int bytes = FMT == RFX_FP2 ? 5120 : FMT == RFX_FP3 ? 7168 : 8704;
};

#ifndef RFX_PREFETCH_MAX_Q
#define RFX_PREFETCH_MAX_Q 2
#endif
constexpr int kPrefetchMaxQ = RFX_PREFETCH_MAX_Q;

// The activation block of every column, held in SGPRs (uniform).
template <int Q>
struct XBlock {
    int x[Q][8];
    float sx[Q];
    int sum[Q];
};

template <int FMT, int Q>
__device__ __forceinline__ XBlock<Q> load_xblock(const GemvArgs &a, int b)
{
    // 32-bit element offsets from one base pointer per array keep the
    // address arithmetic to one SGPR per load (base pair + offset).
    XBlock<Q> xb;
    const sptr_i32 xq = as_scalar_i32(a.xq), xsum = as_scalar_i32(a.xsum);
    const sptr_f32 xs = as_scalar_f32(a.xs);
#pragma unroll
    for (int j = 0; j < Q; j++) {
        const uint32_t xo = ((uint32_t)j * (uint32_t)a.K + 32u * (uint32_t)b) >> 2;
        const uint32_t mo = (uint32_t)j * (uint32_t)a.nb + (uint32_t)b;
#pragma unroll
        for (int i = 0; i < 8; i++)
            xb.x[j][i] = xq[xo + i];
        xb.sx[j] = xs[mo];
        xb.sum[j] = (FMT == RFX_FP4) ? 0 : xsum[mo];
    }
    return xb;
}

// Accumulate one block b of one 64-row tile into acc[Q] (or store dots).
template <int FMT, int Q, bool DOTS>
__device__ __forceinline__ void block_step(const Sel8 &sel, float sw, const XBlock<Q> &xb, int b, int row,
                                           const GemvArgs &a, float (&acc)[Q])
{
#pragma unroll
    for (int j = 0; j < Q; j++) {
        int d = 0;
#pragma unroll
        for (int i = 0; i < 8; i++)
            d = __builtin_amdgcn_sdot4(sel.v[i], xb.x[j][i], d, false);
        if (FMT == RFX_FP2 || FMT == RFX_FP3) {
            // codebook v = 2c - off: D = 2 sum(c x) - off sum(x)
            const int off = FMT == RFX_FP2 ? 3 : 7;
            d = 2 * d - off * xb.sum[j];
        }
        if (DOTS) {
            if (row < a.N)
                a.dots[((size_t)j * a.N + row) * a.nb + b] = d;
        } else {
            acc[j] += (sw * xb.sx[j]) * (float)d;
        }
    }
}

// Registers holding one 64-row x 8-block tile for one lane.
template <int FMT>
struct TileRegs {
    static constexpr int kCode = FMT == RFX_FP2 ? 4 : FMT == RFX_FP3 ? 6 : 8; // code chunks
    u32x4 c[kCode];
    u32x4 sc16; // FP2/FP3: eight fp16 scales
    u32x2 sc8;  // FP4: eight e8m0 bytes
};

template <int FMT>
__device__ __forceinline__ TileRegs<FMT> load_tile(const uint8_t *__restrict__ tile, int lane)
{
    TileRegs<FMT> t;
    const u32x4 *tp = reinterpret_cast<const u32x4 *>(tile) + lane;
#pragma unroll
    for (int k = 0; k < TileRegs<FMT>::kCode; k++)
        t.c[k] = __builtin_nontemporal_load(tp + 64 * k);
    if (FMT == RFX_FP4)
        t.sc8 = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(tile + 8 * 1024) + lane);
    else
        t.sc16 = __builtin_nontemporal_load(tp + 64 * TileRegs<FMT>::kCode);
    return t;
}

template <int FMT, int Q, bool DOTS>
__device__ __forceinline__ void compute_tile(const TileRegs<FMT> &t, int s, int row, const GemvArgs &a,
                                             float (&acc)[Q])
{
    const int b0 = s * 8;
    const int nvalid = min(8, a.nb - b0); // blocks of this tile inside K
    // The next block's activations are fetched while this block is decoded.
    XBlock<Q> xcur = load_xblock<FMT, Q>(a, b0);
#pragma unroll
    for (int bi = 0; bi < 8; bi++) {
        if (bi >= nvalid)
            break;
        // One block of prefetch fits the SGPR budget only for q <= 2; wider
        // blocks are fetched in one batch right before use.
        constexpr bool kPrefetch = Q <= kPrefetchMaxQ;
        XBlock<Q> xnext = xcur;
        if (kPrefetch && bi + 1 < nvalid)
            xnext = load_xblock<FMT, Q>(a, b0 + bi + 1);
        Sel8 sel;
        float sw;
        if (FMT == RFX_FP4) {
            sel = sel_fp4(t.c[bi]);
            const uint32_t e = ((bi < 4 ? t.sc8.x : t.sc8.y) >> (8 * (bi & 3))) & 0xffu;
            sw = ldexpf(1.0f, (int)e - 128);
        } else {
            const uint32_t w0 = (bi & 1) ? t.c[bi >> 1].z : t.c[bi >> 1].x;
            const uint32_t w1 = (bi & 1) ? t.c[bi >> 1].w : t.c[bi >> 1].y;
            if (FMT == RFX_FP3) {
                const u32x4 h4 = t.c[4 + (bi >> 2)];
                const uint32_t h = (bi & 3) == 0 ? h4.x : (bi & 3) == 1 ? h4.y : (bi & 3) == 2 ? h4.z : h4.w;
                sel = sel_fp3(w0, w1, h);
            } else {
                sel = sel_fp2(w0, w1);
            }
            const uint32_t sw2 = (bi >> 1) == 0 ? t.sc16.x : (bi >> 1) == 1 ? t.sc16.y : (bi >> 1) == 2 ? t.sc16.z : t.sc16.w;
            sw = half_bits_to_float((bi & 1) ? (sw2 >> 16) : (sw2 & 0xffffu));
        }
        block_step<FMT, Q, DOTS>(sel, sw, xcur, b0 + bi, row, a, acc);
        if (kPrefetch)
            xcur = xnext;
        else if (bi + 1 < nvalid)
            xcur = load_xblock<FMT, Q>(a, b0 + bi + 1);
    }
}

// One workgroup = W waves on one 64-row group; its tiles [s_begin, s_end)
// are split into contiguous runs, one per wave. Each wave keeps the next
// tile's loads in flight while it decodes the current one.
template <int FMT, int Q, bool DOTS>
__global__ __launch_bounds__(1024) void gemv_kernel(GemvArgs a)
{
    // wave index is uniform per wave; say so, so the tile index, the
    // activation addresses and the loop bounds live in SGPRs.
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    const int g = blockIdx.y, p = blockIdx.x; // grid = (P, G)
    const int row = g * 64 + lane;
    float acc[Q];
#pragma unroll
    for (int j = 0; j < Q; j++)
        acc[j] = 0.0f;

    const int nw = a.P * W, v = p * W + wave;
    const int s_begin = (int)((unsigned)(a.S * v) / (unsigned)nw);
    const int s_end = (int)((unsigned)(a.S * (v + 1)) / (unsigned)nw);
    const uint8_t *gbase = a.W + (size_t)g * a.S * TileFmt<FMT>::bytes;
    if (s_begin < s_end) {
        TileRegs<FMT> cur = load_tile<FMT>(gbase + (size_t)s_begin * TileFmt<FMT>::bytes, lane);
        for (int s = s_begin; s < s_end; s++) {
            TileRegs<FMT> nxt = cur;
            if (s + 1 < s_end)
                nxt = load_tile<FMT>(gbase + (size_t)(s + 1) * TileFmt<FMT>::bytes, lane);
            compute_tile<FMT, Q, DOTS>(cur, s, row, a, acc);
            cur = nxt;
        }
    }
    if (DOTS)
        return;

    // Fixed-order reduction over the waves of this workgroup.
    __shared__ float red[16][Q][64];
#pragma unroll
    for (int j = 0; j < Q; j++)
        red[wave][j][lane] = acc[j];
    __syncthreads();
    if (wave != 0)
        return;
    float val[Q];
#pragma unroll
    for (int j = 0; j < Q; j++) {
        float t = red[0][j][lane];
        for (int w = 1; w < W; w++)
            t += red[w][j][lane];
        val[j] = t;
    }
    if (a.P == 1) {
        if (row < a.N) {
#pragma unroll
            for (int j = 0; j < Q; j++)
                a.y[(size_t)j * a.N + row] = val[j];
        }
        return;
    }
    // Split K over P (a power of two) workgroups: combine the partials up a
    // binary tree. At each node the two children meet in a slot through an
    // atomic exchange (agent scope, coherent across XCDs); the first to
    // arrive leaves its value (stored inverted so the zero-filled slot
    // means "empty"), the second adds it to its own and climbs on. Each
    // node is one two-term fp32 sum, which is exact-order independent
    // (a + b == b + a), so the result does not depend on arrival order.
    // The second arriver clears the slot, leaving the workspace zeroed.
    unsigned *slots = a.slots + (size_t)g * (a.P - 1) * Q * 64;
    bool active[Q];
#pragma unroll
    for (int j = 0; j < Q; j++)
        active[j] = true;
    int node = p, level_base = 0, level_nodes = a.P >> 1;
    for (int span = 1; span < a.P; span <<= 1) {
        const int slot = level_base + (node >> 1);
#pragma unroll
        for (int j = 0; j < Q; j++) {
            if (!active[j])
                continue;
            unsigned *cell = slots + ((size_t)slot * Q + j) * 64 + lane;
            const unsigned old = __hip_atomic_exchange(cell, ~__float_as_uint(val[j]), __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            if (old == 0u) {
                active[j] = false;
            } else {
                val[j] = val[j] + __uint_as_float(~old);
                __hip_atomic_store(cell, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        level_base += level_nodes;
        level_nodes >>= 1;
        node >>= 1;
    }
    if (row < a.N) {
#pragma unroll
        for (int j = 0; j < Q; j++)
            if (active[j])
                a.y[(size_t)j * a.N + row] = val[j];
    }
}

struct LaunchShape {
    int P; // workgroups per row group (power of two)
    int W; // waves per workgroup
};

// Enough waves to give every SIMD a few, each wave one to two tiles; split
// K across workgroups only when the row groups alone cannot fill 256 CUs.
LaunchShape choose_shape(int G, int S)
{
    LaunchShape sh{1, 4};
    const int target_waves = 3072; // 1024 SIMDs x 3
    int P = 1;
    while (P < 8 && G * P * 16 < target_waves && S >= 2 * P * 4)
        P <<= 1;
    int W = (target_waves + G * P - 1) / (G * P);
    W = W < 4 ? 4 : W > 16 ? 16 : W;
    while (W > 1 && W * P > S)
        W--;
    sh.P = P;
    sh.W = W < 1 ? 1 : W;
    return sh;
}

size_t workspace_for(int G, int P, int q)
{
    if (P <= 1)
        return 0;
    return (size_t)G * (P - 1) * q * 64 * sizeof(unsigned);
}

template <int FMT, bool DOTS>
int launch_fmt(const GemvArgs &a, int q, int G, int W, hipStream_t st)
{
    dim3 grid(a.P, G), block(64 * W);
    switch (q) {
    case 1: hipLaunchKernelGGL((gemv_kernel<FMT, 1, DOTS>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<FMT, 2, DOTS>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((gemv_kernel<FMT, 3, DOTS>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<FMT, 4, DOTS>), grid, block, 0, st, a); break;
    default: return fail(RFX_E_INVAL, "q must be 1..4");
    }
    return hip_status("gemv launch");
}

template <bool DOTS>
int launch(int fmt, const GemvArgs &a, int q, int G, int W, hipStream_t st)
{
    switch (fmt) {
    case RFX_FP2: return launch_fmt<RFX_FP2, DOTS>(a, q, G, W, st);
    case RFX_FP3: return launch_fmt<RFX_FP3, DOTS>(a, q, G, W, st);
    case RFX_FP4: return launch_fmt<RFX_FP4, DOTS>(a, q, G, W, st);
    }
    return fail(RFX_E_INVAL, "unknown format");
}

int check_act(const int8_t *xq, const float *xs, const int32_t *xsum, bool need_xs)
{
    int st = check_ptr(xq, 16, "xq");
    if (!st && need_xs)
        st = check_ptr(xs, 4, "xs");
    if (!st)
        st = check_ptr(xsum, 4, "xsum");
    return st;
}

} // namespace

extern "C" {

int rfx_quantize_act(const float *x, int q, int K, int8_t *xq, float *xs, int32_t *xsum, void *stream)
{
    if (q < 1 || K < 32 || K % 32)
        return fail(RFX_E_INVAL, "rfx_quantize_act: bad shape q=%d K=%d", q, K);
    int st = check_ptr(x, 4, "x");
    if (!st)
        st = check_ptr(xq, 4, "xq");
    if (!st)
        st = check_ptr(xs, 4, "xs");
    if (!st)
        st = check_ptr(xsum, 4, "xsum");
    if (st)
        return st;
    const int64_t n = (int64_t)q * K;
    dim3 grid((unsigned)((n + 255) / 256)), block(256);
    hipLaunchKernelGGL(act_quant_kernel, grid, block, 0, (hipStream_t)stream, x, n, xq, xs, xsum);
    return hip_status("act_quant launch");
}

size_t rfx_gemv_workspace_bytes(const rfx_qmat *W, int q)
{
    if (!W || !fmt_ok(W->fmt) || W->rows < 1 || W->cols < 32 || q < 1 || q > 4)
        return 0;
    const int G = (int)ceil_div(W->rows, kTileRows), S = (int)ceil_div(W->cols, kTileCols);
    return workspace_for(G, choose_shape(G, S).P, q);
}

int rfx_gemv(const rfx_qmat *W, const int8_t *xq, const float *xs, const int32_t *xsum, int q,
             float *y, void *ws, size_t ws_bytes, void *stream)
{
    int st = check_qmat(W, "W", false);
    if (st)
        return st;
    if (q < 1 || q > 4)
        return fail(RFX_E_INVAL, "rfx_gemv: q=%d (must be 1..4)", q);
    if ((st = check_act(xq, xs, xsum, true)) || (st = check_ptr(y, 4, "y")))
        return st;
    const int G = (int)ceil_div(W->rows, kTileRows), S = (int)ceil_div(W->cols, kTileCols);
    LaunchShape sh = choose_shape(G, S);
    if (!ws) { // no workspace: one workgroup per row group
        sh.P = 1;
        sh.W = 16;
        while (sh.W > 1 && sh.W > S)
            sh.W--;
    } else {
        if (ws_bytes < workspace_for(G, sh.P, q))
            return fail(RFX_E_WORKSPACE, "rfx_gemv: workspace %zu < %zu bytes", ws_bytes,
                        workspace_for(G, sh.P, q));
        if ((st = check_ptr(ws, 256, "ws")))
            return st;
    }
    GemvArgs a{};
    a.W = static_cast<const uint8_t *>(W->data);
    a.N = W->rows;
    a.K = W->cols;
    a.S = S;
    a.nb = W->cols / 32;
    a.P = sh.P;
    a.xq = xq;
    a.xs = xs;
    a.xsum = xsum;
    a.y = y;
    a.slots = static_cast<unsigned *>(ws);
    return launch<false>(W->fmt, a, q, G, sh.W, (hipStream_t)stream);
}

int rfx_gemv_q1(const rfx_qmat *W, const int8_t *xq, const float *xs, const int32_t *xsum, float *y,
                void *ws, size_t ws_bytes, void *stream)
{
    return rfx_gemv(W, xq, xs, xsum, 1, y, ws, ws_bytes, stream);
}

int rfx_gemv_q4(const rfx_qmat *W, const int8_t *xq, const float *xs, const int32_t *xsum, float *y,
                void *ws, size_t ws_bytes, void *stream)
{
    return rfx_gemv(W, xq, xs, xsum, 4, y, ws, ws_bytes, stream);
}

int rfx_debug_block_dots(const rfx_qmat *W, const int8_t *xq, const int32_t *xsum, int q,
                         int32_t *dots, void *stream)
{
    int st = check_qmat(W, "W", false);
    if (st)
        return st;
    if (q < 1 || q > 4)
        return fail(RFX_E_INVAL, "rfx_debug_block_dots: q=%d", q);
    if ((st = check_act(xq, nullptr, xsum, false)) || (st = check_ptr(dots, 4, "dots")))
        return st;
    GemvArgs a{};
    a.W = static_cast<const uint8_t *>(W->data);
    a.N = W->rows;
    a.K = W->cols;
    a.S = (int)ceil_div(W->cols, kTileCols);
    a.nb = W->cols / 32;
    a.P = 1;
    a.xq = xq;
    a.xsum = xsum;
    a.dots = dots;
    const int G = (int)ceil_div(W->rows, kTileRows);
    return launch<true>(W->fmt, a, q, G, 4, (hipStream_t)stream);
}

} // extern "C"
