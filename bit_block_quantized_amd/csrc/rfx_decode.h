// Device-side decode core shared by the GEMV and MoE kernels (gfx950).
//
// Pages cited (title, site):
//   [HM] "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
//        (hellomarvisaitoday.com), paragraphs numbered from the top.
//
// [HM] para 3: packed blocks are read directly, codebooks are expanded with
// byte-permute instructions in registers and feed integer dot products.
// Here: one lane owns one output row of a 64-row x 8-block tile; the
// activation block is uniform across the wave and lives in SGPRs, used as
// the SGPR operand of v_dot4_i32_i8.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "rfx.h"

namespace rfx {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef const int32_t __attribute__((address_space(4))) *sptr_i32;
typedef const float __attribute__((address_space(4))) *sptr_f32;

// A pointer read from memory (a per-expert table) is generic to the
// compiler, so loads through it become flat loads, which count against
// lgkmcnt as well as vmcnt: every wait for an LDS or scalar result then also
// waits for the weight loads in flight. Device memory and mapped pinned host
// memory are both in the global aperture, so such a pointer is re-typed as
// global (an address-space cast the compiler propagates to the loads).
__device__ __forceinline__ const uint8_t *as_global(const void *p)
{
    typedef const __attribute__((address_space(1))) uint8_t *gptr_u8;
    return (const uint8_t *)(gptr_u8)(uintptr_t)p;
}

// s_waitcnt immediate (gfx9 encoding): lgkmcnt = 0, vmcnt and expcnt at
// their maxima: wait for every outstanding scalar and LDS operation only.
constexpr int kWaitLgkmcnt0 = 0xC07F;

// Uniform pointer -> constant address space, so the compiler reads it with
// scalar loads (s_load_dwordxN) into SGPRs.
__device__ __forceinline__ sptr_i32 as_scalar_i32(const void *p) { return (sptr_i32)(uintptr_t)p; }
__device__ __forceinline__ sptr_f32 as_scalar_f32(const void *p) { return (sptr_f32)(uintptr_t)p; }

template <int FMT>
struct TileFmt {
    static constexpr int bytes = FMT == RFX_FP2 ? 5120 : FMT == RFX_FP3 ? 7168
                               : FMT == RFX_FP2M || FMT == RFX_FP2S ? 6144 : FMT == RFX_Q8 ? 17408
                               : FMT == RFX_FP3E ? 6656 : 8704;
    static constexpr int code_chunks = FMT == RFX_FP2 || FMT == RFX_FP2M || FMT == RFX_FP2S ? 4
                                     : FMT == RFX_FP3 || FMT == RFX_FP3E ? 6
                                     : FMT == RFX_Q8 ? 16 : 8;
    // the activation block sums enter the result (codebook offset or minimum)
    static constexpr bool needs_sum = FMT == RFX_FP2 || FMT == RFX_FP3 || FMT == RFX_FP2M || FMT == RFX_FP3E;
};

// ------------------------------------------------------------------
// Selector / value bytes of one block, computed once for every column.
// ------------------------------------------------------------------
struct Sel8 {
    int v[8];
};

// FP2: word m holds weights 16m..16m+15, group i (x dword 4m+i) in bits
// 2i..2i+1 of each byte. The selector byte is the code c; the codebook is
// v = 2c - 3, so sum(v x) = 2 sum(c x) - 3 sum(x).
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

// FP2S: the codes expanded through FP2's codebook {-3, -1, +1, +3} (bytes
// FD FF 01 03) by one v_perm per four weights. With the signed values each
// half's dot is a plain sum: dwords 0-3 are weights 0..15, dwords 4-7
// weights 16..31, so neither half needs an activation sum.
constexpr uint32_t kFp2Values = 0x0301FFFDu;

__device__ __forceinline__ Sel8 sel_fp2s(uint32_t w0, uint32_t w1)
{
    Sel8 s = sel_fp2(w0, w1);
#pragma unroll
    for (int i = 0; i < 8; i++)
        s.v[i] = (int)__builtin_amdgcn_perm(0u, kFp2Values, (uint32_t)s.v[i]);
    return s;
}

// FP3: low two bits as FP2, high bit of weight 4i+j at bit 8j+i of h;
// selector byte = lo | hi << 2 = the 3-bit code (v = 2c - 7).
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
// v_perm picks per byte on the sign bit. Values are 2 x E2M1 as int8.
constexpr uint32_t kPosLo = 0x03020100u; // 0 1 2 3
constexpr uint32_t kPosHi = 0x0C080604u; // 4 6 8 12
constexpr uint32_t kNegLo = 0xFDFEFF00u; // 0 -1 -2 -3
constexpr uint32_t kNegHi = 0xF4F8FAFCu; // -4 -6 -8 -12

// A constant materialized in a VGPR. VOP3 instructions on gfx9 take no
// literal and read at most one SGPR, so (x & a) | b with two constants
// only becomes one v_and_or_b32 when one of them sits in a VGPR.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c)
{
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
    return r;
}

__device__ __forceinline__ int fp4_expand(uint32_t nib_shifted_word, uint32_t sign_shifted_word, uint32_t k4)
{
    const uint32_t idx = nib_shifted_word & 0x07070707u;
    const uint32_t pos = __builtin_amdgcn_perm(kPosHi, kPosLo, idx);
    const uint32_t neg = __builtin_amdgcn_perm(kNegHi, kNegLo, idx);
    const uint32_t msel = (sign_shifted_word & k4) | 0x03020100u; // one v_and_or_b32
    return (int)__builtin_amdgcn_perm(neg, pos, msel);
}

__device__ __forceinline__ Sel8 sel_fp4(u32x4 c)
{
    Sel8 s;
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const uint32_t k4 = vgpr_const(0x04040404u);
#pragma unroll
    for (int m = 0; m < 4; m++) {
        s.v[2 * m] = fp4_expand(w[m], w[m] >> 1, k4);
        s.v[2 * m + 1] = fp4_expand(w[m] >> 4, w[m] >> 5, k4);
    }
    return s;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)bits16);
}

// ------------------------------------------------------------------
// One 64-row x 8-block tile in registers (one lane = one row).
// ------------------------------------------------------------------
template <int FMT>
struct TileRegs {
    u32x4 c[TileFmt<FMT>::code_chunks];
    u32x4 sc16; // FP2/FP3/FP2M/Q8: eight fp16 scales
    u32x4 mn16; // FP2M: eight fp16 minima; FP2S: the eight second-half scales
    u32x2 sc8;  // FP4 / FP3E: eight e8m0 bytes
};

// Issue order = use order: the scales first, then the code chunks in the
// order blocks 0..7 need them, so that with straight-line code the compiler's
// partial vmcnt waits let block 0 start while later chunks are in flight.
// The scheduling barriers keep the machine scheduler from reordering them.
template <int FMT>
__device__ __forceinline__ TileRegs<FMT> load_tile(const uint8_t *__restrict__ tile, int lane)
{
    TileRegs<FMT> t;
    const u32x4 *tp = reinterpret_cast<const u32x4 *>(tile) + lane;
#define RFX_LD(dst, ptr)                                                                                      \
    do {                                                                                                      \
        dst = __builtin_nontemporal_load(ptr);                                                                \
        __builtin_amdgcn_sched_barrier(0);                                                                    \
    } while (0)
    if (FMT == RFX_FP4) {
        RFX_LD(t.sc8, reinterpret_cast<const u32x2 *>(tile + 8 * 1024) + lane);
#pragma unroll
        for (int k = 0; k < 8; k++)
            RFX_LD(t.c[k], tp + 64 * k);
    } else if (FMT == RFX_Q8) {
        RFX_LD(t.sc16, tp + 64 * 16);
#pragma unroll
        for (int k = 0; k < 16; k++)
            RFX_LD(t.c[k], tp + 64 * k);
    } else if (FMT == RFX_FP3 || FMT == RFX_FP3E) {
        if (FMT == RFX_FP3E)
            RFX_LD(t.sc8, reinterpret_cast<const u32x2 *>(tile + 6 * 1024) + lane);
        else
            RFX_LD(t.sc16, tp + 64 * 6);
        RFX_LD(t.c[4], tp + 64 * 4); // high bits, blocks 0..3
        RFX_LD(t.c[0], tp);
        RFX_LD(t.c[1], tp + 64);
        RFX_LD(t.c[5], tp + 64 * 5); // high bits, blocks 4..7
        RFX_LD(t.c[2], tp + 64 * 2);
        RFX_LD(t.c[3], tp + 64 * 3);
    } else {
        RFX_LD(t.sc16, tp + 64 * 4);
        if (FMT == RFX_FP2M || FMT == RFX_FP2S)
            RFX_LD(t.mn16, tp + 64 * 5);
#pragma unroll
        for (int k = 0; k < 4; k++)
            RFX_LD(t.c[k], tp + 64 * k);
    }
#undef RFX_LD
    return t;
}

// fp16 value bi (0..7) of eight packed in a 16-byte chunk.
__device__ __forceinline__ float half_of(const u32x4 &v, int bi)
{
    const uint32_t w2 = (bi >> 1) == 0 ? v.x : (bi >> 1) == 1 ? v.y : (bi >> 1) == 2 ? v.z : v.w;
    return half_bits_to_float((bi & 1) ? (w2 >> 16) : (w2 & 0xffffu));
}

// A block's second small value: FP2M's minimum (added after the scale),
// FP2S's second-half scale; 0 for the one-scale formats.
template <int FMT>
__device__ __forceinline__ float block_second(const TileRegs<FMT> &t, int bi)
{
    return FMT == RFX_FP2M || FMT == RFX_FP2S ? half_of(t.mn16, bi) : 0.0f;
}

// Selector bytes and dequantization scale of block bi (0..7) of a tile.
// FP2M shares FP2's code layout; its selector byte is the code c itself.
// FP2S: the signed codebook values; sw is the first half's scale.
template <int FMT>
__device__ __forceinline__ void decode_block(const TileRegs<FMT> &t, int bi, Sel8 &sel, float &sw)
{
    if (FMT == RFX_Q8) { // the codes are the int8 values: no expansion
        const u32x4 a = t.c[2 * bi], b = t.c[2 * bi + 1];
        sel.v[0] = (int)a.x, sel.v[1] = (int)a.y, sel.v[2] = (int)a.z, sel.v[3] = (int)a.w;
        sel.v[4] = (int)b.x, sel.v[5] = (int)b.y, sel.v[6] = (int)b.z, sel.v[7] = (int)b.w;
        sw = half_of(t.sc16, bi);
    } else if (FMT == RFX_FP4) {
        sel = sel_fp4(t.c[bi]);
        const uint32_t e = ((bi < 4 ? t.sc8.x : t.sc8.y) >> (8 * (bi & 3))) & 0xffu;
        sw = ldexpf(1.0f, (int)e - 128); // 2 x E2M1 codebook: scale 2^(E-128)
    } else {
        const uint32_t w0 = (bi & 1) ? t.c[bi >> 1].z : t.c[bi >> 1].x;
        const uint32_t w1 = (bi & 1) ? t.c[bi >> 1].w : t.c[bi >> 1].y;
        if (FMT == RFX_FP3 || FMT == RFX_FP3E) {
            const u32x4 h4 = t.c[4 + (bi >> 2)];
            const uint32_t h = (bi & 3) == 0 ? h4.x : (bi & 3) == 1 ? h4.y : (bi & 3) == 2 ? h4.z : h4.w;
            sel = sel_fp3(w0, w1, h);
        } else if (FMT == RFX_FP2S) {
            sel = sel_fp2s(w0, w1);
        } else {
            sel = sel_fp2(w0, w1);
        }
        if (FMT == RFX_FP3E) { // a power-of-two scale 2^(E - 127)
            const uint32_t e = ((bi < 4 ? t.sc8.x : t.sc8.y) >> (8 * (bi & 3))) & 0xffu;
            sw = ldexpf(1.0f, (int)e - 127);
        } else {
            const uint32_t sw2 = (bi >> 1) == 0 ? t.sc16.x : (bi >> 1) == 1 ? t.sc16.y : (bi >> 1) == 2 ? t.sc16.z : t.sc16.w;
            sw = half_bits_to_float((bi & 1) ? (sw2 >> 16) : (sw2 & 0xffffu));
        }
    }
}

// ------------------------------------------------------------------
// Activation columns: int8 codes, fp32 block scales, int32 block sums.
// Column j starts at element xoff[j] (a multiple of 32) of xq and at block
// moff[j] of xs / xsum. Offsets are uniform (SGPRs).
// ------------------------------------------------------------------
template <int Q>
struct XCols {
    const int8_t *xq;
    const float *xs;
    const int32_t *xsum;
    uint32_t xoff[Q];
    uint32_t moff[Q];
};

template <int Q>
struct XBlock {
    int x[Q][8];
    float sx[Q];
    int sum[Q];
};

template <bool NEED_SUM, int Q>
__device__ __forceinline__ XBlock<Q> load_xblock(const XCols<Q> &c, int b)
{
    XBlock<Q> xb;
    const sptr_i32 xq = as_scalar_i32(c.xq), xsum = as_scalar_i32(c.xsum);
    const sptr_f32 xs = as_scalar_f32(c.xs);
#pragma unroll
    for (int j = 0; j < Q; j++) {
        const uint32_t xo = (c.xoff[j] + 32u * (uint32_t)b) >> 2;
        const uint32_t mo = c.moff[j] + (uint32_t)b;
#pragma unroll
        for (int i = 0; i < 8; i++)
            xb.x[j][i] = xq[xo + i];
        xb.sx[j] = xs[mo];
        xb.sum[j] = NEED_SUM ? xsum[mo] : 0;
    }
    return xb;
}

// Exact per-block integer dot D for column j (codebook offset folded in;
// FP2M: D = sum(c x), the minimum enters through the block sum).
template <int FMT, int Q>
__device__ __forceinline__ int block_dot(const Sel8 &sel, const XBlock<Q> &xb, int j)
{
    int d = 0;
#pragma unroll
    for (int i = 0; i < 8; i++)
        d = __builtin_amdgcn_sdot4(sel.v[i], xb.x[j][i], d, false);
    if (FMT == RFX_FP2 || FMT == RFX_FP3 || FMT == RFX_FP3E) {
        const int off = FMT == RFX_FP2 ? 3 : 7; // v = 2c - off
        d = 2 * d - off * xb.sum[j];
    }
    return d;
}

// FP2M: the block is s * c + m, so its dot is sx * (s D + m X), X the
// activation block's code sum (s2 = m). FP2S: sx * (s0 D0 + s1 D1) over the
// two halves (sw = s0, s2 = s1).
template <int FMT, int Q, int NQ>
__device__ __forceinline__ void accumulate_block(const Sel8 &sel, float sw, const XBlock<Q> &xb,
                                                 float (&acc)[Q], float s2 = 0.0f)
{
#pragma unroll
    for (int j = 0; j < NQ; j++) {
        if (FMT == RFX_FP2S) {
            int d0 = 0, d1 = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                d0 = __builtin_amdgcn_sdot4(sel.v[i], xb.x[j][i], d0, false);
                d1 = __builtin_amdgcn_sdot4(sel.v[4 + i], xb.x[j][4 + i], d1, false);
            }
            acc[j] += xb.sx[j] * (sw * (float)d0 + s2 * (float)d1);
        } else if (FMT == RFX_FP2M)
            acc[j] += xb.sx[j] * (sw * (float)block_dot<FMT, Q>(sel, xb, j) + s2 * (float)xb.sum[j]);
        else
            acc[j] += (sw * xb.sx[j]) * (float)block_dot<FMT, Q>(sel, xb, j);
    }
}

// All blocks of one tile (blocks b0 .. b0 + 7 of the row) against one set of
// activation columns. FULL: every tile lies inside K (K % 256 == 0), chosen
// per launch. Otherwise the blocks past K are computed too, with the
// activation index clamped into range and the weight scale forced to zero.
// Either way the code is straight-line: every chunk load is used on every
// path, so the compiler keeps them in flight instead of sinking each into a
// branch, and waits for each block's chunks just before that block.
template <int FMT, int Q, int NQ, bool FULL>
__device__ __forceinline__ void tile_blocks(const TileRegs<FMT> &t, int b0, int nb, const XCols<Q> &xc,
                                            float (&acc)[Q])
{
    XBlock<Q> xn = load_xblock<TileFmt<FMT>::needs_sum, Q>(xc, FULL ? b0 : min(b0, nb - 1));
#pragma unroll
    for (int bi = 0; bi < 8; bi++) {
        // block bi's scalar loads are done here; the next block's are
        // issued now, so they are in flight during this block's work
        // (scalar loads return out of order: a wait covers all of them)
        __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
        const XBlock<Q> xb = xn;
        __builtin_amdgcn_sched_barrier(0);
        if (bi + 1 < 8)
            xn = load_xblock<TileFmt<FMT>::needs_sum, Q>(xc, FULL ? b0 + bi + 1 : min(b0 + bi + 1, nb - 1));
        __builtin_amdgcn_sched_barrier(0);
        Sel8 sel;
        float sw;
        decode_block<FMT>(t, bi, sel, sw);
        float s2 = block_second<FMT>(t, bi);
        if (!FULL) {
            sw = b0 + bi < nb ? sw : 0.0f;
            s2 = b0 + bi < nb ? s2 : 0.0f;
        }
        accumulate_block<FMT, Q, NQ>(sel, sw, xb, acc, s2);
        // keep each block's work after its own chunk wait (the scheduler
        // would otherwise hoist the decodes and wait for the whole tile)
        __builtin_amdgcn_sched_barrier(0);
    }
}

// A gate tile and the matching up tile against the same activation blocks.
template <int FG, int FU, int Q, bool FULL>
__device__ __forceinline__ void tile_blocks2(const TileRegs<FG> &tg, const TileRegs<FU> &tu, int b0, int nb,
                                             const XCols<Q> &xc, float (&ag)[Q], float (&au)[Q])
{
    XBlock<Q> xn = load_xblock<true, Q>(xc, FULL ? b0 : min(b0, nb - 1));
#pragma unroll
    for (int bi = 0; bi < 8; bi++) {
        __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0); // as in tile_blocks
        const XBlock<Q> xb = xn;
        __builtin_amdgcn_sched_barrier(0);
        if (bi + 1 < 8)
            xn = load_xblock<true, Q>(xc, FULL ? b0 + bi + 1 : min(b0 + bi + 1, nb - 1));
        __builtin_amdgcn_sched_barrier(0);
        Sel8 sel;
        float sw;
        decode_block<FG>(tg, bi, sel, sw);
        if (!FULL)
            sw = b0 + bi < nb ? sw : 0.0f;
        accumulate_block<FG, Q, Q>(sel, sw, xb, ag);
        decode_block<FU>(tu, bi, sel, sw);
        if (!FULL)
            sw = b0 + bi < nb ? sw : 0.0f;
        accumulate_block<FU, Q, Q>(sel, sw, xb, au);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// s_waitcnt immediate (gfx9 encoding): vmcnt = 0, expcnt and lgkmcnt at
// their maxima: wait for every outstanding vector memory operation.
constexpr int kWaitVmcnt0 = 0x0F70;

} // namespace dev
} // namespace rfx
