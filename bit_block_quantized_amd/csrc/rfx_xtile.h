// Activation tiles held in VGPRs and the matrix-core block dots (gfx950).
//
// Pages cited (title, site):
//   [HM] "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
//        (hellomarvisaitoday.com), paragraphs numbered from the top.
//
// [HM] para 3: one decoded weight block feeds integer dot products for every
// activation column. With q >= 2 columns those dots run on the matrix core:
// the activation slice of a whole tile (q columns x 256 bytes, plus the
// eight block scales and sums per column) is read with ordinary vector loads
// issued together with the weight tile (vector loads complete in order, so
// block b waits only for its own data; scalar loads complete out of order
// and every use waits for all of them), and a v_mfma_i32_4x4x4_16b_i8 per
// K step takes the decoded weights of each lane's row as one operand and
// the activations, broadcast from one 4-lane group, as the other.
// FP4 (E2M1 codes, [HM] para 2) takes the f16 form of the same matrix op:
// the hardware FP4 -> f16 conversion expands two codes per instruction and
// the lane's activations are turned into f16 once per tile, which needs a
// third of the vector instructions of the byte-permute expansion.
#pragma once

#include "rfx_decode.h"

#include <utility>

namespace rfx {
namespace dev {

// Selector bytes equal to 2c (twice the code) for FP2 / FP3, so that with
// v = 2c - off the block dot is sum(2c * x) + (-off * sum(x)): the second
// term starts the accumulator and needs no instruction after the dots.
__device__ __forceinline__ Sel8 sel2_fp2(uint32_t w0, uint32_t w1)
{
    Sel8 s;
    s.v[0] = (int)((w0 << 1) & 0x06060606u);
    s.v[1] = (int)((w0 >> 1) & 0x06060606u);
    s.v[2] = (int)((w0 >> 3) & 0x06060606u);
    s.v[3] = (int)((w0 >> 5) & 0x06060606u);
    s.v[4] = (int)((w1 << 1) & 0x06060606u);
    s.v[5] = (int)((w1 >> 1) & 0x06060606u);
    s.v[6] = (int)((w1 >> 3) & 0x06060606u);
    s.v[7] = (int)((w1 >> 5) & 0x06060606u);
    return s;
}

// FP3: the high code bit of weight 4i + j sits at bit 8j + i of h; in 2c it
// has weight 8.
__device__ __forceinline__ Sel8 sel2_fp3(uint32_t w0, uint32_t w1, uint32_t h)
{
    Sel8 s = sel2_fp2(w0, w1);
    s.v[0] |= (int)((h << 3) & 0x08080808u);
    s.v[1] |= (int)((h << 2) & 0x08080808u);
    s.v[2] |= (int)((h << 1) & 0x08080808u);
    s.v[3] |= (int)(h & 0x08080808u);
    s.v[4] |= (int)((h >> 1) & 0x08080808u);
    s.v[5] |= (int)((h >> 2) & 0x08080808u);
    s.v[6] |= (int)((h >> 3) & 0x08080808u);
    s.v[7] |= (int)((h >> 4) & 0x08080808u);
    return s;
}

// Selector bytes (2c for FP2/FP3, c for FP2M, signed values for FP4 and
// FP2S) and the weight scale of block BI of a tile (FP2S: its first half's).
template <int FMT, int BI>
__device__ __forceinline__ void decode_block2(const TileRegs<FMT> &t, Sel8 &sel, float &sw)
{
    if (FMT == RFX_Q8) {
        decode_block<FMT>(t, BI, sel, sw);
    } else if (FMT == RFX_FP4) {
        sel = sel_fp4(t.c[BI]);
        const uint32_t e = ((BI < 4 ? t.sc8.x : t.sc8.y) >> (8 * (BI & 3))) & 0xffu;
        sw = ldexpf(1.0f, (int)e - 128);
    } else {
        const uint32_t w0 = (BI & 1) ? t.c[BI >> 1].z : t.c[BI >> 1].x;
        const uint32_t w1 = (BI & 1) ? t.c[BI >> 1].w : t.c[BI >> 1].y;
        if (FMT == RFX_FP3 || FMT == RFX_FP3E) {
            const u32x4 h4 = t.c[4 + (BI >> 2)];
            const uint32_t h = (BI & 3) == 0 ? h4.x : (BI & 3) == 1 ? h4.y : (BI & 3) == 2 ? h4.z : h4.w;
            sel = sel2_fp3(w0, w1, h);
        } else if (FMT == RFX_FP2M) {
            sel = sel_fp2(w0, w1);
        } else if (FMT == RFX_FP2S) {
            sel = sel_fp2s(w0, w1);
        } else {
            sel = sel2_fp2(w0, w1);
        }
        if (FMT == RFX_FP3E) {
            const uint32_t e = ((BI < 4 ? t.sc8.x : t.sc8.y) >> (8 * (BI & 3))) & 0xffu;
            sw = ldexpf(1.0f, (int)e - 127);
        } else {
            const uint32_t sw2 = (BI >> 1) == 0 ? t.sc16.x : (BI >> 1) == 1 ? t.sc16.y : (BI >> 1) == 2 ? t.sc16.z : t.sc16.w;
            sw = half_bits_to_float((BI & 1) ? (sw2 >> 16) : (sw2 & 0xffffu));
        }
    }
}

// Broadcast lane N of each 16-lane row (a DPP move the compiler folds into
// the consuming VALU instruction where it can).
template <int N>
__device__ __forceinline__ int bcast_row(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, 0x150 + N, 0xF, 0xF, true);
}

// ------------------------------------------------------------------
// Matrix-core variant for q >= 2: the q column dots of a block run as
// v_mfma_i32_4x4x4_16b_i8 with the decoded weights as the B operand (lane
// l = row l, four int8 weights per K step) and the activations as the A
// operand. For that MFMA, output lane l, register v is the dot of B's lane
// l with A's lane 4 * abid + v when cbsz = 4 broadcasts one 4-lane group to
// all sixteen (measured on gfx950). So lane l holds the 16-byte chunk l / 4
// of column l % 4's 256-byte tile slice, and K step s of block b takes its
// activations from group 2b + s / 4, component s % 4: one vector load per
// tile feeds every column, and each lane ends with its own row's q dots.
// ------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Per-lane part of one tile's activations: code holds bytes
// [16 (l / 4), 16 (l / 4) + 16) of column min(l % 4, Q - 1)'s 256-byte
// slice; lane n of each 16-lane row (n = l & 15) holds column j's fp32
// scale of block n & 7 in sx[j] and, for FP2/FP3, -off * (block sum) in
// nsum[j] (off = 3 or 7, the codebook offset folded out of the dot; FP2M:
// the block sum itself, which multiplies the block minimum); the block's
// values reach every lane by DPP row broadcast (sx only for FP2M and
// FP2S). sxa: lane m holds the scale of column min(m % 4, Q - 1) for block
// (m / 4) % 8, the A operand of the scale products (scale_products).
template <int Q>
struct XTileM {
    u32x4 code;
    float sx[Q];
    int nsum[Q];
    float sxa;
};

// The formats whose epilogue is (s_w * s_x) * D, scaled through
// scale_products; FP2M and FP2S combine two terms per block and keep the
// broadcast column scales.
template <int FMT>
constexpr bool plain_scale()
{
    return FMT != RFX_FP2M && FMT != RFX_FP2S;
}

template <int FMT, int Q, bool FULL>
__device__ __forceinline__ XTileM<Q> load_xtile_m(const XCols<Q> &xc, int s, int nb, int lane)
{
    XTileM<Q> xt;
    const int n = lane & 15, chunk = lane >> 2;
    const int bc = FULL ? s * 8 + (chunk >> 1) : min(s * 8 + (chunk >> 1), nb - 1);
    const int bs = FULL ? s * 8 + (n & 7) : min(s * 8 + (n & 7), nb - 1);
    // column offset of this lane as a sum of steps (a select between the
    // offsets themselves would be turned into a lane-indexed private array)
    uint32_t xo = xc.xoff[0];
#pragma unroll
    for (int j = 1; j < Q; j++)
        xo += (lane & 3) >= j ? xc.xoff[j] - xc.xoff[j - 1] : 0u;
    xt.code = *reinterpret_cast<const u32x4 *>(xc.xq + xo + (uint32_t)bc * 32u + (uint32_t)(chunk & 1) * 16u);
    if constexpr (plain_scale<FMT>()) {
        const int ba = FULL ? s * 8 + ((lane >> 2) & 7) : min(s * 8 + ((lane >> 2) & 7), nb - 1);
        uint32_t mo = xc.moff[0];
#pragma unroll
        for (int j = 1; j < Q; j++)
            mo += (lane & 3) >= j ? xc.moff[j] - xc.moff[j - 1] : 0u;
        xt.sxa = xc.xs[mo + (uint32_t)ba];
    } else {
#pragma unroll
        for (int j = 0; j < Q; j++)
            xt.sx[j] = xc.xs[xc.moff[j] + (uint32_t)bs];
    }
    if (TileFmt<FMT>::needs_sum) {
        constexpr int off = FMT == RFX_FP2 ? 3 : FMT == RFX_FP3 || FMT == RFX_FP3E ? 7 : -1; // FP2M: +sum
#pragma unroll
        for (int j = 0; j < Q; j++)
            xt.nsum[j] = -off * xc.xsum[xc.moff[j] + (uint32_t)bs];
    }
    return xt;
}

// One K step of block BI: four weights per lane against group 2 BI + S / 4.
template <int BI, int S>
__device__ __forceinline__ i32x4 mfma_step(i32x4 d, const u32x4 &x, int w)
{
    const uint32_t xa = (S & 3) == 0 ? x.x : (S & 3) == 1 ? x.y : (S & 3) == 2 ? x.z : x.w;
    return __builtin_amdgcn_mfma_i32_4x4x4i8((int)xa, w, d, 4, 2 * BI + (S >> 2), 0);
}

// Exact block dots of block BI for the four column slots (slot j is
// column j for j < Q), as two accumulation chains of four steps each, so
// consecutive matrix ops do not wait on one another: d0 takes weights
// 0..15, d1 weights 16..31 (FP2S's two halves). FP2 / FP3 start d0 at
// -off * sum(x) (the codebook offset), so only d0 + d1 means anything.
template <int FMT, int Q, int BI>
__device__ __forceinline__ void block_half_dots_mfma(const Sel8 &sel, const XTileM<Q> &xt, i32x4 &d0, i32x4 &d1)
{
    d0 = i32x4{0, 0, 0, 0};
    d1 = i32x4{0, 0, 0, 0};
    if (FMT == RFX_FP2 || FMT == RFX_FP3 || FMT == RFX_FP3E) {
#pragma unroll
        for (int j = 0; j < Q; j++)
            d0[j] = bcast_row<BI>(xt.nsum[j]);
    }
    d0 = mfma_step<BI, 0>(d0, xt.code, sel.v[0]);
    d1 = mfma_step<BI, 4>(d1, xt.code, sel.v[4]);
    d0 = mfma_step<BI, 1>(d0, xt.code, sel.v[1]);
    d1 = mfma_step<BI, 5>(d1, xt.code, sel.v[5]);
    d0 = mfma_step<BI, 2>(d0, xt.code, sel.v[2]);
    d1 = mfma_step<BI, 6>(d1, xt.code, sel.v[6]);
    d0 = mfma_step<BI, 3>(d0, xt.code, sel.v[3]);
    d1 = mfma_step<BI, 7>(d1, xt.code, sel.v[7]);
}

// Exact block dots of block BI as one accumulation chain (a dependent
// matrix op of the same kind reads the previous result after two wait
// states), started at -off * sum(x) for FP2 / FP3.
template <int FMT, int Q, int BI>
__device__ __forceinline__ i32x4 block_dots_mfma(const Sel8 &sel, const XTileM<Q> &xt)
{
    i32x4 d = {0, 0, 0, 0};
    if (FMT == RFX_FP2 || FMT == RFX_FP3 || FMT == RFX_FP3E) {
#pragma unroll
        for (int j = 0; j < Q; j++)
            d[j] = bcast_row<BI>(xt.nsum[j]);
    }
    d = mfma_step<BI, 0>(d, xt.code, sel.v[0]);
    d = mfma_step<BI, 1>(d, xt.code, sel.v[1]);
    d = mfma_step<BI, 2>(d, xt.code, sel.v[2]);
    d = mfma_step<BI, 3>(d, xt.code, sel.v[3]);
    d = mfma_step<BI, 4>(d, xt.code, sel.v[4]);
    d = mfma_step<BI, 5>(d, xt.code, sel.v[5]);
    d = mfma_step<BI, 6>(d, xt.code, sel.v[6]);
    d = mfma_step<BI, 7>(d, xt.code, sel.v[7]);
    return d;
}

// FP4 on v_mfma_f32_4x4x4_16b_f16. v_cvt_scalef32_pk_f16_fp4 with scale 2
// turns byte b of a code word into two f16 values, 2 x E2M1 of its low and
// of its high nibble (measured on gfx950, all 256 byte values): in word m
// of a block those are weights 8m + b and 8m + 4 + b. K step (m, p) takes
// bytes 2p and 2p + 1, i.e. weights (8m + 2p, 8m + 2p + 4, 8m + 2p + 1,
// 8m + 2p + 5), and the activations must come in that order. Products and
// sums are integers below 2^24, so the f32 accumulation is exact and the
// result equals the int8 path's.
struct XHalf {
    u32x4 h[2]; // h[m % 2]: the lane's A operands of word m, step p in dwords 2p, 2p + 1
};

// The lane's 16 activations (bytes of code) in f16, in the step order
// above: gather the two bytes of each pair, bias them to unsigned
// (x + 128), put each under the f16 exponent byte 0x64 (the value
// 1024 + x + 128) and subtract 1152 (exact: all values are integers below
// 2048).
__device__ __forceinline__ XHalf act_f16_fp4(const u32x4 &code)
{
    const uint32_t w[4] = {code.x, code.y, code.z, code.w};
    const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    uint32_t o[8];
#pragma unroll
    for (int mp = 0; mp < 2; mp++) {
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const uint32_t sel = (uint32_t)(2 * p) | (uint32_t)(2 * p + 1) << 8 | (uint32_t)(2 * p + 4) << 16 |
                                 (uint32_t)(2 * p + 5) << 24;
            const uint32_t t = __builtin_amdgcn_perm(w[2 * mp + 1], w[2 * mp], sel) ^ 0x80808080u;
            const f16x2 lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, t, 0x04020400u)) - bias;
            const f16x2 hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, t, 0x04030401u)) - bias;
            o[4 * mp + 2 * p] = __builtin_bit_cast(uint32_t, lo);
            o[4 * mp + 2 * p + 1] = __builtin_bit_cast(uint32_t, hi);
        }
    }
    XHalf x;
    x.h[0] = u32x4{o[0], o[1], o[2], o[3]};
    x.h[1] = u32x4{o[4], o[5], o[6], o[7]};
    return x;
}

// The two K steps of code word M of block BI.
template <int BI, int M>
__device__ __forceinline__ f32x4 fp4_word_steps(f32x4 d, uint32_t w, const XHalf &xh)
{
    const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 0);
    const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 1);
    const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 2);
    const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 3);
    const u32x4 &xa = xh.h[M & 1];
    const f16x4 a0 = __builtin_bit_cast(f16x4, u32x2{xa.x, xa.y});
    const f16x4 a1 = __builtin_bit_cast(f16x4, u32x2{xa.z, xa.w});
    const f16x4 b0 = {h0[0], h0[1], h1[0], h1[1]};
    const f16x4 b1 = {h2[0], h2[1], h3[0], h3[1]};
    d = __builtin_amdgcn_mfma_f32_4x4x4f16(a0, b0, d, 4, 2 * BI + (M >> 1), 0);
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a1, b1, d, 4, 2 * BI + (M >> 1), 0);
}

// Exact dots of FP4 block BI (its four code words in c) for the four
// column slots, as f32 integers.
template <int BI>
__device__ __forceinline__ f32x4 fp4_block_dots(const u32x4 &c, const XHalf &xh)
{
    f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
    d = fp4_word_steps<BI, 0>(d, c.x, xh);
    d = fp4_word_steps<BI, 1>(d, c.y, xh);
    d = fp4_word_steps<BI, 2>(d, c.z, xh);
    return fp4_word_steps<BI, 3>(d, c.w, xh);
}

// Weight scale of FP4 block BI for the 2 x E2M1 values: 2^(e - 128).
template <int BI>
__device__ __forceinline__ float fp4_scale(const TileRegs<RFX_FP4> &t)
{
    const uint32_t e = ((BI < 4 ? t.sc8.x : t.sc8.y) >> (8 * (BI & 3))) & 0xffu;
    return ldexpf(1.0f, (int)e - 128);
}

// The f16 activations of a tile for FP4 (nothing for the other formats).
template <int FMT>
__device__ __forceinline__ XHalf tile_xhalf(const u32x4 &code)
{
    if constexpr (FMT == RFX_FP4)
        return act_f16_fp4(code);
    else
        return XHalf{};
}

// The scale products of block BI for the lane's row: element j is
// s_w(row) * s_x(column j, block BI). v_mfma_f32_4x4x1_16b_f32's output
// lane l, register v is A(lane 4 (l / 4) + v) * B(lane l) (measured on
// gfx950), and cbsz 4 with abid BI broadcasts lanes 4 BI .. 4 BI + 3 of A
// to every block: those lanes hold block BI's column scales (sxa), B is the
// lane's own weight scale. One product per output rounded once, so each is
// the value of the vector multiply s_w * s_x.
template <int BI>
__device__ __forceinline__ f32x4 scale_products(float sxa, float sw)
{
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_f32_4x4x1f32(sxa, sw, zero, 4, BI, 0);
}

template <int FMT, int Q, int BI, bool FULL>
__device__ __forceinline__ void tile_block_mfma(const TileRegs<FMT> &t, const XTileM<Q> &xt, const XHalf &xh,
                                                int b0, int nb, float (&acc)[Q])
{
    if constexpr (FMT == RFX_FP4) {
        float sw = fp4_scale<BI>(t);
        if (!FULL)
            sw = b0 + BI < nb ? sw : 0.0f;
        const f32x4 d = fp4_block_dots<BI>(t.c[BI], xh);
        const f32x4 sc = scale_products<BI>(xt.sxa, sw);
#pragma unroll
        for (int j = 0; j < Q; j++)
            acc[j] = fmaf(sc[j], d[j], acc[j]);
        __builtin_amdgcn_sched_barrier(0);
        return;
    }
    Sel8 sel;
    float sw;
    decode_block2<FMT, BI>(t, sel, sw);
    float s2 = block_second<FMT>(t, BI);
    if (!FULL) {
        sw = b0 + BI < nb ? sw : 0.0f;
        s2 = b0 + BI < nb ? s2 : 0.0f;
    }
    if (FMT == RFX_FP2S) { // sx * (s0 D0 + s1 D1)
        i32x4 d0, d1;
        block_half_dots_mfma<FMT, Q, BI>(sel, xt, d0, d1);
#pragma unroll
        for (int j = 0; j < Q; j++) {
            const float sxb = __builtin_bit_cast(float, bcast_row<BI>(__builtin_bit_cast(int, xt.sx[j])));
            acc[j] += sxb * (sw * (float)d0[j] + s2 * (float)d1[j]);
        }
        __builtin_amdgcn_sched_barrier(0);
        return;
    }
    const i32x4 d = block_dots_mfma<FMT, Q, BI>(sel, xt);
    if constexpr (FMT == RFX_FP2M) { // sx * (s D + m X)
#pragma unroll
        for (int j = 0; j < Q; j++) {
            const float sxb = __builtin_bit_cast(float, bcast_row<BI>(__builtin_bit_cast(int, xt.sx[j])));
            acc[j] += sxb * (sw * (float)d[j] + s2 * (float)bcast_row<BI>(xt.nsum[j]));
        }
    } else {
        const f32x4 sc = scale_products<BI>(xt.sxa, sw);
#pragma unroll
        for (int j = 0; j < Q; j++)
            acc[j] = fmaf(sc[j], (float)d[j], acc[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int FMT, int Q, bool FULL, int... BI>
__device__ __forceinline__ void tile_blocks_mfma_seq(const TileRegs<FMT> &t, const XTileM<Q> &xt, const XHalf &xh,
                                                     int b0, int nb, float (&acc)[Q], std::integer_sequence<int, BI...>)
{
    (tile_block_mfma<FMT, Q, BI, FULL>(t, xt, xh, b0, nb, acc), ...);
}

// All 8 blocks of one tile on the matrix core. Every lane must be active
// (the scale broadcasts read other lanes).
template <int FMT, int Q, bool FULL>
__device__ __forceinline__ void tile_blocks_mfma(const TileRegs<FMT> &t, const XTileM<Q> &xt, int b0, int nb,
                                                 float (&acc)[Q])
{
    const XHalf xh = tile_xhalf<FMT>(xt.code);
    tile_blocks_mfma_seq<FMT, Q, FULL>(t, xt, xh, b0, nb, acc, std::make_integer_sequence<int, 8>{});
}

// A gate tile and the matching up tile (same format) against one
// activation slice: block BI of both.
template <int F, int Q, int BI, bool FULL>
__device__ __forceinline__ void tile_block2_mfma(const TileRegs<F> &tg, const TileRegs<F> &tu, const XTileM<Q> &xt,
                                                 const XHalf &xh, int b0, int nb, float (&ag)[Q], float (&au)[Q])
{
    static_assert(plain_scale<F>(), "gate/up formats scale as (s_w * s_x) * D");
    if constexpr (F == RFX_FP4) {
        float sg = fp4_scale<BI>(tg), su = fp4_scale<BI>(tu);
        if (!FULL) {
            sg = b0 + BI < nb ? sg : 0.0f;
            su = b0 + BI < nb ? su : 0.0f;
        }
        const f32x4 dg = fp4_block_dots<BI>(tg.c[BI], xh);
        const f32x4 cg = scale_products<BI>(xt.sxa, sg);
#pragma unroll
        for (int j = 0; j < Q; j++)
            ag[j] = fmaf(cg[j], dg[j], ag[j]);
        const f32x4 du = fp4_block_dots<BI>(tu.c[BI], xh);
        const f32x4 cu = scale_products<BI>(xt.sxa, su);
#pragma unroll
        for (int j = 0; j < Q; j++)
            au[j] = fmaf(cu[j], du[j], au[j]);
        __builtin_amdgcn_sched_barrier(0);
        return;
    }
    Sel8 sel;
    float sw;
    decode_block2<F, BI>(tg, sel, sw);
    if (!FULL)
        sw = b0 + BI < nb ? sw : 0.0f;
    i32x4 d = block_dots_mfma<F, Q, BI>(sel, xt);
    const f32x4 cg = scale_products<BI>(xt.sxa, sw);
#pragma unroll
    for (int j = 0; j < Q; j++)
        ag[j] = fmaf(cg[j], (float)d[j], ag[j]);
    decode_block2<F, BI>(tu, sel, sw);
    if (!FULL)
        sw = b0 + BI < nb ? sw : 0.0f;
    d = block_dots_mfma<F, Q, BI>(sel, xt);
    const f32x4 cu = scale_products<BI>(xt.sxa, sw);
#pragma unroll
    for (int j = 0; j < Q; j++)
        au[j] = fmaf(cu[j], (float)d[j], au[j]);
    __builtin_amdgcn_sched_barrier(0);
}

template <int F, int Q, bool FULL, int... BI>
__device__ __forceinline__ void tile_blocks2_mfma_seq(const TileRegs<F> &tg, const TileRegs<F> &tu,
                                                      const XTileM<Q> &xt, const XHalf &xh, int b0, int nb,
                                                      float (&ag)[Q], float (&au)[Q], std::integer_sequence<int, BI...>)
{
    (tile_block2_mfma<F, Q, BI, FULL>(tg, tu, xt, xh, b0, nb, ag, au), ...);
}

template <int F, int Q, bool FULL>
__device__ __forceinline__ void tile_blocks2_mfma(const TileRegs<F> &tg, const TileRegs<F> &tu, const XTileM<Q> &xt,
                                                  int b0, int nb, float (&ag)[Q], float (&au)[Q])
{
    const XHalf xh = tile_xhalf<F>(xt.code);
    tile_blocks2_mfma_seq<F, Q, FULL>(tg, tu, xt, xh, b0, nb, ag, au, std::make_integer_sequence<int, 8>{});
}

// The per-block dots themselves (debug path), block BI.
template <int FMT, int Q, int BI>
__device__ __forceinline__ i32x4 tile_block_dots_mfma(const TileRegs<FMT> &t, const XTileM<Q> &xt)
{
    if constexpr (FMT == RFX_FP4) {
        const f32x4 d = fp4_block_dots<BI>(t.c[BI], act_f16_fp4(xt.code));
        return i32x4{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
    }
    Sel8 sel;
    float sw;
    decode_block2<FMT, BI>(t, sel, sw);
    return block_dots_mfma<FMT, Q, BI>(sel, xt);
}

} // namespace dev
} // namespace rfx
