// FP4 blocks on the block-scaled matrix core of gfx950.
//
// Pages cited (title, site):
//   [HM] "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
//        (hellomarvisaitoday.com), paragraphs numbered from the top.
//
// FP4 blocks are E2M1 codes with one e8m0 exponent per 32 weights ([HM]
// para 2 gives 4.25 bits per weight), which is the operand format of
// v_mfma_scale_f32_16x16x128_f8f6f4: the matrix core reads the packed codes
// as they are stored and applies the block exponent itself, so the weights
// are never expanded on the vector unit. The int8 activations enter as the
// other operand, each split exactly into two FP8 (E4M3) values: x = 16 h + l
// with l = x & 15 in 0..15 and h = x >> 4 in -8..7, both exact in E4M3.
// The activation scales are fp32 per block, which the matrix core cannot
// apply (its scales are powers of two), so each block gets output columns
// of its own: B column n carries only block n % 4 of its 128-wide K slice,
// and the fp32 scaling happens after the product, once per block and row.
//
// Operand layouts of this MFMA (measured on gfx950, A = FP4, B = FP8):
//   A: lane l holds row l % 16, K = 32 (l / 16) + t for nibble t (nibble t at
//      bits 4 (t % 8) of dword t / 8); its scale byte is that (row, 32-block).
//   B: lane l holds column l % 16; byte q covers K = 16 (l / 16) + q for
//      q < 16 and K = 64 + 16 (l / 16) + (q - 16) for q >= 16.
//   D: lane l, register v holds row 4 (l / 16) + v, column l % 16.
// In the tiled FP4 layout chunk c holds block c of every row (lane = row).
// A tile (64 rows x 8 blocks) takes eight products, (16-row group g, h):
// MFMA K-block kb of product (g, h) is tile block 2kb + h, so lane l loads
// chunk 2 (l / 16) + h of row 16g + l % 16 (four 256-byte runs per load)
// and its two scale bytes (blocks 2 (l / 16) and 2 (l / 16) + 1 of that
// row) are adjacent: one 16-bit load per g, the MFMA picks byte h.
// Inside a block the code nibbles are not in K order (weight 8m + 4i + j
// sits in word m, byte j, nibble i): nibble t holds weight
// 8 (t / 8) + 4 (t % 2) + (t % 8) / 2, so B takes the activations in that
// order (one byte permute per output word).
#pragma once

#include "rfx_decode.h"

namespace rfx {
namespace dev {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// E4M3 codes of 0..15 (the low nibble of an int8, unsigned) ...
constexpr uint32_t kE4m3Lo[4] = {0x44403800u, 0x4E4C4A48u, 0x53525150u, 0x57565554u};
// ... and of the high nibble read as a signed 4-bit value: 0..7, then -8..-1.
constexpr uint32_t kE4m3Hi[4] = {0x44403800u, 0x4E4C4A48u, 0xCACCCED0u, 0xB8C0C4C8u};

// Column pairs: pair p of the B operand carries activation columns 2p and
// 2p + 1 (q = 3: column 3 absent). For pair 0, lanes n % 8 < 4 hold the low
// parts (block n % 4) and n % 8 >= 4 the high parts; pair 1 swaps the two,
// so after combining high into low both pairs' sums sit in different lanes
// and share one accumulator: the quad k = n / 4 of each 16-lane row ends
// with column 0, 2, 1, 3 for k = 0, 1, 2, 3.
template <int Q>
struct MxLane {
    static constexpr int NP = (Q + 1) / 2;
    uint32_t tab2[NP], tab3[NP]; // entries 8..15 of this lane's E4M3 table
    uint32_t sh[NP];             // 0: low nibble, 4: high nibble
    uint32_t sb[NP];             // B scale byte of the lane's column: 127 (low part), 131 (high: x 16)
    uint32_t xo[NP];             // byte offset of the lane's 16 activations (column, block 0 of the half)
    uint32_t mo[NP];             // index of the lane's column's scale of block 0
    bool lo[NP];                 // this lane collects the block sum of pair p
    bool put_lo[NP], put_hi[NP]; // the lane's data goes to bytes 0..15 / 16..31 (else zero)
    int bn;                      // block of the half this lane's column carries
};

template <int Q>
__device__ __forceinline__ MxLane<Q> mx_lane(int lane, const XCols<Q> &xc)
{
    MxLane<Q> m;
    const int gb = lane >> 4, n = lane & 15, bn = n & 3;
    m.bn = bn;
    const bool has = (gb >> 1) == (bn & 1); // lane group holds K slots of block bn
#pragma unroll
    for (int p = 0; p < MxLane<Q>::NP; p++) {
        const bool first_half = (n & 7) < 4;
        const bool low_part = p == 0 ? first_half : !first_half;
        const int c = 2 * p + (n >> 3);
        const uint32_t cc = (uint32_t)(c < Q ? c : Q - 1);
        uint32_t xo = xc.xoff[0], mo = xc.moff[0];
#pragma unroll
        for (int j = 1; j < Q; j++) { // per-lane column as a sum of steps
            xo += cc >= (uint32_t)j ? xc.xoff[j] - xc.xoff[j - 1] : 0u;
            mo += cc >= (uint32_t)j ? xc.moff[j] - xc.moff[j - 1] : 0u;
        }
        m.xo[p] = xo + 16u * (uint32_t)(gb & 1);
        m.mo[p] = mo;
        m.lo[p] = low_part && c < Q;
        m.sh[p] = low_part ? 0u : 4u;
        m.sb[p] = low_part ? 127u : 131u;
        m.tab2[p] = low_part ? kE4m3Lo[2] : kE4m3Hi[2];
        m.tab3[p] = low_part ? kE4m3Lo[3] : kE4m3Hi[3];
        m.put_lo[p] = has && c < Q && bn < 2;
        m.put_hi[p] = has && c < Q && bn >= 2;
    }
    return m;
}

// One tile (64 rows x 8 blocks) of FP4 codes ...
struct MxW {
    u32x4 a[8];     // A of (g, h), index 2g + h
    uint32_t sa[4]; // e8m0 bytes of row 16g + l % 16, blocks 2 (l / 16) + {0, 1}
};

// ... and the activation operands of its K range (shared by every weight
// matrix over that range, e.g. an expert's gate and up).
template <int Q>
struct MxX {
    static constexpr int NP = (Q + 1) / 2;
    u32x4 xr[2][NP]; // raw int8 activations for the B operand of (h, pair)
    float sx[2][NP]; // fp32 scale of this lane's (column, block); 0 off-lane
};

// Every address is a uniform base plus a 32-bit lane offset (the
// SGPR-base form of the global loads): A in 16-byte units at chunk
// 2 (l / 16) + h, row 16g + l % 16; the two scale bytes of that row.
__device__ __forceinline__ MxW load_mx_w(const uint8_t *__restrict__ tile, int lane)
{
    MxW w;
    const uint32_t gb = (uint32_t)lane >> 4, n = (uint32_t)lane & 15u;
    const uint32_t ai = 128u * gb + n, si = 4096u + 4u * n + gb; // si in 16-bit units
    const u32x4 *tv = reinterpret_cast<const u32x4 *>(tile);
    const uint16_t *th = reinterpret_cast<const uint16_t *>(tile);
#pragma unroll
    for (int g = 0; g < 4; g++)
        w.sa[g] = th[si + 64u * g];
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int g = 0; g < 4; g++) {
            w.a[2 * g + h] = __builtin_nontemporal_load(tv + (ai + 64u * h + 16u * g));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    return w;
}

// Activation block of (h, lane): s * 8 + 2 bn + h, clamped into K (the
// weights past K are zero). SX = false leaves the scales out (the block-dot
// test hook has none).
template <int Q, bool FULL, bool SX = true>
__device__ __forceinline__ MxX<Q> load_mx_x(int s, int nb, const XCols<Q> &xc, const MxLane<Q> &ml)
{
    MxX<Q> x;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int blk = FULL ? s * 8 + 2 * ml.bn + h : min(s * 8 + 2 * ml.bn + h, nb - 1);
#pragma unroll
        for (int p = 0; p < MxX<Q>::NP; p++) {
            x.xr[h][p] = *reinterpret_cast<const u32x4 *>(xc.xq + (ml.xo[p] + 32u * (uint32_t)blk));
            // masked where it is used (compute_mx): a select here would
            // wait for the load before the tile's weight loads are issued
            x.sx[h][p] = SX ? xc.xs[ml.mo[p] + (uint32_t)blk] : 0.0f;
        }
    }
    return x;
}

template <int Q>
struct MxTile {
    MxW w;
    MxX<Q> x;
};

template <int Q, bool FULL>
__device__ __forceinline__ MxTile<Q> load_mx_tile(const uint8_t *__restrict__ tile, int s, int nb, int lane,
                                                  const XCols<Q> &xc, const MxLane<Q> &ml)
{
    MxTile<Q> t;
    t.x = load_mx_x<Q, FULL>(s, nb, xc, ml);
    t.w = load_mx_w(tile, lane);
    return t;
}

// B operand of one (half, pair): the lane's 16 activations in nibble order,
// split to the lane's part and coded as E4M3, in bytes 0..15 or 16..31.
template <int Q>
__device__ __forceinline__ i32x8 build_b(const u32x4 &x, const MxLane<Q> &ml, int p)
{
    const uint32_t w[4] = {__builtin_amdgcn_perm(x.y, x.x, 0x05010400u), __builtin_amdgcn_perm(x.y, x.x, 0x07030602u),
                           __builtin_amdgcn_perm(x.w, x.z, 0x05010400u), __builtin_amdgcn_perm(x.w, x.z, 0x07030602u)};
    const uint32_t sh = ml.sh[p];
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t idx = (w[k] >> sh) & 0x07070707u;
        const uint32_t lo8 = __builtin_amdgcn_perm(kE4m3Lo[1], kE4m3Lo[0], idx); // same for both parts
        const uint32_t hi8 = __builtin_amdgcn_perm(ml.tab3[p], ml.tab2[p], idx);
        const uint32_t msel = ((w[k] >> (sh + 1u)) & 0x04040404u) | 0x03020100u;
        o[k] = __builtin_amdgcn_perm(hi8, lo8, msel);
    }
    i32x8 b;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        b[k] = (int)(ml.put_lo[p] ? o[k] : 0u);
        b[4 + k] = (int)(ml.put_hi[p] ? o[k] : 0u);
    }
    return b;
}

// The high part of the pair-P column that this lane's low part pairs with:
// 4 lanes up for pair 0, 4 lanes down for pair 1 (0 past the row's end).
template <int P>
__device__ __forceinline__ float high_part(float d)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, d), P == 0 ? 0x104 : 0x114,
                                                                 0xF, 0xF, true));
}

// One product: A (FP4, scale byte H of sa) x B (FP8; the high-part
// columns scaled by 2^4, so a block's two columns simply add up).
template <int H>
__device__ __forceinline__ f32x4 mx_product(const u32x4 &a4, const i32x8 &b, uint32_t sa, uint32_t sb)
{
    const i32x8 a = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w, 0, 0, 0, 0};
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 4, 0, H, (int)sa, 0, (int)sb);
}

// All eight (g, h) products of a tile for each of M weight matrices over
// the same K range (one B operand per (half, pair) serves them all), then
// per output the high part folded into the low one and the fp32 block scale
// applied: acc[m][g][v] collects row 16g + 4 (l / 16) + v of the lane's
// column (see MxLane).
template <int Q, int M>
__device__ __forceinline__ void compute_mx(const MxW (&w)[M], const MxX<Q> &x, const MxLane<Q> &ml,
                                           float (&acc)[M][4][4])
{
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int p = 0; p < MxX<Q>::NP; p++) {
            const i32x8 b = build_b<Q>(x.xr[h][p], ml, p);
            const float sx = ml.lo[p] ? x.sx[h][p] : 0.0f;
#pragma unroll
            for (int m = 0; m < M; m++) {
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const f32x4 d = h == 0 ? mx_product<0>(w[m].a[2 * g], b, w[m].sa[g], ml.sb[p])
                                           : mx_product<1>(w[m].a[2 * g + 1], b, w[m].sa[g], ml.sb[p]);
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        const float hi = p == 0 ? high_part<0>(d[v]) : high_part<1>(d[v]);
                        const float blk = d[v] + hi;
                        acc[m][g][v] = fmaf(sx, blk, acc[m][g][v]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The products of compute_mx for one weight matrix, stopped before the
// activation scale: for every (half, pair, g) the low-part lanes hold
// 2^(E-128) D, E the block exponent and D the block's integer dot, of their
// (column, tile row, tile block), handed to store(col, row, blk, value).
// Same operands, same products and the same high-into-low fold as the
// product path; every lane takes part in the products and the fold.
template <int Q, typename Store>
__device__ __forceinline__ void mx_block_values(const MxW &w, const MxX<Q> &x, const MxLane<Q> &ml, int lane,
                                                Store store)
{
    const int rq = lane >> 4, n = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int p = 0; p < MxX<Q>::NP; p++) {
            const i32x8 b = build_b<Q>(x.xr[h][p], ml, p);
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const f32x4 d = h == 0 ? mx_product<0>(w.a[2 * g], b, w.sa[g], ml.sb[p])
                                       : mx_product<1>(w.a[2 * g + 1], b, w.sa[g], ml.sb[p]);
                float blk[4];
#pragma unroll
                for (int v = 0; v < 4; v++)
                    blk[v] = d[v] + (p == 0 ? high_part<0>(d[v]) : high_part<1>(d[v]));
                if (ml.lo[p]) {
#pragma unroll
                    for (int v = 0; v < 4; v++)
                        store(2 * p + (n >> 3), 16 * g + 4 * rq + v, 2 * ml.bn + h, blk[v]);
                }
            }
        }
    }
}

template <int Q>
__device__ __forceinline__ void compute_mx_tile(const MxTile<Q> &t, const MxLane<Q> &ml, float (&acc)[4][4])
{
    const MxW w[1] = {t.w};
    float (&a1)[1][4][4] = reinterpret_cast<float (&)[1][4][4]>(acc);
    compute_mx<Q, 1>(w, t.x, ml, a1);
}

// Quad sums (the four blocks of a half), then store(col, row, value) for
// the lane's column and its rows 16g + 4 (l / 16) + v of the tile (one lane
// per quad stores).
template <int Q, typename Store>
__device__ __forceinline__ void mx_rows(float (&acc)[4][4], int lane, Store store)
{
    const int n = lane & 15, rq = lane >> 4, k = n >> 2;
    const int col = (k & 1) ? 2 + (k >> 1) : (k >> 1);
#pragma unroll
    for (int g = 0; g < 4; g++) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            float s = acc[g][v];
            s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, true));
            s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, true));
            if ((n & 3) == 0 && col < Q)
                store(col, 16 * g + 4 * rq + v, s);
        }
    }
}

// The per-row partials of every column into red[(wave * Q + col) * 64 + row],
// the layout the GEMV epilogue reads.
template <int Q>
__device__ __forceinline__ void mx_to_red(float (&acc)[4][4], float *red, int wave, int lane)
{
    mx_rows<Q>(acc, lane, [&](int col, int row, float v) { red[(wave * Q + col) * 64 + row] = v; });
}

} // namespace dev
} // namespace rfx
