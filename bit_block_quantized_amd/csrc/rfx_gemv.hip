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
//   - q = 1: the activation block is the same for all 64 lanes, so it is
//     read with scalar loads into SGPRs and used directly as the SGPR
//     operand of v_dot4_i32_i8: no LDS traffic, no cross-lane reduction;
//   - q >= 2: the q column dots of a block run on the matrix core
//     (v_mfma_i32_4x4x4_16b_i8, weights of the lane's row against the
//     activations broadcast from one 4-lane group), fed by one vector load
//     of the tile's activation slice;
//   - FP2/FP3 codebooks are affine in the code (v = 2c - 3, v = 2c - 7), so
//     the selector bytes go straight into v_dot4 and the offset is folded in
//     once per block with the precomputed activation block sum (the FP2M
//     variant's block minimum enters the same way, as m times that sum,
//     after the scale; the FP2S variant expands its codes to the signed
//     values with one v_perm_b32 per four weights and keeps the dots of
//     its two 16-weight halves apart, one per sub-scale); FP4 (E2M1,
//     not affine) expands through two v_perm_b32 table lookups and a v_perm
//     merge on the sign bit;
//   - the 256-column tiles of a row group are split into contiguous runs over
//     the W waves of a workgroup (fixed-order LDS reduce) and, when the row
//     groups alone cannot fill 256 CUs, over P = 2^k workgroups; their
//     partials meet pairwise up a binary tree of exchange slots, each node
//     one two-term fp32 sum, so the result does not depend on arrival order
//     (deterministic, no float atomics, no counters, no L2 write-back);
//   - each wave keeps the next tile's loads in flight while it decodes the
//     current one;
//   - several independent GEMVs can share one launch (gemv_grouped_kernel),
//     so one matrix's last workgroups overlap the next one's weight stream.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "rfx_decode.h"
#include "rfx_mx4.h"
#include "rfx_xtile.h"
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

using namespace rfx::dev;

// ------------------------------------------------------------------
// Activation quantization: one lane per four elements (a 16-byte load and
// one packed 4-byte store), eight lanes per 32-element block. s = amax/127
// (IEEE division), code = clamp(rne(x/s)); the max and the integer sum are
// order-free, so the result is the same as element by element.
// ------------------------------------------------------------------
__global__ __launch_bounds__(256) void act_quant_kernel(const float4 *__restrict__ x, int64_t n4,
                                                        uint32_t *__restrict__ xq,
                                                        float *__restrict__ xs,
                                                        int32_t *__restrict__ xsum)
{
#pragma clang fp contract(off)
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; // group of four
    const bool valid = i < n4; // n4 is a multiple of 8: blocks are whole
    const float4 v4 = valid ? x[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float v[4] = {v4.x, v4.y, v4.z, v4.w};
    float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    for (int o = 4; o > 0; o >>= 1)
        a = fmaxf(a, __shfl_xor(a, o, 8));
    const float s = a / 127.0f;
    uint32_t packed = 0u;
    int sum = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        int qv = 0;
        if (s != 0.0f) {
            float r = rintf(v[k] / s);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            qv = (int)r;
        }
        sum += qv;
        packed |= ((uint32_t)qv & 0xffu) << (8 * k);
    }
    for (int o = 4; o > 0; o >>= 1)
        sum += __shfl_xor(sum, o, 8);
    if (valid) {
        xq[i] = packed;
        if ((threadIdx.x & 7) == 0) {
            xs[i >> 3] = s;
            xsum[i >> 3] = sum;
        }
    }
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

// Activations per block come either from SGPRs (scalar loads per block) or,
// with BC, from a per-tile VGPR slice loaded together with the weight tile,
// and the column dots then run on the matrix core (v_mfma_i32_4x4x4_16b_i8
// with the activations broadcast from one 4-lane group). Scalar loads
// complete out of order, so each block waits for all of its activation
// loads: at q >= 2 that wait and the q v_dot4 chains per block dominate and
// BC wins; at q = 1 the scalar path is as fast and needs fewer VGPRs. The
// multi-tile loop of a lone GEMV (double-buffered tiles) takes the scalar
// path to stay within the register budget of a 1024-thread workgroup.
template <int Q>
constexpr bool use_bcast()
{
    return Q >= 2;
}

// A weight tile and, in broadcast mode, the matching activation slice.
template <int FMT, int Q>
struct WTile {
    TileRegs<FMT> w;
    XTileM<Q> x;
};

template <int FMT, int Q, bool FULL, bool BC>
__device__ __forceinline__ WTile<FMT, Q> load_wtile(const uint8_t *gbase, int s, int lane, const XCols<Q> &xc,
                                                    int nb)
{
    WTile<FMT, Q> t;
    if (BC) // issued first: block 0 needs it together with the first chunk
        t.x = load_xtile_m<FMT, Q, FULL>(xc, s, nb, lane);
    t.w = load_tile<FMT>(gbase + (size_t)s * TileFmt<FMT>::bytes, lane);
    return t;
}

template <int FMT, int Q, bool FULL, int... BI>
__device__ __forceinline__ void store_dots_bcast(const WTile<FMT, Q> &t, int b0, int row, const GemvArgs &a,
                                                 std::integer_sequence<int, BI...>)
{
    // the dots run with every lane active (the broadcasts read other
    // lanes); only the stores are predicated
    (
        [&] {
            int d[Q];
            const i32x4 dm = tile_block_dots_mfma<FMT, Q, BI>(t.w, t.x);
#pragma unroll
            for (int j = 0; j < Q; j++)
                d[j] = dm[j];
            if (b0 + BI < a.nb && row < a.N) {
#pragma unroll
                for (int j = 0; j < Q; j++)
                    a.dots[((size_t)j * a.N + row) * a.nb + b0 + BI] = d[j];
            }
        }(),
        ...);
}

template <int FMT, int Q, bool DOTS, bool FULL, bool BC>
__device__ __forceinline__ void compute_tile(const WTile<FMT, Q> &t, int s, int row, const GemvArgs &a,
                                             const XCols<Q> &xc, float (&acc)[Q])
{
    const int b0 = s * 8;
    if (!DOTS) {
        if (BC)
            tile_blocks_mfma<FMT, Q, FULL>(t.w, t.x, b0, a.nb, acc);
        else
            tile_blocks<FMT, Q, Q, FULL>(t.w, b0, a.nb, xc, acc);
        return;
    }
    // debug path: per-block dots of the blocks inside K
    if (BC) {
        store_dots_bcast<FMT, Q, FULL>(t, b0, row, a, std::make_integer_sequence<int, 8>{});
        return;
    }
#pragma unroll
    for (int bi = 0; bi < 8; bi++) {
        const int b = min(b0 + bi, a.nb - 1);
        const XBlock<Q> xb = load_xblock<TileFmt<FMT>::needs_sum, Q>(xc, b);
        Sel8 sel;
        float sw;
        decode_block<FMT>(t.w, bi, sel, sw);
        if (b0 + bi < a.nb && row < a.N) {
#pragma unroll
            for (int j = 0; j < Q; j++)
                a.dots[((size_t)j * a.N + row) * a.nb + b0 + bi] = block_dot<FMT, Q>(sel, xb, j);
        }
    }
}

// Wave 0 of a workgroup: sum the W waves' partials (fixed order) and
// either store y or climb the split-K exchange tree.
template <int Q>
__device__ __forceinline__ void gemv_finish(const GemvArgs &a, int p, int g, int W, const float *red)
{
    const int lane = threadIdx.x & 63;
    const int row = g * 64 + lane;
    float val[Q];
#pragma unroll
    for (int j = 0; j < Q; j++) {
        float t = red[j * 64 + lane];
        for (int w = 1; w < W; w++)
            t += red[(w * Q + j) * 64 + lane];
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
    // node is one two-term fp32 sum, and a + b == b + a exactly, so the
    // result does not depend on arrival order. The second arriver clears
    // the slot, leaving the workspace zeroed for the next call.
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

// One workgroup = W waves on one 64-row group; its tiles [s_begin, s_end)
// are split into contiguous runs, one per wave. Each wave keeps the next
// tile's loads in flight while it decodes the current one.
//
// Workgroup p (of P) of row group g; red holds W x Q x 64 floats of LDS.
// LBC: the multi-tile loop takes the broadcast path too (two activation
// slices in registers; affordable below 1024 threads per workgroup).
template <int FMT, int Q, bool DOTS, bool FULL, bool LBC = false>
__device__ __forceinline__ void gemv_body(const GemvArgs &a, int p, int g, float *red)
{
    // wave index is uniform per wave; say so, so the tile index, the
    // activation addresses and the loop bounds live in SGPRs.
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    const int row = g * 64 + lane;
    float acc[Q];
    XCols<Q> xc;
    xc.xq = a.xq;
    xc.xs = a.xs;
    xc.xsum = a.xsum;
#pragma unroll
    for (int j = 0; j < Q; j++) {
        acc[j] = 0.0f;
        xc.xoff[j] = (uint32_t)j * (uint32_t)a.K;
        xc.moff[j] = (uint32_t)j * (uint32_t)a.nb;
    }

    const int nw = a.P * W, v = p * W + wave;
    // the division runs on the vector unit; pin its uniform result to SGPRs
    const int s_begin = __builtin_amdgcn_readfirstlane((int)((unsigned)(a.S * v) / (unsigned)nw));
    const int s_end = __builtin_amdgcn_readfirstlane((int)((unsigned)(a.S * (v + 1)) / (unsigned)nw));
    const uint8_t *gbase = a.W + (size_t)g * a.S * TileFmt<FMT>::bytes;
    if (s_end - s_begin == 1) {
        // the common case: one tile per wave, straight-line code, so each
        // block waits only for its own chunks
        constexpr bool BC = use_bcast<Q>();
        const WTile<FMT, Q> t = load_wtile<FMT, Q, FULL, BC>(gbase, s_begin, lane, xc, a.nb);
        compute_tile<FMT, Q, DOTS, FULL, BC>(t, s_begin, row, a, xc, acc);
    } else if (TileFmt<FMT>::code_chunks > 8) {
        // Q8 tiles (64 registers of codes) take one buffer, so that the
        // format does not raise the register budget of the kernels it
        // shares with the smaller formats
        constexpr bool BC = LBC && use_bcast<Q>();
        for (int s = s_begin; s < s_end; s++) {
            const WTile<FMT, Q> t = load_wtile<FMT, Q, FULL, BC>(gbase, s, lane, xc, a.nb);
            compute_tile<FMT, Q, DOTS, FULL, BC>(t, s, row, a, xc, acc);
        }
    } else if (s_begin < s_end) {
        // two tile buffers used in turn (no register copies, which would
        // wait for the loads they copy): tile s + 1 in flight while s is
        // computed. The loop body loads unconditionally and the last one or
        // two tiles run after it: with the next tile's loads under a branch,
        // the compiler's wait for the current tile's first chunk had to
        // assume they were not issued and waited for nearly all of them.
        constexpr bool BC = LBC && use_bcast<Q>();
        WTile<FMT, Q> ta = load_wtile<FMT, Q, FULL, BC>(gbase, s_begin, lane, xc, a.nb), tb;
        int s = s_begin;
        for (; s + 2 < s_end; s += 2) {
            tb = load_wtile<FMT, Q, FULL, BC>(gbase, s + 1, lane, xc, a.nb);
            compute_tile<FMT, Q, DOTS, FULL, BC>(ta, s, row, a, xc, acc);
            ta = load_wtile<FMT, Q, FULL, BC>(gbase, s + 2, lane, xc, a.nb);
            compute_tile<FMT, Q, DOTS, FULL, BC>(tb, s + 1, row, a, xc, acc);
        }
        if (s + 1 < s_end)
            tb = load_wtile<FMT, Q, FULL, BC>(gbase, s + 1, lane, xc, a.nb);
        compute_tile<FMT, Q, DOTS, FULL, BC>(ta, s, row, a, xc, acc);
        if (s + 1 < s_end)
            compute_tile<FMT, Q, DOTS, FULL, BC>(tb, s + 1, row, a, xc, acc);
    }
    if (DOTS)
        return;

    // Fixed-order reduction over the waves of this workgroup: every wave
    // leaves its partials in LDS, wave 0 sums and finishes.
#pragma unroll
    for (int j = 0; j < Q; j++)
        red[(wave * Q + j) * 64 + lane] = acc[j];
    __syncthreads();
    if (wave == 0)
        gemv_finish<Q>(a, p, g, W, red);
}

// FP4 blocks go to the block-scaled matrix core (rfx_mx4.h) for one or two
// activation columns (one column pair of the B operand). From three columns
// on, the two pairs cost more registers (166 per lane: three waves per
// SIMD) and a longer dependency chain per tile than the vector decode with
// the 4x4x4 int8 matrix op saves; measured on the 7168 x 7168 step, the
// FP4 q = 4 job ran faster on that path.
template <int FMT, int Q>
constexpr bool use_mx()
{
    return FMT == RFX_FP4 && Q <= 2;
}

// FP4 on the block-scaled matrix core (rfx_mx4.h): the same tile split,
// K split and epilogue as gemv_body, with each wave's partials moved into
// the row layout of the LDS reduction before it. LBC: the multi-tile loop
// keeps the next tile in flight (two tile buffers; within the register
// budget of a workgroup of at most 256 threads), else it loads and
// computes one tile at a time.
template <int Q, bool FULL, bool LBC>
__device__ __forceinline__ void gemv_body_mx(const GemvArgs &a, int p, int g, float *red)
{
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    XCols<Q> xc;
    xc.xq = a.xq;
    xc.xs = a.xs;
    xc.xsum = a.xsum;
#pragma unroll
    for (int j = 0; j < Q; j++) {
        xc.xoff[j] = (uint32_t)j * (uint32_t)a.K;
        xc.moff[j] = (uint32_t)j * (uint32_t)a.nb;
    }
    const MxLane<Q> ml = mx_lane<Q>(lane, xc);
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int v = 0; v < 4; v++)
            acc[i][v] = 0.0f;

    const int nw = a.P * W, vv = p * W + wave;
    const int s_begin = __builtin_amdgcn_readfirstlane((int)((unsigned)(a.S * vv) / (unsigned)nw));
    const int s_end = __builtin_amdgcn_readfirstlane((int)((unsigned)(a.S * (vv + 1)) / (unsigned)nw));
    const uint8_t *gbase = a.W + (size_t)g * a.S * TileFmt<RFX_FP4>::bytes;
    constexpr int TB = TileFmt<RFX_FP4>::bytes;
    if (LBC && s_end - s_begin > 1) {
        // the loop body loads unconditionally (see gemv_body)
        MxTile<Q> ta = load_mx_tile<Q, FULL>(gbase + (size_t)s_begin * TB, s_begin, a.nb, lane, xc, ml), tb;
        int s = s_begin;
        for (; s + 2 < s_end; s += 2) {
            tb = load_mx_tile<Q, FULL>(gbase + (size_t)(s + 1) * TB, s + 1, a.nb, lane, xc, ml);
            compute_mx_tile<Q>(ta, ml, acc);
            ta = load_mx_tile<Q, FULL>(gbase + (size_t)(s + 2) * TB, s + 2, a.nb, lane, xc, ml);
            compute_mx_tile<Q>(tb, ml, acc);
        }
        if (s + 1 < s_end)
            tb = load_mx_tile<Q, FULL>(gbase + (size_t)(s + 1) * TB, s + 1, a.nb, lane, xc, ml);
        compute_mx_tile<Q>(ta, ml, acc);
        if (s + 1 < s_end)
            compute_mx_tile<Q>(tb, ml, acc);
    } else {
        for (int s = s_begin; s < s_end; s++) {
            const MxTile<Q> t = load_mx_tile<Q, FULL>(gbase + (size_t)s * TB, s, a.nb, lane, xc, ml);
            compute_mx_tile<Q>(t, ml, acc);
        }
    }
    mx_to_red<Q>(acc, red, wave, lane);
    __syncthreads();
    if (wave == 0)
        gemv_finish<Q>(a, p, g, W, red);
}

// Test hook on the block-scaled matrix core: the products gemv_body_mx
// computes, each block's value 2^(E-128) D read before the activation scale
// and multiplied back by 2^(128-E) (exact: a power of two). The stored dot
// is that integer, or INT32_MIN when the value the matrix core produced is
// not one (lost to the fp32 range), so an inexact product never passes.
// Workgroup of W waves on row group g, no K split.
template <int Q, bool FULL>
__device__ __forceinline__ void gemv_dots_mx(const GemvArgs &a, int g)
{
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    XCols<Q> xc;
    xc.xq = a.xq;
    xc.xs = nullptr;
    xc.xsum = a.xsum;
#pragma unroll
    for (int j = 0; j < Q; j++) {
        xc.xoff[j] = (uint32_t)j * (uint32_t)a.K;
        xc.moff[j] = (uint32_t)j * (uint32_t)a.nb;
    }
    const MxLane<Q> ml = mx_lane<Q>(lane, xc);
    constexpr int TB = TileFmt<RFX_FP4>::bytes;
    const int s_begin = __builtin_amdgcn_readfirstlane((int)((unsigned)(a.S * wave) / (unsigned)W));
    const int s_end = __builtin_amdgcn_readfirstlane((int)((unsigned)(a.S * (wave + 1)) / (unsigned)W));
    for (int s = s_begin; s < s_end; s++) {
        const uint8_t *tile = a.W + ((size_t)g * a.S + s) * TB;
        MxTile<Q> t;
        t.x = load_mx_x<Q, FULL, false>(s, a.nb, xc, ml);
        t.w = load_mx_w(tile, lane);
        mx_block_values<Q>(t.w, t.x, ml, lane, [&](int col, int r, int tb, float v) {
            const int row = g * 64 + r, blk = s * 8 + tb;
            if (row < a.N && blk < a.nb) {
                const int e = tile[8192 + r * 8 + tb];
                const float dv = ldexpf(v, 128 - e);
                int di = INT32_MIN;
                if (fabsf(dv) < 2147483648.0f && (float)(int)dv == dv)
                    di = (int)dv;
                a.dots[((size_t)col * a.N + row) * a.nb + blk] = di;
            }
        });
    }
}

// One GEMV; grid = (P, G).
template <int FMT, int Q, bool DOTS, bool FULL>
__global__ __launch_bounds__(1024) void gemv_kernel(GemvArgs a)
{
    __shared__ float red[16 * Q * 64];
    if constexpr (use_mx<FMT, Q>()) {
        if constexpr (DOTS)
            gemv_dots_mx<Q, FULL>(a, blockIdx.y);
        else
            gemv_body_mx<Q, FULL, false>(a, blockIdx.x, blockIdx.y, red);
    } else {
        gemv_body<FMT, Q, DOTS, FULL>(a, blockIdx.x, blockIdx.y, red);
    }
}

// Several independent GEMVs in one launch. The workgroups are the jobs'
// (row group, K split) pairs. When every workgroup of the launch is
// resident at once, the dispatcher places workgroup b on CU b mod n_cu (in
// round b / n_cu; measured on MI355X), so each CU's share is fixed by the
// order, and the launch ends with its most loaded CU: the host orders the
// workgroups so that the CUs' shares cost about the same (balanced_order),
// else they run job by job, the longest work first.
constexpr int kMaxJobs = RFX_MAX_GEMV_JOBS;
constexpr int kMaxOrder = 1024; // workgroups a balanced order covers

// Every job runs W waves per workgroup (one block size per launch), each
// wave a contiguous run of tiles with the next tile in flight. K is split
// over P workgroups only as far as needed to give the launch about two
// waves per SIMD: a launch of several large matrices runs one workgroup
// per row group (no exchange at all, every workgroup resident at once); a
// lone small matrix still fills the chip.
constexpr int kGroupW = 4;

struct GroupArgs {
    GemvArgs job[kMaxJobs];
    int kind[kMaxJobs];         // 8 * fmt + q
    int wg_begin[kMaxJobs + 1]; // job j: workgroups [wg_begin[j], wg_begin[j + 1])
    int n;
    int n_order;                // 0: workgroups job by job; else workgroup b is
    uint16_t order[kMaxOrder];  // order[b] = (job << 12) | index within the job
};

template <bool FULL>
__global__ __launch_bounds__(64 * kGroupW) void gemv_grouped_kernel(GroupArgs ga)
{
    __shared__ float red[kGroupW * 4 * 64];
    const int bid = blockIdx.x;
    int j = 0, local;
    if (ga.n_order) {
        // read straight from the kernel-argument segment (ga is its only
        // argument, at offset 0): indexing the by-value struct with bid makes
        // the compiler copy the whole struct to private memory first
        typedef const __attribute__((address_space(4))) uint16_t *korder_t;
        typedef const __attribute__((address_space(4))) char *kbytes_t;
        const unsigned e =
            ((korder_t)((kbytes_t)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(GroupArgs, order)))[bid];
        j = (int)(e >> 12);
        local = (int)(e & 4095u);
    } else {
        while (j + 1 < ga.n && bid >= ga.wg_begin[j + 1])
            j++;
        local = bid - ga.wg_begin[j];
    }
    j = __builtin_amdgcn_readfirstlane(j);
    local = __builtin_amdgcn_readfirstlane(local);
    const GemvArgs &a = ga.job[j];
    const int p = local & (a.P - 1), g = local / a.P;
#define RFX_JOB(F, QQ)                                                                                        \
    case 8 * F + QQ:                                                                                          \
        if constexpr (use_mx<F, QQ>())                                                                        \
            gemv_body_mx<QQ, FULL, true>(a, p, g, red);                                                       \
        else                                                                                                  \
            gemv_body<F, QQ, false, FULL, true>(a, p, g, red);                                                \
        break;
    switch (ga.kind[j]) {
        RFX_JOB(RFX_FP2, 1) RFX_JOB(RFX_FP2, 2) RFX_JOB(RFX_FP2, 3) RFX_JOB(RFX_FP2, 4)
        RFX_JOB(RFX_FP3, 1) RFX_JOB(RFX_FP3, 2) RFX_JOB(RFX_FP3, 3) RFX_JOB(RFX_FP3, 4)
        RFX_JOB(RFX_FP4, 1) RFX_JOB(RFX_FP4, 2) RFX_JOB(RFX_FP4, 3) RFX_JOB(RFX_FP4, 4)
        RFX_JOB(RFX_FP2M, 1) RFX_JOB(RFX_FP2M, 2) RFX_JOB(RFX_FP2M, 3) RFX_JOB(RFX_FP2M, 4)
        RFX_JOB(RFX_Q8, 1) RFX_JOB(RFX_Q8, 2) RFX_JOB(RFX_Q8, 3) RFX_JOB(RFX_Q8, 4)
        RFX_JOB(RFX_FP2S, 1) RFX_JOB(RFX_FP2S, 2) RFX_JOB(RFX_FP2S, 3) RFX_JOB(RFX_FP2S, 4)
        RFX_JOB(RFX_FP3E, 1) RFX_JOB(RFX_FP3E, 2) RFX_JOB(RFX_FP3E, 3) RFX_JOB(RFX_FP3E, 4)
    default: break;
    }
#undef RFX_JOB
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

template <int FMT, bool DOTS, bool FULL>
int launch_q(const GemvArgs &a, int q, int G, int W, hipStream_t st)
{
    dim3 grid(a.P, G), block(64 * W);
    switch (q) {
    case 1: hipLaunchKernelGGL((gemv_kernel<FMT, 1, DOTS, FULL>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<FMT, 2, DOTS, FULL>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((gemv_kernel<FMT, 3, DOTS, FULL>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<FMT, 4, DOTS, FULL>), grid, block, 0, st, a); break;
    default: return fail(RFX_E_INVAL, "q must be 1..4");
    }
    return hip_status("gemv launch");
}

template <bool DOTS>
int launch(int fmt, const GemvArgs &a, int q, int G, int W, hipStream_t st)
{
    const bool full = a.K % kTileCols == 0; // no partial tiles
    switch (fmt) {
    case RFX_FP2: return full ? launch_q<RFX_FP2, DOTS, true>(a, q, G, W, st) : launch_q<RFX_FP2, DOTS, false>(a, q, G, W, st);
    case RFX_FP3: return full ? launch_q<RFX_FP3, DOTS, true>(a, q, G, W, st) : launch_q<RFX_FP3, DOTS, false>(a, q, G, W, st);
    case RFX_FP4: return full ? launch_q<RFX_FP4, DOTS, true>(a, q, G, W, st) : launch_q<RFX_FP4, DOTS, false>(a, q, G, W, st);
    case RFX_FP2M: return full ? launch_q<RFX_FP2M, DOTS, true>(a, q, G, W, st) : launch_q<RFX_FP2M, DOTS, false>(a, q, G, W, st);
    case RFX_Q8: return full ? launch_q<RFX_Q8, DOTS, true>(a, q, G, W, st) : launch_q<RFX_Q8, DOTS, false>(a, q, G, W, st);
    case RFX_FP2S: return full ? launch_q<RFX_FP2S, DOTS, true>(a, q, G, W, st) : launch_q<RFX_FP2S, DOTS, false>(a, q, G, W, st);
    case RFX_FP3E: return full ? launch_q<RFX_FP3E, DOTS, true>(a, q, G, W, st) : launch_q<RFX_FP3E, DOTS, false>(a, q, G, W, st);
    }
    return fail(RFX_E_INVAL, "unknown format");
}

// P per job (a power of two, at most 8, and no more than its tiles need).
void grouped_shape(const rfx_gemv_job *jobs, int n, int *P)
{
    const int target_waves = 2048; // 1024 SIMDs x 2
    for (int cap = 1;; cap <<= 1) {
        long waves = 0;
        bool can_split = false;
        for (int j = 0; j < n; j++) {
            const int G = (int)ceil_div(jobs[j].W.rows, kTileRows), S = (int)ceil_div(jobs[j].W.cols, kTileCols);
            int p = 1;
            while (p < cap && p * kGroupW < S)
                p <<= 1;
            P[j] = p;
            can_split = can_split || (p == cap && p * kGroupW < S);
            waves += (long)G * p * kGroupW;
        }
        if (waves >= target_waves || !can_split || cap >= 8)
            return;
    }
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

int check_act(const int8_t *xq, const float *xs, const int32_t *xsum, bool need_xs)
{
    int st = check_ptr(xq, 16, "xq");
    if (!st && need_xs)
        st = check_ptr(xs, 4, "xs");
    if (!st)
        st = check_ptr(xsum, 4, "xsum");
    return st;
}

// Compute units of the current device (cached per device).
int cu_count()
{
    static int n_cu[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (!n_cu[dev]) {
        int v = 0;
        n_cu[dev] = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0
                        ? v
                        : 256;
    }
    return n_cu[dev];
}

// Balanced workgroup order of a grouped launch whose workgroups are all
// resident at once (at most three per CU: a workgroup of four waves at the
// kernel's ~140 registers). Cost of a workgroup: its tiles x (tile bytes +
// an amount per activation column beyond the first), a fit of per-CU
// finishing times of the six-GEMV 7168 x 7168 step on MI355X: a column's
// decode share and int8 matrix ops cost about as much as 1450 more weight
// bytes per tile, and about 330 for FP4 on the f16 matrix op (q >= 3; at
// q = 2 FP4 runs on the block-scaled matrix core). Largest cost first,
// each to the CU with the least cost that has a position left (CU c holds
// positions c, c + n_cu, ...), then swaps between the most loaded CU and
// the others while they lower its cost. Deterministic; results do not
// depend on the order (each workgroup computes the same values wherever
// it runs). Orders are cached per launch signature.
bool balanced_order(GroupArgs &ga, int wgs)
{
    const int n_cu = cu_count();
    if (wgs > kMaxOrder || wgs > 3 * n_cu || n_cu > 1024 || wgs < 2)
        return false;
    struct Key {
        int n, wgs, n_cu, sig[kMaxJobs][3];
        bool operator==(const Key &o) const { return std::memcmp(this, &o, sizeof(Key)) == 0; }
    };
    Key key;
    std::memset(&key, 0, sizeof key);
    key.n = ga.n;
    key.wgs = wgs;
    key.n_cu = n_cu;
    for (int j = 0; j < ga.n; j++) {
        key.sig[j][0] = ga.kind[j];
        key.sig[j][1] = ga.wg_begin[j + 1] - ga.wg_begin[j];
        key.sig[j][2] = (int)ceil_div(ga.job[j].S, ga.job[j].P);
    }
    static std::mutex mu;
    static std::vector<std::pair<Key, std::vector<uint16_t>>> cache;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto &e : cache)
        if (e.first == key) {
            std::copy(e.second.begin(), e.second.end(), ga.order);
            ga.n_order = wgs;
            return true;
        }
    struct Item {
        long cost;
        int job, local;
    };
    std::vector<Item> items;
    for (int j = 0; j < ga.n; j++) {
        const int fmt = ga.kind[j] >> 3, q = ga.kind[j] & 7;
        const long per_col = fmt == RFX_FP4 ? 330L : 1450L;
        const long cost = (long)key.sig[j][2] * (tile_bytes(fmt) + per_col * (q - 1));
        for (int l = 0; l < key.sig[j][1]; l++)
            items.push_back(Item{cost, j, l});
    }
    std::stable_sort(items.begin(), items.end(), [](const Item &a, const Item &b) { return a.cost > b.cost; });
    std::vector<long> load(n_cu, 0);
    std::vector<std::vector<int>> held(n_cu); // item indices per CU
    std::vector<int> cap(n_cu);
    for (int c = 0; c < n_cu; c++)
        cap[c] = c < wgs ? (wgs - 1 - c) / n_cu + 1 : 0;
    for (int i = 0; i < (int)items.size(); i++) {
        int best = -1;
        for (int c = 0; c < n_cu; c++)
            if ((int)held[c].size() < cap[c] && (best < 0 || load[c] < load[best]))
                best = c;
        held[best].push_back(i);
        load[best] += items[i].cost;
    }
    for (int it = 0; it < 4 * wgs; it++) {
        int a = 0;
        for (int c = 1; c < n_cu; c++)
            if (load[c] > load[a])
                a = c;
        long gain = 0;
        int bb = -1, ia = -1, ib = -1;
        for (int b = 0; b < n_cu; b++) {
            if (b == a)
                continue;
            for (int x = 0; x < (int)held[a].size(); x++)
                for (int y = 0; y < (int)held[b].size(); y++) {
                    const long d = items[held[a][x]].cost - items[held[b][y]].cost;
                    if (d <= 0 || load[b] + d >= load[a])
                        continue;
                    const long g = load[a] - std::max(load[a] - d, load[b] + d);
                    if (g > gain) {
                        gain = g;
                        bb = b;
                        ia = x;
                        ib = y;
                    }
                }
        }
        if (bb < 0)
            break;
        const long d = items[held[a][ia]].cost - items[held[bb][ib]].cost;
        std::swap(held[a][ia], held[bb][ib]);
        load[a] -= d;
        load[bb] += d;
    }
    std::vector<uint16_t> ord(wgs);
    for (int c = 0; c < n_cu; c++)
        for (int k = 0; k < (int)held[c].size(); k++) {
            const Item &t = items[held[c][k]];
            ord[c + k * n_cu] = (uint16_t)((t.job << 12) | t.local);
        }
    if (cache.size() >= 16)
        cache.erase(cache.begin());
    cache.emplace_back(key, ord);
    std::copy(ord.begin(), ord.end(), ga.order);
    ga.n_order = wgs;
    return true;
}

// ------------------------------------------------------------------
// rfx_gemv_noalloc: rfx_gemv with its split-K exchange slots in a
// file-scope device array instead of a caller workspace, for callers that
// cannot allocate. The largest split choose_shape picks (row groups x
// (P - 1) below 192, q <= 4) needs under 192 KiB of slots.
// ------------------------------------------------------------------
constexpr size_t kNoAllocBytes = 256u << 10;
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices]; // device address of `scratch`, per device

__global__ __launch_bounds__(256) void zero_words_kernel(unsigned *p, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

} // namespace

// Every GPU the library runs on holds its own copy of this array until the
// process ends. In host code the name is only a stand-in: kernels and
// copies take the address hipGetSymbolAddress returns for the current
// device.
static __device__ __align__(256) unsigned scratch[kNoAllocBytes / sizeof(unsigned)];

namespace {

// The current device's address of `scratch`: looked up once per device and
// cleared then (a fill kernel on the caller's stream, ahead of the call's
// own kernels); every completed GEMV leaves its slots zero again.
int scratch_address(void **out, hipStream_t st)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return hip_status("hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(RFX_E_UNSUPPORTED, "rfx_gemv_noalloc: device %d (at most %d devices)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(RFX_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        const size_t n = kNoAllocBytes / sizeof(unsigned);
        hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           static_cast<unsigned *>(p), n);
        if (int rc = hip_status("rfx_gemv_noalloc scratch clear"))
            return rc;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RFX_OK;
}

} // namespace

extern "C" {

int rfx_quantize_act(const float *x, int q, int K, int8_t *xq, float *xs, int32_t *xsum, void *stream)
{
    if (q < 1 || K < 32 || K % 32)
        return fail(RFX_E_INVAL, "rfx_quantize_act: bad shape q=%d K=%d", q, K);
    int st = check_ptr(x, 16, "x");
    if (!st)
        st = check_ptr(xq, 16, "xq");
    if (!st)
        st = check_ptr(xs, 4, "xs");
    if (!st)
        st = check_ptr(xsum, 4, "xsum");
    if (st)
        return st;
    const int64_t n4 = (int64_t)q * K / 4;
    dim3 grid((unsigned)((n4 + 255) / 256)), block(256);
    hipLaunchKernelGGL(act_quant_kernel, grid, block, 0, (hipStream_t)stream, reinterpret_cast<const float4 *>(x),
                       n4, reinterpret_cast<uint32_t *>(xq), xs, xsum);
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

int rfx_gemv_noalloc(const rfx_qmat *W, const int8_t *xq, const float *xs, const int32_t *xsum, int q, float *y,
                     void *stream)
{
    int st = check_qmat(W, "W", false);
    if (st)
        return st;
    if (q < 1 || q > 4)
        return fail(RFX_E_INVAL, "rfx_gemv_noalloc: q=%d (must be 1..4)", q);
    if ((st = check_act(xq, xs, xsum, true)) || (st = check_ptr(y, 4, "y")))
        return st;
    const size_t need = rfx_gemv_workspace_bytes(W, q);
    if (need > kNoAllocBytes)
        return fail(RFX_E_WORKSPACE, "rfx_gemv_noalloc: this shape needs %zu bytes of scratch, more than its %zu",
                    need, kNoAllocBytes);
    void *ws = nullptr;
    if (need && (st = scratch_address(&ws, (hipStream_t)stream)))
        return st;
    // the same launch as rfx_gemv with a workspace: same shape, same kernels
    return rfx_gemv(W, xq, xs, xsum, q, y, ws, ws ? kNoAllocBytes : 0, stream);
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

size_t rfx_gemv_grouped_workspace_bytes(const rfx_gemv_job *jobs, int n_jobs)
{
    if (!jobs || n_jobs < 1 || n_jobs > kMaxJobs)
        return 0;
    for (int j = 0; j < n_jobs; j++) {
        const rfx_qmat &W = jobs[j].W;
        if (!fmt_ok(W.fmt) || W.rows < 1 || W.cols < 32 || jobs[j].q < 1 || jobs[j].q > 4)
            return 0;
    }
    int P[kMaxJobs];
    grouped_shape(jobs, n_jobs, P);
    size_t total = 0;
    for (int j = 0; j < n_jobs; j++)
        total += align256(workspace_for((int)ceil_div(jobs[j].W.rows, kTileRows), P[j], jobs[j].q));
    return total;
}

int rfx_gemv_grouped(const rfx_gemv_job *jobs, int n_jobs, void *ws, size_t ws_bytes, void *stream)
{
    if (!jobs)
        return fail(RFX_E_INVAL, "rfx_gemv_grouped: jobs is NULL");
    if (n_jobs < 1 || n_jobs > kMaxJobs)
        return fail(RFX_E_INVAL, "rfx_gemv_grouped: n_jobs=%d (must be 1..%d)", n_jobs, kMaxJobs);
    // Longest work first: jobs whose workgroups take longest (most VALU per
    // block, see the block decoders) start first and the short ones fill
    // the end of the launch. Only the launch order changes; each job still
    // writes its own outputs.
    int order[kMaxJobs];
    for (int j = 0; j < n_jobs; j++)
        order[j] = j;
    auto cost = [&](int j) {
        const int f = jobs[j].W.fmt, q = jobs[j].q;
        const int base = f == RFX_FP2 ? 30 : f == RFX_FP3 || f == RFX_FP3E ? 45 : f == RFX_FP2M || f == RFX_FP2S ? 38
                       : f == RFX_Q8 ? 20 : 75;
        return base + 12 * q;
    };
    for (int i = 1; i < n_jobs; i++) // stable insertion sort, n <= 16
        for (int k = i; k > 0 && cost(order[k]) > cost(order[k - 1]); k--) {
            const int t = order[k];
            order[k] = order[k - 1];
            order[k - 1] = t;
        }
    int Pj[kMaxJobs];
    grouped_shape(jobs, n_jobs, Pj);
    GroupArgs ga{};
    ga.n = n_jobs;
    bool full = true;
    size_t ws_off = 0;
    int wgs = 0;
    for (int jj = 0; jj < n_jobs; jj++) {
        const int j = order[jj];
        const rfx_gemv_job &jb = jobs[j];
        char name[32];
        snprintf(name, sizeof name, "jobs[%d].W", j);
        int st = check_qmat(&jb.W, name, false);
        if (st)
            return st;
        if (jb.q < 1 || jb.q > 4)
            return fail(RFX_E_INVAL, "rfx_gemv_grouped: jobs[%d].q=%d (must be 1..4)", j, jb.q);
        if ((st = check_act(jb.xq, jb.xs, jb.xsum, true)) || (st = check_ptr(jb.y, 4, "y")))
            return fail(st, "rfx_gemv_grouped: jobs[%d]: %s", j, rfx_last_error());
        const int G = (int)ceil_div(jb.W.rows, kTileRows), S = (int)ceil_div(jb.W.cols, kTileCols);
        const int P = Pj[j];
        GemvArgs &a = ga.job[jj];
        a.W = static_cast<const uint8_t *>(jb.W.data);
        a.N = jb.W.rows;
        a.K = jb.W.cols;
        a.S = S;
        a.nb = jb.W.cols / 32;
        a.P = P;
        a.xq = jb.xq;
        a.xs = jb.xs;
        a.xsum = jb.xsum;
        a.y = jb.y;
        const size_t need = workspace_for(G, P, jb.q);
        a.slots = need ? reinterpret_cast<unsigned *>(static_cast<uint8_t *>(ws) + ws_off) : nullptr;
        ws_off += align256(need);
        ga.kind[jj] = 8 * jb.W.fmt + jb.q;
        ga.wg_begin[jj] = wgs;
        wgs += G * P;
        full = full && jb.W.cols % kTileCols == 0;
    }
    ga.wg_begin[n_jobs] = wgs;
    balanced_order(ga, wgs);
    if (ws_off) {
        if (!ws || ws_bytes < ws_off)
            return fail(RFX_E_WORKSPACE, "rfx_gemv_grouped: workspace %zu < %zu bytes", ws ? ws_bytes : (size_t)0,
                        ws_off);
        int st = check_ptr(ws, 256, "ws");
        if (st)
            return st;
    }
    const hipStream_t hs = (hipStream_t)stream;
    if (full)
        hipLaunchKernelGGL(gemv_grouped_kernel<true>, dim3(wgs), dim3(64 * kGroupW), 0, hs, ga);
    else
        hipLaunchKernelGGL(gemv_grouped_kernel<false>, dim3(wgs), dim3(64 * kGroupW), 0, hs, ga);
    return hip_status("grouped gemv launch");
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
