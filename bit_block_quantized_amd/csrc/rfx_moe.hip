// MoE decode layer for gfx950: router (logits, softmax, top-k, stable
// bucketing of (token, slot) pairs by expert) and the expert FFN (fused
// gate/up + SwiGLU + requantization, then down + shared expert + combine).
//
// Pages cited (title, site):
//   [HM]  "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
//         (hellomarvisaitoday.com), paragraphs numbered from the top.
//   [AIN] "Token Freedom via APU: AMD Ryzen AI MAX+ 395 Runs DeepSeek V4
//         Flash at 32 tok/s on a 284B Model" (ainomam.com), by section.
//   [KK]  the kaikai365.com post on DeepSeek V4 Flash on Strix Halo, by
//         section heading.
//
// The model has 256 routed experts plus one shared expert and activates six
// per token ([AIN] introduction); routed gate/up are stored in FP2, down in
// FP3, dense/sensitive projections in FP4 ([HM] para 2; [KK] ROCmFPX
// section); routing is a TOP_K + ARGSORT step ([HM] para 3; [KK] DSpark
// section). Expert weights stream once per decode step; every expert that
// several tokens picked is decoded once for all of them.
//
// Launches per layer: route (1), gate/up (1), down + combine (1). Each
// kernel finishes its cross-workgroup step with a last-arriver pattern
// (agent-scope write-through stores + an arrival counter), so outputs are
// deterministic and no extra launch is needed.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rfx_decode.h"
#include "rfx_internal.h"
#include "rfx_moe_dev.h"
#include "rfx_moe_ws.h"
#include "rfx_mx4.h"
#include "rfx_xtile.h"

using namespace rfx;
using namespace rfx::dev;
using namespace rfx::moe;

namespace {

// Router for q <= 4 tokens: one workgroup per expert row of Wr. Arrival
// is counted in two levels (kRouteGroup workgroups per sub-counter, then
// one counter over the groups), since atomics on one address serialize;
// the last workgroup to arrive picks the top k per token and buckets the
// pairs.
// ARRIVE = false: logits and quantization only; the top k is picked by
// every gate/up workgroup of the next launch (wg_route).
template <bool ARRIVE>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a)
{
    __shared__ int s_last;
    __shared__ __align__(16) int s_idx[kMaxDecodeQ * kMaxK];
    __shared__ float s_part[4][kMaxDecodeQ];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int e = blockIdx.x;

    // (0) the workgroup's row of Wr: each thread takes up to 8 float4
    //     columns (h = 4 tid + 1024 i), issued before anything waits
    const float *wrow = a.wr + (size_t)e * a.H;
    float4 w4[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int h = tid * 4 + 1024 * i;
        w4[i] = h < a.H ? *reinterpret_cast<const float4 *>(wrow + h) : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // (1) logits of row e: every token's x loaded at once, then a
    //     fixed-order reduction (per thread, the lane butterfly, then the
    //     waves in order)
    float4 x4[kMaxDecodeQ][8];
#pragma unroll
    for (int t = 0; t < kMaxDecodeQ; t++)
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int h = tid * 4 + 1024 * i;
            x4[t][i] = (t < a.q && h < a.H) ? *reinterpret_cast<const float4 *>(a.x + (size_t)t * a.H + h)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    float part[kMaxDecodeQ];
#pragma unroll
    for (int t = 0; t < kMaxDecodeQ; t++) {
        part[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++)
            part[t] = dot4_acc(part[t], w4[i], x4[t][i]);
        for (int o = 32; o > 0; o >>= 1)
            part[t] += __shfl_xor(part[t], o, 64);
    }
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < kMaxDecodeQ; t++)
            s_part[wave][t] = part[t];
    }
    __syncthreads();
    if (tid < a.q) {
        const float l = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
        __hip_atomic_store(a.logits + (size_t)tid * a.E + e, a.wb ? l + a.wb[e] : l, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!ARRIVE) {
        route_quant(a, blockIdx.x, gridDim.x, 4, wave, lane);
        return;
    }
    // (2) arrival. Every workgroup but the last then quantizes its share
    //     of the tokens (late, so that no logit waits for it) and leaves;
    //     the last does its share after the top-k and the bucketing.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    const int ngroups = (gridDim.x + kRouteGroup - 1) / kRouteGroup;
    if (tid == 0) {
        const int g = blockIdx.x / kRouteGroup;
        const unsigned gsize = (unsigned)min(kRouteGroup, (int)gridDim.x - g * kRouteGroup);
        bool last = false;
        if (__hip_atomic_fetch_add(a.cnt + kRouteCntStride * g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            gsize - 1)
            last = __hip_atomic_fetch_add(a.cnt + kRouteCntStride * kRouteMaxGroups, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == (unsigned)ngroups - 1;
        s_last = last;
    }
    __syncthreads();
    if (!s_last) {
        route_quant(a, blockIdx.x, gridDim.x, 4, wave, lane);
        return;
    }

    // (3) last workgroup: top-k, bucketing, counter reset
    route_select(a, ngroups, s_idx);
    route_quant(a, blockIdx.x, gridDim.x, 4, wave, lane);
}

// A gate tile, the matching up tile and, for two or more columns, the
// activation slice for the matrix-core dots (one column keeps the
// scalar-operand v_dot4 path).
template <int FG, int NE>
struct GUTile {
    TileRegs<FG> g, u;
    XTileM<NE> x;
};

template <int FG, int NE>
__device__ __forceinline__ GUTile<FG, NE> load_gu(const uint8_t *gm, const uint8_t *um, int s, int nbH,
                                                  const XCols<NE> &xc, int lane)
{
    GUTile<FG, NE> t;
    if (NE >= 2)
        t.x = load_xtile_m<FG, NE, false>(xc, s, nbH, lane);
    t.g = load_tile<FG>(gm + (size_t)s * TileFmt<FG>::bytes, lane);
    t.u = load_tile<FG>(um + (size_t)s * TileFmt<FG>::bytes, lane);
    return t;
}

template <int FG, int NE>
__device__ __forceinline__ void gateup_tile(const GUTile<FG, NE> &t, int s, int nbH, const XCols<NE> &xc,
                                            float (&ag)[NE], float (&au)[NE])
{
    if (NE >= 2)
        tile_blocks2_mfma<FG, NE, false>(t.g, t.u, t.x, s * 8, nbH, ag, au);
    else
        tile_blocks2<FG, FG, NE, false>(t.g, t.u, s * 8, nbH, xc, ag, au);
}


template <int FG, int NE>
__device__ void gateup_body(const FfnArgs &a, const SlotInfo &si, int g, int lane, int wave, int W,
                            float *red, const int *pairs_lds)
{
    constexpr int FU = FG;
    const SlotCols<NE> cols = slot_cols<NE>(si, a, pairs_lds);
    const int nbH = a.H / 32;
    uint32_t goff[NE], moff[NE];
#pragma unroll
    for (int j = 0; j < NE; j++) {
        goff[j] = (uint32_t)cols.token[j] * (uint32_t)a.H;
        moff[j] = (uint32_t)cols.token[j] * (uint32_t)nbH;
    }
    XCols<NE> xc;
    xc.xq = a.xq;
    xc.xs = a.xs;
    xc.xsum = a.xsum;
#pragma unroll
    for (int j = 0; j < NE; j++) {
        xc.xoff[j] = goff[j];
        xc.moff[j] = moff[j];
    }
    const int S = (a.H + 255) / 256;
    const uint8_t *gm, *um;
    if (si.kind == 2) {
        gm = a.sh_gate;
        um = a.sh_up;
    } else {
        gm = expert_mat(a, 0, si.expert);
        um = expert_mat(a, 1, si.expert);
    }
    gm += (size_t)g * S * TileFmt<FG>::bytes;
    um += (size_t)g * S * TileFmt<FU>::bytes;
    static_assert(FU == FG, "gate and up share a format");
    float ag[NE], au[NE];
#pragma unroll
    for (int j = 0; j < NE; j++) {
        ag[j] = 0.0f;
        au[j] = 0.0f;
    }
    const int s_begin = __builtin_amdgcn_readfirstlane((int)((unsigned)(S * wave) / (unsigned)W));
    const int s_end = __builtin_amdgcn_readfirstlane((int)((unsigned)(S * (wave + 1)) / (unsigned)W));
    // two buffers per stream used in turn: tile s + 1 in flight while s is
    // computed, with no register copies (which would wait for the loads).
    // FP4 tiles take one buffer: their registers set the kernel's budget,
    // and two would halve the workgroups resident per CU.
    if (FG == RFX_FP4) {
        for (int s = s_begin; s < s_end; s++) {
            const GUTile<FG, NE> t = load_gu<FG, NE>(gm, um, s, nbH, xc, lane);
            gateup_tile<FG, NE>(t, s, nbH, xc, ag, au);
        }
    } else if (s_end - s_begin == 1) {
        const GUTile<FG, NE> t = load_gu<FG, NE>(gm, um, s_begin, nbH, xc, lane);
        gateup_tile<FG, NE>(t, s_begin, nbH, xc, ag, au);
    } else if (s_begin < s_end) {
        // every load is issued on every path, so the wait for a tile's
        // first chunk leaves the next tile's loads in flight (with them
        // under a branch, the compiler waited for those too); an odd count
        // of three or more re-reads its last tile once
        GUTile<FG, NE> ta = load_gu<FG, NE>(gm, um, s_begin, nbH, xc, lane), tb;
        int s = s_begin;
        for (; s + 2 < s_end; s += 2) {
            tb = load_gu<FG, NE>(gm, um, s + 1, nbH, xc, lane);
            gateup_tile<FG, NE>(ta, s, nbH, xc, ag, au);
            ta = load_gu<FG, NE>(gm, um, s + 2, nbH, xc, lane);
            gateup_tile<FG, NE>(tb, s + 1, nbH, xc, ag, au);
        }
        tb = load_gu<FG, NE>(gm, um, min(s + 1, s_end - 1), nbH, xc, lane);
        gateup_tile<FG, NE>(ta, s, nbH, xc, ag, au);
        if (s + 1 < s_end)
            gateup_tile<FG, NE>(tb, s + 1, nbH, xc, ag, au);
    }
    // fixed-order reduction over waves; red[w][m][j][row], m = gate/up
#pragma unroll
    for (int j = 0; j < NE; j++) {
        red[((wave * 2 + 0) * kMaxDecodeQ + j) * 64 + lane] = ag[j];
        red[((wave * 2 + 1) * kMaxDecodeQ + j) * 64 + lane] = au[j];
    }
    __syncthreads();
    if (wave == 0)
        gateup_finish<NE>(a, cols, g, lane, W, red);
}

// FP4 gate and up on the block-scaled matrix core (rfx_mx4.h), one column
// pair per two tokens: both matrices' products take the same activation
// operand, built once per (half, column pair). Same tile split, reduction and
// epilogue as gateup_body. SINGLE: one tile buffer (see gateup_body).
template <int NE, bool SINGLE = true>
__device__ void gateup_body_mx(const FfnArgs &a, const SlotInfo &si, int g, int lane, int wave, int W, float *red,
                               const int *pairs_lds)
{
    constexpr int TB = TileFmt<RFX_FP4>::bytes;
    const SlotCols<NE> cols = slot_cols<NE>(si, a, pairs_lds);
    const int nbH = a.H / 32;
    XCols<NE> xc;
    xc.xq = a.xq;
    xc.xs = a.xs;
    xc.xsum = a.xsum;
#pragma unroll
    for (int j = 0; j < NE; j++) {
        xc.xoff[j] = (uint32_t)cols.token[j] * (uint32_t)a.H;
        xc.moff[j] = (uint32_t)cols.token[j] * (uint32_t)nbH;
    }
    const int S = (a.H + 255) / 256;
    const uint8_t *gm, *um;
    if (si.kind == 2) {
        gm = a.sh_gate;
        um = a.sh_up;
    } else {
        gm = expert_mat(a, 0, si.expert);
        um = expert_mat(a, 1, si.expert);
    }
    gm += (size_t)g * S * TB;
    um += (size_t)g * S * TB;
    const MxLane<NE> ml = mx_lane<NE>(lane, xc);
    float acc[2][4][4];
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int v = 0; v < 4; v++)
                acc[m][i][v] = 0.0f;
    const int s_begin = __builtin_amdgcn_readfirstlane((int)((unsigned)(S * wave) / (unsigned)W));
    const int s_end = __builtin_amdgcn_readfirstlane((int)((unsigned)(S * (wave + 1)) / (unsigned)W));
    if (SINGLE) {
        for (int s = s_begin; s < s_end; s++) {
            const MxX<NE> x = load_mx_x<NE, false>(s, nbH, xc, ml);
            MxW w[2];
            w[0] = load_mx_w(gm + (size_t)s * TB, lane);
            w[1] = load_mx_w(um + (size_t)s * TB, lane);
            compute_mx<NE, 2>(w, x, ml, acc);
        }
    } else if (s_begin < s_end) {
        // two buffers used in turn: tile s + 1 in flight while s is computed
        MxW wa[2], wb[2];
        MxX<NE> xa = load_mx_x<NE, false>(s_begin, nbH, xc, ml), xb;
        wa[0] = load_mx_w(gm + (size_t)s_begin * TB, lane);
        wa[1] = load_mx_w(um + (size_t)s_begin * TB, lane);
        for (int s = s_begin; s < s_end; s += 2) {
            if (s + 1 < s_end) {
                xb = load_mx_x<NE, false>(s + 1, nbH, xc, ml);
                wb[0] = load_mx_w(gm + (size_t)(s + 1) * TB, lane);
                wb[1] = load_mx_w(um + (size_t)(s + 1) * TB, lane);
            }
            compute_mx<NE, 2>(wa, xa, ml, acc);
            if (s + 1 >= s_end)
                break;
            if (s + 2 < s_end) {
                xa = load_mx_x<NE, false>(s + 2, nbH, xc, ml);
                wa[0] = load_mx_w(gm + (size_t)(s + 2) * TB, lane);
                wa[1] = load_mx_w(um + (size_t)(s + 2) * TB, lane);
            }
            compute_mx<NE, 2>(wb, xb, ml, acc);
        }
    }
#pragma unroll
    for (int m = 0; m < 2; m++)
        mx_rows<NE>(acc[m], lane, [&](int col, int row, float v) {
            red[((wave * 2 + m) * kMaxDecodeQ + col) * 64 + row] = v;
        });
    __syncthreads();
    if (wave == 0)
        gateup_finish<NE>(a, cols, g, lane, W, red);
}

// ROUTE: the workgroups of routed slots pick the top k from the router
// logits themselves (wg_route) and row group 0 of slot 1 writes the
// routing outputs; the shared expert's workgroups (slot 0) need no routing
// and start on their weights at once.
template <int FG, int FS, bool ROUTE>
__global__ __launch_bounds__(512) void gateup_kernel(FfnArgs a, RouteOut ro)
{
    __shared__ float red[8 * 2 * kMaxDecodeQ * 64];
    __shared__ RouteLds s_route;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    const int *pl = nullptr;
    const int slot = blockIdx.y;
    SlotInfo si;
    if (ROUTE && a.has_shared && slot == 0) {
        si = SlotInfo{2, -1, 0, 0, 0};
    } else {
        if (ROUTE) {
            wg_route(ro, a.q, a.k, a.E, blockIdx.x == 0 && slot == (a.has_shared ? 1 : 0), s_route);
            pl = s_route.pairs;
        }
        si = find_slot(slot, ROUTE ? s_route.eoff : a.expert_off, a.E, a.has_shared);
    }
    if (si.kind == 0)
        return;
    const int ne = si.kind == 2 ? a.q : si.pe - si.pb;
    // FP4 on the block-scaled matrix core: the shared expert (every token,
    // the heaviest slot, whose workgroups share CUs with routed ones) at
    // any token count, routed slots with one or two tokens
    if (si.kind == 2) {
        switch (ne) {
        case 1:
            if constexpr (FS == RFX_FP4)
                gateup_body_mx<1>(a, si, blockIdx.x, lane, wave, W, red, pl);
            else
                gateup_body<FS, 1>(a, si, blockIdx.x, lane, wave, W, red, pl);
            break;
        case 2:
            if constexpr (FS == RFX_FP4)
                gateup_body_mx<2>(a, si, blockIdx.x, lane, wave, W, red, pl);
            else
                gateup_body<FS, 2>(a, si, blockIdx.x, lane, wave, W, red, pl);
            break;
        case 3:
            if constexpr (FS == RFX_FP4)
                gateup_body_mx<3>(a, si, blockIdx.x, lane, wave, W, red, pl);
            else
                gateup_body<FS, 3>(a, si, blockIdx.x, lane, wave, W, red, pl);
            break;
        case 4:
            if constexpr (FS == RFX_FP4)
                gateup_body_mx<4>(a, si, blockIdx.x, lane, wave, W, red, pl);
            else
                gateup_body<FS, 4>(a, si, blockIdx.x, lane, wave, W, red, pl);
            break;
        default: break;
        }
    } else {
        switch (ne) {
        case 1:
            if constexpr (FG == RFX_FP4)
                gateup_body_mx<1>(a, si, blockIdx.x, lane, wave, W, red, pl);
            else
                gateup_body<FG, 1>(a, si, blockIdx.x, lane, wave, W, red, pl);
            break;
        case 2:
            if constexpr (FG == RFX_FP4)
                gateup_body_mx<2>(a, si, blockIdx.x, lane, wave, W, red, pl);
            else
                gateup_body<FG, 2>(a, si, blockIdx.x, lane, wave, W, red, pl);
            break;
        case 3: gateup_body<FG, 3>(a, si, blockIdx.x, lane, wave, W, red, pl); break;
        case 4: gateup_body<FG, 4>(a, si, blockIdx.x, lane, wave, W, red, pl); break;
        default: break;
        }
    }
}

// ------------------------------------------------------------------
// Expert down projection, shared expert and the weighted combine.
// ------------------------------------------------------------------
// MF: one-token slots take the matrix-core dots too (the same exact
// integers and fp32 sums as the scalar-operand path). Chosen per call: in
// calls with two or more tokens most routed slots have one, and the matrix
// core measured 1.6 us faster per q = 4 top-6 layer; at q = 1 the
// scalar-operand path measured 2 us faster per 8-layer step.
template <int FD, int NE>
struct DTile {
    TileRegs<FD> w;
    XTileM<NE> x;
};

template <int FD, int NE, bool MF>
__device__ __forceinline__ DTile<FD, NE> load_dn(const uint8_t *dm, int s, int nbI, const XCols<NE> &xc, int lane)
{
    DTile<FD, NE> t;
    if (NE >= 2 || MF)
        t.x = load_xtile_m<FD, NE, false>(xc, s, nbI, lane);
    t.w = load_tile<FD>(dm + (size_t)s * TileFmt<FD>::bytes, lane);
    return t;
}

template <int FD, int NE, bool MF>
__device__ __forceinline__ void down_tile(const DTile<FD, NE> &t, int s, int nbI, const XCols<NE> &xc,
                                          float (&ao)[NE])
{
    if (NE >= 2 || MF)
        tile_blocks_mfma<FD, NE, false>(t.w, t.x, s * 8, nbI, ao);
    else
        tile_blocks<FD, NE, NE, false>(t.w, s * 8, nbI, xc, ao);
}


template <int FD, int NE, bool MF = false>
__device__ void down_body(const FfnArgs &a, const SlotInfo &si, int g, int lane, int wave, int W, float *red)
{
    const SlotCols<NE> cols = slot_cols<NE>(si, a);
    const int nbI = a.I / 32;
    uint32_t goff[NE], moff[NE];
#pragma unroll
    for (int j = 0; j < NE; j++) {
        goff[j] = (uint32_t)cols.out_idx[j] * (uint32_t)a.I;
        moff[j] = (uint32_t)cols.out_idx[j] * (uint32_t)nbI;
    }
    XCols<NE> xc;
    xc.xq = a.ws.hq;
    xc.xs = a.ws.hs;
    xc.xsum = a.ws.hsum;
#pragma unroll
    for (int j = 0; j < NE; j++) {
        xc.xoff[j] = goff[j];
        xc.moff[j] = moff[j];
    }
    const int S = (a.I + 255) / 256;
    const uint8_t *dm = si.kind == 2 ? a.sh_down : expert_mat(a, 2, si.expert);
    dm += (size_t)g * S * TileFmt<FD>::bytes;
    float ao[NE];
#pragma unroll
    for (int j = 0; j < NE; j++)
        ao[j] = 0.0f;
    const int s_begin = __builtin_amdgcn_readfirstlane((int)((unsigned)(S * wave) / (unsigned)W));
    const int s_end = __builtin_amdgcn_readfirstlane((int)((unsigned)(S * (wave + 1)) / (unsigned)W));
    if (s_end - s_begin == 1) {
        const DTile<FD, NE> t = load_dn<FD, NE, MF>(dm, s_begin, nbI, xc, lane);
        down_tile<FD, NE, MF>(t, s_begin, nbI, xc, ao);
    } else if (s_begin < s_end) {
        // loads on every path, as in gateup_body
        DTile<FD, NE> da = load_dn<FD, NE, MF>(dm, s_begin, nbI, xc, lane), db;
        int s = s_begin;
        for (; s + 2 < s_end; s += 2) {
            db = load_dn<FD, NE, MF>(dm, s + 1, nbI, xc, lane);
            down_tile<FD, NE, MF>(da, s, nbI, xc, ao);
            da = load_dn<FD, NE, MF>(dm, s + 2, nbI, xc, lane);
            down_tile<FD, NE, MF>(db, s + 1, nbI, xc, ao);
        }
        db = load_dn<FD, NE, MF>(dm, min(s + 1, s_end - 1), nbI, xc, lane);
        down_tile<FD, NE, MF>(da, s, nbI, xc, ao);
        if (s + 1 < s_end)
            down_tile<FD, NE, MF>(db, s + 1, nbI, xc, ao);
    }
#pragma unroll
    for (int j = 0; j < NE; j++)
        red[(wave * kMaxDecodeQ + j) * 64 + lane] = ao[j];
    __syncthreads();
    if (wave == 0)
        down_finish<NE>(a, cols, g, lane, W, red);
}

// FP4 down with one or two tokens on the block-scaled matrix core
// (rfx_mx4.h), one tile at a time (a workgroup of up to 1024 threads has
// 128 registers per lane, and the waves mostly get one tile each).
template <int NE>
__device__ void down_body_mx(const FfnArgs &a, const SlotInfo &si, int g, int lane, int wave, int W, float *red)
{
    constexpr int TB = TileFmt<RFX_FP4>::bytes;
    const SlotCols<NE> cols = slot_cols<NE>(si, a);
    const int nbI = a.I / 32;
    XCols<NE> xc;
    xc.xq = a.ws.hq;
    xc.xs = a.ws.hs;
    xc.xsum = a.ws.hsum;
#pragma unroll
    for (int j = 0; j < NE; j++) {
        xc.xoff[j] = (uint32_t)cols.out_idx[j] * (uint32_t)a.I;
        xc.moff[j] = (uint32_t)cols.out_idx[j] * (uint32_t)nbI;
    }
    const int S = (a.I + 255) / 256;
    const uint8_t *dm = si.kind == 2 ? a.sh_down : expert_mat(a, 2, si.expert);
    dm += (size_t)g * S * TB;
    const MxLane<NE> ml = mx_lane<NE>(lane, xc);
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int v = 0; v < 4; v++)
            acc[i][v] = 0.0f;
    const int s_begin = __builtin_amdgcn_readfirstlane((int)((unsigned)(S * wave) / (unsigned)W));
    const int s_end = __builtin_amdgcn_readfirstlane((int)((unsigned)(S * (wave + 1)) / (unsigned)W));
    for (int s = s_begin; s < s_end; s++) {
        const MxTile<NE> t = load_mx_tile<NE, false>(dm + (size_t)s * TB, s, nbI, lane, xc, ml);
        compute_mx_tile<NE>(t, ml, acc);
    }
    mx_rows<NE>(acc, lane, [&](int col, int row, float v) { red[(wave * kMaxDecodeQ + col) * 64 + row] = v; });
    __syncthreads();
    if (wave == 0)
        down_finish<NE>(a, cols, g, lane, W, red);
}

template <int FD, int FSD>
__global__ __launch_bounds__(1024) void down_kernel(FfnArgs a)
{
    __shared__ float red[16 * kMaxDecodeQ * 64];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    const int g = blockIdx.x;
    const SlotInfo si = find_slot(blockIdx.y, a.expert_off, a.E, a.has_shared);
    if (si.kind == 0)
        return;
    const int ne = si.kind == 2 ? a.q : si.pe - si.pb;
    // FP4 with one or two tokens on the block-scaled matrix core (for the
    // shared expert's three or four tokens it measured no faster here)
    if (si.kind == 2) {
        switch (ne) {
        case 1:
            if constexpr (FSD == RFX_FP4)
                down_body_mx<1>(a, si, g, lane, wave, W, red);
            else if (a.q >= 2)
                down_body<FSD, 1, true>(a, si, g, lane, wave, W, red);
            else
                down_body<FSD, 1>(a, si, g, lane, wave, W, red);
            break;
        case 2:
            if constexpr (FSD == RFX_FP4)
                down_body_mx<2>(a, si, g, lane, wave, W, red);
            else
                down_body<FSD, 2>(a, si, g, lane, wave, W, red);
            break;
        case 3: down_body<FSD, 3>(a, si, g, lane, wave, W, red); break;
        case 4: down_body<FSD, 4>(a, si, g, lane, wave, W, red); break;
        default: break;
        }
    } else {
        switch (ne) {
        case 1:
            if constexpr (FD == RFX_FP4)
                down_body_mx<1>(a, si, g, lane, wave, W, red);
            else if (a.q >= 2)
                down_body<FD, 1, true>(a, si, g, lane, wave, W, red);
            else
                down_body<FD, 1>(a, si, g, lane, wave, W, red);
            break;
        case 2:
            if constexpr (FD == RFX_FP4)
                down_body_mx<2>(a, si, g, lane, wave, W, red);
            else
                down_body<FD, 2>(a, si, g, lane, wave, W, red);
            break;
        case 3: down_body<FD, 3>(a, si, g, lane, wave, W, red); break;
        case 4: down_body<FD, 4>(a, si, g, lane, wave, W, red); break;
        default: break;
        }
    }
    // Last slot to finish this row group combines, in fixed slot order:
    // y[t] = o_shared[t] + sum_j w[t][j] * o[t*k + j].
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    __shared__ int s_last;
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(a.ws.comb_cnt + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (unsigned)(si.n_slots - 1);
    __syncthreads();
    if (!s_last)
        return;
    if (wave == 0)
        combine_rows(a, g, lane);
    if (threadIdx.x == 0)
        __hip_atomic_store(a.ws.comb_cnt + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------
// Host-side helpers.
// ------------------------------------------------------------------
int check_layer(const rfx_moe_layer *L)
{
    if (!L)
        return fail(RFX_E_INVAL, "MoE layer descriptor is NULL");
    if (L->n_experts < 1 || L->n_experts > kMaxE)
        return fail(RFX_E_INVAL, "n_experts=%d (must be 1..%d)", L->n_experts, kMaxE);
    if (L->hidden < 32 || L->hidden % 32 || L->inter < 32 || L->inter % 32)
        return fail(RFX_E_INVAL, "hidden=%d inter=%d must be positive multiples of 32", L->hidden, L->inter);
    int st;
    const bool placed = L->expert_data != nullptr;
    if ((st = check_qmat(&L->gate, "gate", true, placed)) || (st = check_qmat(&L->up, "up", true, placed)) ||
        (st = check_qmat(&L->down, "down", true, placed)))
        return st;
    if (placed && (st = check_ptr(L->expert_data, 8, "expert_data")))
        return st;
    if (L->gate.rows != L->inter || L->gate.cols != L->hidden || L->up.rows != L->inter ||
        L->up.cols != L->hidden || L->down.rows != L->hidden || L->down.cols != L->inter)
        return fail(RFX_E_INVAL, "expert matrix shapes do not match hidden=%d inter=%d", L->hidden, L->inter);
    if (L->gate.fmt != L->up.fmt)
        return fail(RFX_E_UNSUPPORTED, "gate and up must share a block format (fused gate/up kernel)");
    for (const rfx_qmat *m : {&L->gate, &L->up, &L->down, &L->sh_gate, &L->sh_up, &L->sh_down})
        if (m->data && (m->fmt == RFX_FP2M || m->fmt == RFX_Q8 || m->fmt == RFX_FP2S || m->fmt == RFX_FP3E))
            return fail(RFX_E_UNSUPPORTED,
                        "the FP2M, FP2S, FP3E and Q8 formats are supported by the GEMV entry points only");
    if (L->sh_gate.data && L->sh_gate.fmt != L->sh_up.fmt)
        return fail(RFX_E_UNSUPPORTED, "shared gate and up must share a block format");
    if (L->gate.count != L->n_experts || L->up.count != L->n_experts || L->down.count != L->n_experts)
        return fail(RFX_E_INVAL, "expert stacks must hold n_experts=%d matrices", L->n_experts);
    if (L->sh_gate.data) {
        if ((st = check_qmat(&L->sh_gate, "sh_gate", false)) || (st = check_qmat(&L->sh_up, "sh_up", false)) ||
            (st = check_qmat(&L->sh_down, "sh_down", false)))
            return st;
        if (L->sh_gate.rows != L->inter || L->sh_gate.cols != L->hidden || L->sh_up.rows != L->inter ||
            L->sh_up.cols != L->hidden || L->sh_down.rows != L->hidden || L->sh_down.cols != L->inter)
            return fail(RFX_E_INVAL, "shared expert shapes do not match hidden/inter");
    }
    return check_ptr(L->router_w, 16, "router_w");
}

template <int FG, bool ROUTE>
int launch_gateup(int fs, const FfnArgs &a, const RouteOut &ro, dim3 grid, dim3 block, hipStream_t st)
{
    const size_t lds = 0;
    switch (fs) {
    case RFX_FP2: hipLaunchKernelGGL((gateup_kernel<FG, RFX_FP2, ROUTE>), grid, block, lds, st, a, ro); break;
    case RFX_FP3: hipLaunchKernelGGL((gateup_kernel<FG, RFX_FP3, ROUTE>), grid, block, lds, st, a, ro); break;
    case RFX_FP4: hipLaunchKernelGGL((gateup_kernel<FG, RFX_FP4, ROUTE>), grid, block, lds, st, a, ro); break;
    }
    return hip_status("gate/up launch");
}

template <int FD>
int launch_down(int fsd, const FfnArgs &a, dim3 grid, dim3 block, hipStream_t st)
{
    const size_t lds = 0;
    switch (fsd) {
    case RFX_FP2: hipLaunchKernelGGL((down_kernel<FD, RFX_FP2>), grid, block, lds, st, a); break;
    case RFX_FP3: hipLaunchKernelGGL((down_kernel<FD, RFX_FP3>), grid, block, lds, st, a); break;
    case RFX_FP4: hipLaunchKernelGGL((down_kernel<FD, RFX_FP4>), grid, block, lds, st, a); break;
    }
    return hip_status("down launch");
}

// Compute units of the current device (cached per device).
int device_cus()
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

// The decode FFN (q <= 4): gate/up then down. ro: the gate/up workgroups
// route from these logits themselves (and write the routing outputs), else
// the routing comes in a's inputs.
int decode_ffn(const rfx_moe_layer *L, const FfnArgs &a, const RouteOut *ro, hipStream_t s)
{
    int st = RFX_OK;
    const int q = a.q, k = a.k;
    const int max_slots = (q * k < L->n_experts ? q * k : L->n_experts) + (a.has_shared ? 1 : 0);
    const int GI = (int)ceil_div(L->inter, 64), GH = (int)ceil_div(L->hidden, 64);
    const int SH = (int)ceil_div(L->hidden, 256), SI = (int)ceil_div(L->inter, 256);
    {
        const int W = waves_for(max_slots * GI, SH, kMaxFfnWaves, kGateUpWaveTarget);
        dim3 grid(GI, max_slots), block(64 * W);
        const RouteOut r = ro ? *ro : RouteOut{};
        switch (a.fmt_g) {
        case RFX_FP2:
            st = ro ? launch_gateup<RFX_FP2, true>(a.fmt_sg, a, r, grid, block, s)
                    : launch_gateup<RFX_FP2, false>(a.fmt_sg, a, r, grid, block, s);
            break;
        case RFX_FP3:
            st = ro ? launch_gateup<RFX_FP3, true>(a.fmt_sg, a, r, grid, block, s)
                    : launch_gateup<RFX_FP3, false>(a.fmt_sg, a, r, grid, block, s);
            break;
        case RFX_FP4:
            st = ro ? launch_gateup<RFX_FP4, true>(a.fmt_sg, a, r, grid, block, s)
                    : launch_gateup<RFX_FP4, false>(a.fmt_sg, a, r, grid, block, s);
            break;
        }
        if (st)
            return st;
    }
    {
        const int W = waves_for(max_slots * GH, SI, kMaxFfnWaves, kDownWaveTarget);
        dim3 grid(GH, max_slots), block(64 * W);
        switch (a.fmt_d) {
        case RFX_FP2: st = launch_down<RFX_FP2>(a.fmt_sd, a, grid, block, s); break;
        case RFX_FP3: st = launch_down<RFX_FP3>(a.fmt_sd, a, grid, block, s); break;
        case RFX_FP4: st = launch_down<RFX_FP4>(a.fmt_sd, a, grid, block, s); break;
        }
    }
    return st;
}

RouteArgs make_route_args(const rfx_moe_layer *L, const float *x, int q, int k, int32_t *topk_idx, float *topk_w,
                          int32_t *pairs_sorted, int32_t *expert_off, int8_t *xq, float *xs, int32_t *xsum,
                          const MoeWs &w)
{
    RouteArgs a{};
    a.x = x;
    a.wr = L->router_w;
    a.wb = L->router_b;
    a.q = q;
    a.k = k;
    a.E = L->n_experts;
    a.H = L->hidden;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.pairs_sorted = pairs_sorted;
    a.expert_off = expert_off;
    a.xq = xq;
    a.xs = xs;
    a.xsum = xsum;
    a.logits = w.logits;
    a.cnt = w.route_cnt;
    return a;
}

FfnArgs make_ffn_args(const rfx_moe_layer *L, int q, int k, const int8_t *xq, const float *xs, const int32_t *xsum,
                      const int32_t *topk_idx, const float *topk_w, const int32_t *pairs_sorted,
                      const int32_t *expert_off, const float *resid, float *y, const MoeWs &w)
{
    FfnArgs a{};
    a.gate = static_cast<const uint8_t *>(L->gate.data);
    a.up = static_cast<const uint8_t *>(L->up.data);
    a.down = static_cast<const uint8_t *>(L->down.data);
    a.gate_stride = (size_t)rfx_qmat_bytes(L->gate.fmt, L->inter, L->hidden);
    a.up_stride = (size_t)rfx_qmat_bytes(L->up.fmt, L->inter, L->hidden);
    a.down_stride = (size_t)rfx_qmat_bytes(L->down.fmt, L->hidden, L->inter);
    a.has_shared = L->sh_gate.data != nullptr;
    a.sh_gate = static_cast<const uint8_t *>(L->sh_gate.data);
    a.sh_up = static_cast<const uint8_t *>(L->sh_up.data);
    a.sh_down = static_cast<const uint8_t *>(L->sh_down.data);
    a.fmt_g = L->gate.fmt;
    a.fmt_u = L->up.fmt;
    a.fmt_d = L->down.fmt;
    a.fmt_sg = a.has_shared ? L->sh_gate.fmt : L->gate.fmt;
    a.fmt_su = a.has_shared ? L->sh_up.fmt : L->up.fmt;
    a.fmt_sd = a.has_shared ? L->sh_down.fmt : L->down.fmt;
    a.E = L->n_experts;
    a.H = L->hidden;
    a.I = L->inter;
    a.q = q;
    a.k = k;
    a.xq = xq;
    a.xs = xs;
    a.xsum = xsum;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.pairs_sorted = pairs_sorted;
    a.expert_off = expert_off;
    a.resid = resid;
    a.y = y;
    a.ws = w;
    a.expert_data = L->expert_data;
    return a;
}

} // namespace

extern "C" {

size_t rfx_moe_workspace_bytes(const rfx_moe_layer *L, int q, int k)
{
    if (!L || q < 1 || k < 1 || L->n_experts < 1 || L->hidden < 32 || L->inter < 32)
        return 0;
    return carve(nullptr, q, k, L->n_experts, L->hidden, L->inter).bytes;
}

int rfx_moe_route_topk(const rfx_moe_layer *L, const float *x, int q, int k, int32_t *topk_idx,
                       float *topk_w, int32_t *pairs_sorted, int32_t *expert_off, int8_t *xq, float *xs,
                       int32_t *xsum, void *ws, size_t ws_bytes, void *stream)
{
    int st = check_layer(L);
    if (st)
        return st;
    if (k < 1 || k > kMaxK || k > L->n_experts)
        return fail(RFX_E_INVAL, "k=%d (must be 1..%d and <= n_experts)", k, kMaxK);
    if (q < 1)
        return fail(RFX_E_INVAL, "q=%d", q);
    if (q > kMaxPrefillQ)
        return fail(RFX_E_UNSUPPORTED, "rfx_moe_route_topk: q=%d > %d", q, kMaxPrefillQ);
    if ((st = check_ptr(x, 16, "x")) || (st = check_ptr(topk_idx, 4, "topk_idx")) ||
        (st = check_ptr(topk_w, 4, "topk_w")) || (st = check_ptr(pairs_sorted, 4, "pairs_sorted")) ||
        (st = check_ptr(expert_off, 4, "expert_off")) || (st = check_ptr(xq, 16, "xq")) ||
        (st = check_ptr(xs, 4, "xs")) || (st = check_ptr(xsum, 4, "xsum")) || (st = check_ptr(ws, 256, "ws")))
        return st;
    if (L->router_b && (st = check_ptr(L->router_b, 4, "router_b")))
        return st;
    MoeWs w = carve(ws, q, k, L->n_experts, L->hidden, L->inter);
    if (ws_bytes < w.bytes)
        return fail(RFX_E_WORKSPACE, "MoE workspace %zu < %zu bytes", ws_bytes, w.bytes);
    if (q > kMaxDecodeQ) // many tokens: the prefill router and bucketing
        return prefill_route(L, x, q, k, topk_idx, topk_w, pairs_sorted, expert_off, xq, xs, xsum, w,
                             (hipStream_t)stream);
    const RouteArgs a = make_route_args(L, x, q, k, topk_idx, topk_w, pairs_sorted, expert_off, xq, xs, xsum, w);
    if (L->hidden > 8192) // one workgroup reads a row as 8 float4 per thread
        return fail(RFX_E_UNSUPPORTED, "router: hidden=%d > 8192 for q <= 4", L->hidden);
    const int grid = L->n_experts; // one workgroup per expert row
    hipLaunchKernelGGL(route_kernel<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream, a);
    return hip_status("route launch");
}

int rfx_moe_ffn(const rfx_moe_layer *L, int q, int k, const int8_t *xq, const float *xs, const int32_t *xsum,
                const int32_t *topk_idx, const float *topk_w, const int32_t *pairs_sorted,
                const int32_t *expert_off, const float *resid, float *y, void *ws, size_t ws_bytes,
                void *stream)
{
    int st = check_layer(L);
    if (st)
        return st;
    if (k < 1 || k > kMaxK || k > L->n_experts || q < 1)
        return fail(RFX_E_INVAL, "q=%d k=%d", q, k);
    if (q > kMaxPrefillQ)
        return fail(RFX_E_UNSUPPORTED, "rfx_moe_ffn: q=%d > %d", q, kMaxPrefillQ);
    if ((st = check_ptr(xq, 16, "xq")) || (st = check_ptr(xs, 4, "xs")) || (st = check_ptr(xsum, 4, "xsum")) ||
        (st = check_ptr(topk_idx, 4, "topk_idx")) || (st = check_ptr(topk_w, 4, "topk_w")) ||
        (st = check_ptr(pairs_sorted, 4, "pairs_sorted")) || (st = check_ptr(expert_off, 4, "expert_off")) ||
        (st = check_ptr(y, 4, "y")) || (st = check_ptr(ws, 256, "ws")))
        return st;
    MoeWs w = carve(ws, q, k, L->n_experts, L->hidden, L->inter);
    if (ws_bytes < w.bytes)
        return fail(RFX_E_WORKSPACE, "MoE workspace %zu < %zu bytes", ws_bytes, w.bytes);
    if (resid && (st = check_ptr(resid, 16, "resid")))
        return st;
    if (q > kMaxDecodeQ) // many tokens: grouped matrix-core path
        return prefill_ffn(L, q, k, xq, xs, topk_w, pairs_sorted, expert_off, resid, y, w, (hipStream_t)stream);
    const FfnArgs a = make_ffn_args(L, q, k, xq, xs, xsum, topk_idx, topk_w, pairs_sorted, expert_off, resid, y, w);
    return decode_ffn(L, a, nullptr, (hipStream_t)stream);
}

int rfx_moe_forward(const rfx_moe_layer *L, const float *x, int q, int k, const float *resid, float *y,
                    int32_t *topk_idx, float *topk_w, int32_t *pairs_sorted, int32_t *expert_off, int8_t *xq,
                    float *xs, int32_t *xsum, void *ws, size_t ws_bytes, unsigned flags, void *stream)
{
    int st = check_layer(L);
    if (st)
        return st;
    if (k < 1 || k > kMaxK || k > L->n_experts || q < 1)
        return fail(RFX_E_INVAL, "q=%d k=%d (k must be 1..%d and <= n_experts)", q, k, kMaxK);
    if (q > kMaxPrefillQ)
        return fail(RFX_E_UNSUPPORTED, "rfx_moe_forward: q=%d > %d", q, kMaxPrefillQ);
    if (flags & ~(unsigned)RFX_FORWARD_ONE_LAUNCH)
        return fail(RFX_E_INVAL, "rfx_moe_forward: unknown flags 0x%x", flags);
    if ((st = check_ptr(x, 16, "x")) || (st = check_ptr(y, 4, "y")) || (st = check_ptr(topk_idx, 4, "topk_idx")) ||
        (st = check_ptr(topk_w, 4, "topk_w")) || (st = check_ptr(pairs_sorted, 4, "pairs_sorted")) ||
        (st = check_ptr(expert_off, 4, "expert_off")) || (st = check_ptr(xq, 16, "xq")) ||
        (st = check_ptr(xs, 4, "xs")) || (st = check_ptr(xsum, 4, "xsum")) || (st = check_ptr(ws, 256, "ws")))
        return st;
    if (L->router_b && (st = check_ptr(L->router_b, 4, "router_b")))
        return st;
    if (resid && (st = check_ptr(resid, 16, "resid")))
        return st;
    const MoeWs w = carve(ws, q, k, L->n_experts, L->hidden, L->inter);
    if (ws_bytes < w.bytes)
        return fail(RFX_E_WORKSPACE, "MoE workspace %zu < %zu bytes", ws_bytes, w.bytes);
    const FfnArgs fa = make_ffn_args(L, q, k, xq, xs, xsum, topk_idx, topk_w, pairs_sorted, expert_off, resid, y, w);
    const RouteArgs ra = make_route_args(L, x, q, k, topk_idx, topk_w, pairs_sorted, expert_off, xq, xs, xsum, w);
    if ((flags & RFX_FORWARD_ONE_LAUNCH) && layer_kernel_takes(fa, q, k))
        return launch_layer(fa, ra, (hipStream_t)stream);
    // Routing inside the gate/up workgroups costs each of them the top-k
    // selection (~2 us before its weights start to stream), which pays for
    // the router launch's arrival phase only when the gate/up grid runs in
    // one round of one workgroup per compute unit (measured at q = 1 top-4:
    // 28.2 against 29.4 us per layer; at q = 4 the workgroups run in
    // several rounds per CU, each paying the selection again).
    const int gu_wgs = (int)ceil_div(L->inter, 64) * ((q * k < L->n_experts ? q * k : L->n_experts) +
                                                      (fa.has_shared ? 1 : 0));
    if (q > kMaxDecodeQ || L->hidden > 8192 || gu_wgs > device_cus()) {
        if ((st = rfx_moe_route_topk(L, x, q, k, topk_idx, topk_w, pairs_sorted, expert_off, xq, xs, xsum, ws,
                                     ws_bytes, stream)))
            return st;
        return rfx_moe_ffn(L, q, k, xq, xs, xsum, topk_idx, topk_w, pairs_sorted, expert_off, resid, y, ws, ws_bytes,
                           stream);
    }
    // the router launch computes the logits and quantizes x, and every
    // routed gate/up workgroup picks the top k from the logits
    hipLaunchKernelGGL(route_kernel<false>, dim3(L->n_experts), dim3(256), 0, (hipStream_t)stream, ra);
    if ((st = hip_status("route launch")))
        return st;
    const RouteOut ro{w.logits, topk_idx, topk_w, pairs_sorted, expert_off};
    return decode_ffn(L, fa, &ro, (hipStream_t)stream);
}

int rfx_moe_forward_single_launch(const rfx_moe_layer *L, int q, int k)
{
    int st = check_layer(L);
    if (st)
        return st;
    if (k < 1 || k > kMaxK || k > L->n_experts || q < 1)
        return fail(RFX_E_INVAL, "q=%d k=%d", q, k);
    const MoeWs w = carve(nullptr, q, k, L->n_experts, L->hidden, L->inter);
    const FfnArgs fa = make_ffn_args(L, q, k, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, w);
    return layer_kernel_takes(fa, q, k) ? 1 : 0;
}

int rfx_moe_forward_status(const rfx_moe_layer *L, int q, int k, void *ws, size_t ws_bytes, void *stream)
{
    int st = check_layer(L);
    if (st)
        return st;
    if (k < 1 || k > kMaxK || q < 1)
        return fail(RFX_E_INVAL, "q=%d k=%d", q, k);
    if ((st = check_ptr(ws, 256, "ws")))
        return st;
    const MoeWs w = carve(ws, q, k, L->n_experts, L->hidden, L->inter);
    if (ws_bytes < w.bytes)
        return fail(RFX_E_WORKSPACE, "MoE workspace %zu < %zu bytes", ws_bytes, w.bytes);
    unsigned *word = w.sync + kSyncErr * kSyncLine;
    unsigned err = 0;
    const hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(&err, word, sizeof(err), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return hip_status("rfx_moe_forward_status");
    if (!err)
        return RFX_OK;
    const unsigned zero = 0;
    if (hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return hip_status("rfx_moe_forward_status");
    return fail(RFX_E_TIMEOUT, "a bounded wait of the single-launch MoE layer kernel ran out; the outputs of that "
                               "call are undefined");
}

int rfx_moe_debug_hidden(const rfx_moe_layer *L, int q, int k, const void *ws, size_t ws_bytes, float *h,
                         int8_t *hq, float *hs, void *stream)
{
    int st = check_layer(L);
    if (st)
        return st;
    if (q < 1 || q > kMaxPrefillQ || k < 1 || k > kMaxK)
        return fail(RFX_E_INVAL, "q=%d k=%d", q, k);
    if (!ws)
        return fail(RFX_E_INVAL, "ws is NULL");
    if (h && q > kMaxDecodeQ)
        return fail(RFX_E_UNSUPPORTED, "rfx_moe_debug_hidden: h (fp32) is not kept for q > %d", kMaxDecodeQ);
    MoeWs w = carve(const_cast<void *>(ws), q, k, L->n_experts, L->hidden, L->inter);
    if (ws_bytes < w.bytes)
        return fail(RFX_E_WORKSPACE, "rfx_moe_debug_hidden: workspace %zu < %zu bytes for q=%d k=%d", ws_bytes,
                    w.bytes, q, k);
    const size_t NP = (size_t)q * k + q;
    const hipStream_t s = (hipStream_t)stream;
    if (h && hipMemcpyAsync(h, w.h, NP * L->inter * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return hip_status("debug copy h");
    if (hq && hipMemcpyAsync(hq, w.hq, NP * L->inter, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return hip_status("debug copy hq");
    if (hs && hipMemcpyAsync(hs, w.hs, NP * (L->inter / 32) * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return hip_status("debug copy hs");
    return RFX_OK;
}

int rfx_moe_debug_prefill(const rfx_moe_layer *L, int q, int k, const int8_t *xq, const float *xs,
                          const float *topk_w, const int32_t *pairs_sorted, const int32_t *expert_off, void *ws,
                          size_t ws_bytes, int probe_expert, int probe_first, float *h, int32_t *dots_gate,
                          int32_t *dots_up, int32_t *dots_down, void *stream)
{
    int st = check_layer(L);
    if (st)
        return st;
    if (q <= kMaxDecodeQ || q > kMaxPrefillQ || k < 1 || k > kMaxK || k > L->n_experts)
        return fail(RFX_E_INVAL, "rfx_moe_debug_prefill: q=%d k=%d (q must be %d..%d)", q, k, kMaxDecodeQ + 1,
                    kMaxPrefillQ);
    const bool has_shared = L->sh_gate.data != nullptr;
    if (probe_expert < 0 || probe_expert > L->n_experts || (probe_expert == L->n_experts && !has_shared) ||
        probe_first < 0 || probe_first % kPrefillChunk)
        return fail(RFX_E_INVAL, "rfx_moe_debug_prefill: probe (expert %d, first %d)", probe_expert, probe_first);
    if ((st = check_ptr(xq, 16, "xq")) || (st = check_ptr(xs, 4, "xs")) || (st = check_ptr(topk_w, 4, "topk_w")) ||
        (st = check_ptr(pairs_sorted, 4, "pairs_sorted")) || (st = check_ptr(expert_off, 4, "expert_off")) ||
        (st = check_ptr(ws, 256, "ws")))
        return st;
    if ((h && (st = check_ptr(h, 4, "h"))) || (dots_gate && (st = check_ptr(dots_gate, 4, "dots_gate"))) ||
        (dots_up && (st = check_ptr(dots_up, 4, "dots_up"))) ||
        (dots_down && (st = check_ptr(dots_down, 4, "dots_down"))))
        return st;
    MoeWs w = carve(ws, q, k, L->n_experts, L->hidden, L->inter);
    if (ws_bytes < w.bytes)
        return fail(RFX_E_WORKSPACE, "MoE workspace %zu < %zu bytes", ws_bytes, w.bytes);
    PrefillDebug dbg{};
    dbg.h = h;
    dbg.probe_expert = probe_expert;
    dbg.probe_first = probe_first;
    dbg.dots[0] = dots_gate;
    dbg.dots[1] = dots_up;
    dbg.dots[2] = dots_down;
    return prefill_ffn(L, q, k, xq, xs, topk_w, pairs_sorted, expert_off, nullptr, nullptr, w, (hipStream_t)stream,
                       &dbg);
}

} // extern "C"
