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
#include "rfx_moe_ws.h"
#include "rfx_mx4.h"
#include "rfx_xtile.h"

using namespace rfx;
using namespace rfx::dev;

namespace {

// ------------------------------------------------------------------
// Shared device helpers.
// ------------------------------------------------------------------

// Activation quantization of one 32-element block held by 32 lanes
// (lanes 0-31 or 32-63 of a wave): s = amax/127, code = clamp(rne(v/s)).
__device__ __forceinline__ void quant32(float v, int8_t *q_out, float *s_out, int32_t *sum_out,
                                        bool write_meta)
{
#pragma clang fp contract(off)
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
    *q_out = (int8_t)qv;
    if (write_meta) {
        *s_out = s;
        *sum_out = sum;
    }
}

// ------------------------------------------------------------------
// Router (decode: q <= 4 tokens).
// ------------------------------------------------------------------
struct RouteArgs {
    const float *x;  // [q][H]
    const float *wr; // [E][H]
    const float *wb; // [E] or null
    int q, k, E, H;
    int32_t *topk_idx;
    float *topk_w;
    int32_t *pairs_sorted;
    int32_t *expert_off;
    int8_t *xq;
    float *xs;
    int32_t *xsum;
    float *logits;
    unsigned *cnt;
};

// Wave-wide reductions through DPP row shifts and row broadcasts (no LDS
// traffic); the result is read from lane 63, where the prefix completes.
// Lanes a DPP step does not reach take the identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t identity, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROW_MASK, 0xF, false);
}

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, uint32_t identity, Op op)
{
    v = op(v, dpp_u32<0x111, 0xF>(identity, v)); // row_shr:1
    v = op(v, dpp_u32<0x112, 0xF>(identity, v)); // row_shr:2
    v = op(v, dpp_u32<0x114, 0xF>(identity, v)); // row_shr:4
    v = op(v, dpp_u32<0x118, 0xF>(identity, v)); // row_shr:8
    v = op(v, dpp_u32<0x142, 0xA>(identity, v)); // row_bcast:15 into rows 1, 3
    v = op(v, dpp_u32<0x143, 0xC>(identity, v)); // row_bcast:31 into rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_umax(uint32_t v)
{
    return wave_reduce_u32(v, 0u, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}

__device__ __forceinline__ uint32_t wave_umin(uint32_t v)
{
    return wave_reduce_u32(v, 0xFFFFFFFFu, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}

__device__ __forceinline__ float wave_fsum(float v)
{
    return __uint_as_float(wave_reduce_u32(__float_as_uint(v), 0u, [](uint32_t x, uint32_t y) {
        return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
    }));
}

// Total order of fp32 logits as unsigned keys (larger logit, larger key).
__device__ __forceinline__ uint32_t logit_key(float l)
{
    const uint32_t u = __float_as_uint(l);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of logit_key.
__device__ __forceinline__ float key_logit(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Candidate order of the top-k: larger key first, equal keys by lower id.
__device__ __forceinline__ void order_pair(uint32_t &ka, int &ia, uint32_t &kb, int &ib)
{
    const bool sw = kb > ka || (kb == ka && ib < ia);
    const uint32_t k0 = sw ? kb : ka, k1 = sw ? ka : kb;
    const int i0 = sw ? ib : ia, i1 = sw ? ia : ib;
    ka = k0;
    kb = k1;
    ia = i0;
    ib = i1;
}

// One wave: softmax over the E <= 256 logits of token t, held 4 per lane
// (expert lane + 64 r), and the top k by logit, equal logits to the lower
// id. Each lane sorts its four candidates once; a round then takes the
// wave maximum of the lane heads and the lowest id among the heads equal
// to it (one ballot; a second reduction only when several lanes tie), and
// that lane drops its head. Lane j keeps pick j. Writes topk_idx / topk_w
// and s_idx[t*k + j]. The last workgroup runs this once per call, with a
// cold instruction cache, so the loops stay rolled and the code short.
__device__ void wave_topk(const float (&l)[4], int E, int k, int t, int lane, int32_t *topk_idx, float *topk_w,
                          int *s_idx)
{
    uint32_t key[4];
    int id[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
        id[r] = lane + 64 * r;
        key[r] = id[r] < E ? logit_key(l[r]) : 0u; // 0 is below every finite logit
    }
    order_pair(key[0], id[0], key[1], id[1]);
    order_pair(key[2], id[2], key[3], id[3]);
    order_pair(key[0], id[0], key[2], id[2]);
    order_pair(key[1], id[1], key[3], id[3]);
    order_pair(key[1], id[1], key[2], id[2]);

    uint32_t my_key = 0u, top_key = 0u;
    int my_id = 0;
#pragma unroll 1
    for (int j = 0; j < k; j++) {
        const uint32_t best = wave_umax(key[0]);
        const unsigned long long tied = __ballot(key[0] == best);
        int e;
        if (__popcll(tied) == 1)
            e = __builtin_amdgcn_readlane(id[0], __ffsll((long long)tied) - 1);
        else
            e = (int)wave_umin(key[0] == best ? (uint32_t)id[0] : 0xFFFFFFFFu);
        if (lane == (e & 63)) { // the winner's lane drops its head
            key[0] = key[1];
            key[1] = key[2];
            key[2] = key[3];
            key[3] = 0u;
            id[0] = id[1];
            id[1] = id[2];
            id[2] = id[3];
            id[3] = 0x7FFFFFFF;
        }
        if (lane == j) {
            my_key = best;
            my_id = e;
        }
        top_key = j == 0 ? best : top_key;
    }
    // softmax denominator against the largest logit
    const float m = key_logit(top_key);
    float zz = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; r++)
        zz += lane + 64 * r < E ? expf(l[r] - m) : 0.0f;
    const float z = wave_fsum(zz);
    if (lane < k) {
        topk_idx[t * k + lane] = my_id;
        topk_w[t * k + lane] = expf(key_logit(my_key) - m) / z;
        s_idx[t * k + lane] = my_id;
    }
}

// Quantization of the router's tokens for the experts: 32 lanes per
// 32-element block, blocks spread over all workgroups of the router.
__device__ __forceinline__ void route_quant(const RouteArgs &a, int wave, int lane)
{
    const int nblk = a.q * (a.H / 32);
    for (int base = (blockIdx.x * 4 + wave) * 2; base < nblk; base += gridDim.x * 8) {
        const int blk = base + (lane >> 5);
        const bool valid = blk < nblk;
        const int i = blk * 32 + (lane & 31);
        const float v = valid ? a.x[i] : 0.0f;
        int8_t qv;
        float sv;
        int32_t sm;
        quant32(v, &qv, &sv, &sm, true);
        if (valid) {
            a.xq[i] = qv;
            if ((lane & 31) == 0) {
                a.xs[blk] = sv;
                a.xsum[blk] = sm;
            }
        }
    }
}

// Router for q <= 4 tokens: one workgroup per expert row of Wr. Arrival
// is counted in two levels (kRouteGroup workgroups per sub-counter, then
// one counter over the groups), since atomics on one address serialize;
// the last workgroup to arrive picks the top k per token and buckets the
// pairs.
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
            part[t] += w4[i].x * x4[t][i].x + w4[i].y * x4[t][i].y + w4[i].z * x4[t][i].z + w4[i].w * x4[t][i].w;
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
        route_quant(a, wave, lane);
        return;
    }

    // (3) last workgroup: softmax and top-k, one wave per token (the
    //     pair list's unused tail holds a key above every expert)
    const int np = a.q * a.k;
    if (tid >= np && tid < kMaxDecodeQ * kMaxK)
        s_idx[tid] = 0x7FFFFFFF;
    if (wave < a.q) {
        const int t = wave;
        float l[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int ee = lane + 64 * r;
            l[r] = ee < a.E ? __hip_atomic_load(a.logits + (size_t)t * a.E + ee, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT)
                            : -INFINITY;
        }
        wave_topk(l, a.E, a.k, t, lane, a.topk_idx, a.topk_w, s_idx);
    }
    __syncthreads();

    // (4) stable bucketing of the np = q*k <= 32 pairs by expert (pair
    //     p = t*k + j): position = pairs of lower experts + earlier pairs
    //     of the same one; expert_off[ee] = pairs of experts below ee.
    //     Every thread reads the list as int4 words and compares eight
    //     entries per step, skipping steps past np.
    const int mine = tid < np ? s_idx[tid] : 0;
    int pos = 0, before = 0;
#pragma unroll
    for (int c = 0; c < kMaxDecodeQ * kMaxK; c += 8) {
        if (c < np) {
            const int4 u = reinterpret_cast<const int4 *>(s_idx)[c / 4];
            const int4 v = reinterpret_cast<const int4 *>(s_idx)[c / 4 + 1];
            const int pe[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 8; i++) {
                pos += (pe[i] < mine || (pe[i] == mine && c + i < tid)) ? 1 : 0;
                before += pe[i] < tid ? 1 : 0;
            }
        }
    }
    if (tid < np)
        a.pairs_sorted[pos] = tid;
    if (tid < a.E)
        a.expert_off[tid] = before;
    if (tid == 0)
        a.expert_off[a.E] = np;
    if (tid < ngroups)
        __hip_atomic_store(a.cnt + kRouteCntStride * tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0)
        __hip_atomic_store(a.cnt + kRouteCntStride * kRouteMaxGroups, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    route_quant(a, wave, lane);
}

// ------------------------------------------------------------------
// Slot plan: slot 0 is the shared expert (when present), then the routed
// experts that have pairs, in id order. The FFN grids are (row group,
// slot) with the row group fastest, so the shared expert (the slot with
// the most tokens and, for sensitive layers, the heaviest format) is
// dispatched first.
// ------------------------------------------------------------------
struct SlotInfo {
    int kind;   // 0 = none, 1 = routed expert, 2 = shared expert
    int expert; // routed expert id
    int pb, pe; // pair range in pairs_sorted
    int n_slots;
};

__device__ __forceinline__ SlotInfo find_slot(int slot, const int32_t *__restrict__ expert_off, int E,
                                              bool has_shared)
{
    __shared__ SlotInfo s_info;
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 64) {
        // lane holds experts lane + 64 r (r < 4); all eight offsets are
        // loaded at once (clamped indices, no branches) and kept, so the
        // found expert's pair range needs no second round trip
        int lo[4], hi[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int e = min(lane + 64 * r, E);
            lo[r] = expert_off[e];
            hi[r] = expert_off[min(e + 1, E)];
        }
        const int rslot = has_shared ? slot - 1 : slot; // routed rank (-1: the shared slot)
        int total = 0, found_r = -1;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const bool act = (lane + 64 * r) < E && hi[r] > lo[r];
            const unsigned long long bal = __ballot(act);
            const int rank = total + __popcll(bal & ((1ull << lane) - 1ull));
            if (act && rank == rslot)
                found_r = r;
            total += __popcll(bal);
        }
        if (lane == 0) {
            s_info.n_slots = total + (has_shared ? 1 : 0);
            s_info.kind = (has_shared && slot == 0) ? 2 : 0;
            s_info.expert = -1;
            s_info.pb = s_info.pe = 0;
        }
        __builtin_amdgcn_wave_barrier();
        if (found_r >= 0) { // exactly one lane
            s_info.kind = 1;
            s_info.expert = lane + 64 * found_r;
            s_info.pb = found_r == 0 ? lo[0] : found_r == 1 ? lo[1] : found_r == 2 ? lo[2] : lo[3];
            s_info.pe = found_r == 0 ? hi[0] : found_r == 1 ? hi[1] : found_r == 2 ? hi[2] : hi[3];
        }
    }
    __syncthreads();
    const SlotInfo r = s_info;
    return r;
}

// ------------------------------------------------------------------
// Expert gate/up + SwiGLU + requantization of h.
// ------------------------------------------------------------------
struct FfnArgs {
    // routed stacks and shared expert (data pointers, per-matrix byte strides)
    const uint8_t *gate, *up, *down;
    size_t gate_stride, up_stride, down_stride;
    const uint8_t *sh_gate, *sh_up, *sh_down;
    int fmt_g, fmt_u, fmt_d, fmt_sg, fmt_su, fmt_sd;
    int E, H, I, q, k;
    bool has_shared;
    const int8_t *xq;
    const float *xs;
    const int32_t *xsum;
    const int32_t *topk_idx;
    const float *topk_w;
    const int32_t *pairs_sorted;
    const int32_t *expert_off;
    const float *resid; // [q][H] or null
    float *y;           // [q][H]
    MoeWs ws;
};

// Column j of a slot: its h / output row index and its activation token.
template <int NE>
struct SlotCols {
    int out_idx[NE]; // pair id (routed) or q*k + t (shared)
    int token[NE];
};

template <int NE>
__device__ __forceinline__ SlotCols<NE> slot_cols(const SlotInfo &si, const FfnArgs &a)
{
    SlotCols<NE> c;
    const sptr_i32 ps = as_scalar_i32(a.pairs_sorted);
#pragma unroll
    for (int j = 0; j < NE; j++) {
        if (si.kind == 2) {
            c.token[j] = j;
            c.out_idx[j] = a.q * a.k + j;
        } else {
            const int p = ps[si.pb + j];
            c.token[j] = p / a.k;
            c.out_idx[j] = p;
        }
    }
    return c;
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

// Wave 0: sum the W waves' gate and up partials of row g * 64 + lane (fixed
// order), SwiGLU, and the per-32 requantization of h.
template <int NE>
__device__ __forceinline__ void gateup_finish(const FfnArgs &a, const SlotCols<NE> &cols, int g, int lane, int W,
                                              const float *red)
{
#define RED_GU(w, m, j) red[(((w) * 2 + (m)) * kMaxDecodeQ + (j)) * 64 + lane]
    const int row = g * 64 + lane; // row of the intermediate dimension
    const int nbI = a.I / 32;
#pragma unroll
    for (int j = 0; j < NE; j++) {
        float gv = RED_GU(0, 0, j), uv = RED_GU(0, 1, j);
        for (int w = 1; w < W; w++) {
            gv += RED_GU(w, 0, j);
            uv += RED_GU(w, 1, j);
        }
#undef RED_GU
        // SwiGLU: silu(g) * u
        const float hv = row < a.I ? gv / (1.0f + expf(-gv)) * uv : 0.0f;
        const size_t idx = (size_t)cols.out_idx[j];
        int8_t qv;
        float sv;
        int32_t sm;
        quant32(hv, &qv, &sv, &sm, true);
        if (row < a.I) {
            a.ws.h[idx * a.I + row] = hv;
            a.ws.hq[idx * a.I + row] = qv;
            if ((lane & 31) == 0) {
                a.ws.hs[idx * nbI + (row >> 5)] = sv;
                a.ws.hsum[idx * nbI + (row >> 5)] = sm;
            }
        }
    }
}

template <int FG, int NE>
__device__ void gateup_body(const FfnArgs &a, const SlotInfo &si, int g, int lane, int wave, int W,
                            float *red)
{
    constexpr int FU = FG;
    const SlotCols<NE> cols = slot_cols<NE>(si, a);
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
        gm = a.gate + a.gate_stride * (size_t)si.expert;
        um = a.up + a.up_stride * (size_t)si.expert;
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
    } else if (s_begin < s_end) {
        GUTile<FG, NE> ta = load_gu<FG, NE>(gm, um, s_begin, nbH, xc, lane), tb;
        for (int s = s_begin; s < s_end; s += 2) {
            if (s + 1 < s_end)
                tb = load_gu<FG, NE>(gm, um, s + 1, nbH, xc, lane);
            gateup_tile<FG, NE>(ta, s, nbH, xc, ag, au);
            if (s + 1 >= s_end)
                break;
            if (s + 2 < s_end)
                ta = load_gu<FG, NE>(gm, um, s + 2, nbH, xc, lane);
            gateup_tile<FG, NE>(tb, s + 1, nbH, xc, ag, au);
        }
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
__device__ void gateup_body_mx(const FfnArgs &a, const SlotInfo &si, int g, int lane, int wave, int W, float *red)
{
    constexpr int TB = TileFmt<RFX_FP4>::bytes;
    const SlotCols<NE> cols = slot_cols<NE>(si, a);
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
        gm = a.gate + a.gate_stride * (size_t)si.expert;
        um = a.up + a.up_stride * (size_t)si.expert;
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

template <int FG, int FS>
__global__ __launch_bounds__(512) void gateup_kernel(FfnArgs a)
{
    __shared__ float red[8 * 2 * kMaxDecodeQ * 64];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    const SlotInfo si = find_slot(blockIdx.y, a.expert_off, a.E, a.has_shared);
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
                gateup_body_mx<1>(a, si, blockIdx.x, lane, wave, W, red);
            else
                gateup_body<FS, 1>(a, si, blockIdx.x, lane, wave, W, red);
            break;
        case 2:
            if constexpr (FS == RFX_FP4)
                gateup_body_mx<2>(a, si, blockIdx.x, lane, wave, W, red);
            else
                gateup_body<FS, 2>(a, si, blockIdx.x, lane, wave, W, red);
            break;
        case 3:
            if constexpr (FS == RFX_FP4)
                gateup_body_mx<3>(a, si, blockIdx.x, lane, wave, W, red);
            else
                gateup_body<FS, 3>(a, si, blockIdx.x, lane, wave, W, red);
            break;
        case 4:
            if constexpr (FS == RFX_FP4)
                gateup_body_mx<4>(a, si, blockIdx.x, lane, wave, W, red);
            else
                gateup_body<FS, 4>(a, si, blockIdx.x, lane, wave, W, red);
            break;
        default: break;
        }
    } else {
        switch (ne) {
        case 1:
            if constexpr (FG == RFX_FP4)
                gateup_body_mx<1>(a, si, blockIdx.x, lane, wave, W, red);
            else
                gateup_body<FG, 1>(a, si, blockIdx.x, lane, wave, W, red);
            break;
        case 2:
            if constexpr (FG == RFX_FP4)
                gateup_body_mx<2>(a, si, blockIdx.x, lane, wave, W, red);
            else
                gateup_body<FG, 2>(a, si, blockIdx.x, lane, wave, W, red);
            break;
        case 3: gateup_body<FG, 3>(a, si, blockIdx.x, lane, wave, W, red); break;
        case 4: gateup_body<FG, 4>(a, si, blockIdx.x, lane, wave, W, red); break;
        default: break;
        }
    }
}

// ------------------------------------------------------------------
// Expert down projection, shared expert and the weighted combine.
// ------------------------------------------------------------------
template <int FD, int NE>
struct DTile {
    TileRegs<FD> w;
    XTileM<NE> x;
};

template <int FD, int NE>
__device__ __forceinline__ DTile<FD, NE> load_dn(const uint8_t *dm, int s, int nbI, const XCols<NE> &xc, int lane)
{
    DTile<FD, NE> t;
    if (NE >= 2)
        t.x = load_xtile_m<FD, NE, false>(xc, s, nbI, lane);
    t.w = load_tile<FD>(dm + (size_t)s * TileFmt<FD>::bytes, lane);
    return t;
}

template <int FD, int NE>
__device__ __forceinline__ void down_tile(const DTile<FD, NE> &t, int s, int nbI, const XCols<NE> &xc,
                                          float (&ao)[NE])
{
    if (NE >= 2)
        tile_blocks_mfma<FD, NE, false>(t.w, t.x, s * 8, nbI, ao);
    else
        tile_blocks<FD, NE, NE, false>(t.w, s * 8, nbI, xc, ao);
}

// Wave 0: sum the W waves' partials of output row g * 64 + lane (fixed
// order) and leave them in o for the combine.
template <int NE>
__device__ __forceinline__ void down_finish(const FfnArgs &a, const SlotCols<NE> &cols, int g, int lane, int W,
                                            const float *red)
{
    const int row = g * 64 + lane;
#pragma unroll
    for (int j = 0; j < NE; j++) {
        float v = red[j * 64 + lane];
        for (int w = 1; w < W; w++)
            v += red[(w * kMaxDecodeQ + j) * 64 + lane];
        if (row < a.H)
            __hip_atomic_store(a.ws.o + (size_t)cols.out_idx[j] * a.H + row, v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int FD, int NE>
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
    const uint8_t *dm = si.kind == 2 ? a.sh_down : a.down + a.down_stride * (size_t)si.expert;
    dm += (size_t)g * S * TileFmt<FD>::bytes;
    float ao[NE];
#pragma unroll
    for (int j = 0; j < NE; j++)
        ao[j] = 0.0f;
    const int s_begin = __builtin_amdgcn_readfirstlane((int)((unsigned)(S * wave) / (unsigned)W));
    const int s_end = __builtin_amdgcn_readfirstlane((int)((unsigned)(S * (wave + 1)) / (unsigned)W));
    if (s_begin < s_end) {
        DTile<FD, NE> da = load_dn<FD, NE>(dm, s_begin, nbI, xc, lane), db;
        for (int s = s_begin; s < s_end; s += 2) {
            if (s + 1 < s_end)
                db = load_dn<FD, NE>(dm, s + 1, nbI, xc, lane);
            down_tile<FD, NE>(da, s, nbI, xc, ao);
            if (s + 1 >= s_end)
                break;
            if (s + 2 < s_end)
                da = load_dn<FD, NE>(dm, s + 2, nbI, xc, lane);
            down_tile<FD, NE>(db, s + 1, nbI, xc, ao);
        }
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
    const uint8_t *dm = si.kind == 2 ? a.sh_down : a.down + a.down_stride * (size_t)si.expert;
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
    const int row = g * 64 + lane;
    if (wave == 0 && row < a.H) {
        // every load issued before the first sum (one round trip, not one
        // per pair), then the sums in the fixed order
        float os[kMaxDecodeQ], rs[kMaxDecodeQ], ov[kMaxDecodeQ][kMaxK];
#pragma unroll
        for (int t = 0; t < kMaxDecodeQ; t++) {
            os[t] = 0.0f;
            rs[t] = 0.0f;
            if (t < a.q) {
                if (a.has_shared)
                    os[t] = __hip_atomic_load(a.ws.o + (size_t)(a.q * a.k + t) * a.H + row, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                if (a.resid)
                    rs[t] = a.resid[(size_t)t * a.H + row];
            }
#pragma unroll
            for (int j = 0; j < kMaxK; j++)
                ov[t][j] = t < a.q && j < a.k ? __hip_atomic_load(a.ws.o + (size_t)(t * a.k + j) * a.H + row,
                                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                              : 0.0f;
        }
#pragma unroll
        for (int t = 0; t < kMaxDecodeQ; t++) {
            if (t >= a.q)
                break;
            float acc = os[t];
            if (a.resid)
                acc = rs[t] + acc;
#pragma unroll
            for (int j = 0; j < kMaxK; j++)
                if (j < a.k)
                    acc += a.topk_w[t * a.k + j] * ov[t][j];
            a.y[(size_t)t * a.H + row] = acc;
        }
    }
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
    if ((st = check_qmat(&L->gate, "gate", true)) || (st = check_qmat(&L->up, "up", true)) ||
        (st = check_qmat(&L->down, "down", true)))
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

template <int FG>
int launch_gateup(int fs, const FfnArgs &a, dim3 grid, dim3 block, hipStream_t st)
{
    const size_t lds = 0;
    switch (fs) {
    case RFX_FP2: hipLaunchKernelGGL((gateup_kernel<FG, RFX_FP2>), grid, block, lds, st, a); break;
    case RFX_FP3: hipLaunchKernelGGL((gateup_kernel<FG, RFX_FP3>), grid, block, lds, st, a); break;
    case RFX_FP4: hipLaunchKernelGGL((gateup_kernel<FG, RFX_FP4>), grid, block, lds, st, a); break;
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

int waves_for(int wgs, int tiles, int max_waves)
{
    const int target = 3072; // ~3 waves per SIMD over 256 CUs
    int W = (target + wgs - 1) / wgs;
    W = W < 1 ? 1 : W > max_waves ? max_waves : W;
    return W > tiles ? tiles : W;
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
    if (L->hidden > 8192) // one workgroup reads a row as 8 float4 per thread
        return fail(RFX_E_UNSUPPORTED, "router: hidden=%d > 8192 for q <= 4", L->hidden);
    const int grid = L->n_experts; // one workgroup per expert row
    hipLaunchKernelGGL(route_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, a);
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
    if (q > kMaxDecodeQ) // many tokens: grouped int8 MFMA path
        return prefill_ffn(L, q, k, xq, xs, topk_w, pairs_sorted, expert_off, resid, y, w, (hipStream_t)stream);
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
    const int max_slots = (q * k < L->n_experts ? q * k : L->n_experts) + (a.has_shared ? 1 : 0);
    const hipStream_t s = (hipStream_t)stream;
    const int GI = (int)ceil_div(L->inter, 64), GH = (int)ceil_div(L->hidden, 64);
    const int SH = (int)ceil_div(L->hidden, 256), SI = (int)ceil_div(L->inter, 256);
    {
        const int W = waves_for(max_slots * GI, SH, 8);
        dim3 grid(GI, max_slots), block(64 * W);
        switch (a.fmt_g) {
        case RFX_FP2: st = launch_gateup<RFX_FP2>(a.fmt_sg, a, grid, block, s); break;
        case RFX_FP3: st = launch_gateup<RFX_FP3>(a.fmt_sg, a, grid, block, s); break;
        case RFX_FP4: st = launch_gateup<RFX_FP4>(a.fmt_sg, a, grid, block, s); break;
        }
        if (st)
            return st;
    }
    {
        const int W = waves_for(max_slots * GH, SI, 16);
        dim3 grid(GH, max_slots), block(64 * W);
        switch (a.fmt_d) {
        case RFX_FP2: st = launch_down<RFX_FP2>(a.fmt_sd, a, grid, block, s); break;
        case RFX_FP3: st = launch_down<RFX_FP3>(a.fmt_sd, a, grid, block, s); break;
        case RFX_FP4: st = launch_down<RFX_FP4>(a.fmt_sd, a, grid, block, s); break;
        }
    }
    return st;
}

int rfx_moe_debug_hidden(const rfx_moe_layer *L, int q, int k, const void *ws, float *h, int8_t *hq, float *hs,
                         void *stream)
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

} // extern "C"
