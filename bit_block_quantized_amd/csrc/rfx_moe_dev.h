// Device code shared by the MoE decode kernels: the three-launch path
// (route, gate/up, down + combine) and the single-launch layer kernel.
// Router pieces (activation quantization, top-k, bucketing), the slot plan,
// the FFN arguments, and the per-row-group finish and combine steps.
//
// Pages cited (title, site):
//   [HM]  "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
//         (hellomarvisaitoday.com), paragraphs numbered from the top.
//   [AIN] "Token Freedom via APU: AMD Ryzen AI MAX+ 395 Runs DeepSeek V4
//         Flash at 32 tok/s on a 284B Model" (ainomam.com), by section.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "rfx_decode.h"
#include "rfx_internal.h"
#include "rfx_moe_ws.h"

namespace rfx {
namespace moe {

using namespace rfx::dev;

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
// that lane drops its head. Lane j keeps pick j. Writes s_idx[t*k + j]
// and, unless topk_idx is null, topk_idx / topk_w. The last workgroup runs this once per call, with a
// cold instruction cache, so the loops stay rolled and the code short.
inline __device__ void wave_topk(const float (&l)[4], int E, int k, int t, int lane, int32_t *topk_idx, float *topk_w,
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
        if (topk_idx) {
            topk_idx[t * k + lane] = my_id;
            topk_w[t * k + lane] = expf(key_logit(my_key) - m) / z;
        }
        s_idx[t * k + lane] = my_id;
    }
}

// Router logits: acc + w . x over one float4 of a row, as an explicit
// chain of fused multiply-adds, so that every kernel computing logits
// rounds them the same way (the compiler's own contraction of a written-out
// sum of products depends on the code around it).
__device__ __forceinline__ float dot4_acc(float acc, const float4 &w, const float4 &x)
{
    acc = fmaf(w.x, x.x, acc);
    acc = fmaf(w.y, x.y, acc);
    acc = fmaf(w.z, x.z, acc);
    return fmaf(w.w, x.w, acc);
}

// Quantization of the router's tokens for the experts: 32 lanes per
// 32-element block, blocks spread over the n_wg router workgroups (W waves
// each); wg is this workgroup's index among them.
__device__ __forceinline__ void route_quant(const RouteArgs &a, int wg, int n_wg, int W, int wave, int lane)
{
    const int nblk = a.q * (a.H / 32);
    for (int base = (wg * W + wave) * 2; base < nblk; base += n_wg * W * 2) {
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

// The router's last workgroup, after every logit is stored: softmax and
// top-k per token (wave t for token t), then the stable bucketing of the
// pairs by expert and the reset of the arrival counters (ngroups
// sub-counters and the one over them). Every thread of the workgroup calls
// it; blockDim.x >= 256 >= E. s_idx: shared int[kMaxDecodeQ * kMaxK],
// 16-byte aligned.
__device__ __forceinline__ void route_select(const RouteArgs &a, int ngroups, int *s_idx)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // softmax and top-k, one wave per token (the pair list's unused tail
    // holds a key above every expert)
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

    // stable bucketing of the np = q*k <= 32 pairs by expert (pair
    // p = t*k + j): position = pairs of lower experts + earlier pairs
    // of the same one; expert_off[ee] = pairs of experts below ee.
    // Every thread reads the list as int4 words and compares eight
    // entries per step, skipping steps past np.
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
}

// ------------------------------------------------------------------
// Routing inside each FFN workgroup. When the router's logits come
// complete from the previous launch, every gate/up workgroup can pick the
// top k and bucket the pairs itself (a few hundred instructions) instead of
// the router launch finding its last workgroup through arrival counters and
// that workgroup reading the logits back: the launch boundary is the only
// barrier. The operations and their order are route_select's, so the
// results are the same bit for bit; one workgroup also writes the routing
// outputs, which the down launch and the caller read.
// ------------------------------------------------------------------
struct RouteOut {
    const float *logits; // [q][E] router logits (with bias), complete
    int32_t *topk_idx;   // [q][k]
    float *topk_w;       // [q][k]
    int32_t *pairs_sorted;
    int32_t *expert_off; // [E + 1]
};

struct RouteLds {
    __align__(16) int idx[kMaxDecodeQ * kMaxK]; // expert of pair p = t*k + j
    int pairs[kMaxDecodeQ * kMaxK];             // pairs_sorted
    int eoff[kMaxE + 1];                        // expert_off
};

__device__ __forceinline__ void wg_route(const RouteOut &ro, int q, int k, int E, bool out, RouteLds &s)
{
    const int tid = threadIdx.x, lane = tid & 63, nt = blockDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), W = nt >> 6;
    const int np = q * k;
    for (int i = np + tid; i < kMaxDecodeQ * kMaxK; i += nt)
        s.idx[i] = 0x7FFFFFFF;
    for (int t = wave; t < q; t += W) {
        float l[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int ee = lane + 64 * r;
            l[r] = ee < E ? ro.logits[(size_t)t * E + ee] : -INFINITY;
        }
        wave_topk(l, E, k, t, lane, out ? ro.topk_idx : nullptr, ro.topk_w, s.idx);
    }
    __syncthreads();
    // stable bucketing (route_select's counts), the whole pair list read
    // once as int4 words (a broadcast: every lane reads the same words);
    // the unused tail holds a key above every expert, so it counts nowhere
    int pe[kMaxDecodeQ * kMaxK];
#pragma unroll
    for (int c = 0; c < kMaxDecodeQ * kMaxK / 4; c++) {
        const int4 u = reinterpret_cast<const int4 *>(s.idx)[c];
        pe[4 * c] = u.x;
        pe[4 * c + 1] = u.y;
        pe[4 * c + 2] = u.z;
        pe[4 * c + 3] = u.w;
    }
    if (tid < np) {
        const int mine = s.idx[tid];
        int pos = 0;
#pragma unroll
        for (int i = 0; i < kMaxDecodeQ * kMaxK; i++)
            pos += (pe[i] < mine || (pe[i] == mine && i < tid)) ? 1 : 0;
        s.pairs[pos] = tid;
        if (out)
            ro.pairs_sorted[pos] = tid;
    }
    for (int e = tid; e <= E; e += nt) {
        int before = 0;
#pragma unroll
        for (int i = 0; i < kMaxDecodeQ * kMaxK; i++)
            before += pe[i] < e ? 1 : 0;
        s.eoff[e] = before;
        if (out)
            ro.expert_off[e] = before;
    }
    __syncthreads();
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
    const void *const *expert_data; // placement table [3][E] or null
};

// Matrix m (0 gate, 1 up, 2 down) of routed expert e: from the placement
// table when there is one, else from the stack.
__device__ __forceinline__ const uint8_t *expert_mat(const FfnArgs &a, int m, int e)
{
    if (a.expert_data)
        return as_global(a.expert_data[m * a.E + e]);
    return m == 0 ? a.gate + a.gate_stride * (size_t)e
         : m == 1 ? a.up + a.up_stride * (size_t)e : a.down + a.down_stride * (size_t)e;
}

// Column j of a slot: its h / output row index and its activation token.
template <int NE>
struct SlotCols {
    int out_idx[NE]; // pair id (routed) or q*k + t (shared)
    int token[NE];
};

// pairs_lds: the sorted pairs in LDS (routing inside the workgroup), else
// null and they are read from a.pairs_sorted.
template <int NE>
__device__ __forceinline__ SlotCols<NE> slot_cols(const SlotInfo &si, const FfnArgs &a,
                                                  const int *pairs_lds = nullptr)
{
    SlotCols<NE> c;
    const sptr_i32 ps = as_scalar_i32(a.pairs_sorted);
#pragma unroll
    for (int j = 0; j < NE; j++) {
        if (si.kind == 2) {
            c.token[j] = j;
            c.out_idx[j] = a.q * a.k + j;
        } else {
            const int p = pairs_lds ? __builtin_amdgcn_readfirstlane(pairs_lds[si.pb + j]) : ps[si.pb + j];
            c.token[j] = p / a.k;
            c.out_idx[j] = p;
        }
    }
    return c;
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

// Wave 0 of the last slot to finish output row group g: the weighted
// combine y[t] = resid[t] + o_shared[t] + sum_j w[t][j] * o[t*k + j], in
// this fixed order.
__device__ __forceinline__ void combine_rows(const FfnArgs &a, int g, int lane)
{
    const int row = g * 64 + lane;
    if (row < a.H) {
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
}

// Waves per workgroup of the decode gate/up and down kernels: about
// `target` waves over the chip (gate/up 3072, three per SIMD; down twice
// that, kDownWaveTarget: its workgroups hold ~120 registers, four waves
// per SIMD, and measured 1-2 us faster per q = 4 layer with four waves
// per workgroup than with two), rounded down to a power of two (a
// workgroup's waves then spread evenly over the four SIMDs of a CU: six
// waves at ~160 registers left room for one workgroup per CU and measured
// 4.6 us slower per q = 4 top-4 layer than four), at most max_waves, at
// most one per tile (each wave takes a contiguous share of the row group's
// tiles; the shares' fp32 partials are summed in wave order, so this choice
// fixes the summation order and is shared by both decode paths). Host code.
constexpr int kGateUpWaveTarget = 3072;
constexpr int kDownWaveTarget = 6144;
inline int waves_for(int wgs, int tiles, int max_waves, int target)
{
    int W = (target + wgs - 1) / wgs;
    W = W < 1 ? 1 : W > max_waves ? max_waves : W;
    while (W & (W - 1))
        W &= W - 1;
    return W > tiles ? tiles : W;
}

// The single-launch layer kernel (rfx_moe_layer.hip): whether it takes a
// call (q <= 4, the formats it is built for, the grid within its counters)
// and its launch. Arguments are validated by the caller.
bool layer_kernel_takes(const FfnArgs &f, int q, int k);
int launch_layer(const FfnArgs &f, const RouteArgs &r, hipStream_t stream);

} // namespace moe
} // namespace rfx
