// Prefill-sized MoE layer for gfx950: router over many tokens, stable
// bucketing of the (token, slot) pairs by expert, and the expert FFN as
// grouped int8 MFMA tiles with a per-block fp32 rescale.
//
// Pages cited (title, site):
//   [HM]  "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
//         (hellomarvisaitoday.com), paragraphs numbered from the top.
//   [KK]  the kaikai365.com post on DeepSeek V4 Flash on Strix Halo, by
//         section heading.
//
// Routing is a TOP_K and an ARGSORT step ([HM] para 3; [KK] DSpark
// section): after the argsort every expert's tokens are contiguous, so with
// thousands of tokens each expert's FFN is a small dense contraction
// (tens of tokens x 2048 x 4096). There the packed FP2/FP3/FP4 blocks are
// expanded through their codebooks into int8 operand tiles in LDS and fed to
// v_mfma_i32_16x16x32_i8: one MFMA K step is exactly one 32-weight block, so
// its int32 result is the exact block dot D, which is then scaled by the
// weight and activation block scales in fp32 (the same sum as the decode
// kernels, over the same blocks in the same order per output).
//
// Launches per layer: act quant, router logits (fp32 matrix core), softmax /
// top-k, bucket (one workgroup), gate/up (+ SwiGLU + requantization), down,
// combine.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rfx_decode.h"
#include "rfx_internal.h"
#include "rfx_moe_ws.h"

using namespace rfx;
using namespace rfx::dev;

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------
// Router logits x . Wr^T (+ b) in fp32 on the matrix core
// (v_mfma_f32_16x16x4_f32): one workgroup per 16 tokens x 32 experts, its
// four waves splitting H into contiguous runs of 32 columns (so each SIMD
// has four independent load streams in flight) and summed in fixed order
// through LDS. Per 16-column chunk, lane l holds x[t0 + l%16][k0 +
// 4(l/16) ..+3] and the same four columns of expert rows e0 + l%16 and
// e0 + 16 + l%16; step s of the chunk feeds component s of each, so the
// matrix op's K index l/16 stands for column k0 + 4(l/16) + s on both
// operands and every product pairs equal columns. Output lane l, register
// v: token t0 + 4(l/16) + v, expert e0 + l%16 (second tile: + 16). Rows
// past T or E are read clamped and never stored.
// ------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct LogitArgs {
    const float *x;  // [T][H]
    const float *wr; // [E][H]
    const float *wb; // [E] or null
    int T, E, H;     // H % 32 == 0
    float *logits;   // [T][E]
};

constexpr int kLogitWaves = 4;

__global__ __launch_bounds__(64 * kLogitWaves) void prefill_logits_kernel(LogitArgs a)
{
    __shared__ f32x4 red[kLogitWaves][2][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 32;
    const int r = lane & 15, kq = (lane >> 4) * 4;
    const float *xp = a.x + (size_t)min(t0 + r, a.T - 1) * a.H + kq;
    const float *w0 = a.wr + (size_t)min(e0 + r, a.E - 1) * a.H + kq;
    const float *w1 = a.wr + (size_t)min(e0 + 16 + r, a.E - 1) * a.H + kq;
    const int nc = a.H / 32;
    const int c_begin = nc * wave / kLogitWaves, c_end = nc * (wave + 1) / kLogitWaves;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int c32 = c_begin; c32 < c_end; c32++) {
        const int k0 = 32 * c32;
        f32x4 xv[2], wv0[2], wv1[2];
#pragma unroll
        for (int c = 0; c < 2; c++) {
            xv[c] = *reinterpret_cast<const f32x4 *>(xp + k0 + 16 * c);
            wv0[c] = *reinterpret_cast<const f32x4 *>(w0 + k0 + 16 * c);
            wv1[c] = *reinterpret_cast<const f32x4 *>(w1 + k0 + 16 * c);
        }
#pragma unroll
        for (int c = 0; c < 2; c++)
#pragma unroll
            for (int st = 0; st < 4; st++) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[c][st], wv0[c][st], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[c][st], wv1[c][st], acc1, 0, 0, 0);
            }
    }
    red[wave][0][lane] = acc0;
    red[wave][1][lane] = acc1;
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int w = 1; w < kLogitWaves; w++) { // fixed order: wave 0, 1, 2, 3
        acc0 += red[w][0][lane];
        acc1 += red[w][1][lane];
    }
    const int ea = e0 + r, eb = e0 + 16 + r;
    const float ba = a.wb && ea < a.E ? a.wb[ea] : 0.0f, bb = a.wb && eb < a.E ? a.wb[eb] : 0.0f;
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int t = t0 + 4 * (lane >> 4) + v;
        if (t < a.T) {
            if (ea < a.E)
                a.logits[(size_t)t * a.E + ea] = acc0[v] + ba;
            if (eb < a.E)
                a.logits[(size_t)t * a.E + eb] = acc1[v] + bb;
        }
    }
}

// ------------------------------------------------------------------
// Router selection: softmax over all experts, top-k by logit with ties to
// the lower id, weights = the chosen probabilities. One wave per token,
// kRouteTB tokens per workgroup, logits from prefill_logits_kernel.
// ------------------------------------------------------------------
constexpr int kRouteTB = 8; // tokens per workgroup

struct RouteArgs {
    const float *logits; // [T][E]
    int T, k, E;
    int32_t *topk_idx;
    float *topk_w;
};

__global__ __launch_bounds__(256) void prefill_route_kernel(RouteArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t0 = blockIdx.x * kRouteTB;

    // one wave per token: softmax and top-k
    for (int tt = wave; tt < kRouteTB; tt += 4) {
        const int t = t0 + tt;
        if (t >= a.T)
            break;
        float l[4];
        bool taken[4];
        float m = -INFINITY;
        for (int r = 0; r < 4; r++) {
            const int ee = lane + 64 * r;
            l[r] = ee < a.E ? a.logits[(size_t)t * a.E + ee] : -INFINITY;
            taken[r] = ee >= a.E;
            m = fmaxf(m, l[r]);
        }
        for (int o = 32; o > 0; o >>= 1)
            m = fmaxf(m, __shfl_xor(m, o, 64));
        float z = 0.0f;
        for (int r = 0; r < 4; r++)
            z += (lane + 64 * r) < a.E ? expf(l[r] - m) : 0.0f;
        for (int o = 32; o > 0; o >>= 1)
            z += __shfl_xor(z, o, 64);
        for (int j = 0; j < a.k; j++) {
            float bv = -INFINITY;
            int be = 0x7fffffff;
            for (int r = 0; r < 4; r++) {
                const int ee = lane + 64 * r;
                if (!taken[r] && (l[r] > bv || (l[r] == bv && ee < be))) {
                    bv = l[r];
                    be = ee;
                }
            }
            for (int o = 32; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oe = __shfl_xor(be, o, 64);
                if (ov > bv || (ov == bv && oe < be)) {
                    bv = ov;
                    be = oe;
                }
            }
            for (int r = 0; r < 4; r++)
                if (lane + 64 * r == be)
                    taken[r] = true;
            if (lane == 0) {
                a.topk_idx[(size_t)t * a.k + j] = be;
                a.topk_w[(size_t)t * a.k + j] = expf(bv - m) / z;
            }
        }
    }
}

// ------------------------------------------------------------------
// Stable bucketing (one workgroup of 16 waves). Wave w owns a contiguous
// segment of the pairs. Pass 1 counts experts per wave; a scan gives each
// (wave, expert) its first output slot; pass 2 walks the segment in order,
// 64 pairs at a time, ranking equal experts among the lanes with ballots,
// so equal experts keep their pair order. Also writes expert_off and the
// work items of the FFN kernels.
// ------------------------------------------------------------------
struct BucketArgs {
    const int32_t *topk_idx;
    int np, T, E;
    bool shared;
    int32_t *pairs_sorted;
    int32_t *expert_off;
    int32_t *items;
};

// Block-wide exclusive scan of one value per thread among the first 256
// threads of a 1024-thread workgroup (all threads must call it).
__device__ int scan256_exclusive(int v, int *buf)
{
    const int tid = threadIdx.x;
    if (tid < 256)
        buf[tid] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        int add = 0;
        if (tid < 256 && tid >= o)
            add = buf[tid - o];
        __syncthreads();
        if (tid < 256)
            buf[tid] += add;
        __syncthreads();
    }
    const int incl = tid < 256 ? buf[tid] : 0;
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(1024) void bucket_kernel(BucketArgs a)
{
    __shared__ int cnt[16][kMaxE];
    __shared__ int buf[256];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < 16 * kMaxE; i += 1024)
        (&cnt[0][0])[i] = 0;
    __syncthreads();
    const int seg = (a.np + 15) / 16;
    const int p_begin = min(wave * seg, a.np), p_end = min(p_begin + seg, a.np);
    for (int p = p_begin + lane; p < p_end; p += 64)
        atomicAdd(&cnt[wave][a.topk_idx[p]], 1);
    __syncthreads();

    // totals and offsets per expert; each (wave, expert) gets its first slot
    int tot = 0;
    if (tid < a.E)
        for (int w = 0; w < 16; w++)
            tot += cnt[w][tid];
    const int off = scan256_exclusive(tid < a.E ? tot : 0, buf);
    if (tid < a.E) {
        int run = off;
        for (int w = 0; w < 16; w++) {
            const int c = cnt[w][tid];
            cnt[w][tid] = run;
            run += c;
        }
        a.expert_off[tid] = off;
    }
    if (tid == 0)
        a.expert_off[a.E] = a.np;
    __syncthreads();

    // ordered placement; e = 511 marks an idle lane (never matches a real id)
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int base = p_begin; base < p_end; base += 64) {
        const int p = base + lane;
        const bool valid = p < p_end;
        const int e = valid ? a.topk_idx[p] : 511;
        unsigned long long m = ~0ull;
#pragma unroll
        for (int bit = 0; bit < 9; bit++) {
            const unsigned long long bb = __ballot((e >> bit) & 1);
            m &= ((e >> bit) & 1) ? bb : ~bb;
        }
        const int rank = __popcll(m & lt);
        const int n = __popcll(m);
        int slot = 0;
        if (valid)
            slot = cnt[wave][e] + rank;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            a.pairs_sorted[slot] = p;
            if (rank == n - 1)
                cnt[wave][e] = slot + 1;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }

    // FFN work items: chunks of kPrefillChunk tokens per expert, in expert
    // order, then the shared expert's chunks
    const int chunks = tid < a.E ? (tot + kPrefillChunk - 1) / kPrefillChunk : 0;
    const int istart = scan256_exclusive(chunks, buf);
    if (tid < a.E)
        for (int c = 0; c < chunks; c++) {
            a.items[1 + 2 * (istart + c)] = tid;
            a.items[2 + 2 * (istart + c)] = c * kPrefillChunk;
        }
    __shared__ int s_routed;
    if (tid == 255)
        s_routed = istart + chunks;
    __syncthreads();
    const int routed = s_routed;
    const int sh_chunks = a.shared ? (a.T + kPrefillChunk - 1) / kPrefillChunk : 0;
    for (int c = tid; c < sh_chunks; c += 1024) {
        a.items[1 + 2 * (routed + c)] = a.E;
        a.items[2 + 2 * (routed + c)] = c * kPrefillChunk;
    }
    if (tid == 0)
        a.items[0] = routed + sh_chunks;
}

// ------------------------------------------------------------------
// Grouped FFN on MFMA.
// ------------------------------------------------------------------
struct FfnArgs {
    const uint8_t *gate, *up, *down; // routed stacks
    size_t gate_stride, up_stride, down_stride;
    const uint8_t *sh_gate, *sh_up, *sh_down;
    int E, H, I, T, k;
    const int8_t *xq; // [T][H]
    const float *xs;  // [T][H/32]
    const int32_t *pairs_sorted;
    const int32_t *expert_off;
    const float *topk_w;
    const float *resid;
    float *y;
    MoeWs ws;
};

struct Item {
    int expert; // E = the shared expert
    int first;  // first token of the chunk within the expert's list
    int n;      // tokens in the chunk (1..64)
};

__device__ __forceinline__ Item load_item(const FfnArgs &a, int idx, bool &ok)
{
    Item it{};
    const int n_items = __builtin_amdgcn_readfirstlane(a.ws.items[0]);
    ok = idx < n_items;
    if (!ok)
        return it;
    it.expert = __builtin_amdgcn_readfirstlane(a.ws.items[1 + 2 * idx]);
    it.first = __builtin_amdgcn_readfirstlane(a.ws.items[2 + 2 * idx]);
    const int total = it.expert == a.E ? a.T : a.expert_off[it.expert + 1] - a.expert_off[it.expert];
    it.n = __builtin_amdgcn_readfirstlane(min(kPrefillChunk, total - it.first));
    return it;
}

// Row of h / o (pair id, or T*k + token for the shared expert) and the
// token of slot i of an item.
__device__ __forceinline__ void slot_rows(const FfnArgs &a, const Item &it, int i, int &row, int &token)
{
    if (it.expert == a.E) {
        token = it.first + i;
        row = a.T * a.k + token;
    } else {
        const int p = a.pairs_sorted[a.expert_off[it.expert] + it.first + i];
        token = p / a.k;
        row = p;
    }
}

// Expand block b of row tr of one tile into 32 int8 codebook values (8
// dwords, weights 4d..4d+3 in dword d) and its weight scale.
template <int FMT>
__device__ __forceinline__ void expand_block(const uint8_t *tile, int tr, int b, uint32_t (&v)[8], float &sw)
{
    if (FMT == RFX_FP4) {
        const u32x4 c = *reinterpret_cast<const u32x4 *>(tile + b * 1024 + tr * 16);
        const Sel8 sv = sel_fp4(c);
#pragma unroll
        for (int d = 0; d < 8; d++)
            v[d] = (uint32_t)sv.v[d];
        const uint32_t e = tile[8192 + tr * 8 + b];
        sw = ldexpf(1.0f, (int)e - 128);
    } else {
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(tile + (b >> 1) * 1024 + tr * 16 + (b & 1) * 8);
        const uint32_t w[2] = {lo.x, lo.y};
        uint32_t h = 0;
        if (FMT == RFX_FP3)
            h = *reinterpret_cast<const uint32_t *>(tile + (4 + (b >> 2)) * 1024 + tr * 16 + (b & 3) * 4);
#pragma unroll
        for (int d = 0; d < 8; d++) {
            uint32_t sel = (w[d >> 2] >> (2 * (d & 3))) & 0x03030303u;
            if (FMT == RFX_FP3) {
                sel |= ((h >> d) & 0x01010101u) << 2;
                // {-7 -5 -3 -1 | 1 3 5 7}
                v[d] = __builtin_amdgcn_perm(0x07050301u, 0xFFFDFBF9u, sel);
            } else {
                // {-3 -1 1 3}
                v[d] = __builtin_amdgcn_perm(0u, 0x0301FFFDu, sel);
            }
        }
        const int sc = FMT == RFX_FP3 ? 6 : 4;
        sw = half_bits_to_float(*reinterpret_cast<const uint16_t *>(tile + sc * 1024 + tr * 16 + b * 2));
    }
}

// LDS operand fragments of v_mfma_i32_16x16x32_i8: lane l of a 16-row
// (A) or 16-token (B) tile holds row / token l % 16, k = 8 (l / 16) .. +7
// of one 32-k block. Fragment [tile][block][lane] = 8 bytes.
__device__ __forceinline__ void put_frag(uint2 *frag_base, int r16, const uint32_t (&v)[8])
{
#pragma unroll
    for (int kg = 0; kg < 4; kg++)
        frag_base[r16 + 16 * kg] = make_uint2(v[2 * kg], v[2 * kg + 1]);
}

// Stage the activation slice of K tile s for up to 64 slots into LDS B
// fragments (4 token tiles x 8 blocks x 64 lanes) and their block scales.
// Thread (slot i = tid / 4, quarter qd = tid % 4) moves blocks 2qd, 2qd+1.
// Slots past n and blocks past nb are zero.
__device__ __forceinline__ void stage_b(const int8_t *rows, const float *scales, size_t row_stride,
                                        size_t scale_stride, const int *slot_src, int n, int s, int nb,
                                        uint2 *lB, float *lsx)
{
    const int tid = threadIdx.x;
    const int i = tid >> 2, qd = tid & 3;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int b = 2 * qd + h;
        const int blk = s * 8 + b;
        uint32_t v[8];
        float sx = 0.0f;
        if (i < n && blk < nb) {
            const int src = slot_src[i];
            const u32x4 *p = reinterpret_cast<const u32x4 *>(rows + (size_t)src * row_stride + (size_t)blk * 32);
            const u32x4 c0 = p[0], c1 = p[1];
            v[0] = c0.x;
            v[1] = c0.y;
            v[2] = c0.z;
            v[3] = c0.w;
            v[4] = c1.x;
            v[5] = c1.y;
            v[6] = c1.z;
            v[7] = c1.w;
            sx = scales[(size_t)src * scale_stride + blk];
        } else {
#pragma unroll
            for (int d = 0; d < 8; d++)
                v[d] = 0u;
        }
        put_frag(lB + ((i >> 4) * 8 + b) * 64, i & 15, v);
        lsx[b * 64 + i] = sx;
    }
}

// One K tile of MFMA work for one wave: a 16-row A tile against up to 4
// token tiles over 8 blocks. acc[tt][r] is row 4 (lane / 16) + r of the
// tile, token 16 tt + lane % 16. lsw: the tile's row scales, block stride
// sw_stride. Each MFMA is one block: its int32 result is the exact block
// dot, scaled by (weight scale x activation scale) into fp32.
__device__ __forceinline__ void mfma_tile(const uint2 *lA_tile, const float *lsw, int sw_stride, const uint2 *lB,
                                          const float *lsx, int ntt, int lane, float (&acc)[4][4])
{
#pragma unroll
    for (int b = 0; b < 8; b++) {
        const uint2 av = lA_tile[b * 64 + lane];
        const long a8 = (long)(((unsigned long)av.y << 32) | av.x);
        const float4 sw = *reinterpret_cast<const float4 *>(lsw + b * sw_stride + 4 * (lane >> 4));
#pragma unroll
        for (int tt = 0; tt < 4; tt++) {
            if (tt >= ntt)
                break;
            const uint2 bv = lB[(tt * 8 + b) * 64 + lane];
            const long b8 = (long)(((unsigned long)bv.y << 32) | bv.x);
            const i32x4 zero = {0, 0, 0, 0};
            const i32x4 d = __builtin_amdgcn_mfma_i32_16x16x32_i8(a8, b8, zero, 0, 0, 0);
            const float sx = lsx[b * 64 + 16 * tt + (lane & 15)];
            acc[tt][0] += (float)d[0] * (sw.x * sx);
            acc[tt][1] += (float)d[1] * (sw.y * sx);
            acc[tt][2] += (float)d[2] * (sw.z * sx);
            acc[tt][3] += (float)d[3] * (sw.w * sx);
        }
    }
}

// LDS map of the FFN kernels (bytes): A fragments 16 KB, B fragments 16 KB,
// row scales 2 KB, slot scales 2 KB, slot maps 512 B. The SwiGLU epilogue
// reuses the fragment area for the [2][32][65] fp32 gate/up tile.
constexpr int kLdsA = 0, kLdsB = 16384, kLdsSw = 32768, kLdsSx = 34816, kLdsRow = 36864, kLdsTok = 37120;
constexpr int kLdsBytes = 37376;

__device__ __forceinline__ void zero_acc(float (&acc)[4][4])
{
#pragma unroll
    for (int tt = 0; tt < 4; tt++)
#pragma unroll
        for (int r = 0; r < 4; r++)
            acc[tt][r] = 0.0f;
}

// Slot -> (h / o row, token) maps of an item, in LDS.
__device__ __forceinline__ void fill_slots(const FfnArgs &a, const Item &it, int *slot_row, int *slot_tok)
{
    const int tid = threadIdx.x;
    if (tid < kPrefillChunk) {
        int row = 0, tok = 0;
        if (tid < it.n)
            slot_rows(a, it, tid, row, tok);
        slot_row[tid] = row;
        slot_tok[tid] = tok;
    }
}

// Gate/up: one workgroup = 32 intermediate rows of gate and of up x one
// item. Wave w: matrix w >> 1 (gate, up), row tile w & 1. Epilogue:
// h = silu(g) * u and the per-32 requantization of h, whose 32-row block
// is exactly this workgroup's rows.
template <int F>
__device__ void gateup_body(const FfnArgs &a, const Item &it, const uint8_t *gm, const uint8_t *um, char *smem)
{
    uint2 *lA = reinterpret_cast<uint2 *>(smem + kLdsA); // [2 mat][2 rt][8 b][64]
    uint2 *lB = reinterpret_cast<uint2 *>(smem + kLdsB); // [4 tt][8 b][64]
    float *lsw = reinterpret_cast<float *>(smem + kLdsSw); // [2 mat][8 b][32 rows]
    float *lsx = reinterpret_cast<float *>(smem + kLdsSx); // [8 b][64 slots]
    int *slot_row = reinterpret_cast<int *>(smem + kLdsRow);
    int *slot_tok = reinterpret_cast<int *>(smem + kLdsTok);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r0 = blockIdx.x * 32, g = r0 >> 6, half = r0 & 63;
    const int S = (a.H + 255) / 256, nbH = a.H / 32;
    constexpr int TBYTES = TileFmt<F>::bytes;
    fill_slots(a, it, slot_row, slot_tok);
    __syncthreads();
    const int ntt = (it.n + 15) >> 4;
    float acc[4][4];
    zero_acc(acc);
    const int mat = wave >> 1, rt = wave & 1;
    for (int s = 0; s < S; s++) {
        {
            // A: thread -> (row r, block b) of gate and of up
            const int r = tid & 31, b = tid >> 5;
#pragma unroll
            for (int m = 0; m < 2; m++) {
                const uint8_t *tile = (m == 0 ? gm : um) + ((size_t)g * S + s) * TBYTES;
                uint32_t v[8];
                float sw = 0.0f;
                if (s * 8 + b < nbH) {
                    expand_block<F>(tile, half + r, b, v, sw);
                } else {
#pragma unroll
                    for (int d = 0; d < 8; d++)
                        v[d] = 0u;
                }
                put_frag(lA + ((m * 2 + (r >> 4)) * 8 + b) * 64, r & 15, v);
                lsw[(m * 8 + b) * 32 + r] = sw;
            }
        }
        stage_b(a.xq, a.xs, (size_t)a.H, (size_t)nbH, slot_tok, it.n, s, nbH, lB, lsx);
        __syncthreads();
        mfma_tile(lA + (mat * 2 + rt) * 8 * 64, lsw + mat * 8 * 32 + 16 * rt, 32, lB, lsx, ntt, lane, acc);
        __syncthreads();
    }

    // epilogue: gate and up tiles meet in LDS
    float *hb = reinterpret_cast<float *>(smem + kLdsA); // [2][32][65]
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
        if (tt >= ntt)
            break;
#pragma unroll
        for (int r = 0; r < 4; r++)
            hb[(mat * 32 + 16 * rt + 4 * (lane >> 4) + r) * 65 + 16 * tt + (lane & 15)] = acc[tt][r];
    }
    __syncthreads();
    {
#pragma clang fp contract(off)
        const int i = tid >> 2, rg = tid & 3;
        float hv[8];
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float gv = hb[(8 * rg + j) * 65 + i], uv = hb[(32 + 8 * rg + j) * 65 + i];
            hv[j] = gv / (1.0f + expf(-gv)) * uv; // SwiGLU: silu(g) * u
            amax = fmaxf(amax, fabsf(hv[j]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        const float sc = amax / 127.0f;
        uint32_t packed[2] = {0u, 0u};
        int sum = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            int qv = 0;
            if (sc != 0.0f) {
                float rr = rintf(hv[j] / sc);
                rr = fminf(fmaxf(rr, -127.0f), 127.0f);
                qv = (int)rr;
            }
            sum += qv;
            packed[j >> 2] |= ((uint32_t)qv & 0xffu) << (8 * (j & 3));
        }
        sum += __shfl_xor(sum, 1, 64);
        sum += __shfl_xor(sum, 2, 64);
        if (i < it.n) {
            const size_t row = (size_t)slot_row[i];
            *reinterpret_cast<uint2 *>(a.ws.hq + row * a.I + r0 + 8 * rg) = make_uint2(packed[0], packed[1]);
            if (rg == 0) {
                a.ws.hs[row * (a.I / 32) + blockIdx.x] = sc;
                a.ws.hsum[row * (a.I / 32) + blockIdx.x] = sum;
            }
        }
    }
}

template <int FG, int FS>
__global__ __launch_bounds__(256) void prefill_gateup_kernel(FfnArgs a)
{
    __shared__ __align__(16) char smem[kLdsBytes];
    bool ok;
    const Item it = load_item(a, blockIdx.y, ok);
    if (!ok)
        return;
    if (it.expert == a.E)
        gateup_body<FS>(a, it, a.sh_gate, a.sh_up, smem);
    else
        gateup_body<FG>(a, it, a.gate + a.gate_stride * (size_t)it.expert, a.up + a.up_stride * (size_t)it.expert,
                        smem);
}

// Down: one workgroup = 64 output rows x one item; wave w = row tile w.
// o[row of slot][output row] in fp32 for the combine.
template <int F>
__device__ void down_body(const FfnArgs &a, const Item &it, const uint8_t *dm, char *smem)
{
    uint2 *lA = reinterpret_cast<uint2 *>(smem + kLdsA); // [4 rt][8 b][64]
    uint2 *lB = reinterpret_cast<uint2 *>(smem + kLdsB);
    float *lsw = reinterpret_cast<float *>(smem + kLdsSw); // [8 b][64 rows]
    float *lsx = reinterpret_cast<float *>(smem + kLdsSx);
    int *slot_row = reinterpret_cast<int *>(smem + kLdsRow);
    int *slot_tok = reinterpret_cast<int *>(smem + kLdsTok);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x;
    const int S = (a.I + 255) / 256, nbI = a.I / 32;
    constexpr int TBYTES = TileFmt<F>::bytes;
    fill_slots(a, it, slot_row, slot_tok);
    __syncthreads();
    const int ntt = (it.n + 15) >> 4;
    float acc[4][4];
    zero_acc(acc);
    for (int s = 0; s < S; s++) {
        const uint8_t *tile = dm + ((size_t)g * S + s) * TBYTES;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int u = tid + 256 * h;
            const int r = u & 63, b = u >> 6;
            uint32_t v[8];
            float sw = 0.0f;
            if (s * 8 + b < nbI) {
                expand_block<F>(tile, r, b, v, sw);
            } else {
#pragma unroll
                for (int d = 0; d < 8; d++)
                    v[d] = 0u;
            }
            put_frag(lA + ((r >> 4) * 8 + b) * 64, r & 15, v);
            lsw[b * 64 + r] = sw;
        }
        stage_b(a.ws.hq, a.ws.hs, (size_t)a.I, (size_t)nbI, slot_row, it.n, s, nbI, lB, lsx);
        __syncthreads();
        mfma_tile(lA + wave * 8 * 64, lsw + 16 * wave, 64, lB, lsx, ntt, lane, acc);
        __syncthreads();
    }
    const int orow = g * 64 + 16 * wave + 4 * (lane >> 4);
    if (orow < a.H) {
#pragma unroll
        for (int tt = 0; tt < 4; tt++) {
            const int i = 16 * tt + (lane & 15);
            if (tt < ntt && i < it.n)
                *reinterpret_cast<float4 *>(a.ws.o + (size_t)slot_row[i] * a.H + orow) =
                    make_float4(acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]);
        }
    }
}

template <int FD, int FSD>
__global__ __launch_bounds__(256) void prefill_down_kernel(FfnArgs a)
{
    __shared__ __align__(16) char smem[kLdsBytes];
    bool ok;
    const Item it = load_item(a, blockIdx.y, ok);
    if (!ok)
        return;
    if (it.expert == a.E)
        down_body<FSD>(a, it, a.sh_down, smem);
    else
        down_body<FD>(a, it, a.down + a.down_stride * (size_t)it.expert, smem);
}

// y[t] = resid[t] + o_shared[t] + sum_j w[t][j] o[t*k + j], slot order.
__global__ __launch_bounds__(256) void prefill_combine_kernel(FfnArgs a, bool has_shared)
{
    const int t = blockIdx.y;
    const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (h >= a.H)
        return;
    float4 acc = has_shared ? *reinterpret_cast<const float4 *>(a.ws.o + ((size_t)a.T * a.k + t) * a.H + h)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.resid) {
        const float4 r = *reinterpret_cast<const float4 *>(a.resid + (size_t)t * a.H + h);
        acc = make_float4(r.x + acc.x, r.y + acc.y, r.z + acc.z, r.w + acc.w);
    }
    for (int j = 0; j < a.k; j++) {
        const float w = a.topk_w[(size_t)t * a.k + j];
        const float4 o = *reinterpret_cast<const float4 *>(a.ws.o + ((size_t)t * a.k + j) * a.H + h);
        acc.x += w * o.x;
        acc.y += w * o.y;
        acc.z += w * o.z;
        acc.w += w * o.w;
    }
    *reinterpret_cast<float4 *>(a.y + (size_t)t * a.H + h) = acc;
}

template <int FG>
int launch_gateup(int fs, const FfnArgs &a, dim3 grid, hipStream_t st)
{
    switch (fs) {
    case RFX_FP2: hipLaunchKernelGGL((prefill_gateup_kernel<FG, RFX_FP2>), grid, dim3(256), 0, st, a); break;
    case RFX_FP3: hipLaunchKernelGGL((prefill_gateup_kernel<FG, RFX_FP3>), grid, dim3(256), 0, st, a); break;
    case RFX_FP4: hipLaunchKernelGGL((prefill_gateup_kernel<FG, RFX_FP4>), grid, dim3(256), 0, st, a); break;
    }
    return hip_status("prefill gate/up launch");
}

template <int FD>
int launch_down(int fsd, const FfnArgs &a, dim3 grid, hipStream_t st)
{
    switch (fsd) {
    case RFX_FP2: hipLaunchKernelGGL((prefill_down_kernel<FD, RFX_FP2>), grid, dim3(256), 0, st, a); break;
    case RFX_FP3: hipLaunchKernelGGL((prefill_down_kernel<FD, RFX_FP3>), grid, dim3(256), 0, st, a); break;
    case RFX_FP4: hipLaunchKernelGGL((prefill_down_kernel<FD, RFX_FP4>), grid, dim3(256), 0, st, a); break;
    }
    return hip_status("prefill down launch");
}

} // namespace

namespace rfx {

int prefill_route(const rfx_moe_layer *L, const float *x, int q, int k, int32_t *topk_idx, float *topk_w,
                  int32_t *pairs_sorted, int32_t *expert_off, int8_t *xq, float *xs, int32_t *xsum,
                  const MoeWs &w, hipStream_t stream)
{
    int st = rfx_quantize_act(x, q, L->hidden, xq, xs, xsum, stream);
    if (st)
        return st;
    LogitArgs la{};
    la.x = x;
    la.wr = L->router_w;
    la.wb = L->router_b;
    la.T = q;
    la.E = L->n_experts;
    la.H = L->hidden;
    la.logits = w.logits;
    hipLaunchKernelGGL(prefill_logits_kernel, dim3((q + 15) / 16, (L->n_experts + 31) / 32), dim3(64 * kLogitWaves),
                       0, stream, la);
    if ((st = hip_status("prefill logits launch")))
        return st;
    RouteArgs ra{};
    ra.logits = w.logits;
    ra.T = q;
    ra.k = k;
    ra.E = L->n_experts;
    ra.topk_idx = topk_idx;
    ra.topk_w = topk_w;
    hipLaunchKernelGGL(prefill_route_kernel, dim3((q + kRouteTB - 1) / kRouteTB), dim3(256), 0, stream, ra);
    if ((st = hip_status("prefill route launch")))
        return st;
    BucketArgs ba{};
    ba.topk_idx = topk_idx;
    ba.np = q * k;
    ba.T = q;
    ba.E = L->n_experts;
    ba.shared = L->sh_gate.data != nullptr;
    ba.pairs_sorted = pairs_sorted;
    ba.expert_off = expert_off;
    ba.items = w.items;
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(1024), 0, stream, ba);
    return hip_status("bucket launch");
}

int prefill_ffn(const rfx_moe_layer *L, int q, int k, const int8_t *xq, const float *xs, const float *topk_w,
                const int32_t *pairs_sorted, const int32_t *expert_off, const float *resid, float *y,
                const MoeWs &w, hipStream_t stream)
{
    FfnArgs a{};
    a.gate = static_cast<const uint8_t *>(L->gate.data);
    a.up = static_cast<const uint8_t *>(L->up.data);
    a.down = static_cast<const uint8_t *>(L->down.data);
    a.gate_stride = (size_t)rfx_qmat_bytes(L->gate.fmt, L->inter, L->hidden);
    a.up_stride = (size_t)rfx_qmat_bytes(L->up.fmt, L->inter, L->hidden);
    a.down_stride = (size_t)rfx_qmat_bytes(L->down.fmt, L->hidden, L->inter);
    const bool has_shared = L->sh_gate.data != nullptr;
    a.sh_gate = static_cast<const uint8_t *>(L->sh_gate.data);
    a.sh_up = static_cast<const uint8_t *>(L->sh_up.data);
    a.sh_down = static_cast<const uint8_t *>(L->sh_down.data);
    a.E = L->n_experts;
    a.H = L->hidden;
    a.I = L->inter;
    a.T = q;
    a.k = k;
    a.xq = xq;
    a.xs = xs;
    a.pairs_sorted = pairs_sorted;
    a.expert_off = expert_off;
    a.topk_w = topk_w;
    a.resid = resid;
    a.y = y;
    a.ws = w;
    const int fsg = has_shared ? L->sh_gate.fmt : L->gate.fmt;
    const int fsd = has_shared ? L->sh_down.fmt : L->down.fmt;
    const int items = prefill_max_items(q, k, L->n_experts);
    int st = 0;
    {
        const dim3 grid(L->inter / 32, items);
        switch (L->gate.fmt) {
        case RFX_FP2: st = launch_gateup<RFX_FP2>(fsg, a, grid, stream); break;
        case RFX_FP3: st = launch_gateup<RFX_FP3>(fsg, a, grid, stream); break;
        case RFX_FP4: st = launch_gateup<RFX_FP4>(fsg, a, grid, stream); break;
        }
        if (st)
            return st;
    }
    {
        const dim3 grid((L->hidden + 63) / 64, items);
        switch (L->down.fmt) {
        case RFX_FP2: st = launch_down<RFX_FP2>(fsd, a, grid, stream); break;
        case RFX_FP3: st = launch_down<RFX_FP3>(fsd, a, grid, stream); break;
        case RFX_FP4: st = launch_down<RFX_FP4>(fsd, a, grid, stream); break;
        }
        if (st)
            return st;
    }
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((L->hidden / 4 + 255) / 256, q), dim3(256), 0, stream, a,
                       has_shared);
    return hip_status("prefill combine launch");
}

} // namespace rfx
