// Prefill-sized MoE layer for gfx950: router over many tokens, stable
// bucketing of the (token, slot) pairs by expert, and the expert FFN as
// grouped matrix-core tiles with a per-block fp32 rescale.
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
// expanded through their codebooks into matrix-core operand fragments and
// multiplied with the int8 activations one 32-weight block per instruction,
// so each result is the exact integer block dot D, which is then scaled by
// the weight and activation block scales in fp32 (the same sum as the
// decode kernels, over the same blocks in the same order per output).
// The operands are the codes' integer values held as f16 (exact: at most
// 12 and 127 in magnitude) on v_mfma_f32_16x16x32_f16, whose fp32 result
// needs no conversion before the rescale.
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
// Grouped FFN on the matrix core.
//
// Each work item is up to 64 tokens of one expert. A workgroup of eight
// waves takes one item and a range of output rows; per 256-column K tile
// the item's activations are staged once into LDS as f16 operand
// fragments (direct-to-LDS loads from an f16 copy of the int8 codes, made
// once per layer), and every wave decodes the packed blocks of its own rows
// straight from memory into f16 fragments through the codebook (byte
// permutes of a table of f16 high bytes: every codebook value is a small
// integer whose f16 low byte is zero). v_mfma_f32_16x16x32_f16 then takes
// one 32-weight block per instruction: its operands are the int8 codes'
// exact integer values and its fp32 sum of 32 products (each at most
// 12 x 127, the sum below 2^24) is the exact block dot D, the integer dot
// product of the method ([HM] para 3) carried in an fp32 register. D is
// then scaled by the weight and activation block scales: one multiply and
// one fused multiply-add per output and block.
//
// MFMA operands: A = activations (lane l: token l % 16 of the token tile,
// K group l / 16 = values 8 (l / 16) .. +7 of the block), B = weights
// (lane l: row l % 16 of the row tile, the same K group); output lane l,
// register v: token 4 (l / 16) + v, row l % 16. A lane's eight weights are
// taken from the packed words in the order the bit layout stores them,
// which for every format is K order 8g .. 8g + 7.
// ------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kFfnWaves = 8;
constexpr int kFfnThreads = 64 * kFfnWaves;
constexpr int kGateRows = 16 * kFfnWaves;    // gate/up: one tile of gate and one of up per wave
constexpr int kDownRows = 32 * kFfnWaves;    // down: two row tiles per wave

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
    // test hook (DBG kernels only): fp32 h of every row, and the block dots
    // of one work item, [row][slot][block] per matrix (gate, up, down)
    float *dbg_h;
    int probe_expert, probe_first;
    int32_t *dots[3];
    const void *const *expert_data; // placement table [3][E] or null
    const uint16_t *xh; // f16 copy of xq [T][H] (workspace)
    uint16_t *hh;       // f16 copy of h~ [rows][I] (workspace)
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

// f16 high bytes of the codebook values (the low bytes are zero).
// FP2 {-3, -1, 1, 3}; FP3 {-7, -5, ..., 7}; FP4 magnitudes {0, 1, 2, 3, 4,
// 6, 8, 12} (2 x E2M1), the sign going to bit 7.
constexpr uint32_t kH2 = 0x423CBCC2u;
constexpr uint32_t kH3Lo = 0xBCC2C5C7u, kH3Hi = 0x4745423Cu;
constexpr uint32_t kH4Lo = 0x42403C00u, kH4Hi = 0x4A484644u;

// One lane's packed words of half a 256-column tile (4 blocks): per block,
// the word that holds its K group (FP3: the low-bit word, then the
// high-bit word), and its row's four block scales.
template <int F>
struct WHalf {
    uint32_t c[F == RFX_FP3 ? 8 : 4];
    uint32_t s[F == RFX_FP4 ? 1 : 2];
};

// Half hf of tile `tile`, row r (0..63), lane K group g.
template <int F>
__device__ __forceinline__ WHalf<F> load_whalf(const uint8_t *__restrict__ tile, int r, int g, int hf)
{
    WHalf<F> w;
    const uint8_t *rp = tile + r * 16;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int b = 4 * hf + j;
        if constexpr (F == RFX_FP4) {
            w.c[j] = *reinterpret_cast<const uint32_t *>(rp + b * 1024 + g * 4);
        } else {
            const uint32_t lo = *reinterpret_cast<const uint32_t *>(rp + (b >> 1) * 1024 + (b & 1) * 8 + (g >> 1) * 4);
            if constexpr (F == RFX_FP3) {
                w.c[2 * j] = lo;
                w.c[2 * j + 1] = *reinterpret_cast<const uint32_t *>(rp + (4 + hf) * 1024 + j * 4);
            } else {
                w.c[j] = lo;
            }
        }
    }
    if constexpr (F == RFX_FP4) {
        w.s[0] = *reinterpret_cast<const uint32_t *>(tile + 8192 + r * 8 + 4 * hf);
    } else {
        const u32x2 sc = *reinterpret_cast<const u32x2 *>(rp + (F == RFX_FP3 ? 6 : 4) * 1024 + 8 * hf);
        w.s[0] = sc.x;
        w.s[1] = sc.y;
    }
    return w;
}

// Weights 8g..8g+7 of block j of the half as eight f16 values.
template <int F>
__device__ __forceinline__ f16x8 wfrag(const WHalf<F> &w, int j, int g)
{
    uint32_t ha, hb; // f16 high bytes of weights 8g..8g+3 and 8g+4..8g+7
    if constexpr (F == RFX_FP4) {
        // word g: weight 8g + 4i + j at bits 8j + 4i
        const uint32_t na = w.c[j] & 0x0F0F0F0Fu, nb = (w.c[j] >> 4) & 0x0F0F0F0Fu;
        ha = __builtin_amdgcn_perm(kH4Hi, kH4Lo, na & 0x07070707u) | ((na << 4) & 0x80808080u);
        hb = __builtin_amdgcn_perm(kH4Hi, kH4Lo, nb & 0x07070707u) | ((nb << 4) & 0x80808080u);
    } else {
        // word g / 2: weight 16m + 4i + j at bits 8j + 2i; the K group
        // takes i = 2 (g % 2) and i + 1
        const uint32_t word = F == RFX_FP3 ? w.c[2 * j] : w.c[j];
        const uint32_t sh = 4u * (uint32_t)(g & 1);
        uint32_t sa = (word >> sh) & 0x03030303u, sb = (word >> (sh + 2u)) & 0x03030303u;
        if constexpr (F == RFX_FP3) {
            // high bit of weight 4i + j at bit 8j + i, i = 2g and 2g + 1
            const uint32_t h = w.c[2 * j + 1] >> (2u * (uint32_t)g);
            sa |= (h & 0x01010101u) << 2;
            sb |= ((h >> 1) & 0x01010101u) << 2;
            ha = __builtin_amdgcn_perm(kH3Hi, kH3Lo, sa);
            hb = __builtin_amdgcn_perm(kH3Hi, kH3Lo, sb);
        } else {
            ha = __builtin_amdgcn_perm(0u, kH2, sa);
            hb = __builtin_amdgcn_perm(0u, kH2, sb);
        }
    }
    const u32x4 v = {__builtin_amdgcn_perm(0u, ha, 0x010C000Cu), __builtin_amdgcn_perm(0u, ha, 0x030C020Cu),
                     __builtin_amdgcn_perm(0u, hb, 0x010C000Cu), __builtin_amdgcn_perm(0u, hb, 0x030C020Cu)};
    return __builtin_bit_cast(f16x8, v);
}

// Weight scale of block j of the half, for the lane's row.
template <int F>
__device__ __forceinline__ float wscale(const WHalf<F> &w, int j)
{
    if constexpr (F == RFX_FP4) {
        const uint32_t e = (w.s[0] >> (8 * j)) & 0xffu;
        return ldexpf(1.0f, (int)e - 128);
    } else {
        const uint32_t s2 = w.s[j >> 1];
        return half_bits_to_float((j & 1) ? (s2 >> 16) : (s2 & 0xffffu));
    }
}

// Four int8 codes -> two dwords of f16 (exact: f16 holds 1024 + u exactly
// for u = x + 128 in 0..255).
__device__ __forceinline__ void i8x4_to_f16(uint32_t x, uint32_t &p01, uint32_t &p23)
{
    const uint32_t u = x ^ 0x80808080u;
    const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    p01 = __builtin_bit_cast(uint32_t,
                             __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off);
    p23 = __builtin_bit_cast(uint32_t,
                             __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off);
}

// LDS map (bytes): two buffers of activation fragments [4 token tiles][8
// blocks][64 lanes] x 16 B (32 KB each) and of slot scales [8 blocks][64
// slots] fp32 (2 KB each); slot maps 2 x 256 B. The epilogue reuses the
// fragment area.
constexpr int kLdsFrag = 0, kLdsSx = 65536, kLdsRow = 69632, kLdsTok = 69888;
constexpr int kLdsBytes = 70144;

// Activation staging by direct loads into LDS (global_load_lds_dwordx4):
// the item's rows come from an f16 copy of the int8 codes (exact), written
// once per layer, so the K loop spends no registers and no conversion on
// them. Wave w stages block w of a K tile: fragment (tt, w) of every token
// tile tt < NT (lane l: 16 bytes of slot 16 tt + l % 16, values
// 8 (l / 16) .. + 7 of the block, which is the MFMA A-operand layout) and
// the slots' fp32 scales of the block. Slots past n read the row the slot
// map gives them (row 0) and blocks past nb the last block: their products
// are never stored (slots) or never issued (blocks).
__device__ __forceinline__ void lds_dma16(const void *src, void *lds_dst)
{
    typedef const __attribute__((address_space(1))) void *gptr;
    typedef __attribute__((address_space(3))) void *lptr;
    __builtin_amdgcn_global_load_lds((gptr)(uintptr_t)src, (lptr)(uint32_t)(uintptr_t)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ void lds_dma4(const void *src, void *lds_dst)
{
    typedef const __attribute__((address_space(1))) void *gptr;
    typedef __attribute__((address_space(3))) void *lptr;
    __builtin_amdgcn_global_load_lds((gptr)(uintptr_t)src, (lptr)(uint32_t)(uintptr_t)lds_dst, 4, 0, 0);
}

template <int NT>
struct ActDma {
    uint32_t frag[NT]; // byte offsets of the lane's fragment rows in the f16 copy
    uint32_t sc;       // byte offset of the lane's slot row of scales
};

template <int NT>
__device__ __forceinline__ ActDma<NT> act_dma_setup(const int *slot_src, size_t row_stride, int nb)
{
    const int lane = threadIdx.x & 63;
    ActDma<NT> d;
#pragma unroll
    for (int tt = 0; tt < NT; tt++)
        d.frag[tt] = (uint32_t)slot_src[16 * tt + (lane & 15)] * (uint32_t)(row_stride * 2) + 16u * (uint32_t)(lane >> 4);
    d.sc = (uint32_t)slot_src[lane] * (uint32_t)(nb * 4);
    return d;
}

template <int NT>
__device__ __forceinline__ void act_dma(const ActDma<NT> &d, const uint16_t *rows, const float *scales, int s,
                                        int nb, char *frag_buf, char *sx_buf)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int blk = min(s * 8 + wave, nb - 1);
    const char *rb = reinterpret_cast<const char *>(rows) + (size_t)blk * 64;
#pragma unroll
    for (int tt = 0; tt < NT; tt++)
        lds_dma16(rb + d.frag[tt], frag_buf + (tt * 8 + wave) * 1024);
    lds_dma4(reinterpret_cast<const char *>(scales) + (size_t)blk * 4 + d.sc, sx_buf + wave * 256);
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

// Blocks 4 hf .. 4 hf + 3 of K tile s for one wave: its M 16-row weight
// tiles w[m] (rows r0[m] .. + 15) against the item's NT token tiles.
// acc[m][tt][v]: token 16 tt + 4 (l / 16) + v, row r0[m] + l % 16. The
// token tiles run as a pipeline: tile tt's products are issued before tile
// tt - 1's results are scaled, and tile tt + 1's operands are read from LDS
// meanwhile. With DBG and dots[m] set, each block dot is also stored,
// [row][slot][block].
template <int F, int M, int NT, bool DBG, typename Hook>
__device__ __forceinline__ void ffn_half(const WHalf<F> (&w)[M], const uint32_t *frag, const float *lsx, int n,
                                         int s, int hf, int nb, float (&acc)[M][NT][4], int32_t *const (&dots)[M],
                                         const int (&r0)[M], int R, Hook &&after_first)
{
    const int lane = threadIdx.x & 63, g = lane >> 4;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const u32x4 *fr = reinterpret_cast<const u32x4 *>(frag) + lane;
    // the scale products sw(row) * sx(token) of a 16 x 16 output tile come
    // from v_mfma_f32_4x4x1_16b_f32: its output lane l, register v is
    // A(lane 4 (l / 4) + v) * B(lane l) (measured on gfx950), which is the
    // 16x16x32 product's layout (token 4 (l / 16) + v, row l % 16) when lane
    // l holds the scale of token 4 (l / 16) + l % 4 as A and its row's
    // scale as B. One product per output, rounded once: the same value as
    // the vector multiply it replaces, with four fewer VALU operations per
    // output tile and block.
    const float *sxl = lsx + 4 * g + (lane & 3);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int b = 4 * hf + j;
        if (s * 8 + b >= nb)
            break;
        f16x8 av = __builtin_bit_cast(f16x8, fr[b * 64]);
        float sa = sxl[b * 64];
        f16x8 wv[M];
        float sw[M];
#pragma unroll
        for (int m = 0; m < M; m++) {
            wv[m] = wfrag<F>(w[m], j, g);
            sw[m] = wscale<F>(w[m], j);
        }
        if (j == 0) {
            __builtin_amdgcn_sched_barrier(0);
            after_first();
            __builtin_amdgcn_sched_barrier(0);
        }
        f32x4 dp[M];
        float sa_prev = sa;
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
            f16x8 av_n = av;
            float sa_n = sa;
            if (tt + 1 < NT) {
                av_n = __builtin_bit_cast(f16x8, fr[((tt + 1) * 8 + b) * 64]);
                sa_n = sxl[b * 64 + 16 * (tt + 1)];
            }
            f32x4 dc[M];
#pragma unroll
            for (int m = 0; m < M; m++)
                dc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, wv[m], zero, 0, 0, 0);
            if (tt > 0) {
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const f32x4 sc = __builtin_amdgcn_mfma_f32_4x4x1f32(sa_prev, sw[m], zero, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; v++)
                        acc[m][tt - 1][v] = fmaf(dp[m][v], sc[v], acc[m][tt - 1][v]);
                }
            }
            if (DBG) {
#pragma unroll
                for (int m = 0; m < M; m++) {
                    if (!dots[m])
                        continue;
                    const int row = r0[m] + (lane & 15);
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        const int slot = 16 * tt + 4 * g + v;
                        if (slot < n && row < R)
                            dots[m][((size_t)row * 64 + slot) * nb + s * 8 + b] = (int)dc[m][v];
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < M; m++)
                dp[m] = dc[m];
            sa_prev = sa;
            av = av_n;
            sa = sa_n;
        }
#pragma unroll
        for (int m = 0; m < M; m++) {
            const f32x4 sc = __builtin_amdgcn_mfma_f32_4x4x1f32(sa_prev, sw[m], zero, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; v++)
                acc[m][NT - 1][v] = fmaf(dp[m][v], sc[v], acc[m][NT - 1][v]);
        }
    }
}

// The K loop of one workgroup, software-pipelined. Activations: while K
// tile s is computed from one LDS buffer, tile s + 1's rows load into
// staging registers and go to the other buffer after the compute (one
// barrier per tile). Weights: half tiles in two register sets used in
// turn, the next half loading while the current one is computed. The wave's
// M row tiles start at r0[m] in mat[m] (a wave whose rows are past R only
// stages activations). Every load is issued on every path (a wave past R
// reads row group 0, the last step re-reads its own tile), so each wait
// covers only the loads it needs: with loads under a branch the compiler
// waited for all of them before every LDS store.
template <int F, int M, int NT, bool DBG>
__device__ __forceinline__ void ffn_pipe(const uint8_t *const (&mat)[M], const int (&r0)[M], int R, int S, int nb,
                                         const uint16_t *act, const float *act_s, size_t act_stride,
                                         const int *slot_src, int n, char *smem, float (&acc)[M][NT][4],
                                         int32_t *const (&dots)[M])
{
    constexpr int TB = TileFmt<F>::bytes;
    const int lane = threadIdx.x & 63, g = lane >> 4;
    const bool rows_ok = r0[0] < R;
    const uint8_t *tb[M];
    int rin[M];
#pragma unroll
    for (int m = 0; m < M; m++) {
        const int rr = rows_ok ? r0[m] : 0;
        tb[m] = mat[m] + (size_t)(rr >> 6) * S * TB;
        rin[m] = (rr & 63) + (lane & 15);
    }
    const ActDma<NT> ad = act_dma_setup<NT>(slot_src, act_stride, nb);
    WHalf<F> wa[M], wb[M];
#pragma unroll
    for (int m = 0; m < M; m++)
        wa[m] = load_whalf<F>(tb[m], rin[m], g, 0);
    act_dma<NT>(ad, act, act_s, 0, nb, smem + kLdsFrag, smem + kLdsSx);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    for (int s = 0; s < S; s++) {
        const uint32_t *frag = reinterpret_cast<const uint32_t *>(smem + kLdsFrag + (s & 1) * 32768);
        const float *lsx = reinterpret_cast<const float *>(smem + kLdsSx + (s & 1) * 2048);
        const int sn = s + 1 < S ? s + 1 : s;
#pragma unroll
        for (int m = 0; m < M; m++)
            wb[m] = load_whalf<F>(tb[m] + (size_t)s * TB, rin[m], g, 1);
        if (rows_ok)
            ffn_half<F, M, NT, DBG>(wa, frag, lsx, n, s, 0, nb, acc, dots, r0, R, [] {});
        // The next tile's activations (direct to LDS) and its first weight
        // half are issued once this half's first block has its weights:
        // while a direct-to-LDS load is in flight the compiler waits for
        // every outstanding load (vmcnt(0)) wherever it waits for one, so
        // none may be pending where wb is waited for.
        const auto stage = [&] {
            act_dma<NT>(ad, act, act_s, sn, nb, smem + kLdsFrag + ((s + 1) & 1) * 32768,
                        smem + kLdsSx + ((s + 1) & 1) * 2048);
#pragma unroll
            for (int m = 0; m < M; m++)
                wa[m] = load_whalf<F>(tb[m] + (size_t)sn * TB, rin[m], g, 0);
        };
        if (rows_ok) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0); // wb: the only loads in flight
            ffn_half<F, M, NT, DBG>(wb, frag, lsx, n, s, 1, nb, acc, dots, r0, R, stage);
        }
        if (!rows_ok)
            stage();
        // the next tile's staging has landed in every wave before any reads it
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
    }
}

// Gate/up: one workgroup = 128 intermediate rows of gate and of up x one
// item; wave w: rows 16w..16w+15 of both. Epilogue: h = silu(g) * u and
// the per-32 requantization of h (a 32-row block is two waves' rows).
template <int F, int NT, bool DBG>
__device__ void gateup_body(const FfnArgs &a, const Item &it, const uint8_t *gm, const uint8_t *um, char *smem)
{
    const int *slot_row = reinterpret_cast<const int *>(smem + kLdsRow);
    const int *slot_tok = reinterpret_cast<const int *>(smem + kLdsTok);
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rw = blockIdx.x * kGateRows + 16 * wave; // this wave's first row
    const int S = (a.H + 255) / 256, nbH = a.H / 32;
    const bool probe = DBG && it.expert == a.probe_expert && it.first == a.probe_first;
    int32_t *const dots[2] = {probe ? a.dots[0] : nullptr, probe ? a.dots[1] : nullptr};
    const uint8_t *const mats[2] = {gm, um};
    const int r0[2] = {rw, rw};
    float acc[2][NT][4] = {};
    ffn_pipe<F, 2, NT, DBG>(mats, r0, a.I, S, nbH, a.xh, a.xs, (size_t)a.H, slot_tok, it.n, smem, acc, dots);
    const bool rows_ok = rw < a.I;

    // epilogue: h, amax over this wave's 16 rows per token, then over the
    // 32-row block (waves 2j, 2j + 1) through LDS
    float *amax_l = reinterpret_cast<float *>(smem + kLdsFrag);                   // [8 waves][64 slots]
    int8_t *hq_l = reinterpret_cast<int8_t *>(smem + kLdsFrag + kFfnWaves * 256); // [64 slots][128 rows]
    float h[NT][4], am[NT][4];
    {
#pragma clang fp contract(off)
#pragma unroll
        for (int tt = 0; tt < NT; tt++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float gv = acc[0][tt][v], uv = acc[1][tt][v];
                h[tt][v] = gv / (1.0f + expf(-gv)) * uv; // SwiGLU: silu(g) * u
                float m = fabsf(h[tt][v]);
#pragma unroll
                for (int o = 1; o < 16; o <<= 1)
                    m = fmaxf(m, __shfl_xor(m, o, 16));
                am[tt][v] = m;
            }
    }
    if (DBG && a.dbg_h && rows_ok) {
#pragma unroll
        for (int tt = 0; tt < NT; tt++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int i = 16 * tt + 4 * g + v;
                if (i < it.n)
                    a.dbg_h[(size_t)slot_row[i] * a.I + rw + (lane & 15)] = h[tt][v];
            }
    }
    if ((lane & 15) == 0) {
#pragma unroll
        for (int tt = 0; tt < NT; tt++)
#pragma unroll
            for (int v = 0; v < 4; v++)
                amax_l[wave * 64 + 16 * tt + 4 * g + v] = am[tt][v];
    }
    __syncthreads();
    {
#pragma clang fp contract(off)
#pragma unroll
        for (int tt = 0; tt < NT; tt++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int i = 16 * tt + 4 * g + v;
                const float amax = fmaxf(am[tt][v], amax_l[(wave ^ 1) * 64 + i]);
                const float sc = amax / 127.0f;
                int qv = 0;
                if (sc != 0.0f) {
                    float rr = rintf(h[tt][v] / sc);
                    rr = fminf(fmaxf(rr, -127.0f), 127.0f);
                    qv = (int)rr;
                }
                hq_l[i * kGateRows + 16 * wave + (lane & 15)] = (int8_t)qv;
                if ((wave & 1) == 0 && (lane & 15) == 0 && i < it.n && rows_ok)
                    a.ws.hs[(size_t)slot_row[i] * (a.I / 32) + (rw >> 5)] = sc;
            }
    }
    __syncthreads();
    {
        // 64 slots x 128 rows of codes, 16 bytes per thread
        const int i = tid >> 3, piece = tid & 7;
        const int row = blockIdx.x * kGateRows + 16 * piece;
        if (i < it.n && row < a.I) {
            const u32x4 c = *reinterpret_cast<const u32x4 *>(hq_l + i * kGateRows + 16 * piece);
            *reinterpret_cast<u32x4 *>(a.ws.hq + (size_t)slot_row[i] * a.I + row) = c;
            // the same codes as f16, which the down launch stages
            uint32_t f[8];
            i8x4_to_f16(c.x, f[0], f[1]);
            i8x4_to_f16(c.y, f[2], f[3]);
            i8x4_to_f16(c.z, f[4], f[5]);
            i8x4_to_f16(c.w, f[6], f[7]);
            const u32x4 f0 = {f[0], f[1], f[2], f[3]}, f1 = {f[4], f[5], f[6], f[7]};
            u32x4 *hp = reinterpret_cast<u32x4 *>(a.hh + (size_t)slot_row[i] * a.I + row);
            hp[0] = f0;
            hp[1] = f1;
        }
    }
}

template <int F, bool DBG>
__device__ void gateup_dispatch(const FfnArgs &a, const Item &it, const uint8_t *gm, const uint8_t *um, char *smem)
{
    switch ((it.n + 15) >> 4) {
    case 1: gateup_body<F, 1, DBG>(a, it, gm, um, smem); break;
    case 2: gateup_body<F, 2, DBG>(a, it, gm, um, smem); break;
    case 3: gateup_body<F, 3, DBG>(a, it, gm, um, smem); break;
    default: gateup_body<F, 4, DBG>(a, it, gm, um, smem); break;
    }
}

template <int FG, int FS, bool DBG>
__global__ __launch_bounds__(kFfnThreads, 4) void prefill_gateup_kernel(FfnArgs a)
{
    __shared__ __align__(16) char smem[kLdsBytes];
    bool ok;
    const Item it = load_item(a, blockIdx.y, ok);
    if (!ok)
        return;
    fill_slots(a, it, reinterpret_cast<int *>(smem + kLdsRow), reinterpret_cast<int *>(smem + kLdsTok));
    __syncthreads();
    if (it.expert == a.E)
        gateup_dispatch<FS, DBG>(a, it, a.sh_gate, a.sh_up, smem);
    else
        gateup_dispatch<FG, DBG>(a, it, expert_mat(a, 0, it.expert), expert_mat(a, 1, it.expert), smem);
}

// Down: one workgroup = 256 output rows x one item; wave w: rows
// 32w..32w+31 (two row tiles). o[row of slot][output row] in fp32 for the
// combine.
template <int F, int NT, bool DBG>
__device__ void down_body(const FfnArgs &a, const Item &it, const uint8_t *dm, char *smem)
{
    const int *slot_row = reinterpret_cast<const int *>(smem + kLdsRow);
    const int lane = threadIdx.x & 63, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rw = blockIdx.x * kDownRows + 32 * wave;
    const int S = (a.I + 255) / 256, nbI = a.I / 32;
    const bool probe = DBG && it.expert == a.probe_expert && it.first == a.probe_first;
    int32_t *const dots[2] = {probe ? a.dots[2] : nullptr, probe ? a.dots[2] : nullptr};
    const uint8_t *const mats[2] = {dm, dm};
    const int r0[2] = {rw, rw + 16};
    float acc[2][NT][4] = {};
    ffn_pipe<F, 2, NT, DBG>(mats, r0, a.H, S, nbI, a.hh, a.ws.hs, (size_t)a.I, slot_row, it.n, smem, acc, dots);
    if (rw >= a.H)
        return;
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const int row = r0[m] + (lane & 15);
        if (row >= a.H)
            continue;
#pragma unroll
        for (int tt = 0; tt < NT; tt++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int i = 16 * tt + 4 * g + v;
                if (i < it.n)
                    a.ws.o[(size_t)slot_row[i] * a.H + row] = acc[m][tt][v];
            }
    }
}

template <int F, bool DBG>
__device__ void down_dispatch(const FfnArgs &a, const Item &it, const uint8_t *dm, char *smem)
{
    switch ((it.n + 15) >> 4) {
    case 1: down_body<F, 1, DBG>(a, it, dm, smem); break;
    case 2: down_body<F, 2, DBG>(a, it, dm, smem); break;
    case 3: down_body<F, 3, DBG>(a, it, dm, smem); break;
    default: down_body<F, 4, DBG>(a, it, dm, smem); break;
    }
}

// Three waves per SIMD for down (152 registers with FP3 weights, none
// spilled), four for gate/up (128, where the wider occupancy paid more
// than the few spilled registers cost, measured).
template <int FD, int FSD, bool DBG>
__global__ __launch_bounds__(kFfnThreads, 3) void prefill_down_kernel(FfnArgs a)
{
    __shared__ __align__(16) char smem[kLdsBytes];
    bool ok;
    const Item it = load_item(a, blockIdx.y, ok);
    if (!ok)
        return;
    fill_slots(a, it, reinterpret_cast<int *>(smem + kLdsRow), reinterpret_cast<int *>(smem + kLdsTok));
    __syncthreads();
    if (it.expert == a.E)
        down_dispatch<FSD, DBG>(a, it, a.sh_down, smem);
    else
        down_dispatch<FD, DBG>(a, it, expert_mat(a, 2, it.expert), smem);
}

// f16 copy of the int8 token codes (exact), 16 per thread; n % 16 == 0.
__global__ __launch_bounds__(256) void codes_f16_kernel(const int8_t *xq, uint16_t *xh, size_t n)
{
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 16;
    if (i >= n)
        return;
    const u32x4 c = *reinterpret_cast<const u32x4 *>(xq + i);
    uint32_t f[8];
    i8x4_to_f16(c.x, f[0], f[1]);
    i8x4_to_f16(c.y, f[2], f[3]);
    i8x4_to_f16(c.z, f[4], f[5]);
    i8x4_to_f16(c.w, f[6], f[7]);
    const u32x4 f0 = {f[0], f[1], f[2], f[3]}, f1 = {f[4], f[5], f[6], f[7]};
    u32x4 *p = reinterpret_cast<u32x4 *>(xh + i);
    p[0] = f0;
    p[1] = f1;
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

template <int FG, bool DBG>
int launch_gateup(int fs, const FfnArgs &a, dim3 grid, hipStream_t st)
{
    switch (fs) {
    case RFX_FP2: hipLaunchKernelGGL((prefill_gateup_kernel<FG, RFX_FP2, DBG>), grid, dim3(kFfnThreads), 0, st, a); break;
    case RFX_FP3: hipLaunchKernelGGL((prefill_gateup_kernel<FG, RFX_FP3, DBG>), grid, dim3(kFfnThreads), 0, st, a); break;
    case RFX_FP4: hipLaunchKernelGGL((prefill_gateup_kernel<FG, RFX_FP4, DBG>), grid, dim3(kFfnThreads), 0, st, a); break;
    }
    return hip_status("prefill gate/up launch");
}

template <int FD, bool DBG>
int launch_down(int fsd, const FfnArgs &a, dim3 grid, hipStream_t st)
{
    switch (fsd) {
    case RFX_FP2: hipLaunchKernelGGL((prefill_down_kernel<FD, RFX_FP2, DBG>), grid, dim3(kFfnThreads), 0, st, a); break;
    case RFX_FP3: hipLaunchKernelGGL((prefill_down_kernel<FD, RFX_FP3, DBG>), grid, dim3(kFfnThreads), 0, st, a); break;
    case RFX_FP4: hipLaunchKernelGGL((prefill_down_kernel<FD, RFX_FP4, DBG>), grid, dim3(kFfnThreads), 0, st, a); break;
    }
    return hip_status("prefill down launch");
}

template <bool DBG>
int launch_ffn(const rfx_moe_layer *L, const FfnArgs &a, int items, int fsg, int fsd, hipStream_t stream)
{
    int st = 0;
    const dim3 ggrid((L->inter + kGateRows - 1) / kGateRows, items);
    switch (L->gate.fmt) {
    case RFX_FP2: st = launch_gateup<RFX_FP2, DBG>(fsg, a, ggrid, stream); break;
    case RFX_FP3: st = launch_gateup<RFX_FP3, DBG>(fsg, a, ggrid, stream); break;
    case RFX_FP4: st = launch_gateup<RFX_FP4, DBG>(fsg, a, ggrid, stream); break;
    }
    if (st)
        return st;
    const dim3 dgrid((L->hidden + kDownRows - 1) / kDownRows, items);
    switch (L->down.fmt) {
    case RFX_FP2: st = launch_down<RFX_FP2, DBG>(fsd, a, dgrid, stream); break;
    case RFX_FP3: st = launch_down<RFX_FP3, DBG>(fsd, a, dgrid, stream); break;
    case RFX_FP4: st = launch_down<RFX_FP4, DBG>(fsd, a, dgrid, stream); break;
    }
    return st;
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
                const MoeWs &w, hipStream_t stream, const PrefillDebug *dbg)
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
    a.probe_expert = -1;
    a.probe_first = -1;
    a.expert_data = L->expert_data;
    // f16 copies in the workspace's h region (prefill keeps no fp32 h); the
    // kernels address their rows with 32-bit byte offsets
    if ((size_t)(q * k + q) * L->inter * 2 >= ((size_t)1 << 32) || (size_t)q * L->hidden * 2 >= ((size_t)1 << 32))
        return fail(RFX_E_UNSUPPORTED, "prefill: f16 activation copies of %d tokens exceed 4 GiB", q);
    a.hh = reinterpret_cast<uint16_t *>(w.h);
    a.xh = a.hh + (size_t)(q * k + q) * L->inter;
    {
        const size_t n = (size_t)q * L->hidden;
        hipLaunchKernelGGL(codes_f16_kernel, dim3((unsigned)((n / 16 + 255) / 256)), dim3(256), 0, stream, xq,
                           const_cast<uint16_t *>(a.xh), n);
        int st = hip_status("prefill f16 codes launch");
        if (st)
            return st;
    }
    const int fsg = has_shared ? L->sh_gate.fmt : L->gate.fmt;
    const int fsd = has_shared ? L->sh_down.fmt : L->down.fmt;
    const int items = prefill_max_items(q, k, L->n_experts);
    if (dbg) {
        a.dbg_h = dbg->h;
        a.probe_expert = dbg->probe_expert;
        a.probe_first = dbg->probe_first;
        for (int m = 0; m < 3; m++)
            a.dots[m] = dbg->dots[m];
        return launch_ffn<true>(L, a, items, fsg, fsd, stream);
    }
    int st = launch_ffn<false>(L, a, items, fsg, fsd, stream);
    if (st)
        return st;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((L->hidden / 4 + 255) / 256, q), dim3(256), 0, stream, a,
                       has_shared);
    return hip_status("prefill combine launch");
}

} // namespace rfx
