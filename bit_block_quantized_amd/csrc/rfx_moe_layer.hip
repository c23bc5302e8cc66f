// Single-launch MoE decode layer for gfx950 (q <= 4 tokens): router
// logits, top-k and bucketing, activation quantization, every active
// expert's gate/up + SwiGLU + h requantization, down, the shared expert and
// the weighted combine (plus the residual) in one kernel.
//
// Pages cited (title, site):
//   [HM]  "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
//         (hellomarvisaitoday.com), paragraphs numbered from the top.
//   [KK]  the kaikai365.com post on DeepSeek V4 Flash on Strix Halo, by
//         section heading.
//
// [HM] para 3 verifies several positions in one fused pass, and [KK]
// (DSpark section) runs the decode step as one fused graph; decode at one
// to four tokens is bound by latency, not by bandwidth, so here the layer's
// steps overlap inside one launch instead of following each other as
// kernels. The arithmetic is that of the three-launch path (rfx_moe.hip),
// step for step and with the same split of each row group over waves, so
// the results are the same bit for bit; only the schedule differs:
//   - workgroups take roles by index: a few quantize the tokens, then the
//     router rows, then gate/up (the shared expert's row groups, then each
//     routed slot's), then down;
//   - the shared expert needs no routing, so its gate/up streams its
//     weights while the router runs;
//   - the last router workgroup publishes one 32-bit word per slot (token
//     count, expert, pair ids) once the tokens are quantized, so a routed
//     workgroup learns all it needs from the one word it polls and issues
//     its weight and activation loads at once;
//   - each down workgroup issues its first weight tile as soon as it knows
//     its expert and then waits only for its own slot's h~ (a count of the
//     slot's finished gate/up row groups);
//   - the last down workgroup of an output row group combines, as in the
//     three-launch path.
// Waits: one lane polls an agent-scope word; a producer makes its stores
// visible with an agent-scope release before it counts or publishes. A
// consumer reads data produced in the launch only after its word says the
// data is final, and no workgroup reads a line of it earlier, so no cache
// can hold an older copy (caches start the launch clean): the rows of h~
// are whole 128-byte lines when I is a multiple of 1024; otherwise a row
// can share a line with another slot's row, and the consumer invalidates
// with an agent-scope acquire before it reads. A workgroup only waits for
// workgroups of lower index, which the dispatcher places first, so no wait
// depends on a workgroup that cannot run. Each wait is also bounded in time
// (the wall clock): one that runs out sets an abort word that ends every
// other wait of the call, and a sticky error word that
// rfx_moe_forward_status reports. Every workgroup counts itself out at its
// end; the last one clears the call's counters.
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

// A bounded wait gives up after 0.2 s of the wall clock (a whole layer
// takes tens of microseconds); the tick count comes from the device's
// wall-clock rate.
constexpr int kSpinMs = 200;

// Slot word: bit 31 published, bits 28..30 token count (0: unused slot),
// bits 20..27 expert, bits 5j..5j+4 pair id j (pairs in increasing order).
constexpr unsigned kSlotPublished = 0x80000000u;

struct LayerArgs {
    FfnArgs f;
    RouteArgs r;
    unsigned *sync; // [kSyncWords]
    int n_quant;    // workgroups that quantize x (the first ones)
    int n_route;    // router workgroups (RPW expert rows each)
    int n_gu;       // gate/up workgroups: max_slots x gi
    int n_wg;       // the grid
    int max_slots;
    int gi, gh;     // row groups of 64 in inter / hidden
    int w_gu, w_dn; // waves that take tiles in a gate/up / down workgroup (the
                    // three-launch kernels' counts; the other waves idle)
    int acquire;    // rows of h~ share lines: acquire before reading them
    uint64_t spin_ticks;
};

__device__ __forceinline__ unsigned *sync_word(const LayerArgs &L, int i) { return L.sync + i * kSyncLine; }

__device__ __forceinline__ unsigned load_agent(const unsigned *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tile share [s_begin, s_end) of wave `wave` of W over S tiles; waves past
// W have none.
__device__ __forceinline__ void wave_tiles(int S, int wave, int W, int &s_begin, int &s_end)
{
    s_begin = __builtin_amdgcn_readfirstlane(wave < W ? (int)((unsigned)(S * wave) / (unsigned)W) : S);
    s_end = __builtin_amdgcn_readfirstlane(wave < W ? (int)((unsigned)(S * (wave + 1)) / (unsigned)W) : S);
}

// Lane 0: poll word `w` until done(value), bounded in time; 0 on timeout or
// abort, else the value.
template <typename Done>
__device__ __forceinline__ unsigned poll(const LayerArgs &L, int w, Done done)
{
    const unsigned *p = sync_word(L, w);
    unsigned v = load_agent(p);
    if (done(v))
        return v;
    const uint64_t t0 = wall_clock64();
    for (;;) {
        __builtin_amdgcn_s_sleep(2);
        v = load_agent(p);
        if (done(v))
            return v;
        if (load_agent(sync_word(L, kSyncAbort)) != 0u)
            return 0u;
        if (wall_clock64() - t0 > L.spin_ticks) {
            __hip_atomic_store(sync_word(L, kSyncAbort), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_or(sync_word(L, kSyncErr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return 0u;
        }
    }
}

// Every thread of the workgroup: wait until counter `w` reaches target.
// ACQ: acquire at agent scope afterwards (when L.acquire). False if the
// wait ran out or the call was aborted (the workgroup then skips its work).
template <bool ACQ>
__device__ __forceinline__ bool wait_count(const LayerArgs &L, int w, unsigned target)
{
    __shared__ int s_ok;
    __syncthreads(); // every thread has read the previous result
    if (threadIdx.x == 0) {
        const bool ok = poll(L, w, [target](unsigned v) { return v >= target; }) >= target;
        if (ACQ && L.acquire)
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_ok = ok;
    }
    __syncthreads();
    return s_ok != 0;
}

// Every thread: the routing word of `slot` (0 on timeout or abort).
__device__ __forceinline__ unsigned wait_slot(const LayerArgs &L, int slot)
{
    __shared__ unsigned s_w;
    __syncthreads();
    if (threadIdx.x == 0)
        s_w = poll(L, kSyncSlot + slot, [](unsigned v) { return (v & kSlotPublished) != 0u; });
    __syncthreads();
    return s_w;
}

// Every thread: this workgroup's stores done, then one lane adds 1 to
// counter `w` with an agent-scope release.
__device__ __forceinline__ void signal_add(const LayerArgs &L, int w)
{
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(sync_word(L, w), 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------
// Quantization role: the tokens' blocks over the n_quant workgroups.
// Router role: RPW expert rows per workgroup (256 threads each), the
// logits as in route_kernel, two-level arrival; the last workgroup picks
// the top k, buckets the pairs and, once the tokens are quantized,
// publishes the slot words.
// ------------------------------------------------------------------

// The last router workgroup, after route_select: one word per slot, slots
// in the three-launch kernels' order (the shared expert first, then the
// routed experts with pairs in id order). s_idx[p] is the expert of pair p.
__device__ __forceinline__ void publish_slots(const LayerArgs &L, const int *s_idx)
{
    const RouteArgs &a = L.r;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int np = a.q * a.k;
    __shared__ int s_cnt[4];
    __shared__ unsigned s_word[kMaxSlots];
    int ne = 0;
    unsigned pk = 0;
    if (tid < a.E) { // expert e = tid: its pairs in increasing order (at most q)
        for (int p = 0; p < np; p++)
            if (s_idx[p] == tid) {
                pk |= (unsigned)p << (5 * ne);
                ne++;
            }
    }
    const unsigned long long bal = __ballot(ne > 0);
    if (lane == 0 && wave < 4)
        s_cnt[wave] = __popcll(bal);
    if (tid < kMaxSlots)
        s_word[tid] = kSlotPublished; // unused unless an expert takes it
    __syncthreads();
    if (ne > 0) {
        int rank = __popcll(bal & ((1ull << lane) - 1ull));
        for (int w = 0; w < wave; w++)
            rank += s_cnt[w];
        s_word[rank + (L.f.has_shared ? 1 : 0)] = kSlotPublished | ((unsigned)ne << 28) | ((unsigned)tid << 20) | pk;
    }
    // the route outputs (plain stores) out before the words
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        for (int s = L.f.has_shared ? 1 : 0; s < L.max_slots; s++)
            __hip_atomic_store(sync_word(L, kSyncSlot + s), s_word[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int RPW, int QMAX>
__device__ __forceinline__ void route_role(const LayerArgs &L, int r)
{
    const RouteArgs &a = L.r;
    constexpr int W = 4 * RPW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sub = wave >> 2, t8 = tid & 255;
    const int e = r * RPW + sub;
    const bool has_row = e < a.E;
    __shared__ float s_part[W][QMAX];
    __shared__ int s_last;
    __shared__ __align__(16) int s_idx[kMaxDecodeQ * kMaxK];

    // row e of Wr: up to 8 float4 columns per thread (h = 4 t8 + 1024 i)
    const float *wrow = a.wr + (size_t)(has_row ? e : 0) * a.H;
    float4 w4[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int h = t8 * 4 + 1024 * i;
        w4[i] = has_row && h < a.H ? *reinterpret_cast<const float4 *>(wrow + h) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // one token at a time (x stays in 32 registers); per thread, the lane
    // butterfly, then the row's four waves in order, as in route_kernel
    float part[QMAX];
#pragma unroll
    for (int t = 0; t < QMAX; t++) {
        part[t] = 0.0f;
        if (t < a.q) {
            float4 x4[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int h = t8 * 4 + 1024 * i;
                x4[i] = h < a.H ? *reinterpret_cast<const float4 *>(a.x + (size_t)t * a.H + h)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int i = 0; i < 8; i++)
                part[t] = dot4_acc(part[t], w4[i], x4[i]);
        }
        for (int o = 32; o > 0; o >>= 1)
            part[t] += __shfl_xor(part[t], o, 64);
    }
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < QMAX; t++)
            s_part[wave][t] = part[t];
    }
    __syncthreads();
    if (has_row && t8 < a.q) {
        const int w0 = 4 * sub;
        const float l = ((s_part[w0][t8] + s_part[w0 + 1][t8]) + s_part[w0 + 2][t8]) + s_part[w0 + 3][t8];
        __hip_atomic_store(a.logits + (size_t)t8 * a.E + e, a.wb ? l + a.wb[e] : l, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // arrival over the n_route workgroups, in two levels
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    const int ngroups = (L.n_route + kRouteGroup - 1) / kRouteGroup;
    if (tid == 0) {
        const int g = r / kRouteGroup;
        const unsigned gsize = (unsigned)min(kRouteGroup, L.n_route - g * kRouteGroup);
        bool last = false;
        if (__hip_atomic_fetch_add(a.cnt + kRouteCntStride * g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            gsize - 1)
            last = __hip_atomic_fetch_add(a.cnt + kRouteCntStride * kRouteMaxGroups, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == (unsigned)ngroups - 1;
        s_last = last;
    }
    __syncthreads();
    if (s_last) {
        route_select(a, ngroups, s_idx);
        if (wait_count<false>(L, kSyncXq, (unsigned)L.n_quant))
            publish_slots(L, s_idx);
    }
}

template <int RPW>
__device__ __forceinline__ void quant_role(const LayerArgs &L, int r)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    route_quant(L.r, r, L.n_quant, 4 * RPW, wave, lane);
    signal_add(L, kSyncXq);
}

// ------------------------------------------------------------------
// Gate/up role. Weight tiles are issued first, then the wait for the
// quantized tokens, then the activation slices; the loop and the finish
// are those of the three-launch kernel. Every column count takes the
// matrix-core dots (the one-column scalar-operand path of the three-launch
// kernel reads the activations through the scalar cache, which does not
// see data written during the launch); both give the same exact dots and
// the same fp32 sums.
// ------------------------------------------------------------------

// Columns of a slot: the shared expert's are the tokens themselves; a
// routed slot's come from its word.
template <int NE>
__device__ __forceinline__ SlotCols<NE> slot_cols_word(bool shared, unsigned word, const FfnArgs &a)
{
    SlotCols<NE> c;
#pragma unroll
    for (int j = 0; j < NE; j++) {
        if (shared) {
            c.token[j] = j;
            c.out_idx[j] = a.q * a.k + j;
        } else {
            const int p = (int)((word >> (5 * j)) & 31u);
            c.token[j] = p / a.k;
            c.out_idx[j] = p;
        }
    }
    return c;
}

template <int NE>
__device__ __forceinline__ XCols<NE> xcols(const int8_t *xq, const float *xs, const int32_t *xsum,
                                           const int (&row)[NE], int len)
{
    XCols<NE> xc;
    xc.xq = xq;
    xc.xs = xs;
    xc.xsum = xsum;
#pragma unroll
    for (int j = 0; j < NE; j++) {
        xc.xoff[j] = (uint32_t)row[j] * (uint32_t)len;
        xc.moff[j] = (uint32_t)row[j] * (uint32_t)(len / 32);
    }
    return xc;
}

// What a gate/up or down workgroup knows of its slot.
struct Slot {
    bool shared;
    int expert;
    unsigned word;
};

template <int FG, int NE>
struct GUTileM {
    TileRegs<FG> g, u;
    XTileM<NE> x;
};

template <int FG, int NE>
__device__ __forceinline__ bool gu_body(const LayerArgs &L, const Slot &sl, int g, int lane, int wave, int W,
                                        float *red)
{
    const FfnArgs &a = L.f;
    constexpr int TB = TileFmt<FG>::bytes;
    const int nbH = a.H / 32, S = (a.H + 255) / 256;
    const uint8_t *gm = (sl.shared ? a.sh_gate : expert_mat(a, 0, sl.expert)) + (size_t)g * S * TB;
    const uint8_t *um = (sl.shared ? a.sh_up : expert_mat(a, 1, sl.expert)) + (size_t)g * S * TB;
    int s_begin, s_end;
    wave_tiles(S, wave, W, s_begin, s_end);
    // the first two tiles' weights go out at once (a routed slot's tokens
    // are quantized before its word is published; the shared slot waits
    // for them after issuing its weights); the loop then has the
    // three-launch kernel's shape (tile s + 1 issued before tile s is
    // computed: two tiles of registers)
    GUTileM<FG, NE> ta, tb;
    if (s_begin < s_end) {
        ta.g = load_tile<FG>(gm + (size_t)s_begin * TB, lane);
        ta.u = load_tile<FG>(um + (size_t)s_begin * TB, lane);
    }
    if (s_begin + 1 < s_end) {
        tb.g = load_tile<FG>(gm + (size_t)(s_begin + 1) * TB, lane);
        tb.u = load_tile<FG>(um + (size_t)(s_begin + 1) * TB, lane);
    }
    if (sl.shared && !wait_count<false>(L, kSyncXq, (unsigned)L.n_quant))
        return false;
    const SlotCols<NE> cols = slot_cols_word<NE>(sl.shared, sl.word, a);
    const XCols<NE> xc = xcols<NE>(a.xq, a.xs, a.xsum, cols.token, a.H);
    float ag[NE], au[NE];
#pragma unroll
    for (int j = 0; j < NE; j++) {
        ag[j] = 0.0f;
        au[j] = 0.0f;
    }
    if (s_begin < s_end) {
        ta.x = load_xtile_m<FG, NE, false>(xc, s_begin, nbH, lane);
        if (s_begin + 1 < s_end)
            tb.x = load_xtile_m<FG, NE, false>(xc, s_begin + 1, nbH, lane);
        for (int s = s_begin; s < s_end; s += 2) {
            if (s > s_begin && s + 1 < s_end) {
                tb.x = load_xtile_m<FG, NE, false>(xc, s + 1, nbH, lane);
                tb.g = load_tile<FG>(gm + (size_t)(s + 1) * TB, lane);
                tb.u = load_tile<FG>(um + (size_t)(s + 1) * TB, lane);
            }
            tile_blocks2_mfma<FG, NE, false>(ta.g, ta.u, ta.x, s * 8, nbH, ag, au);
            if (s + 1 >= s_end)
                break;
            if (s + 2 < s_end) {
                ta.x = load_xtile_m<FG, NE, false>(xc, s + 2, nbH, lane);
                ta.g = load_tile<FG>(gm + (size_t)(s + 2) * TB, lane);
                ta.u = load_tile<FG>(um + (size_t)(s + 2) * TB, lane);
            }
            tile_blocks2_mfma<FG, NE, false>(tb.g, tb.u, tb.x, (s + 1) * 8, nbH, ag, au);
        }
    }
#pragma unroll
    for (int j = 0; j < NE; j++) {
        red[((wave * 2 + 0) * kMaxDecodeQ + j) * 64 + lane] = ag[j];
        red[((wave * 2 + 1) * kMaxDecodeQ + j) * 64 + lane] = au[j];
    }
    __syncthreads();
    if (wave == 0)
        gateup_finish<NE>(a, cols, g, lane, W, red);
    return true;
}

// FP4 gate/up on the block-scaled matrix core, one tile buffer (as the
// three-launch kernel), the first tile issued before the wait.
template <int NE>
__device__ __forceinline__ bool gu_body_mx(const LayerArgs &L, const Slot &sl, int g, int lane, int wave, int W,
                                           float *red)
{
    const FfnArgs &a = L.f;
    constexpr int TB = TileFmt<RFX_FP4>::bytes;
    const int nbH = a.H / 32, S = (a.H + 255) / 256;
    const uint8_t *gm = (sl.shared ? a.sh_gate : expert_mat(a, 0, sl.expert)) + (size_t)g * S * TB;
    const uint8_t *um = (sl.shared ? a.sh_up : expert_mat(a, 1, sl.expert)) + (size_t)g * S * TB;
    int s_begin, s_end;
    wave_tiles(S, wave, W, s_begin, s_end);
    MxW w[2];
    if (s_begin < s_end) {
        w[0] = load_mx_w(gm + (size_t)s_begin * TB, lane);
        w[1] = load_mx_w(um + (size_t)s_begin * TB, lane);
    }
    if (sl.shared && !wait_count<false>(L, kSyncXq, (unsigned)L.n_quant))
        return false;
    const SlotCols<NE> cols = slot_cols_word<NE>(sl.shared, sl.word, a);
    const XCols<NE> xc = xcols<NE>(a.xq, a.xs, a.xsum, cols.token, a.H);
    const MxLane<NE> ml = mx_lane<NE>(lane, xc);
    float acc[2][4][4];
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int v = 0; v < 4; v++)
                acc[m][i][v] = 0.0f;
    for (int s = s_begin; s < s_end; s++) {
        if (s > s_begin) {
            w[0] = load_mx_w(gm + (size_t)s * TB, lane);
            w[1] = load_mx_w(um + (size_t)s * TB, lane);
        }
        const MxX<NE> x = load_mx_x<NE, false>(s, nbH, xc, ml);
        compute_mx<NE, 2>(w, x, ml, acc);
    }
#pragma unroll
    for (int m = 0; m < 2; m++)
        mx_rows<NE>(acc[m], lane, [&](int col, int row, float v) {
            red[((wave * 2 + m) * kMaxDecodeQ + col) * 64 + row] = v;
        });
    __syncthreads();
    if (wave == 0)
        gateup_finish<NE>(a, cols, g, lane, W, red);
    return true;
}

// Format F with NE columns: the block-scaled matrix core for FP4 up to
// MXMAX columns, else the int8 matrix-core dots.
template <int F, int NE, int MXMAX>
__device__ __forceinline__ bool gu_any(const LayerArgs &L, const Slot &sl, int g, int lane, int wave, int W,
                                       float *red)
{
    if constexpr (F == RFX_FP4 && NE <= MXMAX)
        return gu_body_mx<NE>(L, sl, g, lane, wave, W, red);
    else
        return gu_body<F, NE>(L, sl, g, lane, wave, W, red);
}

template <int F, int MXMAX, int QMAX>
__device__ __forceinline__ bool gu_ne(int ne, const LayerArgs &L, const Slot &sl, int g, int lane, int wave, int W,
                                      float *red)
{
    switch (ne) {
    case 1: return gu_any<F, 1, MXMAX>(L, sl, g, lane, wave, W, red);
    case 2:
        if constexpr (QMAX >= 2)
            return gu_any<F, 2, MXMAX>(L, sl, g, lane, wave, W, red);
        break;
    case 3:
        if constexpr (QMAX >= 3)
            return gu_any<F, 3, MXMAX>(L, sl, g, lane, wave, W, red);
        break;
    case 4:
        if constexpr (QMAX >= 4)
            return gu_any<F, 4, MXMAX>(L, sl, g, lane, wave, W, red);
        break;
    default: break;
    }
    return false;
}

// The slot of a gate/up or down workgroup: the shared expert's at once,
// a routed one's from its published word. ne = 0: unused slot (or the
// wait ran out, when the word is 0).
__device__ __forceinline__ Slot find_slot_word(const LayerArgs &L, int slot, int &ne)
{
    Slot sl;
    if (slot == 0 && L.f.has_shared) {
        sl.shared = true;
        sl.expert = -1;
        sl.word = 0;
        ne = L.f.q;
    } else {
        sl.shared = false;
        sl.word = wait_slot(L, slot);
        sl.expert = (int)((sl.word >> 20) & 255u);
        ne = (int)((sl.word >> 28) & 7u);
    }
    return sl;
}

template <int FG, int FS, int QMAX>
__device__ __forceinline__ void gateup_role(const LayerArgs &L, int u, float *red)
{
    const int slot = u / L.gi, g = u - slot * L.gi;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int ne;
    const Slot sl = find_slot_word(L, slot, ne);
    if (ne == 0)
        return;
    // FP4 on the block-scaled matrix core as in the three-launch kernel:
    // the shared expert at any token count, routed slots at one or two
    const bool ok = sl.shared ? gu_ne<FS, 4, QMAX>(ne, L, sl, g, lane, wave, L.w_gu, red)
                              : gu_ne<FG, 2, QMAX>(ne, L, sl, g, lane, wave, L.w_gu, red);
    if (ok)
        signal_add(L, kSyncH + slot);
}

// ------------------------------------------------------------------
// Down role: the first weight tile, then the wait for the slot's h~, then
// the activation slices; the finish and the combine are those of the
// three-launch kernel.
// ------------------------------------------------------------------
template <int FD, int NE>
struct DTileM {
    TileRegs<FD> w;
    XTileM<NE> x;
};

template <int FD, int NE>
__device__ __forceinline__ bool dn_body(const LayerArgs &L, const Slot &sl, int slot, int g, int lane, int wave,
                                        int W, float *red)
{
    const FfnArgs &a = L.f;
    constexpr int TB = TileFmt<FD>::bytes;
    const int nbI = a.I / 32, S = (a.I + 255) / 256;
    const uint8_t *dm = (sl.shared ? a.sh_down : expert_mat(a, 2, sl.expert)) + (size_t)g * S * TB;
    int s_begin, s_end;
    wave_tiles(S, wave, W, s_begin, s_end);
    DTileM<FD, NE> da, db;
    if (s_begin < s_end)
        da.w = load_tile<FD>(dm + (size_t)s_begin * TB, lane);
    if (s_begin + 1 < s_end)
        db.w = load_tile<FD>(dm + (size_t)(s_begin + 1) * TB, lane);
    if (!wait_count<true>(L, kSyncH + slot, (unsigned)L.gi))
        return false;
    const SlotCols<NE> cols = slot_cols_word<NE>(sl.shared, sl.word, a);
    const XCols<NE> xc = xcols<NE>(a.ws.hq, a.ws.hs, a.ws.hsum, cols.out_idx, a.I);
    float ao[NE];
#pragma unroll
    for (int j = 0; j < NE; j++)
        ao[j] = 0.0f;
    if (s_begin < s_end) {
        da.x = load_xtile_m<FD, NE, false>(xc, s_begin, nbI, lane);
        if (s_begin + 1 < s_end)
            db.x = load_xtile_m<FD, NE, false>(xc, s_begin + 1, nbI, lane);
        for (int s = s_begin; s < s_end; s += 2) {
            if (s > s_begin && s + 1 < s_end) {
                db.x = load_xtile_m<FD, NE, false>(xc, s + 1, nbI, lane);
                db.w = load_tile<FD>(dm + (size_t)(s + 1) * TB, lane);
            }
            tile_blocks_mfma<FD, NE, false>(da.w, da.x, s * 8, nbI, ao);
            if (s + 1 >= s_end)
                break;
            if (s + 2 < s_end) {
                da.x = load_xtile_m<FD, NE, false>(xc, s + 2, nbI, lane);
                da.w = load_tile<FD>(dm + (size_t)(s + 2) * TB, lane);
            }
            tile_blocks_mfma<FD, NE, false>(db.w, db.x, (s + 1) * 8, nbI, ao);
        }
    }
#pragma unroll
    for (int j = 0; j < NE; j++)
        red[(wave * kMaxDecodeQ + j) * 64 + lane] = ao[j];
    __syncthreads();
    if (wave == 0)
        down_finish<NE>(a, cols, g, lane, W, red);
    return true;
}

// FP4 down with one or two tokens on the block-scaled matrix core.
template <int NE>
__device__ __forceinline__ bool dn_body_mx(const LayerArgs &L, const Slot &sl, int slot, int g, int lane, int wave,
                                           int W, float *red)
{
    const FfnArgs &a = L.f;
    constexpr int TB = TileFmt<RFX_FP4>::bytes;
    const int nbI = a.I / 32, S = (a.I + 255) / 256;
    const uint8_t *dm = (sl.shared ? a.sh_down : expert_mat(a, 2, sl.expert)) + (size_t)g * S * TB;
    int s_begin, s_end;
    wave_tiles(S, wave, W, s_begin, s_end);
    MxW w;
    if (s_begin < s_end)
        w = load_mx_w(dm + (size_t)s_begin * TB, lane);
    if (!wait_count<true>(L, kSyncH + slot, (unsigned)L.gi))
        return false;
    const SlotCols<NE> cols = slot_cols_word<NE>(sl.shared, sl.word, a);
    const XCols<NE> xc = xcols<NE>(a.ws.hq, a.ws.hs, a.ws.hsum, cols.out_idx, a.I);
    const MxLane<NE> ml = mx_lane<NE>(lane, xc);
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int v = 0; v < 4; v++)
            acc[i][v] = 0.0f;
    for (int s = s_begin; s < s_end; s++) {
        MxTile<NE> t;
        t.w = s > s_begin ? load_mx_w(dm + (size_t)s * TB, lane) : w;
        t.x = load_mx_x<NE, false>(s, nbI, xc, ml);
        compute_mx_tile<NE>(t, ml, acc);
    }
    mx_rows<NE>(acc, lane, [&](int col, int row, float v) { red[(wave * kMaxDecodeQ + col) * 64 + row] = v; });
    __syncthreads();
    if (wave == 0)
        down_finish<NE>(a, cols, g, lane, W, red);
    return true;
}

template <int F, int NE>
__device__ __forceinline__ bool dn_any(const LayerArgs &L, const Slot &sl, int slot, int g, int lane, int wave, int W,
                                       float *red)
{
    if constexpr (F == RFX_FP4 && NE <= 2)
        return dn_body_mx<NE>(L, sl, slot, g, lane, wave, W, red);
    else
        return dn_body<F, NE>(L, sl, slot, g, lane, wave, W, red);
}

template <int F, int QMAX>
__device__ __forceinline__ bool dn_ne(int ne, const LayerArgs &L, const Slot &sl, int slot, int g, int lane,
                                      int wave, int W, float *red)
{
    switch (ne) {
    case 1: return dn_any<F, 1>(L, sl, slot, g, lane, wave, W, red);
    case 2:
        if constexpr (QMAX >= 2)
            return dn_any<F, 2>(L, sl, slot, g, lane, wave, W, red);
        break;
    case 3:
        if constexpr (QMAX >= 3)
            return dn_any<F, 3>(L, sl, slot, g, lane, wave, W, red);
        break;
    case 4:
        if constexpr (QMAX >= 4)
            return dn_any<F, 4>(L, sl, slot, g, lane, wave, W, red);
        break;
    default: break;
    }
    return false;
}

template <int FD, int FSD, int QMAX>
__device__ __forceinline__ void down_role(const LayerArgs &L, int d, float *red)
{
    const FfnArgs &a = L.f;
    const int slot = d / L.gh, g = d - slot * L.gh;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int ne;
    const Slot sl = find_slot_word(L, slot, ne);
    if (!sl.shared && sl.word == 0)
        return; // the wait ran out
    if (ne > 0) {
        const bool ok = sl.shared ? dn_ne<FSD, QMAX>(ne, L, sl, slot, g, lane, wave, L.w_dn, red)
                                  : dn_ne<FD, QMAX>(ne, L, sl, slot, g, lane, wave, L.w_dn, red);
        if (!ok)
            return;
    }
    // every slot of this output row group arrives (an unused one at once);
    // the last combines
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    __shared__ int s_last;
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(a.ws.comb_cnt + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (unsigned)(L.max_slots - 1);
    __syncthreads();
    if (!s_last)
        return;
    if (wave == 0)
        combine_rows(a, g, lane);
    if (threadIdx.x == 0)
        __hip_atomic_store(a.ws.comb_cnt + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every workgroup at its end (past all its waits): count out in two levels;
// the last clears the call's counters (the sticky error word stays).
__device__ __forceinline__ void layer_exit(const LayerArgs &L, int b)
{
    __syncthreads();
    if (threadIdx.x != 0)
        return;
    const int grp = b / kExitGroup, ngrp = (L.n_wg + kExitGroup - 1) / kExitGroup;
    const unsigned gsize = (unsigned)min(kExitGroup, L.n_wg - grp * kExitGroup);
    if (__hip_atomic_fetch_add(sync_word(L, kSyncExit + grp), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
        gsize - 1)
        return;
    if (__hip_atomic_fetch_add(sync_word(L, kSyncExitTop), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
        (unsigned)ngrp - 1)
        return;
    const int words[] = {kSyncXq, kSyncAbort, kSyncExitTop};
    for (int w : words)
        __hip_atomic_store(sync_word(L, w), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int s = 0; s < L.max_slots; s++) {
        __hip_atomic_store(sync_word(L, kSyncH + s), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(sync_word(L, kSyncSlot + s), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int g = 0; g < ngrp; g++)
        __hip_atomic_store(sync_word(L, kSyncExit + g), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FG, int FS, int FD, int FSD, int RPW, int QMAX>
__global__ __launch_bounds__(256 * RPW) void layer_kernel(LayerArgs L)
{
    __shared__ float red[4 * RPW * 2 * kMaxDecodeQ * 64];
    const int b = blockIdx.x, r0 = L.n_quant, g0 = r0 + L.n_route, d0 = g0 + L.n_gu;
    if (b < r0)
        quant_role<RPW>(L, b);
    else if (b < g0)
        route_role<RPW, QMAX>(L, b - r0);
    else if (b < d0)
        gateup_role<FG, FS, QMAX>(L, b - g0, red);
    else
        down_role<FD, FSD, QMAX>(L, b - d0, red);
    layer_exit(L, b);
}

// Router rows per workgroup (256 threads each): the block must hold the
// gate/up and down wave counts.
int rows_per_wg(int w_gu, int w_dn) { return w_gu > 4 || w_dn > 4 ? 2 : 1; }

// Wall-clock ticks in kSpinMs on the current device (cached per device).
uint64_t spin_ticks()
{
    static uint64_t ticks[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 100000ull * kSpinMs;
    if (!ticks[dev]) {
        int khz = 0;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
            khz = 100000;
        ticks[dev] = (uint64_t)khz * kSpinMs;
    }
    return ticks[dev];
}

template <int RPW, int QMAX>
void launch_one(const LayerArgs &L, hipStream_t stream)
{
    hipLaunchKernelGGL((layer_kernel<RFX_FP2, RFX_FP4, RFX_FP3, RFX_FP4, RPW, QMAX>), dim3(L.n_wg), dim3(256 * RPW),
                       0, stream, L);
}

} // namespace

namespace rfx {
namespace moe {

bool layer_kernel_takes(const FfnArgs &f, int q, int k)
{
    if (q < 1 || q > kMaxDecodeQ || f.H > 8192 || f.E > 256)
        return false;
    if (f.fmt_g != RFX_FP2 || f.fmt_u != RFX_FP2 || f.fmt_d != RFX_FP3)
        return false;
    if (f.has_shared && (f.fmt_sg != RFX_FP4 || f.fmt_su != RFX_FP4 || f.fmt_sd != RFX_FP4))
        return false;
    const int max_slots = (q * k < f.E ? q * k : f.E) + (f.has_shared ? 1 : 0);
    const int gi = (int)ceil_div(f.I, 64), gh = (int)ceil_div(f.H, 64);
    const int rpw = rows_per_wg(waves_for(max_slots * gi, (int)ceil_div(f.H, 256), kMaxFfnWaves, kGateUpWaveTarget),
                                waves_for(max_slots * gh, (int)ceil_div(f.I, 256), kMaxFfnWaves, kDownWaveTarget));
    const int64_t n_wg = ceil_div((int64_t)q * (f.H / 32), 8 * rpw) + ceil_div(f.E, rpw) + (int64_t)max_slots * (gi + gh);
    return n_wg <= (int64_t)kMaxExitGroups * kExitGroup;
}

int launch_layer(const FfnArgs &f, const RouteArgs &r, hipStream_t stream)
{
    LayerArgs L{};
    L.f = f;
    L.r = r;
    L.sync = f.ws.sync;
    const int q = f.q, k = f.k;
    L.max_slots = (q * k < f.E ? q * k : f.E) + (f.has_shared ? 1 : 0);
    L.gi = (int)ceil_div(f.I, 64);
    L.gh = (int)ceil_div(f.H, 64);
    L.w_gu = waves_for(L.max_slots * L.gi, (int)ceil_div(f.H, 256), kMaxFfnWaves, kGateUpWaveTarget);
    L.w_dn = waves_for(L.max_slots * L.gh, (int)ceil_div(f.I, 256), kMaxFfnWaves, kDownWaveTarget);
    const int rpw = rows_per_wg(L.w_gu, L.w_dn), W = 4 * rpw;
    L.n_route = (int)ceil_div(f.E, rpw);
    L.n_quant = (int)ceil_div((int64_t)q * (f.H / 32), 2 * W); // two blocks per wave
    L.n_gu = L.max_slots * L.gi;
    L.n_wg = L.n_quant + L.n_route + L.n_gu + L.max_slots * L.gh;
    L.acquire = f.I % 1024 != 0;
    L.spin_ticks = spin_ticks();
    const int qm = q == 1 ? 1 : q == 2 ? 2 : 4;
    switch (rpw * 8 + qm) {
    case 2 * 8 + 1: launch_one<2, 1>(L, stream); break;
    case 2 * 8 + 2: launch_one<2, 2>(L, stream); break;
    case 2 * 8 + 4: launch_one<2, 4>(L, stream); break;
    case 1 * 8 + 1: launch_one<1, 1>(L, stream); break;
    case 1 * 8 + 2: launch_one<1, 2>(L, stream); break;
    default: launch_one<1, 4>(L, stream); break;
    }
    return hip_status("MoE layer launch");
}

} // namespace moe
} // namespace rfx
