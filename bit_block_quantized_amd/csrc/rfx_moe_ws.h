// MoE layer workspace layout and the limits shared by the decode (q <= 4)
// and prefill (q > 4) paths.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "rfx.h"

namespace rfx {

constexpr int kMaxK = 8;          // experts per token
constexpr int kMaxE = 256;        // routed experts per layer
constexpr int kMaxDecodeQ = 4;    // tokens handled by the decode kernels
constexpr int kMaxFfnWaves = 8;   // waves per decode FFN workgroup
constexpr int kPrefillChunk = 64; // tokens per work item of the prefill kernels
constexpr int kMaxPrefillQ = 1 << 16;
// Arrival counters of the decode router: one per kRouteGroup workgroups,
// then one over the groups, each on its own 128-byte line.
constexpr int kRouteGroup = 16;
constexpr int kRouteMaxGroups = kMaxE / kRouteGroup;
constexpr int kRouteCntStride = 32; // 32-bit words between counters

// Counters of the single-launch decode layer kernel (rfx_moe_layer.hip),
// each on its own 128-byte line: activation quantization done, abort (a
// bounded wait ran out), the sticky timeout word, the exit count over the
// groups; then per slot the gate/up row groups done (h~ of the slot
// complete) and the slot's routing word (published bit, token count,
// expert, pair ids); then the exit count per group of kExitGroup
// workgroups.
constexpr int kSyncLine = 32; // 32-bit words per counter line
constexpr int kSyncXq = 0, kSyncAbort = 1, kSyncErr = 2, kSyncExitTop = 3, kSyncH = 4;
constexpr int kMaxSlots = kMaxDecodeQ * kMaxK + 1;
constexpr int kSyncSlot = kSyncH + kMaxSlots;
constexpr int kSyncExit = kSyncSlot + kMaxSlots;
constexpr int kExitGroup = 64;
constexpr int kMaxExitGroups = 128; // at most 8192 workgroups per launch
constexpr int kSyncWords = (kSyncExit + kMaxExitGroups) * kSyncLine;

// Work items of the prefill FFN: (expert, first token) per chunk of up to
// kPrefillChunk tokens of one expert, then the shared expert's chunks.
inline int prefill_max_items(int q, int k, int E)
{
    return E + (q * k + kPrefillChunk - 1) / kPrefillChunk + (q + kPrefillChunk - 1) / kPrefillChunk;
}

// Workspace regions (bytes, 256-aligned). Zero-filled once by the caller;
// counters return to zero at the end of every call. Rows of h, hq, hs,
// hsum and o are indexed by pair id t*k + j, then q*k + t for the shared
// expert.
struct MoeWs {
    float *logits;      // [q][E] (decode)
    unsigned *route_cnt; // [kRouteMaxGroups + 1] counters, kRouteCntStride words apart
    float *h;           // [NP][I]   NP = q*k + q (decode keeps it for inspection; prefill
                        // holds f16 copies of h~ [NP][I] and of the token codes [q][H] here)
    int8_t *hq;         // [NP][I]
    float *hs;          // [NP][I/32]
    int32_t *hsum;      // [NP][I/32]
    float *o;           // [NP][H]
    unsigned *comb_cnt; // [H/64 + 1]
    int32_t *items;     // [0] = count, then (expert, first token) pairs (prefill)
    unsigned *sync;     // [kSyncWords] counters of the single-launch decode kernel
    size_t bytes;
};

inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }

inline MoeWs carve(void *base, int q, int k, int E, int H, int I)
{
    MoeWs w{};
    const size_t NP = (size_t)q * k + q;
    size_t off = 0;
    auto take = [&](size_t n) -> size_t {
        const size_t o = off;
        off += align256(n);
        return o;
    };
    const size_t o_logits = take((size_t)q * E * 4);
    const size_t o_rc = take((size_t)(kRouteMaxGroups + 1) * kRouteCntStride * 4);
    // prefill (q > kMaxDecodeQ) keeps no fp32 h: the region holds f16 copies
    // of h~ ([NP][I]) and of the token codes ([q][H]) instead
    const size_t h_bytes = q > kMaxDecodeQ ? (NP * I * 2 + (size_t)q * H * 2 > NP * I * 4 ? NP * I * 2 + (size_t)q * H * 2 : NP * I * 4) : NP * I * 4;
    const size_t o_h = take(h_bytes);
    const size_t o_hq = take(NP * I);
    const size_t o_hs = take(NP * (I / 32) * 4);
    const size_t o_hsum = take(NP * (I / 32) * 4);
    const size_t o_o = take(NP * H * 4);
    const size_t o_cc = take((size_t)(H / 64 + 1) * 4);
    const size_t o_it = take((size_t)(1 + 2 * prefill_max_items(q, k, E)) * 4);
    const size_t o_sy = take((size_t)kSyncWords * 4);
    w.bytes = off;
    char *b = static_cast<char *>(base);
    if (b) {
        w.logits = reinterpret_cast<float *>(b + o_logits);
        w.route_cnt = reinterpret_cast<unsigned *>(b + o_rc);
        w.h = reinterpret_cast<float *>(b + o_h);
        w.hq = reinterpret_cast<int8_t *>(b + o_hq);
        w.hs = reinterpret_cast<float *>(b + o_hs);
        w.hsum = reinterpret_cast<int32_t *>(b + o_hsum);
        w.o = reinterpret_cast<float *>(b + o_o);
        w.comb_cnt = reinterpret_cast<unsigned *>(b + o_cc);
        w.items = reinterpret_cast<int32_t *>(b + o_it);
        w.sync = reinterpret_cast<unsigned *>(b + o_sy);
    }
    return w;
}

// Prefill path (q > kMaxDecodeQ), rfx_prefill.hip. Arguments are validated
// by the caller (the C entry points in rfx_moe.hip).
int prefill_route(const rfx_moe_layer *L, const float *x, int q, int k, int32_t *topk_idx, float *topk_w,
                  int32_t *pairs_sorted, int32_t *expert_off, int8_t *xq, float *xs, int32_t *xsum,
                  const MoeWs &w, hipStream_t stream);
// Test-hook stores of the prefill FFN kernels: the fp32 h of every row
// ([q*k + q][I], or null) and, for the work item (probe_expert,
// probe_first), the block dots of gate, up ([I][64][H/32]) and down
// ([H][64][I/32]) (any may be null).
struct PrefillDebug {
    float *h;
    int probe_expert, probe_first;
    int32_t *dots[3];
};
// dbg non-null: the gate/up and down kernels with the test-hook stores,
// no combine.
int prefill_ffn(const rfx_moe_layer *L, int q, int k, const int8_t *xq, const float *xs, const float *topk_w,
                const int32_t *pairs_sorted, const int32_t *expert_off, const float *resid, float *y,
                const MoeWs &w, hipStream_t stream, const PrefillDebug *dbg = nullptr);

} // namespace rfx
