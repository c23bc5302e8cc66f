/*
 * rfx — ROCmFPX-style block-quantized decode kernels for AMD Instinct MI355X
 * (gfx950, CDNA4). C ABI.
 *
 * Pages cited (title, site):
 *   [HM]  "DeepSeek V4 Flash hits 32 tok/s on AMD Ryzen AI MAX+ 395"
 *         (hellomarvisaitoday.com), paragraphs numbered from the top.
 *   [AIN] "Token Freedom via APU: AMD Ryzen AI MAX+ 395 Runs DeepSeek V4
 *         Flash at 32 tok/s on a 284B Model" (ainomam.com), by section.
 *   [KK]  the kaikai365.com post on DeepSeek V4 Flash on Strix Halo, by
 *         section heading.
 *
 * Conventions for every entry point:
 *   - Return value: RFX_OK (0) or a negative RFX_E_* status. Nothing throws
 *     across the ABI. rfx_last_error() gives a thread-local message for the
 *     last failure.
 *   - Arguments are validated synchronously, before any HIP call, so bad
 *     shapes, null pointers and bad alignment fail the same way on a host
 *     without a GPU.
 *   - Device entry points enqueue on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream) and return at once; there is no
 *     implicit synchronisation. A launch failure returns RFX_E_HIP.
 *   - The caller allocates every buffer. The library allocates nothing and
 *     keeps no device state. Where a workspace is taken it must be
 *     zero-filled before its first use; every completed call leaves its
 *     counters at zero again, so one zero fill serves any number of calls.
 *     A workspace must not be shared by calls that can run concurrently.
 *   - Device pointers must be 16-byte aligned unless stated otherwise.
 *   - Floating-point inputs are assumed finite on the device side; the host
 *     encoder checks and rejects non-finite weights.
 */
#ifndef RFX_H
#define RFX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    RFX_OK = 0,
    RFX_E_INVAL = -1,      /* bad shape, format, count or null pointer */
    RFX_E_ALIGN = -2,      /* pointer not aligned as required */
    RFX_E_RANGE = -3,      /* non-finite weight, or fp16 scale overflow */
    RFX_E_UNSUPPORTED = -4,/* valid request this library does not implement */
    RFX_E_WORKSPACE = -5,  /* workspace missing or too small */
    RFX_E_HIP = -6,        /* a HIP runtime call or launch failed */
    RFX_E_TIMEOUT = -7     /* a bounded device-side wait ran out (rfx_moe_forward_status) */
};

/* Block formats. A block is 32 consecutive weights of one row along the
 * reduction dimension, stored as packed codes plus one scale ([HM] para 2
 * lets a block carry a single small scale or a pair; the three named formats
 * here use one, the FP2M and FP2S variants two).
 *   RFX_FP2: 2-bit codes, codebook {-3,-1,+1,+3}, fp16 scale: 10 B / block
 *   RFX_FP3: 3-bit codes, codebook {-7,-5,...,+7}, fp16 scale: 14 B / block
 *   RFX_FP4: 4-bit OCP E2M1 codes (value = 2 x E2M1, |v| <= 12), one e8m0
 *            exponent byte E, scale 2^(E-128): 17 B / block (MXFP4)
 * 10 / 14 / 17 bytes are the pages' 2.50 / 3.50 / 4.25 bits per weight
 * ([HM] para 2; [KK] mixed-precision section).
 *   RFX_FP2M: variant with a scale and a minimum per block (a reading of
 *            the two-value block the same paragraph allows, not one of the
 *            named formats): 2-bit codes c in 0..3, weight = s * c + m, fp16
 *            s then fp16 m: 12 B / block (3.0 bits per weight). Supported
 *            by the encoder, the layout routines and the GEMV entry points;
 *            the MoE and prefill layers return RFX_E_UNSUPPORTED for it.
 *   RFX_Q8:  a tier above FP4 (the same paragraph keeps dense and sensitive
 *            projections at FP4 or higher; this tier is a reading): 32 int8
 *            codes in weight order, then an fp16 scale s; weight = s * c:
 *            34 B / block (8.5 bits per weight). Same support as RFX_FP2M.
 *   RFX_FP2S: variant with two sub-scales (the same paragraph's pair of
 *            small values read as two scales): FP2 codes and codebook;
 *            weights 0..15 take fp16 scale s0, weights 16..31 fp16 scale
 *            s1; codes, s0, s1: 12 B / block (3.0 bits per weight). Same
 *            support as RFX_FP2M.
 *   RFX_FP3E: a 3-bit tier at about 3.3 bits per weight (the figure
 *            another system on the pages gives for its 3-bit experts,
 *            without a layout; this one is a reading): FP3's codes and
 *            codebook, then one e8m0 byte E, weight = 2^(E-127) x value:
 *            13 B / block (3.25 bits per weight). Same support as RFX_FP2M. */
enum { RFX_FP2 = 2, RFX_FP3 = 3, RFX_FP4 = 4, RFX_Q8 = 8, RFX_FP2M = 12, RFX_FP3E = 13, RFX_FP2S = 16 };

const char *rfx_status_str(int status);
const char *rfx_last_error(void);
const char *rfx_version(void);

int rfx_block_bytes(int fmt); /* 10 / 14 / 17 / 12 (FP2M) / 34 (Q8) / 12 (FP2S) / 13 (FP3E), or RFX_E_INVAL */
int rfx_code_bytes(int fmt);  /* 8 / 12 / 16 / 8 / 32 / 8 / 12 */
int rfx_scale_bytes(int fmt); /* bytes after the codes: 2 / 2 / 1 / 4 / 2 / 4 / 1 */

/* ------------------------------------------------------------------ */
/* Host-side encoder (synchronous, host memory).                       */
/* ------------------------------------------------------------------ */

/* Quantize 32 fp32 weights into one canonical block: code bytes, then the
 * scale (fp16 little-endian, or the e8m0 byte).
 * Scale: FP2/FP3 s = fp16_rne(amax / 3 or 7) computed in fp32; FP4 E =
 * clamp(floor(log2 amax) - 2 + 127, 0, 254) (OCP MX rule), amax = 0 -> 0.
 * Code: nearest codebook value to w/s (fp32 division; FP4: w * 2^(128-E));
 * ties go to the larger magnitude for FP2/FP3 (0 -> +1) and to the even
 * E2M1 mantissa for FP4. A zero (or underflowed) FP2/FP3 scale codes every
 * weight as +1 with s = 0.
 * FP2M: m = fp16_rne(min w); s = fp16_rne(max(max w - m, 0) / 3) in fp32;
 * code = nearest of 0..3 to (w - m) / s in fp32, ties to the larger; s = 0
 * codes every weight as 0. Block: codes, s, m (both fp16 little-endian).
 * Q8: s = fp16_rne(amax / 127) in fp32; code = clamp(round half to even of
 * w / s in fp32, -127, 127) stored as the two's-complement byte; s = 0
 * codes every weight as 0. Code byte t is weight t.
 * FP2S: each half h (weights 16h..16h+15) is encoded as an FP2 block with
 * its own amax: s_h = fp16_rne(amax_h / 3) in fp32, FP2 codes and ties;
 * s_h = 0 codes the half's weights as +1. Block: codes, s0, s1 (fp16 LE).
 * FP3E: E = clamp(floor(log2 amax) - 2 + 127, 0, 254), amax = 0 -> 0;
 * code = FP3's nearest value to w * 2^(127-E) (exact), ties to the larger
 * magnitude, saturating at +-7. Block: codes, E.
 * Bit layout of the code bytes, as little-endian 32-bit words:
 *   FP2 (and FP2M, FP2S): weight 16m+4i+j (m<2, i,j<4) at word m bits [8j+2i, 8j+2i+2)
 *   FP3 (and FP3E): low two bits as FP2 in words 0-1; high bit of weight 4i+j (i<8)
 *        at word 2 bit 8j+i
 *   FP4: weight 8m+4i+j (m<4, i<2, j<4) at word m bits [8j+4i, 8j+4i+4)
 * Returns RFX_E_RANGE for a non-finite weight or an fp16 scale (or FP2M
 * minimum) overflow. */
int rfx_quantize_block(int fmt, const float *w32, uint8_t *blk);
int rfx_dequantize_block(int fmt, const uint8_t *blk, float *w32);

/* ------------------------------------------------------------------ */
/* Device weight layout.                                               */
/* ------------------------------------------------------------------ */
/* A matrix of `rows` x `cols` (cols % 32 == 0) is stored as tiles of 64 rows
 * by 256 columns (8 blocks). Tile (g, s) covers rows 64g..64g+63 and blocks
 * 8s..8s+7 and sits at byte offset (g * S + s) * tile_bytes, S = ceil(cols/
 * 256). Inside a tile, 16-byte chunks are interleaved by row so that one
 * 64-lane load of chunk c reads 1 KiB of contiguous memory:
 *   byte offset of (chunk c, row r in 0..63) = c * 1024 + r * 16.
 *   FP2 (tile 5120 B): chunks 0-3 = codes of blocks 2c, 2c+1 (8 B each);
 *       chunk 4 = the eight fp16 scales.
 *   FP3 (tile 7168 B): chunks 0-3 = low-bit words of blocks 2c, 2c+1;
 *       chunks 4-5 = high-bit words of blocks 4(c-4)..4(c-4)+3 (4 B each);
 *       chunk 6 = the eight fp16 scales.
 *   FP4 (tile 8704 B): chunks 0-7 = codes of block c; then 64 rows x 8 B of
 *       e8m0 scales at byte 8192 + r * 8.
 *   FP2M (tile 6144 B): chunks 0-4 as FP2; chunk 5 = the eight fp16 minima.
 *   FP2S (tile 6144 B): chunks 0-3 as FP2; chunk 4 = the eight first-half
 *       scales s0; chunk 5 = the eight second-half scales s1.
 *   FP3E (tile 6656 B): chunks 0-5 as FP3; then 64 rows x 8 B of e8m0
 *       bytes at byte 6144 + r * 8.
 *   Q8 (tile 17408 B): chunk 2b + h = code bytes 16h..16h+15 of block b;
 *       chunk 16 = the eight fp16 scales.
 * Rows beyond `rows` and blocks beyond cols/32 are zero (scale 0). Block
 * bits are exactly those of the canonical block. A stack of `count`
 * matrices (MoE experts) places matrix e at e * rfx_qmat_bytes(...). */
typedef struct rfx_qmat {
    int32_t fmt;      /* RFX_FP2 / RFX_FP3 / RFX_FP4 */
    int32_t rows;     /* N (output features), >= 1 */
    int32_t cols;     /* K (reduction length), multiple of 32 */
    int32_t count;    /* matrices in the stack, >= 1 */
    const void *data; /* device, count * rfx_qmat_bytes(fmt, rows, cols), 256-B aligned */
} rfx_qmat;

int64_t rfx_qmat_bytes(int fmt, int64_t rows, int64_t cols); /* one matrix, padded */

/* fp32 row-major [rows][cols] (host) -> tiled layout (host buffer of
 * rfx_qmat_bytes). Uses up to `threads` host threads (<= 0: hardware
 * concurrency). Same encoder as rfx_quantize_block. */
int rfx_quantize_matrix(int fmt, const float *W, int64_t rows, int64_t cols, void *tiled,
                        int threads);
/* Tiled layout (host) -> canonical blocks [rows][cols/32][block_bytes]. */
int rfx_export_blocks(int fmt, const void *tiled, int64_t rows, int64_t cols, uint8_t *blocks);
/* Canonical blocks (host) -> tiled layout (host), for pre-quantized data. */
int rfx_import_blocks(int fmt, const uint8_t *blocks, int64_t rows, int64_t cols, void *tiled);

/* ------------------------------------------------------------------ */
/* Activations.                                                        */
/* ------------------------------------------------------------------ */
/* Quantize q columns of K fp32 values (K % 32 == 0), device to device.
 * Per 32-block: s = amax / 127 (fp32, IEEE division), code = clamp(round
 * half to even(x / s), -127, 127), all-zero block -> s = 0, codes 0; xsum =
 * the block's integer sum of codes (used by the FP2/FP3 decoders, whose
 * codebooks are affine in the code). Integer activations feed the integer
 * dot products ([HM] para 3).
 * x fp32 [q][K]; xq int8 [q][K]; xs fp32 [q][K/32]; xsum int32 [q][K/32].
 * q >= 1. x and xq need 16-B alignment, xs and xsum 4-B (RFX_E_ALIGN). */
int rfx_quantize_act(const float *x, int q, int K, int8_t *xq, float *xs, int32_t *xsum,
                     void *stream);

/* ------------------------------------------------------------------ */
/* Fused dequantize-and-multiply (GEMV).                                */
/* ------------------------------------------------------------------ */
/* y[j][n] = sum_b S[n][b] * xs[j][b] * D[j][n][b], D the exact integer dot
 * of block b of row n with column j's int8 block. Packed blocks are read
 * once from HBM and expanded in registers; each decoded weight is applied
 * to all q columns ([HM] para 3; [AIN] optimization-trio section: decode
 * once for the four verification columns). fp32 accumulation.
 * W: count must be 1 (use W->data of one expert for stacks). q in 1..4.
 * xq [q][K], xs/xsum [q][K/32] as produced by rfx_quantize_act; y fp32
 * [q][N] (4-B aligned).
 * ws: zero-filled workspace of rfx_gemv_workspace_bytes(W, q) bytes, or
 * NULL to run without splitting K across workgroups (slower for small N). */
size_t rfx_gemv_workspace_bytes(const rfx_qmat *W, int q);
int rfx_gemv(const rfx_qmat *W, const int8_t *xq, const float *xs, const int32_t *xsum, int q,
             float *y, void *ws, size_t ws_bytes, void *stream);
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): rfx_gemv
 * with the split-K exchange slots in a 256 KiB array the library holds on
 * each GPU it runs on (from the first call on that GPU until the process
 * ends) instead of a workspace argument. Same arguments otherwise, same
 * kernels, launch shape and results as rfx_gemv with a workspace. It calls
 * no hipMalloc / hipFree; the first call on a device looks the array up and
 * clears it with a fill kernel on `stream`, and every completed call leaves
 * it clear. All calls on one GPU share the array: calls that can overlap
 * on one GPU (other streams, other threads) race and must not be issued.
 * Errors: those of rfx_gemv; RFX_E_WORKSPACE if a shape would need more
 * than the array holds (no valid shape does: the largest split needs under
 * 192 KiB); RFX_E_HIP if the array's address cannot be obtained. */
int rfx_gemv_noalloc(const rfx_qmat *W, const int8_t *xq, const float *xs, const int32_t *xsum, int q,
                     float *y, void *stream);
int rfx_gemv_q1(const rfx_qmat *W, const int8_t *xq, const float *xs, const int32_t *xsum,
                float *y, void *ws, size_t ws_bytes, void *stream);
int rfx_gemv_q4(const rfx_qmat *W, const int8_t *xq, const float *xs, const int32_t *xsum,
                float *y, void *ws, size_t ws_bytes, void *stream);

/* Several independent GEMVs in one launch (up to RFX_MAX_GEMV_JOBS), each
 * with its own matrix, q and activation / output buffers, computing exactly
 * what rfx_gemv computes for it. One job's last workgroups overlap the next
 * job's weight stream, so a batch of projections that do not depend on one
 * another (a decode step's query / key / value, or gate and up) pays the
 * launch and reduction tail once instead of once per matrix. Jobs may mix
 * formats, shapes and q; whatever their order in `jobs`, the ones with the
 * most decode work per workgroup start first. Each job's result depends
 * only on its own shape (fixed-order reduction), so it is deterministic,
 * though not bit-identical to a lone rfx_gemv (its K split may differ).
 * Field rules are rfx_gemv's; output buffers must not overlap.
 * ws: zero-filled workspace of rfx_gemv_grouped_workspace_bytes(jobs,
 * n_jobs) bytes, 256-B aligned (NULL allowed when that is 0); left zeroed
 * on return. Launches that share a workspace must not overlap.
 * Errors: RFX_E_INVAL (n_jobs outside 1..RFX_MAX_GEMV_JOBS, or a bad job:
 * the message names its index), RFX_E_ALIGN, RFX_E_WORKSPACE, RFX_E_HIP. */
#define RFX_MAX_GEMV_JOBS 16
typedef struct rfx_gemv_job {
    rfx_qmat W;          /* count must be 1 */
    int32_t q;           /* 1..4 */
    int32_t reserved;
    const int8_t *xq;    /* [q][W.cols] */
    const float *xs;     /* [q][W.cols / 32] */
    const int32_t *xsum; /* [q][W.cols / 32] */
    float *y;            /* [q][W.rows] */
} rfx_gemv_job;
size_t rfx_gemv_grouped_workspace_bytes(const rfx_gemv_job *jobs, int n_jobs);
int rfx_gemv_grouped(const rfx_gemv_job *jobs, int n_jobs, void *ws, size_t ws_bytes, void *stream);

/* Test hook: the decode path rfx_gemv takes for the same format and q,
 * storing every per-block integer dot D[j][n][b] (int32 [q][N][K/32])
 * instead of the scaled sum: the dot of the block's codebook values with the
 * activation codes (FP2M: of the codes 0..3; FP2S: over both halves,
 * D0 + D1). FP4 with q <= 2 runs on the block-scaled matrix core, which
 * applies the block exponent inside the product; there the hook reads each
 * block's product 2^(E-128) D before the activation scale and multiplies it
 * back by 2^(128-E), storing INT32_MIN for a block whose product is not an
 * exact integer multiple (a value lost to the fp32 range). No xs is read. */
int rfx_debug_block_dots(const rfx_qmat *W, const int8_t *xq, const int32_t *xsum, int q,
                         int32_t *dots, void *stream);

/* Measurement aid (not part of the method): reads `bytes` (a positive
 * multiple of 16; buf 16-B aligned, device) once with the nontemporal
 * 16-byte loads the GEMV kernels use, XOR-folding every 32-bit word, over
 * n_out workgroups (1..2^20) of 256 threads; workgroup i writes its fold to
 * out[i] (device, n_out words), so the XOR of out[0..n_out) is the XOR of
 * all the buffer's words. Its time gives the HBM read rate for that load
 * form. Errors: RFX_E_INVAL / RFX_E_ALIGN before any HIP call. */
int rfx_read_reference(const void *buf, size_t bytes, uint32_t *out, int n_out, void *stream);

/* ------------------------------------------------------------------ */
/* MoE layer: decode (q <= 4 tokens) and prefill (q > 4).               */
/* ------------------------------------------------------------------ */
/* Routed experts: gate and up (rows = inter, cols = hidden) and down
 * (rows = hidden, cols = inter), `n_experts` stacked each ([HM] para 2 and
 * [KK] ROCmFPX section: gate/up in FP2, down in FP3; any of RFX_FP2, RFX_FP3
 * and RFX_FP4 is accepted, RFX_FP2M, RFX_FP2S, RFX_FP3E and RFX_Q8 are not). Shared expert: sh_* with count 1 (FP4 for sensitive layers),
 * or sh_gate.data == NULL for none. Router: fp32 [n_experts][hidden]
 * weights and an optional fp32 [n_experts] bias. */
typedef struct rfx_moe_layer {
    int32_t hidden;    /* H, multiple of 32 */
    int32_t inter;     /* I, multiple of 32 */
    int32_t n_experts; /* E, 1..256 */
    int32_t reserved;
    rfx_qmat gate, up, down;
    rfx_qmat sh_gate, sh_up, sh_down;
    const float *router_w; /* device fp32 [E][H] */
    const float *router_b; /* device fp32 [E], or NULL */
    /* Expert placement (optional). NULL: routed expert e of gate / up / down
     * is matrix e of that stack. Otherwise a device-readable table of 3 * E
     * pointers, [gate e = 0..E-1][up e][down e], each to one expert matrix in
     * the tiled layout (256-B aligned), which may sit in device memory or in
     * mapped pinned host memory (hipHostMalloc): the kernels read either
     * directly, so hot experts can stay in HBM and cold ones in host memory
     * ([AIN] dual-GPU section: experts are independent and can be split
     * across devices by how often they are used). The stacks then give only
     * format, shape and count; their data may be NULL. */
    const void *const *expert_data;
} rfx_moe_layer;

size_t rfx_moe_workspace_bytes(const rfx_moe_layer *L, int q, int k);

/* Router for q tokens ([HM] para 3 and [KK] DSpark section: dedicated
 * TOP_K and ARGSORT kernels). logits l = x.Wr^T + b (fp32); experts ranked
 * by logit, equal logits to the lower id; top-k picked; weights = softmax
 * over all experts of the picked logits, not renormalised. Pairs p = t*k+j
 * are grouped by expert with a stable sort: pairs_sorted [q*k], expert_off
 * [E+1] (exclusive prefix sum of per-expert counts). The tokens are also
 * quantized for the experts (as rfx_quantize_act).
 * x fp32 [q][H]; topk_idx int32 [q][k]; topk_w fp32 [q][k]; 1 <= k <= 8.
 * q in 1..4 (decode and speculative verification): one launch, every
 * expert row of Wr read once for all q tokens. q in 5..65536 (prefill):
 * act quant, the logits on the fp32 matrix core into ws, a softmax / top-k
 * kernel (one wave per token) and a one-workgroup stable bucketing that
 * also writes the FFN's work items (chunks of up to 64 tokens of one
 * expert) into ws; rfx_moe_ffn must then get the same ws, q and k. The
 * router reads x in 16-byte words: x needs 16-B alignment. */
int rfx_moe_route_topk(const rfx_moe_layer *L, const float *x, int q, int k, int32_t *topk_idx,
                       float *topk_w, int32_t *pairs_sorted, int32_t *expert_off, int8_t *xq,
                       float *xs, int32_t *xsum, void *ws, size_t ws_bytes, void *stream);

/* Expert FFN and combine. For every pair (t, j) with expert e: g = G_e.x~_t,
 * u = U_e.x~_t, h = silu(g) * u, h~ = activation-quantized h, o = D_e.h~;
 * shared expert likewise with weight 1; y_t = resid_t + o_shared + sum_j
 * w_tj o_tj in slot order (deterministic, no float atomics). resid fp32
 * [q][H] or NULL (no residual; it may alias neither y nor ws); y fp32
 * [q][H]. ws: the workspace given to rfx_moe_route_topk may be reused.
 * q <= 4: block-dequant GEMV kernels, each active expert streamed once for
 * its tokens. q > 4 (prefill, needs the ws written by rfx_moe_route_topk):
 * per work item (up to 64 tokens of one expert) and 128 / 256 rows, the
 * packed blocks are expanded through their codebooks into matrix-core
 * operands holding the codes' integer values (as f16, exact) and multiplied
 * with the int8 activations (as f16, exact) on v_mfma_f32_16x16x32_f16, one
 * instruction per 32-weight block, so each fp32 result is the exact integer
 * block dot, then scaled by the weight and activation block scales in fp32
 * ([HM] para 3: integer dot products over the packed codes). The prefill
 * path keeps f16 copies of the token codes and of h~ in ws and returns
 * RFX_E_UNSUPPORTED when either copy would exceed 4 GiB. */
int rfx_moe_ffn(const rfx_moe_layer *L, int q, int k, const int8_t *xq, const float *xs,
                const int32_t *xsum, const int32_t *topk_idx, const float *topk_w,
                const int32_t *pairs_sorted, const int32_t *expert_off, const float *resid,
                float *y, void *ws, size_t ws_bytes, void *stream);

/* The whole layer, rfx_moe_route_topk then rfx_moe_ffn, in one call with
 * the same arguments, outputs and results (bit for bit). flags = 0: three
 * kernel launches. When the gate/up grid holds at most one workgroup per
 * compute unit (q = 1 at the pages' sizes), the router launch only
 * computes the logits and quantizes x, and every routed gate/up workgroup
 * picks the top k and buckets the pairs itself from the logits (one of
 * them writes topk_idx, topk_w, pairs_sorted and expert_off): the launch
 * boundary replaces the router's arrival counters. Otherwise the two calls.
 * flags = RFX_FORWARD_ONE_LAUNCH: for
 * q <= 4 with routed gate/up in RFX_FP2, down in RFX_FP3 and the shared
 * expert (if any) in RFX_FP4 ([HM] para 2 and [KK] ROCmFPX section), one
 * kernel launch ([HM] para 3: several positions verified in one fused
 * pass; [KK] DSpark section: the decode step as one fused graph):
 * workgroups with the token-quantization, router, gate/up and down roles
 * run together, the shared expert's gate/up streams while the router
 * runs, the router publishes one word per expert slot, and each down
 * workgroup fetches its weights before its slot's h~ is complete; they
 * synchronize through counters in ws with time-bounded waits. It is not
 * faster than the three launches on MI355X at these sizes (both are bound
 * by the same chain of dependent memory round trips), so it is not the
 * default. Other formats and q > 4 take the two calls either way;
 * rfx_moe_forward_single_launch(L, q, k) says whether the one-launch kernel
 * can take a call (1 / 0; < 0: a bad layer). x fp32 [q][H], 16-B aligned;
 * resid fp32 [q][H] or NULL, and may be x itself; y must alias none of x,
 * resid and ws. ws: rfx_moe_workspace_bytes(L, q, k) bytes, zero-filled
 * before its first use (the counters return to zero at the end of every
 * call); calls that share a ws must not overlap. Errors: those of the two
 * calls; RFX_E_INVAL for unknown flags. */
#define RFX_FORWARD_ONE_LAUNCH 1u
int rfx_moe_forward(const rfx_moe_layer *L, const float *x, int q, int k, const float *resid, float *y,
                    int32_t *topk_idx, float *topk_w, int32_t *pairs_sorted, int32_t *expert_off,
                    int8_t *xq, float *xs, int32_t *xsum, void *ws, size_t ws_bytes, unsigned flags,
                    void *stream);
int rfx_moe_forward_single_launch(const rfx_moe_layer *L, int q, int k);

/* After rfx_moe_forward calls on ws (synchronizes the stream): RFX_OK, or
 * RFX_E_TIMEOUT if a wait of the one-launch kernel ran out of its time
 * bound since the last status call (the outputs of that call are
 * undefined; the word is cleared). */
int rfx_moe_forward_status(const rfx_moe_layer *L, int q, int k, void *ws, size_t ws_bytes, void *stream);

/* Test hook: after rfx_moe_ffn with the same workspace (ws_bytes as given
 * to it; RFX_E_WORKSPACE when smaller than rfx_moe_workspace_bytes(L, q,
 * k)), copy out the intermediate activations of the last call: h fp32
 * [(q*k)+q][I] (pairs in pair order, then the shared expert per token),
 * h~ int8 and its scales. Any output pointer may be NULL. The prefill path
 * (q > 4) does not keep the fp32 h: h must be NULL there
 * (RFX_E_UNSUPPORTED otherwise); rfx_moe_debug_prefill gives it. */
int rfx_moe_debug_hidden(const rfx_moe_layer *L, int q, int k, const void *ws, size_t ws_bytes, float *h,
                         int8_t *hq, float *hs, void *stream);

/* Test hook of the prefill path (5 <= q <= 65536): after rfx_moe_route_topk
 * with the same ws, q and k, runs the gate/up and down kernels of
 * rfx_moe_ffn (not the combine) with extra stores: h fp32 [(q*k)+q][I] (the
 * SwiGLU output each h~ row was requantized from), and for the one work
 * item of expert probe_expert (n_experts = the shared expert) whose tokens
 * start at position probe_first (a multiple of 64) of that expert's token
 * list, every block dot the matrix core produced: dots_gate and dots_up
 * int32 [I][64][H/32], dots_down int32 [H][64][I/32], indexed [output row]
 * [token slot within the item][block]; slots past the item's tokens are
 * left untouched. Any output pointer may be NULL. The workspace's h~, its
 * scales and o are rewritten as rfx_moe_ffn writes them. Errors:
 * RFX_E_INVAL (q, k, probe), RFX_E_ALIGN, RFX_E_WORKSPACE, RFX_E_HIP. */
int rfx_moe_debug_prefill(const rfx_moe_layer *L, int q, int k, const int8_t *xq, const float *xs,
                          const float *topk_w, const int32_t *pairs_sorted, const int32_t *expert_off, void *ws,
                          size_t ws_bytes, int probe_expert, int probe_first, float *h, int32_t *dots_gate,
                          int32_t *dots_up, int32_t *dots_down, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RFX_H */
