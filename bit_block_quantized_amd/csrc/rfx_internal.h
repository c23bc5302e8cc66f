// Internal declarations shared by the host code and the HIP launchers of
// librfx. Not part of the public ABI (that is include/rfx.h).
#pragma once

#include <cstddef>
#include <cstdint>

#include "rfx.h"

namespace rfx {

// Tiled device layout: 64 rows x 8 blocks (256 columns) per tile; inside a
// tile, 16-byte chunks interleaved by row (chunk c, row r at c*1024 + r*16).
constexpr int kTileRows = 64;
constexpr int kTileBlocks = 8;
constexpr int kTileCols = 32 * kTileBlocks; // 256
constexpr int kChunk = 1024;                                // 64 rows x 16 B
constexpr int kMaxBlockBytes = 34;                          // the largest canonical block (Q8)

constexpr int tile_bytes(int fmt)
{
    return fmt == RFX_FP2 ? 5 * kChunk : fmt == RFX_FP3 ? 7 * kChunk : fmt == RFX_FP4 ? 8 * kChunk + 512
         : fmt == RFX_FP2M || fmt == RFX_FP2S ? 6 * kChunk : fmt == RFX_Q8 ? 17 * kChunk
         : fmt == RFX_FP3E ? 6 * kChunk + 512 : 0;
}

inline bool fmt_ok(int fmt)
{
    return fmt == RFX_FP2 || fmt == RFX_FP3 || fmt == RFX_FP4 || fmt == RFX_FP2M || fmt == RFX_Q8 || fmt == RFX_FP2S ||
           fmt == RFX_FP3E;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Thread-local error message (set by fail()).
int fail(int status, const char *fmt, ...);

// Validation helpers (host only, no HIP calls).
// data_optional: a NULL data pointer is accepted (the MoE stacks when a
// per-expert placement table is given).
int check_qmat(const rfx_qmat *W, const char *what, bool allow_stack, bool data_optional = false);
int check_ptr(const void *p, size_t align, const char *what);

// Last HIP error as an RFX status (RFX_OK if none).
int hip_status(const char *where);

} // namespace rfx
