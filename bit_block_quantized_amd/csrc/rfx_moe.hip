// MoE decode layer: router (top-k + stable bucketing) and expert FFN.
// (Placeholder entry points; the kernels follow.)
#include <hip/hip_runtime.h>

#include "rfx_internal.h"

using namespace rfx;

extern "C" {

size_t rfx_moe_workspace_bytes(const rfx_moe_layer *, int, int) { return 0; }

int rfx_moe_route_topk(const rfx_moe_layer *, const float *, int, int, int32_t *, float *, int32_t *,
                       int32_t *, int8_t *, float *, int32_t *, void *, size_t, void *)
{
    return fail(RFX_E_UNSUPPORTED, "rfx_moe_route_topk: not built yet");
}

int rfx_moe_ffn(const rfx_moe_layer *, int, int, const int8_t *, const float *, const int32_t *,
                const int32_t *, const float *, const int32_t *, const int32_t *, float *, void *,
                size_t, void *)
{
    return fail(RFX_E_UNSUPPORTED, "rfx_moe_ffn: not built yet");
}

int rfx_moe_debug_hidden(const rfx_moe_layer *, int, int, const void *, float *, int8_t *, float *,
                         void *)
{
    return fail(RFX_E_UNSUPPORTED, "rfx_moe_debug_hidden: not built yet");
}

} // extern "C"
