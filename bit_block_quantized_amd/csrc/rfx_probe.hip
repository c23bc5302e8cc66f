// Streaming-read reference for gfx950: reads a buffer once with the
// nontemporal 16-byte vector loads the block-GEMV kernels use and folds
// every 32-bit word by XOR, so that its time measures the read rate HBM
// delivers to this load form (the ceiling the decode kernels stream
// against), and its result can be checked.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rfx_internal.h"

using namespace rfx;

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(const u32x4 &v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Grid-stride over 16-byte vectors, four loads in flight per thread.
__global__ __launch_bounds__(256) void read_ref_kernel(const u32x4 *__restrict__ p, size_t n16, uint32_t *out)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t h = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        h ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
    }
    for (; i < n16; i += stride)
        h ^= fold(__builtin_nontemporal_load(p + i));
    for (int o = 32; o > 0; o >>= 1)
        h ^= (uint32_t)__shfl_xor((int)h, o, 64);
    __shared__ uint32_t s[4];
    if ((threadIdx.x & 63) == 0)
        s[threadIdx.x >> 6] = h;
    __syncthreads();
    if (threadIdx.x == 0)
        out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

} // namespace

extern "C" {

int rfx_read_reference(const void *buf, size_t bytes, uint32_t *out, int n_out, void *stream)
{
    int st = check_ptr(buf, 16, "buf");
    if (!st)
        st = check_ptr(out, 4, "out");
    if (st)
        return st;
    if (bytes == 0 || bytes % 16)
        return fail(RFX_E_INVAL, "rfx_read_reference: bytes=%zu (a positive multiple of 16)", bytes);
    if (n_out < 1 || n_out > (1 << 20))
        return fail(RFX_E_INVAL, "rfx_read_reference: n_out=%d (1..2^20)", n_out);
    hipLaunchKernelGGL(read_ref_kernel, dim3((unsigned)n_out), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4 *>(buf), bytes / 16, out);
    return hip_status("read reference launch");
}

} // extern "C"
