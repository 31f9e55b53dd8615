// Measurement utility: the streaming-read bandwidth the part delivers, the
// practical ceiling next to the published 8 TB/s HBM peak against which the
// kernels' achieved bandwidth is also reported. Each workgroup reads one
// contiguous chunk of the buffer with 16-byte non-temporal loads (four in
// flight per thread) and folds the words into one value per thread, stored
// so the loads cannot be dropped.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
    const size_t per = n16 / gridDim.x;
    const u32x4* base = src + per * blockIdx.x;
    uint32_t acc = 0;
    size_t i = threadIdx.x;
    for (; i + 3 * blockDim.x < per; i += 4 * blockDim.x) {
        const u32x4 a = __builtin_nontemporal_load(base + i);
        const u32x4 b = __builtin_nontemporal_load(base + i + blockDim.x);
        const u32x4 c = __builtin_nontemporal_load(base + i + 2 * blockDim.x);
        const u32x4 d = __builtin_nontemporal_load(base + i + 3 * blockDim.x);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
               d.z ^ d.w;
    }
    for (; i < per; i += blockDim.x) {
        const u32x4 a = __builtin_nontemporal_load(base + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" int mi_hbm_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                                  void* stream) {
    if (!src || !sink || workgroups < 1 || workgroups > 65536 || bytes % 16 != 0 ||
        bytes / 16 < static_cast<size_t>(workgroups))
        return MI_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return MI_ERR_INVALID_ARG;
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), bytes / 16,
                       sink);
    return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}
