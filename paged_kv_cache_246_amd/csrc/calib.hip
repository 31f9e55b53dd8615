// Calibration utilities.
// * The streaming-read bandwidth the part delivers, the practical ceiling
//   next to the published 8 TB/s HBM peak against which the kernels'
//   achieved bandwidth is also reported. Each workgroup reads one contiguous
//   chunk of the buffer with 16-byte non-temporal loads (four in flight per
//   thread) and folds the words into one value per thread, stored so the
//   loads cannot be dropped.
// * The per-KV-head scales of an 8-bit KV pool from sample rows of k and v
//   (the largest finite magnitude of each head maps to the largest E4M3
//   value).
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

// One workgroup per (KV head g, K or V): each thread folds the magnitudes of
// the head's values over 16-byte pieces of the sample rows. A bf16 magnitude
// (bits & 0x7FFF) orders like an integer, and those with an all-ones
// exponent (infinities, NaN) are skipped. The workgroup takes the largest
// and thread 0 stores s = (a * margin) / 448 in float32, or 1.0 when s is not
// positive and finite.
constexpr int kCalibThreads = 256;
constexpr float kE4m3Max = 448.0f;
__global__ __launch_bounds__(kCalibThreads) void calibrate_scales_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int32_t rows, int32_t hkv,
    int32_t head_dim, float margin, float* __restrict__ scales) {
    __shared__ uint32_t s_max[kCalibThreads / 64];
    const int g = blockIdx.x;
    const bool is_v = blockIdx.y == 1;
    const uint16_t* src = is_v ? v : k;
    const int pieces = head_dim / 8;
    const size_t total = static_cast<size_t>(rows) * pieces;
    uint32_t m = 0;
    for (size_t i = threadIdx.x; i < total; i += kCalibThreads) {
        const size_t r = i / pieces;
        const int c = static_cast<int>(i - r * pieces);
        const uint4 w = *reinterpret_cast<const uint4*>(src + (r * hkv + g) * head_dim + 8 * c);
        const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t mag = (words[e] >> (16 * h)) & 0x7FFFu;
                if (mag < 0x7F80u) m = max(m, mag);
            }
        }
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), x)));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t a = s_max[0];
#pragma unroll
        for (int w = 1; w < kCalibThreads / 64; ++w) a = max(a, s_max[w]);
        const float amax = __uint_as_float(a << 16);
        float s = (amax * margin) / kE4m3Max;
        if (!(s > 0.0f && s <= 3.402823466e38f)) s = 1.0f;
        scales[(is_v ? hkv : 0) + g] = s;
    }
}

}  // namespace

extern "C" int mi_kv_pool_calibrate_scales(mi_kv_pool_t p, const uint16_t* k, const uint16_t* v,
                                           int32_t rows, float margin, void* stream) {
    if (!p || !mikv::pool_has_device(p) || !mikv::pool_fp8(p) || !k || !v || rows < 1 ||
        !(margin > 0.0f && margin <= 3.402823466e38f))
        return MI_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(k) % 16 != 0 || reinterpret_cast<uintptr_t>(v) % 16 != 0)
        return MI_ERR_INVALID_ARG;
    hipLaunchKernelGGL(calibrate_scales_kernel, dim3(p->num_kv_heads, 2), dim3(kCalibThreads), 0,
                       static_cast<hipStream_t>(stream), k, v, rows, p->num_kv_heads, p->head_dim, margin,
                       p->scales);
    return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}

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
