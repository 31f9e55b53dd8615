// Device-side E4M3 (OCP 8-bit float, "FN" variant: bias 7, no infinities,
// largest finite 448) encoding of the 8-bit KV cache.
//
// vLLM-based inference-framework report, "FP8 KV Cache quantisation": the
// cache is held in FP8. A bf16 value x under scale s is stored as the code
// nearest to float32(x) / s (one correctly rounded float32 division), ties to
// the even code, magnitudes beyond 448 saturating, NaN as 0x7F.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mikv_dev {

// The hardware conversion rounds to nearest even; it is fed the clamped
// magnitude and the sign is applied separately, so signed zeros, saturation
// and NaN follow the rule above exactly.
__device__ __forceinline__ uint32_t e4m3_encode_sat(float x) {
    if (x != x) return 0x7Fu;
    const float a = fminf(fabsf(x), 448.0f);
    const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, a, 0, false)) & 0xFFu;
    return c | ((__float_as_uint(x) >> 31) << 7);
}

// Code of bf16 bits h under scale s.
__device__ __forceinline__ uint32_t e4m3_quantize_bf16(uint16_t h, float s) {
    return e4m3_encode_sat(__uint_as_float(static_cast<uint32_t>(h) << 16) / s);
}

// Eight bf16 (one uint4) -> eight codes (one uint2), same scale.
__device__ __forceinline__ uint2 e4m3_quantize_bf16x8(uint4 w, float s) {
    const uint32_t in[4] = {w.x, w.y, w.z, w.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = e4m3_quantize_bf16(static_cast<uint16_t>(in[e] & 0xFFFFu), s);
        const uint32_t hi = e4m3_quantize_bf16(static_cast<uint16_t>(in[e] >> 16), s);
        out[e / 2] |= (lo | (hi << 8)) << (16 * (e & 1));
    }
    return make_uint2(out[0], out[1]);
}

}  // namespace mikv_dev
