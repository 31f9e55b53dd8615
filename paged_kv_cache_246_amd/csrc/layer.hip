// Full decoder-layer decode step (placeholder until the MFMA GEMM path lands).
#include <hip/hip_runtime.h>

#include "internal.h"

extern "C" size_t mi_decoder_layer_workspace_bytes(const mi_layer_config*, mi_kv_pool_t, int32_t,
                                                   int32_t) {
    return 0;
}

extern "C" int mi_decoder_layer_decode(mi_kv_pool_t, const mi_layer_config*, const mi_layer_weights*,
                                       const uint16_t*, uint16_t*, const int32_t*, int32_t,
                                       const int32_t*, int32_t, int32_t, void*, size_t, void*) {
    return MI_ERR_UNSUPPORTED;
}
