// Paged KV pool: handle, device buffers, free-block stack, size formulas.
//
// mini-infer README, "Project overview": the KV cache is a pool of blocks
// plus a free-block pool; each request owns a BlockTable of block ids.
// nxmr.cn inference-techniques article, section 2.1: a request of n tokens
// holds ceil(n / block_size) pages, each popped from the list of free pages.
// That list is a stack here: the last id freed is the next one handed out.
// The article grows the pool when the list runs dry; a fixed pool reports
// MI_ERR_NO_FREE_BLOCKS instead.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "internal.h"

extern "C" const char* mi_status_string(int status) {
    switch (status) {
        case MI_OK: return "ok";
        case MI_ERR_INVALID_ARG: return "invalid argument";
        case MI_ERR_OUT_OF_MEMORY: return "out of memory";
        case MI_ERR_NO_FREE_BLOCKS: return "no free KV blocks";
        case MI_ERR_HIP: return "HIP runtime error";
        case MI_ERR_UNSUPPORTED: return "unsupported shape";
        case MI_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MI_ERR_DEVICE_FAULT: return "device-side fault recorded";
        case MI_ERR_SCRATCH_TOO_SMALL: return "call needs more than the fixed scratch array";
        default: return "unknown status";
    }
}

extern "C" int mi_kv_pool_init(mi_kv_pool_t* out, int32_t num_blocks, int32_t block_size,
                               int32_t num_kv_heads, int32_t head_dim, void* k_cache,
                               void* v_cache, uint32_t flags) {
    if (!out) return MI_ERR_INVALID_ARG;
    *out = nullptr;
    if (num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0)
        return MI_ERR_INVALID_ARG;
    if (flags & ~static_cast<uint32_t>(MI_POOL_HOST_ONLY | MI_POOL_KV_FP8 | MI_POOL_SWAP_STAGING |
                                       MI_POOL_DECODE_DOT))
        return MI_ERR_INVALID_ARG;
    if ((k_cache == nullptr) != (v_cache == nullptr)) return MI_ERR_INVALID_ARG;
    if ((flags & MI_POOL_HOST_ONLY) && k_cache) return MI_ERR_INVALID_ARG;
    if (block_size != mikv::kBlockSize) return MI_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return MI_ERR_UNSUPPORTED;

    mi_kv_pool_s* p = new (std::nothrow) mi_kv_pool_s();
    if (!p) return MI_ERR_OUT_OF_MEMORY;
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    p->num_kv_heads = num_kv_heads;
    p->head_dim = head_dim;
    p->flags = flags;
    try {
        p->stack.resize(static_cast<size_t>(num_blocks));
        p->allocated.assign(static_cast<size_t>(num_blocks), 0);
    } catch (...) {
        delete p;
        return MI_ERR_OUT_OF_MEMORY;
    }
    for (int32_t i = 0; i < num_blocks; ++i) p->stack[i] = num_blocks - 1 - i;

    if (!(flags & MI_POOL_HOST_ONLY)) {
        if (hipGetDevice(&p->device) != hipSuccess) {
            delete p;
            return MI_ERR_HIP;
        }
        const size_t bytes = static_cast<size_t>(num_blocks) * num_kv_heads * block_size *
                             head_dim * mikv::pool_elem_bytes(p);
        if (k_cache) {
            p->k = k_cache;
            p->v = v_cache;
        } else {
            if (hipMalloc(&p->k, bytes) != hipSuccess) {
                delete p;
                return MI_ERR_OUT_OF_MEMORY;
            }
            if (hipMalloc(&p->v, bytes) != hipSuccess) {
                (void)hipFree(p->k);
                delete p;
                return MI_ERR_OUT_OF_MEMORY;
            }
            p->owns_cache = true;
        }
        bool ok = hipMalloc(reinterpret_cast<void**>(&p->err), 256) == hipSuccess &&
                  hipMemset(p->err, 0, 256) == hipSuccess &&
                  mikv::setup_noalloc_scratch() == MI_OK;
        if (ok && (flags & MI_POOL_SWAP_STAGING)) {
            const size_t blk = bytes / static_cast<size_t>(num_blocks);
            p->stage_blocks = std::min(mikv::kSwapStageBytes / blk, static_cast<size_t>(num_blocks));
            ok = hipMalloc(&p->stage, 2 * p->stage_blocks * blk) == hipSuccess;
            if (!ok) p->stage = nullptr;
        }
        if (ok && mikv::pool_fp8(p)) {
            const std::vector<float> one(2 * static_cast<size_t>(num_kv_heads), 1.0f);
            ok = hipMalloc(reinterpret_cast<void**>(&p->scales), one.size() * sizeof(float)) == hipSuccess &&
                 hipMemcpy(p->scales, one.data(), one.size() * sizeof(float), hipMemcpyHostToDevice) ==
                     hipSuccess;
        }
        if (!ok || hipDeviceSynchronize() != hipSuccess) {
            if (p->err) (void)hipFree(p->err);
            if (p->scales) (void)hipFree(p->scales);
            if (p->stage) (void)hipFree(p->stage);
            if (p->owns_cache) {
                (void)hipFree(p->k);
                (void)hipFree(p->v);
            }
            delete p;
            return MI_ERR_HIP;
        }
    }
    *out = p;
    return MI_OK;
}

extern "C" int mi_kv_pool_set_scales(mi_kv_pool_t p, const float* k_scales, const float* v_scales) {
    if (!p || !mikv::pool_fp8(p)) return MI_ERR_INVALID_ARG;
    const int hkv = p->num_kv_heads;
    std::vector<float> s(2 * static_cast<size_t>(hkv), 1.0f);
    for (int g = 0; g < hkv; ++g) {
        if (k_scales) s[g] = k_scales[g];
        if (v_scales) s[hkv + g] = v_scales[g];
    }
    for (float x : s)
        if (!(x > 0.0f) || !std::isfinite(x)) return MI_ERR_INVALID_ARG;
    if (!mikv::pool_has_device(p)) return MI_OK;      // host-only pool: nothing on a device
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(p->scales, s.data(), s.size() * sizeof(float), hipMemcpyHostToDevice) != hipSuccess)
        return MI_ERR_HIP;
    return MI_OK;
}

extern "C" int mi_kv_pool_get_scales(mi_kv_pool_t p, float* k_scales, float* v_scales) {
    if (!p || !mikv::pool_fp8(p) || !mikv::pool_has_device(p) || (!k_scales && !v_scales))
        return MI_ERR_INVALID_ARG;
    const int hkv = p->num_kv_heads;
    std::vector<float> s(2 * static_cast<size_t>(hkv));
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(s.data(), p->scales, s.size() * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
        return MI_ERR_HIP;
    for (int g = 0; g < hkv; ++g) {
        if (k_scales) k_scales[g] = s[g];
        if (v_scales) v_scales[g] = s[hkv + g];
    }
    return MI_OK;
}

extern "C" int mi_kv_pool_destroy(mi_kv_pool_t p) {
    if (!p) return MI_OK;
    int st = MI_OK;
    if (p->err && hipFree(p->err) != hipSuccess) st = MI_ERR_HIP;
    if (p->scales && hipFree(p->scales) != hipSuccess) st = MI_ERR_HIP;
    if (p->stage && hipFree(p->stage) != hipSuccess) st = MI_ERR_HIP;
    if (p->owns_cache) {
        if (hipFree(p->k) != hipSuccess) st = MI_ERR_HIP;
        if (hipFree(p->v) != hipSuccess) st = MI_ERR_HIP;
    }
    delete p;
    return st;
}

extern "C" int mi_kv_pool_get(mi_kv_pool_t p, void** k_cache, void** v_cache) {
    if (!p) return MI_ERR_INVALID_ARG;
    if (k_cache) *k_cache = p->k;
    if (v_cache) *v_cache = p->v;
    return MI_OK;
}

extern "C" int mi_kv_pool_shape(mi_kv_pool_t p, int32_t* nb, int32_t* bs, int32_t* hkv,
                                int32_t* d) {
    if (!p) return MI_ERR_INVALID_ARG;
    if (nb) *nb = p->num_blocks;
    if (bs) *bs = p->block_size;
    if (hkv) *hkv = p->num_kv_heads;
    if (d) *d = p->head_dim;
    return MI_OK;
}

extern "C" int mi_kv_alloc_blocks(mi_kv_pool_t p, int32_t n, int32_t* out_ids) {
    if (!p || n < 0 || (n > 0 && !out_ids)) return MI_ERR_INVALID_ARG;
    if (static_cast<size_t>(n) > p->stack.size()) return MI_ERR_NO_FREE_BLOCKS;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = p->stack.back();
        p->stack.pop_back();
        p->allocated[id] = 1;
        out_ids[i] = id;
    }
    return MI_OK;
}

extern "C" int mi_kv_free_blocks(mi_kv_pool_t p, int32_t n, const int32_t* ids) {
    if (!p || n < 0 || (n > 0 && !ids)) return MI_ERR_INVALID_ARG;
    // validate everything first so a bad request frees nothing
    std::vector<uint8_t> seen;
    try {
        seen.assign(static_cast<size_t>(p->num_blocks), 0);
    } catch (...) {
        return MI_ERR_OUT_OF_MEMORY;
    }
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = ids[i];
        if (id < 0 || id >= p->num_blocks || !p->allocated[id] || seen[id])
            return MI_ERR_INVALID_ARG;
        seen[id] = 1;
    }
    for (int32_t i = 0; i < n; ++i) {
        p->allocated[ids[i]] = 0;
        p->stack.push_back(ids[i]);
    }
    return MI_OK;
}

extern "C" int32_t mi_kv_num_free_blocks(mi_kv_pool_t p) {
    if (!p) return MI_ERR_INVALID_ARG;
    return static_cast<int32_t>(p->stack.size());
}

extern "C" int32_t mi_kv_blocks_needed(int32_t num_tokens, int32_t block_size) {
    if (num_tokens < 0 || block_size <= 0) return MI_ERR_INVALID_ARG;
    return static_cast<int32_t>((static_cast<int64_t>(num_tokens) + block_size - 1) / block_size);
}

extern "C" uint64_t mi_kv_cache_bytes(int64_t batch, int64_t layers, int64_t max_seq_len,
                                      int64_t num_kv_heads, int64_t head_dim) {
    if (batch < 0 || layers < 0 || max_seq_len < 0 || num_kv_heads < 0 || head_dim < 0) return 0;
    return 2ull * static_cast<uint64_t>(batch) * static_cast<uint64_t>(layers) *
           static_cast<uint64_t>(max_seq_len) * static_cast<uint64_t>(num_kv_heads) *
           static_cast<uint64_t>(head_dim) * 2ull;
}

extern "C" int mi_kv_pool_check_errors(mi_kv_pool_t p, uint32_t* fault_bits) {
    if (fault_bits) *fault_bits = 0;
    if (!p) return MI_ERR_INVALID_ARG;
    if (!mikv::pool_has_device(p)) return MI_OK;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return MI_ERR_HIP;
    if (prev != p->device && hipSetDevice(p->device) != hipSuccess) return MI_ERR_HIP;
    uint32_t bits = 0;
    int st = MI_OK;
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&bits, p->err, sizeof(bits), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemset(p->err, 0, sizeof(bits)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
        st = MI_ERR_HIP;
    if (prev != p->device) (void)hipSetDevice(prev);
    if (fault_bits) *fault_bits = bits;
    if (st != MI_OK) return st;
    return bits ? MI_ERR_DEVICE_FAULT : MI_OK;
}
