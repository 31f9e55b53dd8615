// KV offload: block copies between a pool and a host swap space.
//
// On-device LLM inference course project, optional task "KV Cache
// Offloading": inactive KV blocks are moved out to CPU memory and brought
// back when needed. A block is the same [Hkv, 16, D] tile in both places.
//
// The copies are DMA transfers; a transfer per block costs far more than its
// 32-64 KiB take on the link, so pairs are ordered by host slot and runs of
// consecutive slots move in one transfer. When the device side of a run is
// not consecutive too, the blocks are first packed (swap-out) or last
// unpacked (swap-in) by a kernel through the pool's device staging buffer
// (allocated with the pool, MI_POOL_SWAP_STAGING), so every run is a single
// transfer whatever the device ids; a pool without staging moves such a run
// one block per transfer. Nothing here allocates device memory. Ids and
// slots are validated on the host before anything is queued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "internal.h"

namespace {

constexpr int kIdsPerLaunch = 256;

struct IdBatch {
    int32_t ids[kIdsPerLaunch];
};

// grid (count, 2): workgroup (i, c) copies block ids.ids[i] of cache c
// (0 = K, 1 = V) between the pool and staging slot i; UNPACK: staging -> pool.
template <bool UNPACK>
__global__ __launch_bounds__(256) void stage_blocks_kernel(char* __restrict__ pool_k,
                                                           char* __restrict__ pool_v,
                                                           char* __restrict__ stage, IdBatch ids,
                                                           size_t blk_bytes, size_t stage_half) {
    const int i = blockIdx.x;
    char* pool = blockIdx.y == 0 ? pool_k : pool_v;
    char* pb = pool + static_cast<size_t>(ids.ids[i]) * blk_bytes;
    char* sb = stage + blockIdx.y * stage_half + static_cast<size_t>(i) * blk_bytes;
    const size_t n16 = blk_bytes / 16;
    for (size_t e = threadIdx.x; e < n16; e += blockDim.x) {
        if (UNPACK)
            reinterpret_cast<uint4*>(pb)[e] = reinterpret_cast<const uint4*>(sb)[e];
        else
            reinterpret_cast<uint4*>(sb)[e] = reinterpret_cast<const uint4*>(pb)[e];
    }
}

// out: pairs are (device block, host slot); in: (host slot, device block).
int swap_blocks(mi_kv_pool_t p, char* host_k, char* host_v, int32_t host_slots,
                const int32_t* pairs, int32_t n, bool out, void* stream) {
    if (!p || !mikv::pool_has_device(p) || host_slots < 0 || n < 0) return MI_ERR_INVALID_ARG;
    if (n == 0) return MI_OK;
    if (!pairs || !host_k || !host_v) return MI_ERR_INVALID_ARG;
    std::vector<int32_t> dev(static_cast<size_t>(n)), slot(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) {
        dev[i] = out ? pairs[2 * i] : pairs[2 * i + 1];
        slot[i] = out ? pairs[2 * i + 1] : pairs[2 * i];
        if (dev[i] < 0 || dev[i] >= p->num_blocks || slot[i] < 0 || slot[i] >= host_slots)
            return MI_ERR_INVALID_ARG;
    }
    {   // every destination (host slot out, device block in) named once
        std::vector<uint8_t> seen(static_cast<size_t>(out ? host_slots : p->num_blocks), 0);
        for (int32_t i = 0; i < n; ++i) {
            const int32_t d = out ? slot[i] : dev[i];
            if (seen[d]) return MI_ERR_INVALID_ARG;
            seen[d] = 1;
        }
    }
    const size_t blk = static_cast<size_t>(p->num_kv_heads) * p->block_size * p->head_dim *
                       mikv::pool_elem_bytes(p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipMemcpyKind kind = out ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
    char* pk = static_cast<char*>(p->k);
    char* pv = static_cast<char*>(p->v);

    std::vector<int32_t> order(static_cast<size_t>(n));
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return slot[a] < slot[b]; });

    // runs of consecutive host slots; a run whose device ids are consecutive
    // too goes straight between pool and host
    std::vector<std::pair<int32_t, int32_t>> runs;          // [begin, end) in `order`
    for (int32_t i = 0; i < n;) {
        int32_t j = i + 1;
        while (j < n && slot[order[j]] == slot[order[j - 1]] + 1) ++j;
        runs.emplace_back(i, j);
        i = j;
    }
    auto copy = [&](char* dk, char* dv, const char* sk, const char* sv, size_t bytes) {
        return hipMemcpyAsync(dk, sk, bytes, kind, st) == hipSuccess &&
               hipMemcpyAsync(dv, sv, bytes, kind, st) == hipSuccess;
    };
    char* stage = static_cast<char*>(p->stage);
    const size_t half = p->stage_blocks * blk;
    for (const auto& run : runs) {
        bool direct = true;
        for (int32_t k = run.first + 1; k < run.second; ++k)
            direct &= dev[order[k]] == dev[order[k - 1]] + 1;
        const size_t h0 = static_cast<size_t>(slot[order[run.first]]) * blk;
        if (direct) {
            const size_t d0 = static_cast<size_t>(dev[order[run.first]]) * blk;
            const size_t bytes = static_cast<size_t>(run.second - run.first) * blk;
            const bool ok = out ? copy(host_k + h0, host_v + h0, pk + d0, pv + d0, bytes)
                                : copy(pk + d0, pv + d0, host_k + h0, host_v + h0, bytes);
            if (!ok) return MI_ERR_HIP;
            continue;
        }
        if (!stage) {        // no staging buffer: one transfer per block
            for (int32_t k = run.first; k < run.second; ++k) {
                const size_t d0 = static_cast<size_t>(dev[order[k]]) * blk;
                const size_t hk = static_cast<size_t>(slot[order[k]]) * blk;
                const bool ok = out ? copy(host_k + hk, host_v + hk, pk + d0, pv + d0, blk)
                                    : copy(pk + d0, pv + d0, host_k + hk, host_v + hk, blk);
                if (!ok) return MI_ERR_HIP;
            }
            continue;
        }
        // through the staging buffer, a chunk at a time
        for (int32_t c0 = run.first; c0 < run.second;) {
            const int32_t cnt = static_cast<int32_t>(std::min<size_t>(
                {p->stage_blocks, static_cast<size_t>(run.second - c0), static_cast<size_t>(kIdsPerLaunch)}));
            IdBatch ids{};
            for (int32_t k = 0; k < cnt; ++k) ids.ids[k] = dev[order[c0 + k]];
            const size_t hoff = static_cast<size_t>(slot[order[c0]]) * blk;
            const size_t bytes = static_cast<size_t>(cnt) * blk;
            if (out) {
                hipLaunchKernelGGL(stage_blocks_kernel<false>, dim3(cnt, 2), dim3(256), 0, st, pk, pv,
                                   stage, ids, blk, half);
                if (hipGetLastError() != hipSuccess) return MI_ERR_HIP;
                if (!copy(host_k + hoff, host_v + hoff, stage, stage + half, bytes)) return MI_ERR_HIP;
            } else {
                if (!copy(stage, stage + half, host_k + hoff, host_v + hoff, bytes)) return MI_ERR_HIP;
                hipLaunchKernelGGL(stage_blocks_kernel<true>, dim3(cnt, 2), dim3(256), 0, st, pk, pv,
                                   stage, ids, blk, half);
                if (hipGetLastError() != hipSuccess) return MI_ERR_HIP;
            }
            c0 += cnt;
        }
    }
    return MI_OK;
}

}  // namespace

extern "C" int mi_kv_swap_out(mi_kv_pool_t p, void* host_k, void* host_v, int32_t host_slots,
                              const int32_t* pairs, int32_t n, void* stream) {
    return swap_blocks(p, static_cast<char*>(host_k), static_cast<char*>(host_v), host_slots, pairs,
                       n, true, stream);
}

extern "C" int mi_kv_swap_in(mi_kv_pool_t p, const void* host_k, const void* host_v,
                             int32_t host_slots, const int32_t* pairs, int32_t n, void* stream) {
    return swap_blocks(p, const_cast<char*>(static_cast<const char*>(host_k)),
                       const_cast<char*>(static_cast<const char*>(host_v)), host_slots, pairs, n,
                       false, stream);
}
