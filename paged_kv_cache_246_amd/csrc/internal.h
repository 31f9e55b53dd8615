// Internal declarations shared by the host sources of libmikv.
#pragma once

#include <cstddef>
#include <cmath>
#include <cstdint>
#include <vector>

#include "mikv.h"

struct mi_kv_pool_s {
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    int32_t num_kv_heads = 0;
    int32_t head_dim = 0;
    uint32_t flags = 0;
    int device = -1;
    void* k = nullptr;               // device [N, Hkv, bs, D]: bf16 bits, or E4M3 codes
    void* v = nullptr;
    float* scales = nullptr;         // device [2 * Hkv] (8-bit pools): K scales, then V scales
    void* stage = nullptr;           // device staging of scattered swaps (MI_POOL_SWAP_STAGING)
    size_t stage_blocks = 0;         // blocks of K (and again of V) the staging holds
    bool owns_cache = false;
    uint32_t* err = nullptr;         // device words: [0] error (MI_FAULT_* bits), [1] prefill redo
    mutable uint32_t prefill_gen = 0;  // generation number of the last prefill call on the pool
    std::vector<int32_t> stack;      // free-block LIFO; back() is handed out next
    std::vector<uint8_t> allocated;  // 1 if the id is currently handed out
};

namespace mikv {

constexpr int kBlockSize = 16;
constexpr size_t kSwapStageBytes = size_t{64} << 20;   // swap staging per cache (K, and again V)
constexpr int kPrefillRedoWord = 1;        // index of the prefill redo word in the pool's device words

// RoPE inverse frequencies theta^(-2i/D), i < D/2, computed on the host in
// float64 and passed to the kernels by value.
struct RopeTable {
    double inv_freq[64];
};
inline RopeTable make_rope_table(double theta, int head_dim) {
    RopeTable t{};
    for (int i = 0; i < head_dim / 2 && i < 64; ++i) t.inv_freq[i] = std::pow(theta, -2.0 * i / head_dim);
    return t;
}

inline bool pool_fp8(const mi_kv_pool_s* p) { return (p->flags & MI_POOL_KV_FP8) != 0; }
inline int pool_elem_bytes(const mi_kv_pool_s* p) { return pool_fp8(p) ? 1 : 2; }

inline bool pool_has_device(const mi_kv_pool_s* p) {
    return p && !(p->flags & MI_POOL_HOST_ONLY) && p->k && p->v && p->err;
}

inline bool supported_group(int32_t hq, int32_t hkv) {
    return hq > 0 && hkv > 0 && hq % hkv == 0 && hq / hkv >= 1 && hq / hkv <= 8;
}

constexpr int kMaxBatch = 1024;            // sequences per attention call
constexpr int kMaxAttnWaves = 4096;        // upper bound of the attention grid
constexpr int kDefaultSplitTokens = 32;    // minimum tokens per wave's share
constexpr int kMaxLayerBatch = 32;         // rows of the decoder-layer projections
constexpr int kLayerDimMultiple = 256;     // hidden, intermediate, Hq * D multiples

// Minimum tokens per attention wave's share chosen by the library.
int32_t default_split_tokens(int32_t batch, int32_t num_kv_heads, int32_t max_context_len);

// Attention grid size: resident waves, capped by the work bound.
int attention_grid_waves(int32_t batch, int32_t hkv, int32_t max_ctx, int32_t min_tiles, int resident);

// Workspace bytes of the attention partials (two slots per wave).
size_t attention_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t split_tokens);

// Launches (attention.hip). Arguments are validated by the caller.
int launch_write_decode_kv(const mi_kv_pool_s* p, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, uint16_t* q_rot, const int32_t* table,
                           int32_t mbps, const int32_t* ctx, int32_t batch, int32_t hq,
                           double theta, void* stream);
int launch_write_prefill_kv(const mi_kv_pool_s* p, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, uint16_t* q_rot, const int32_t* table, int32_t mbps,
                            const int32_t* ctx, const int32_t* cu, int32_t batch, int32_t tokens,
                            int32_t hq, double theta, void* stream);
int launch_paged_prefill(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                         const int32_t* table, int32_t mbps, const int32_t* ctx, const int32_t* cu,
                         int32_t batch, int32_t total, int32_t max_new, int32_t hq, float scale,
                         void* stream);
// default_split: the caller asked for the library's split (split_tokens 0),
// which lets small workloads take the per-segment form (no combine launch).
int launch_paged_gqa_decode(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                            const int32_t* table, int32_t mbps, const int32_t* ctx,
                            int32_t batch, int32_t hq, float scale, int32_t max_ctx,
                            int32_t split_tokens, void* ws, void* stream, bool default_split);
// The decoder layer's attention (the default split): the query as a bf16
// pair (q_hi + q_lo, [B, Hq, D] each), the output in float32 [B, Hq, D];
// workspace as for launch_paged_gqa_decode.
int launch_layer_attention(const mi_kv_pool_s* p, const uint16_t* q_hi, const uint16_t* q_lo,
                           float* out, const int32_t* table, int32_t mbps, const int32_t* ctx,
                           int32_t batch, int32_t hq, float scale, int32_t max_ctx, void* ws,
                           void* stream);
// mi_paged_gqa_decode with its partials in the library's fixed device
// scratch array instead of a workspace (no allocation).
int launch_paged_gqa_decode_noalloc(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                                    const int32_t* table, int32_t mbps, const int32_t* ctx,
                                    int32_t batch, int32_t hq, float scale, int32_t max_ctx,
                                    void* stream);
// Takes the current device's address of the scratch array (once per device;
// called at pool creation with the pool's device current).
int setup_noalloc_scratch();
void* noalloc_scratch(int device);

// write_decode_kv and the attention in one launch (plus the combine).
int launch_decode_step(const mi_kv_pool_s* p, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, uint16_t* q_rot, uint16_t* out, const int32_t* table,
                       int32_t mbps, const int32_t* ctx, int32_t batch, int32_t hq, double theta,
                       float scale, int32_t max_ctx, void* ws, void* stream);

}  // namespace mikv
