/*
 * mikv -- paged-KV grouped-query-attention decode for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libmikv.so. Everything crossing this boundary is a plain pointer
 * (host or device, as stated per argument), an integer or a float. bf16
 * tensors are passed as uint16_t bit patterns; every tensor is row-major and
 * contiguous. No call synchronises the device unless its comment says so.
 *
 * The operations follow the pages this library implements:
 *  - mini-infer README, "Project overview": the KV cache is a pool of
 *    fixed-size blocks with a free-block pool and one BlockTable per request;
 *    "decode_batch key steps": gather each request's K/V through its
 *    BlockTable, run the batched forward, write the new token's K/V back
 *    (write_decode_kv).
 *  - On-device LLM inference course project, section 2.1: RMSNorm, RoPE,
 *    QKV projection with grouped-query attention (query head h reads KV head
 *    h / (Hq / Hkv), as repeat_interleave of the KV heads gives), SwiGLU MLP,
 *    decoder layer with residuals and two norms, KV-cache append.
 *  - nxmr.cn inference-techniques article: section 2.1, a request of n
 *    tokens holds ceil(n / block_size) pages popped from a free list;
 *    section 5.1, the numerically stable softmax; section 4.1, attention
 *    scores in FP32.
 *  - MegEngine/InferLLM article, section 4.2 "problem two": KV bytes =
 *    2 * batch * layers * seq_len * hidden * sizeof(dtype).
 *
 * Conventions (readings where the pages are silent):
 *  - Pool layout: per layer one K pool and one V pool, each
 *    [num_blocks, num_kv_heads, block_size, head_dim] bf16.
 *  - block_table: int32 [batch, max_blocks_per_seq], device memory. Row b
 *    maps logical block j of sequence b to a physical block id in
 *    [0, num_blocks). Entries at j >= ceil((context_lens[b] + 1) / block_size)
 *    are never read (tests fill them with -1).
 *  - context_lens: int32 [batch], device memory, the number of tokens cached
 *    BEFORE this step. The new token goes to logical position context_lens[b],
 *    which is also its RoPE position; attention covers context_lens[b] + 1
 *    tokens, the new one included. Both per-step calls take the same array;
 *    the caller advances it afterwards.
 *  - RoPE pairs dimension i with i + head_dim/2, inv_freq_i =
 *    theta^(-2i/head_dim), integer positions; q and the new k are rotated,
 *    v never. Cached K is stored already rotated.
 *  - Supported shapes: block_size 16, head_dim 64 or 128, num_q_heads a
 *    multiple of num_kv_heads with group size 1..8. Others return
 *    MI_ERR_UNSUPPORTED.
 *
 * Ownership: every device pointer argument (q, k, v, outputs, tables,
 * lengths, workspaces, weights) is owned by the caller and must stay valid
 * until the work queued on `stream` has finished; the library keeps no
 * reference after the call returns. A pool handle is owned by the library
 * and freed by mi_kv_pool_destroy. A pool handle is not thread-safe.
 *
 * Errors: every call returns MI_OK or a negative status, never aborts and
 * never prints. Device-resident values (block ids, lengths) cannot be checked
 * without a sync: the kernels range-check every block id and length they
 * read, skip the access when it is out of range, and record the fault in a
 * per-pool device error word that mi_kv_pool_check_errors reads back.
 *
 * `stream` is a hipStream_t passed as void*; NULL means the null stream.
 */
#ifndef MIKV_H
#define MIKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MI_OK = 0,
    MI_ERR_INVALID_ARG = -1,          /* null pointer, negative size, bad flag */
    MI_ERR_OUT_OF_MEMORY = -2,        /* host or device allocation failed */
    MI_ERR_NO_FREE_BLOCKS = -3,       /* free-block pool cannot satisfy the request */
    MI_ERR_HIP = -4,                  /* a HIP runtime call or kernel launch failed */
    MI_ERR_UNSUPPORTED = -5,          /* valid but unsupported shape */
    MI_ERR_WORKSPACE_TOO_SMALL = -6,  /* workspace_bytes below the size query */
    MI_ERR_DEVICE_FAULT = -7,         /* mi_kv_pool_check_errors found a recorded fault */
    MI_ERR_SCRATCH_TOO_SMALL = -8     /* the call needs more than MI_NOALLOC_SCRATCH_BYTES */
};

/* Device error-word bits (mi_kv_pool_check_errors). */
enum {
    MI_FAULT_BLOCK_ID = 1u,           /* a block-table entry outside [0, num_blocks) */
    MI_FAULT_CONTEXT_LEN = 2u         /* a length < 0, beyond the table row or beyond max_context_len */
};

/* Pool flags. */
enum {
    MI_POOL_HOST_ONLY = 1u,           /* block bookkeeping only: no device memory, no kernels */
    MI_POOL_KV_FP8 = 2u,              /* 8-bit cache: E4M3 codes with per-KV-head scales */
    MI_POOL_SWAP_STAGING = 4u,        /* device staging for scattered KV swaps (mi_kv_swap_out/in) */
    MI_POOL_DECODE_DOT = 8u           /* mi_paged_gqa_decode on vector-ALU dot products, not MFMA */
};

/* Static description of a status code. Never NULL. */
const char* mi_status_string(int status);

typedef struct mi_kv_pool_s* mi_kv_pool_t;

/*
 * Create a paged KV pool of one layer (mini-infer "KVCacheManager": block
 * tensor plus free-block pool).
 *  out          host pointer receiving the handle
 *  num_blocks   > 0
 *  block_size   must be 16
 *  num_kv_heads > 0
 *  head_dim     64 or 128
 *  k_cache, v_cache  both NULL: the library allocates both pools in device
 *               memory (contents undefined) and frees them on destroy. Both
 *               non-NULL: caller-owned device buffers of
 *               num_blocks*num_kv_heads*block_size*head_dim elements each
 *               (bf16 bits, or 1-byte E4M3 codes with MI_POOL_KV_FP8), never
 *               freed by the library. One NULL and one not: MI_ERR_INVALID_ARG.
 *  flags        any OR of
 *               MI_POOL_HOST_ONLY: no device memory (k_cache/v_cache must be
 *                 NULL) and every kernel call on the pool returns
 *                 MI_ERR_INVALID_ARG;
 *               MI_POOL_KV_FP8: the cache holds 8-bit E4M3 codes (OCP "FN"
 *                 variant: bias 7, no infinities, largest finite 448) of
 *                 value / scale, with one K scale and one V scale per KV head
 *                 (all 1.0 until mi_kv_pool_set_scales). vLLM-based
 *                 inference-framework report, "FP8 KV Cache quantisation": the
 *                 cache is held in FP8 to cut the bytes the attention moves;
 *               MI_POOL_SWAP_STAGING: also allocate a device staging buffer
 *                 for KV swaps (two halves of min(64 MiB, pool bytes), freed
 *                 on destroy), with which mi_kv_swap_out/in move a run of
 *                 scattered device blocks in one transfer;
 *               MI_POOL_DECODE_DOT: mi_paged_gqa_decode computes q.k and the
 *                 weighted V sum with packed bf16 dot products and fp32 FMAs
 *                 on the vector ALUs (one query head at a time per tile)
 *                 instead of the matrix cores: a second implementation of
 *                 the same operation, kept to compare the two designs, with
 *                 the same partition, workspace and tolerance. The other
 *                 entry points (decode step, layer, prefill, allocation-free
 *                 decode) are unaffected.
 * The free-block stack starts full; the first allocation returns ids 0, 1, ...
 * The current HIP device at this call is the pool's device.
 */
int mi_kv_pool_init(mi_kv_pool_t* out, int32_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim,
                    void* k_cache, void* v_cache, uint32_t flags);

/*
 * Per-KV-head scales of an 8-bit pool (nxmr.cn inference-techniques article,
 * section 2.2: heads with different value ranges need their own scales).
 * k_scales, v_scales: host arrays [num_kv_heads] of finite values > 0, or
 * NULL for all 1.0. A bf16 value x is stored as the code nearest to
 * float32(x) / scale (one float32 division, then round to nearest even,
 * saturating at +-448, NaN -> 0x7F) and read back as code_value * scale.
 * Set the scales before anything is written: codes already in the cache are
 * not converted. Synchronises the device. MI_ERR_INVALID_ARG for a bf16 pool
 * or a bad scale (nothing changed).
 */
int mi_kv_pool_set_scales(mi_kv_pool_t pool, const float* k_scales, const float* v_scales);

/*
 * Read back the per-KV-head scales of an 8-bit pool (as set or calibrated)
 * into host arrays [num_kv_heads]; either may be NULL. Synchronises the
 * device. MI_ERR_INVALID_ARG for a bf16 or host-only pool or two NULLs.
 */
int mi_kv_pool_get_scales(mi_kv_pool_t pool, float* k_scales, float* v_scales);

/*
 * Quantise whole bf16 caches into an 8-bit pool: k_src, v_src are device
 * bf16 pools of the same [num_blocks, num_kv_heads, 16, head_dim] shape
 * (e.g. filled by a bf16 prefill); every element is stored as its code under
 * its KV head's scale (the rule of mi_kv_pool_set_scales). Asynchronous on
 * stream. MI_ERR_INVALID_ARG for a bf16 or host-only pool or NULL sources.
 */
int mi_kv_pool_quantize(mi_kv_pool_t pool, const uint16_t* k_src, const uint16_t* v_src,
                        void* stream);

/*
 * Calibrate the per-KV-head scales of an 8-bit pool from sample rows, e.g. a
 * prefill chunk (nxmr.cn inference-techniques article, section 2.2: a group
 * is scaled by its largest magnitude so that this value maps to the largest
 * code; read here for E4M3 and static per-head scales). For each KV head and
 * each of K and V:
 *     s = (a * margin) / 448      (two float32 operations)
 * where a is the largest |x| over the head's finite sample values; s = 1.0
 * when that is not positive and finite (no finite nonzero sample).
 *  k, v    device bf16 [rows, num_kv_heads, head_dim] (the layout of
 *          mi_write_prefill_kv's k and v), 16-byte aligned, rows >= 1
 *  margin  finite and > 0. At 1 the sample's largest value stores as +-448;
 *          above 1 leaves headroom for larger later values, which would
 *          otherwise saturate.
 * The new scales replace the pool's on `stream` (asynchronous). Calibrate
 * before anything is written, as with mi_kv_pool_set_scales.
 * MI_ERR_INVALID_ARG for a bf16 or host-only pool, NULL or misaligned
 * inputs, rows < 1 or a bad margin (nothing launched).
 */
int mi_kv_pool_calibrate_scales(mi_kv_pool_t pool, const uint16_t* k, const uint16_t* v, int32_t rows,
                                float margin, void* stream);

/* Free the handle, library-owned pools and the error word. NULL is a no-op. */
int mi_kv_pool_destroy(mi_kv_pool_t pool);

/* Device pointers of the K and V pools (NULL for a host-only pool). */
int mi_kv_pool_get(mi_kv_pool_t pool, void** k_cache, void** v_cache);

/* Shape query: any output pointer may be NULL. */
int mi_kv_pool_shape(mi_kv_pool_t pool, int32_t* num_blocks, int32_t* block_size,
                     int32_t* num_kv_heads, int32_t* head_dim);

/*
 * Free-block pool (nxmr.cn article, section 2.1: pop one free page per page
 * needed). A LIFO stack: freed ids are handed out again last-in first-out.
 *  mi_kv_alloc_blocks  pops n ids into host array out_ids[n]; if fewer than n
 *                      are free, returns MI_ERR_NO_FREE_BLOCKS and pops none.
 *  mi_kv_free_blocks   pushes host array ids[n] back in order; an id out of
 *                      range, not allocated, or repeated returns
 *                      MI_ERR_INVALID_ARG and frees none.
 *  mi_kv_num_free_blocks  free count, or a negative status for a NULL pool.
 *  mi_kv_blocks_needed ceil(num_tokens / block_size) for num_tokens >= 0.
 */
int mi_kv_alloc_blocks(mi_kv_pool_t pool, int32_t n, int32_t* out_ids);
int mi_kv_free_blocks(mi_kv_pool_t pool, int32_t n, const int32_t* ids);
int32_t mi_kv_num_free_blocks(mi_kv_pool_t pool);
int32_t mi_kv_blocks_needed(int32_t num_tokens, int32_t block_size);

/*
 * Bytes of the K and V caches by the InferLLM article's formula, section 4.2
 * problem two, with hidden = num_kv_heads * head_dim and 2-byte elements.
 */
uint64_t mi_kv_cache_bytes(int64_t batch, int64_t layers, int64_t max_seq_len,
                           int64_t num_kv_heads, int64_t head_dim);

/*
 * Read and clear the pool's device error word (MI_FAULT_* bits) into
 * *fault_bits (host pointer, may be NULL). Synchronises the device. Returns
 * MI_ERR_DEVICE_FAULT if any bit was set, else MI_OK.
 */
int mi_kv_pool_check_errors(mi_kv_pool_t pool, uint32_t* fault_bits);

/*
 * write_decode_kv: RoPE, then append (mini-infer "decode_batch" step 4;
 * course project 2.1 RoPE and KV-cache append).
 *  q      device bf16 [batch, num_q_heads, head_dim]
 *  k, v   device bf16 [batch, num_kv_heads, head_dim]
 *  q_rot  device bf16 [batch, num_q_heads, head_dim]; may alias q exactly
 *  For each sequence b at pos = context_lens[b]: K[slot] = bf16(RoPE(k, pos)),
 *  V[slot] = v (bit copy) for every kv head, q_rot = bf16(RoPE(q, pos)), where
 *  slot = (block_table[b][pos / 16], pos % 16). The angle and the rotation are
 *  computed in float64 and rounded once to bf16 (nearest, ties to even).
 *  With an 8-bit pool (MI_POOL_KV_FP8) the slot receives the E4M3 codes of
 *  that bf16 K and of v under the head's scales (mi_kv_pool_set_scales).
 *  batch == 0 is a no-op.
 */
int mi_write_decode_kv(mi_kv_pool_t pool,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       uint16_t* q_rot,
                       const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t batch,
                       int32_t num_q_heads, double rope_theta, void* stream);

/*
 * Prefill write (mini-infer README: prefill runs as its own forward before a
 * request joins the batched decode steps; course project 2.1: prefill stage,
 * then decode, appending to the KV cache). One chunk of n_b new tokens per
 * sequence b at positions context_lens[b] .. context_lens[b] + n_b - 1,
 * packed over the batch:
 *  q      device bf16 [total_tokens, num_q_heads, head_dim]
 *  k, v   device bf16 [total_tokens, num_kv_heads, head_dim]
 *  q_rot  device bf16 [total_tokens, num_q_heads, head_dim]; may alias q
 *  cu_seqlens  device int32 [batch + 1]: 0 = cu[0] <= cu[1] <= ... <= cu[batch]
 *         = total_tokens; row i of q/k/v with cu[b] <= i < cu[b+1] is new token
 *         i - cu[b] of sequence b.
 *  context_lens  device int32 [batch]: tokens cached before the chunk.
 * Every new token gets the same RoPE, rounding and store as
 * mi_write_decode_kv at its position (E4M3 codes under the head's scales for
 * an 8-bit pool); the table row must cover context_lens[b] + n_b tokens.
 */
int mi_write_prefill_kv(mi_kv_pool_t pool, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, uint16_t* q_rot, const int32_t* block_table,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        const int32_t* cu_seqlens, int32_t batch, int32_t total_tokens,
                        int32_t num_q_heads, double rope_theta, void* stream);

/*
 * Causal paged GQA attention of a prefill chunk (after mi_write_prefill_kv):
 * the new token at position p of sequence b attends over positions 0 .. p of
 * that sequence through its block table (cached prefix and the chunk),
 *     out[i,h] = sum_{t <= p} softmax(scale * <q_rot[i,h], K[slot(b,t), g]>)_t V[slot(b,t), g]
 * with g = h / (num_q_heads / num_kv_heads). fp32 accumulation on MFMA, one
 * rounding to bf16 (no split). Each query's softmax is first taken relative
 * to the largest score of its first key tile, which is never raised; if any
 * later score exceeds it by more than 2^64 (in weight), the call repeats the
 * chunk with the running-maximum form (nxmr.cn article, section 5.1) in a
 * second launch, gated by a generation-numbered word in the pool, so prefill
 * calls on one pool must run one after another on one stream. (A captured
 * call replays with its generation number: once a replay has needed the
 * repeat, later replays repeat too -- same results, more time.)
 *  q_rot, out  device bf16 [total_tokens, num_q_heads, head_dim], no aliasing
 *  max_new_tokens  host-side bound of every n_b (sizes the grid); a larger
 *         n_b, cu beyond total_tokens or a chunk past the table row is a fault
 *         (error word) and that sequence's rows are not written.
 *  batch <= 65535. No workspace. An 8-bit pool's codes are read back as
 *  code * scale, as in mi_paged_gqa_decode.
 */
int mi_paged_prefill_attention(mi_kv_pool_t pool, const uint16_t* q_rot, uint16_t* out,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* cu_seqlens,
                               int32_t batch, int32_t total_tokens, int32_t max_new_tokens,
                               int32_t num_q_heads, float softmax_scale, void* stream);

/*
 * Workspace bytes needed by mi_paged_gqa_decode for this batch when every
 * context_lens[b] <= max_context_len (fp32 split-K partials plus padding).
 */
size_t mi_paged_gqa_decode_workspace_bytes(mi_kv_pool_t pool, int32_t batch,
                                           int32_t num_q_heads,
                                           int32_t max_context_len);

/*
 * Paged GQA decode attention (mini-infer gather + attention, fused: the
 * gather through the block table is never materialised). For each sequence b
 * and query head h, with g = h / (num_q_heads / num_kv_heads) and
 * L = context_lens[b] + 1:
 *     s_t = scale * <q_rot[b,h], K[slot(b,t), g]>,  t < L
 *     out[b,h] = sum_t softmax(s)_t V[slot(b,t), g]
 * (with an 8-bit pool, K and V are the codes times their head's scales). The
 * work is split over the device in equal shares of tiles (split-K online
 * softmax): q.K in fp32 from exact bf16 products, the softmax weights
 * exp2-based in fp32 and rounded to bf16 for the weighted sum of V (fp32
 * accumulation), partial results merged in fp32, one rounding to bf16.
 * Short segments (max_context_len + 1 <= 384 and at most 512 (sequence, kv
 * head) pairs, with the library's split) are split over the waves of one
 * workgroup per pair instead and merged on chip: one launch, the workspace
 * untouched.
 *  batch   0 .. 1024 (more: MI_ERR_UNSUPPORTED)
 *  q_rot   device bf16 [batch, num_q_heads, head_dim] (as written by
 *          mi_write_decode_kv)
 *  out     device bf16 [batch, num_q_heads, head_dim]; must not alias q_rot
 *  softmax_scale  <= 0 selects 1/sqrt(head_dim)
 *  max_context_len  host-side upper bound of context_lens[b]; sizes the grid
 *          and the workspace. A larger length is a fault (error word) and
 *          that sequence's output is undefined.
 *  workspace  device buffer of at least the queried bytes (caller-owned,
 *          contents need not be initialised).
 * Tail slots of the last block and blocks past the sequence may hold any
 * bits (NaN included): they are excluded by selection, never by
 * multiplication with zero. The reduction order depends only on logical
 * positions, so results are bit-identical under any relabelling of physical
 * blocks.
 */
int mi_paged_gqa_decode(mi_kv_pool_t pool, const uint16_t* q_rot, uint16_t* out,
                        const int32_t* block_table, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t batch,
                        int32_t num_q_heads, float softmax_scale,
                        int32_t max_context_len,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Same as mi_paged_gqa_decode with an explicit split size: split_tokens is
 * the minimum number of tokens in one wave's share of the work (a positive
 * multiple of 16; small workloads then use fewer, longer shares), or 0 for
 * the library's choice (32). The workspace query for an explicit split size
 * is mi_paged_gqa_decode_split_workspace_bytes.
 */
int mi_paged_gqa_decode_split(mi_kv_pool_t pool, const uint16_t* q_rot, uint16_t* out,
                              const int32_t* block_table, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t batch,
                              int32_t num_q_heads, float softmax_scale,
                              int32_t max_context_len, int32_t split_tokens,
                              void* workspace, size_t workspace_bytes, void* stream);
size_t mi_paged_gqa_decode_split_workspace_bytes(mi_kv_pool_t pool, int32_t batch,
                                                 int32_t num_q_heads,
                                                 int32_t max_context_len,
                                                 int32_t split_tokens);

/*
 * Debug export of the gather step (mini-infer gather_batch_kv): bit copies of
 * K and V of positions [0, context_lens[b] + len_extra) of every sequence and
 * kv head into k_out / v_out, device arrays [batch, num_kv_heads, l_max,
 * head_dim] of the pool's element type (bf16 bits, or E4M3 codes). Positions
 * at or beyond that length are not written.
 * len_extra is 0 or 1; every context_lens[b] + len_extra must be <= l_max.
 */
int mi_gather_kv(mi_kv_pool_t pool, const int32_t* block_table,
                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                 int32_t batch, int32_t len_extra,
                 void* k_out, void* v_out, int32_t l_max, void* stream);

/* ------------------------------------------------------------------------
 * Full decoder-layer decode step (course project 2.1: RMSNorm, QKV with
 * GQA, RoPE, KV append, attention, o_proj, residual, RMSNorm, SwiGLU,
 * residual), pre-norm:
 *   r1 = RMSNorm(x) * ln1_w;  [q|k|v] = r1 W_qkv^T
 *   write_decode_kv (RoPE, append);  o = paged GQA attention
 *   x2 = x + o W_o^T;  r2 = RMSNorm(x2) * ln2_w
 *   x_out = x2 + (silu(r2 W_gate^T) * (r2 W_up^T)) W_down^T
 * Weights are device bf16 in nn.Linear layout [out_features, in_features];
 * w_qkv rows are q (num_q_heads*head_dim), then k, then v
 * (num_kv_heads*head_dim each). The projections run on bf16 MFMA with fp32
 * accumulation; norms, RoPE angle and softmax in fp32/fp64 as above.
 * Supported: hidden and intermediate multiples of 256, batch 1..32.
 * ------------------------------------------------------------------------ */
typedef struct {
    int32_t hidden;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t intermediate;
    float rms_eps;
    double rope_theta;
} mi_layer_config;

typedef struct {
    const uint16_t* ln1_w;    /* [hidden] */
    const uint16_t* w_qkv;    /* [(num_q_heads + 2*num_kv_heads)*head_dim, hidden] */
    const uint16_t* w_o;      /* [hidden, num_q_heads*head_dim] */
    const uint16_t* ln2_w;    /* [hidden] */
    const uint16_t* w_gate;   /* [intermediate, hidden] */
    const uint16_t* w_up;     /* [intermediate, hidden] */
    const uint16_t* w_down;   /* [hidden, intermediate] */
} mi_layer_weights;

/* Workspace bytes needed by mi_decoder_layer_decode (host-side query). */
size_t mi_decoder_layer_workspace_bytes(const mi_layer_config* cfg, mi_kv_pool_t pool,
                                        int32_t batch, int32_t max_context_len);

/*
 * One decode step of one layer for `batch` sequences.
 *  cfg, w    host pointers to the structs above (read during the call only)
 *  x_in      device bf16 [batch, hidden]
 *  x_out     device bf16 [batch, hidden]; must not alias x_in
 *  block_table, max_blocks_per_seq, context_lens, max_context_len: as for
 *            mi_paged_gqa_decode (the new token is appended at context_lens[b])
 *  workspace device buffer of at least mi_decoder_layer_workspace_bytes
 */
int mi_decoder_layer_decode(mi_kv_pool_t pool, const mi_layer_config* cfg,
                            const mi_layer_weights* w,
                            const uint16_t* x_in, uint16_t* x_out,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t batch,
                            int32_t max_context_len,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Continuous-batching step planner (host only): block lifecycle and admission
 * over a pool's free-block stack, with the KV-protection brakes of the
 * vLLM-based inference-framework report ("SLO-aware, KV-cache protecting
 * scheduler": free KV space below a critical threshold stops new prefills
 * -- hard brake; running decodes with free space below a safety threshold
 * stop them too -- soft brake; otherwise requests proceed) and the
 * mini-infer scheduler's waiting/running queues (prefill alone, then batched
 * decode, admission at every step).
 *
 * The planner takes blocks from and returns them to `pool` (mi_kv_alloc_blocks
 * / mi_kv_free_blocks): while it lives, nothing else may allocate from that
 * pool. It is not thread-safe.
 */
typedef struct mi_sched_s* mi_sched_t;

enum { MI_BRAKE_PROCEED = 0, MI_BRAKE_SOFT = 1, MI_BRAKE_HARD = 2 };

typedef struct {
    int32_t num_prefill;     /* rows 0 .. num_prefill-1 of the step's outputs */
    int32_t num_decode;      /* the following num_decode rows */
    int32_t num_preempted;   /* entries of preempted_ids */
    int32_t num_finished;    /* entries of finished_ids */
    int32_t brake;           /* MI_BRAKE_* seen by the step's first admission check */
    int32_t free_blocks;     /* free blocks after the step's allocations */
    int32_t num_swapped_out; /* entries of swapped_ids */
    int32_t num_swap_out;    /* (device block, host slot) pairs in swap_out */
    int32_t num_swap_in;     /* (host slot, device block) pairs in swap_in */
} mi_sched_counts;

/*
 * max_blocks_per_seq  block-table row length of the plans (and the longest
 *                     request: ceil((prompt + max_new) / 16) blocks)
 * max_running         most requests running at once (rows of a plan)
 * hard_free_frac, soft_free_frac  thresholds on free / pool blocks in [0, 1]
 *                     (the report's values: 0.10 and 0.30); "below" is strict.
 */
int mi_sched_create(mi_sched_t* out, mi_kv_pool_t pool, int32_t max_blocks_per_seq,
                    int32_t max_running, double hard_free_frac, double soft_free_frac);
/* Returns every block still held by running requests to the pool. */
int mi_sched_destroy(mi_sched_t sched);

/*
 * Queue a request (FIFO). MI_ERR_UNSUPPORTED if prompt_tokens + max_new_tokens
 * needs more blocks than a table row or the whole pool (it could never run);
 * MI_ERR_INVALID_ARG for counts < 1.
 */
int mi_sched_submit(mi_sched_t sched, int64_t request_id, int32_t prompt_tokens,
                    int32_t max_new_tokens);
int32_t mi_sched_num_waiting(mi_sched_t sched);
int32_t mi_sched_num_running(mi_sched_t sched);
int32_t mi_sched_num_swapped(mi_sched_t sched);

/*
 * KV offload (course project, optional task "KV Cache Offloading": inactive
 * KV blocks go to CPU memory and come back when needed, under an eviction
 * policy). Gives the planner a host swap space of host_slots blocks (call
 * before the first step; 0 = none). A preemption victim (picked by the
 * eviction policy, mi_sched_set_eviction) whose blocks fit the free host slots is then
 * swapped out instead of recomputed: it keeps its context and comes back
 * before anything new is admitted (swapped requests in swap order, regardless
 * of the brakes), with its blocks copied back into fresh device blocks.
 */
int mi_sched_set_swap_space(mi_sched_t sched, int32_t host_slots);

/*
 * Eviction policy of the planner (the same optional task: "design an eviction
 * policy -- LRU / FIFO / by layer / by token segment"). It picks the running
 * request that makes room when the pool runs dry, for swap-out and for
 * recompute preemption alike:
 *  MI_EVICT_LIFO  the most recently admitted running request (the default;
 *                 vLLM's preemption order);
 *  MI_EVICT_FIFO  the running request that entered the running set first
 *                 (admitted, or swapped back in, earliest);
 *  MI_EVICT_LRU   the least recently used running request: every step reads
 *                 the KV of every running request, so this is the FIFO
 *                 victim (identical plans).
 * May be changed between steps. MI_ERR_INVALID_ARG for another value.
 */
enum { MI_EVICT_LIFO = 0, MI_EVICT_FIFO = 1, MI_EVICT_LRU = 2 };
int mi_sched_set_eviction(mi_sched_t sched, int32_t policy);

/*
 * Plan one engine step (host arrays, capacity max_running rows each):
 *  1. requests that produced max_new_tokens retire (ids in finished_ids) and
 *     return their blocks;
 *  2. every running request gets the block its decode write at position
 *     context_len needs (ceil((context_len + 1) / 16) blocks), in admission
 *     order; on an empty pool the running request the eviction policy picks
 *     is preempted (blocks returned; re-queued first, to be prefilled again over
 *     its prompt and generated tokens; id in preempted_ids);
 *  3. waiting requests are admitted in order while a row is free, no brake
 *     holds (free / pool re-measured before each admission) and the pool
 *     holds ceil(prompt / 16) blocks; the first that cannot be admitted
 *     stops admission;
 *  4. rows: the admitted prefills (context_lens 0, new_tokens = prompt), then
 *     the decodes (context_lens = tokens cached, new_tokens 1), with their
 *     block-table rows in block_table [max_running, max_blocks_per_seq]
 *     (-1 padded) -- the inputs of mi_write_prefill_kv /
 *     mi_paged_prefill_attention and mi_write_decode_kv / mi_paged_gqa_decode.
 *     The plan is taken as executed: a prefill yields a request's first
 *     token, a decode one more.
 * With swap space (mi_sched_set_swap_space): swapped_ids [max_running] gets
 * the requests swapped out this step, swap_out [max_running *
 * max_blocks_per_seq][2] the (device block, host slot) pairs to copy out and
 * swap_in (same capacity) the (host slot, device block) pairs to copy back
 * (swapped-in requests decode in this step, after the others). Execute in
 * order: mi_kv_swap_out, mi_kv_swap_in, then the prefill and decode kernels.
 */
int mi_sched_step(mi_sched_t sched, mi_sched_counts* counts, int64_t* seq_ids,
                  int32_t* context_lens, int32_t* new_tokens, int32_t* block_table,
                  int64_t* preempted_ids, int64_t* finished_ids, int64_t* swapped_ids,
                  int32_t* swap_out, int32_t* swap_in);

/*
 * Block copies between a pool and a host swap space (KV offload). host_k,
 * host_v: host arrays [host_slots, num_kv_heads, 16, head_dim] of the pool's
 * element type (bf16 bits or E4M3 codes), page-locked for asynchronous
 * copies (e.g. hipHostMalloc); pairs: host array of n (device block, host
 * slot) pairs for swap_out, n (host slot, device block) pairs for swap_in;
 * each destination (slot out, block in) at most once. Every id and slot is
 * checked before anything is copied (MI_ERR_INVALID_ARG). Pairs are ordered
 * by host slot and each run of consecutive slots moves in one DMA transfer
 * queued on stream, asynchronous for page-locked host memory (the host
 * arrays must stay alive until the stream reaches them); scattered device
 * blocks of a run are packed / unpacked by a kernel through the pool's
 * staging buffer (pools created with MI_POOL_SWAP_STAGING, in chunks of its
 * size), else moved one block per transfer. No device memory is allocated.
 * Swaps on one pool must be ordered on one stream.
 */
int mi_kv_swap_out(mi_kv_pool_t pool, void* host_k, void* host_v, int32_t host_slots,
                   const int32_t* pairs, int32_t n, void* stream);
int mi_kv_swap_in(mi_kv_pool_t pool, const void* host_k, const void* host_v, int32_t host_slots,
                  const int32_t* pairs, int32_t n, void* stream);

/*
 * One decode step in one attention launch (mini-infer "decode_batch":
 * write_decode_kv of the new token, then attention over the gathered cache;
 * course project 2.1: RoPE, KV-cache append, GQA): the effect of
 * mi_write_decode_kv followed by mi_paged_gqa_decode with the same
 * arguments, without the separate write launch. The wave that reads a
 * sequence's last tile for a kv head first writes that head's new k (RoPE)
 * and v into the slot, so the cache after the call and q_rot are
 * bit-identical to mi_write_decode_kv's. The query operand of the attention
 * is rotated by each wave itself in float32 (within one bf16 rounding of the
 * float64 rotation), so out can differ from the two-call path in the last
 * bits, within the same tolerance of the exact result.
 *  q, k, v  device bf16 as for mi_write_decode_kv (not modified)
 *  q_rot    device bf16 [batch, num_q_heads, head_dim] receiving RoPE(q), or
 *           NULL; must not alias q or out
 *  out      device bf16 [batch, num_q_heads, head_dim]; must not alias q
 *  rope_theta, softmax_scale, max_context_len, workspace: as for
 *           mi_write_decode_kv and mi_paged_gqa_decode (workspace query:
 *           mi_paged_gqa_decode_workspace_bytes)
 * A sequence whose length is out of range (a recorded fault) gets no cache
 * write and NaN outputs. batch == 0 is a no-op.
 */
int mi_paged_gqa_decode_step(mi_kv_pool_t pool, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, uint16_t* q_rot, uint16_t* out,
                             const int32_t* block_table, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t batch,
                             int32_t num_q_heads, double rope_theta, float softmax_scale,
                             int32_t max_context_len, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * mi_paged_gqa_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, results and default split as mi_paged_gqa_decode
 * (the same kernels, bit-identical outputs), but no workspace: the split-K
 * partials go to a fixed device array of MI_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends (its address on a device
 * is taken when the first pool is created there). The call allocates nothing.
 * The partials need 2 * W * G * (4 * head_dim + 8) bytes for a grid of W
 * waves (three per compute unit, fewer for small workloads): 6.4 MB at
 * G = 8, head_dim = 128 on 256 compute units. A call that would need more
 * returns MI_ERR_SCRATCH_TOO_SMALL and launches nothing. Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller; every slot a
 * call reads it has written itself, so nothing needs clearing between calls.
 */
#define MI_NOALLOC_SCRATCH_BYTES (8u << 20)
int mi_paged_gqa_decode_noalloc(mi_kv_pool_t pool, const uint16_t* q_rot, uint16_t* out,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t batch,
                                int32_t num_q_heads, float softmax_scale,
                                int32_t max_context_len, void* stream);

/*
 * Measurement utility (not a step of the method): reads `bytes` of device
 * memory at `src` (16-byte aligned, bytes a multiple of 16) with 16-byte
 * non-temporal loads, each of `workgroups` workgroups of 256 threads one
 * contiguous chunk (a tail of fewer than `workgroups` 16-byte units is not
 * read), and stores one folded word per thread into `sink` (device,
 * workgroups * 256 uint32, caller-owned). Timing it gives the streaming-read
 * bandwidth the part delivers, the practical ceiling next to the published
 * HBM peak. Asynchronous on `stream`; MI_ERR_INVALID_ARG for null pointers,
 * misalignment or workgroups outside 1..65536 or above bytes / 16.
 */
int mi_hbm_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MIKV_H */
