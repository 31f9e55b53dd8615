"""write_decode_kv, gather through the block table, paged GQA decode attention.

Test infrastructure only. Everything is float64; the only roundings are the
bf16 stores the definition itself makes (the cache and the boundary outputs).

Pages followed:

* mini-infer README, "decode_batch key steps": gather each request's cached
  K/V from the block tensor through its BlockTable, run the batched forward,
  write the new token's K/V back into the block tensor (write_decode_kv).
* Course project, section 2.1: RoPE; grouped-query attention, where the KV
  heads are shared by groups of query heads (sdpa with enable_gqa, or
  repeat_interleave of the KV heads): query head h reads KV head h // G with
  G = Hq / Hkv; the KV cache grows by appending one token per decode step.
* nxmr.cn inference-techniques article, section 5.1: the numerically stable
  softmax -- subtract the row max, exponentiate, divide by the row sum, then
  weight V; section 4.1: attention scores are kept in FP32 or better.

Readings where the pages are silent:

* context_lens[b] counts tokens cached BEFORE this step; the new token is
  written at logical position ctx_b (also its RoPE position) and attention
  covers L_b = ctx_b + 1 tokens, the new one included.
* RoPE rotates q and the new k, never v; cached K is stored rotated.
* softmax scale 1 / sqrt(D) unless given.
"""
import numpy as np

from . import bf16
from . import fp8
from . import paged
from . import rope


def write_decode_kv(k_pool, v_pool, q, k, v, block_table, context_lens,
                    block_size, theta):
    """Append the new token's rotated K and its V; rotate q.

    k_pool, v_pool : uint16 bf16 bits [N, Hkv, bs, D] (not modified)
    q              : uint16 [B, Hq, D];  k, v : uint16 [B, Hkv, D]
    block_table    : int [B, MB];        context_lens : int [B] (pre-step)

    Returns (k_pool_new, v_pool_new, q_rot_bits, q_rot_f64). q_rot_f64 is the
    unrounded rotation (what a fused layer keeps internally).
    """
    k_new = np.array(k_pool, dtype=np.uint16, copy=True)
    v_new = np.array(v_pool, dtype=np.uint16, copy=True)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    q_rot = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        pos = int(context_lens[b])
        blk, off = paged.slot(block_table[b], pos, block_size)
        for g in range(Hkv):
            k_new[blk, g, off, :] = bf16.encode(rope.apply(bf16.decode(k[b, g]), pos, theta))
            v_new[blk, g, off, :] = v[b, g]
        for h in range(Hq):
            q_rot[b, h] = rope.apply(bf16.decode(q[b, h]), pos, theta)
    return k_new, v_new, bf16.encode(q_rot), q_rot


def gather_kv(k_pool, v_pool, block_table, block_size, b, g, length):
    """Contiguous copies of K and V of sequence b, kv head g, positions [0, length).

    Bit copies (the pool's element type: bf16 bits or 8-bit codes) in logical
    order -- the gather_batch_kv step.
    """
    D = k_pool.shape[-1]
    ks = np.empty((length, D), dtype=k_pool.dtype)
    vs = np.empty((length, D), dtype=v_pool.dtype)
    for p in range(length):
        blk, off = paged.slot(block_table[b], p, block_size)
        ks[p] = k_pool[blk, g, off]
        vs[p] = v_pool[blk, g, off]
    return ks, vs


def attend(q_vec, K, V, scale):
    """One query against L keys: softmax(K q * scale) V, the stable form.

    q_vec [D], K [L, D], V [L, D], all float64.
    """
    s = (K @ q_vec) * scale
    m = np.max(s)
    p = np.exp(s - m)
    return (p @ V) / np.sum(p)


def partial_attend(q_vec, K, V, scale):
    """The softmax statistics of one piece of the key range (the split-K step
    of the decode path; nxmr.cn section 5.1's stable form kept unnormalised):
    m = max of the scores, l = sum of exp(s - m), acc = sum of exp(s - m) V.
    An empty piece returns (-inf, 0, 0).
    """
    s = (K @ q_vec) * scale
    if s.size == 0:
        return -np.inf, 0.0, np.zeros(V.shape[1])
    m = np.max(s)
    p = np.exp(s - m)
    return m, np.sum(p), p @ V


def combine_partials(parts):
    """Merge the (m, l, acc) of the pieces of one key range: with M = max m_i,
    out = sum_i exp(m_i - M) acc_i / sum_i exp(m_i - M) l_i. Pieces are taken
    in the order given (the result is the same for any order in exact
    arithmetic). Pinned by tests/test_oracle_combine.py: equal to attend()
    over the whole range for any split, empty pieces included.
    """
    M = max(m for m, _, _ in parts)
    l = 0.0
    acc = 0.0
    for m, li, ai in parts:
        if m == -np.inf:
            continue
        w = np.exp(m - M)
        l = l + w * li
        acc = acc + w * ai
    return acc / l


def paged_gqa_decode(q_rot, k_pool, v_pool, block_table, context_lens, block_size,
                     scale=None, q_is_bits=True):
    """Paged GQA decode attention: every query head of every sequence attends
    over the L_b = ctx_b + 1 cached tokens of its KV head.

    q_rot : [B, Hq, D] bf16 bits (or float64 if q_is_bits is False)
    k_pool, v_pool : bf16 bits [N, Hkv, bs, D] (already holding the new token)
    Returns float64 [B, Hq, D].
    """
    qf = bf16.decode(q_rot) if q_is_bits else np.asarray(q_rot, dtype=np.float64)
    B, Hq, D = qf.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(np.float64(D))
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b]) + 1
        for g in range(Hkv):
            ks, vs = gather_kv(k_pool, v_pool, block_table, block_size, b, g, L)
            K = bf16.decode(ks)
            V = bf16.decode(vs)
            for h in range(g * G, (g + 1) * G):
                out[b, h] = attend(qf[b, h], K, V, scale)
    return out


def decode_step(k_pool, v_pool, q, k, v, block_table, context_lens, block_size,
                theta, scale=None):
    """write_decode_kv followed by paged attention (the attention half of a
    decoder-layer decode step). Returns (out_f64, k_pool_new, v_pool_new, q_rot_bits)."""
    k_new, v_new, q_rot_bits, _ = write_decode_kv(
        k_pool, v_pool, q, k, v, block_table, context_lens, block_size, theta)
    out = paged_gqa_decode(q_rot_bits, k_new, v_new, block_table, context_lens,
                           block_size, scale)
    return out, k_new, v_new, q_rot_bits


# ---------------------------------------------------------------- 8-bit cache
# vLLM-based inference-framework project report, "FP8 KV Cache quantisation":
# the cache holds FP8 codes; the attention reads them back dequantised. Codec
# and scale convention in oracle.fp8.

def write_decode_kv_fp8(k_pool8, v_pool8, q, k, v, block_table, context_lens,
                        block_size, theta, k_scales, v_scales):
    """write_decode_kv into an 8-bit cache: the new token's K is rotated and
    rounded to bf16 exactly as for the bf16 cache, then K and V are quantised
    with their KV head's scale (oracle.fp8.quantize) and stored at the slot.

    k_pool8, v_pool8 : uint8 codes [N, Hkv, bs, D] (not modified)
    k_scales, v_scales : [Hkv] float32 scales
    Returns (k_pool_new, v_pool_new, q_rot_bits, q_rot_f64).
    """
    k_new = np.array(k_pool8, dtype=np.uint8, copy=True)
    v_new = np.array(v_pool8, dtype=np.uint8, copy=True)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    q_rot = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        pos = int(context_lens[b])
        blk, off = paged.slot(block_table[b], pos, block_size)
        for g in range(Hkv):
            k_rot = bf16.decode(bf16.encode(rope.apply(bf16.decode(k[b, g]), pos, theta)))
            k_new[blk, g, off, :] = fp8.quantize(k_rot, k_scales[g])
            v_new[blk, g, off, :] = fp8.quantize(bf16.decode(v[b, g]), v_scales[g])
        for h in range(Hq):
            q_rot[b, h] = rope.apply(bf16.decode(q[b, h]), pos, theta)
    return k_new, v_new, bf16.encode(q_rot), q_rot


def paged_gqa_decode_fp8(q_rot, k_pool8, v_pool8, block_table, context_lens, block_size,
                         k_scales, v_scales, scale=None, q_is_bits=True):
    """Paged GQA decode attention over an 8-bit cache: gather the codes through
    the block table, dequantise them with their KV head's scales, then the
    same stable softmax attention as paged_gqa_decode. Returns float64
    [B, Hq, D]."""
    qf = bf16.decode(q_rot) if q_is_bits else np.asarray(q_rot, dtype=np.float64)
    B, Hq, D = qf.shape
    Hkv = k_pool8.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(np.float64(D))
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b]) + 1
        for g in range(Hkv):
            ks, vs = gather_kv(k_pool8, v_pool8, block_table, block_size, b, g, L)
            K = fp8.dequantize(ks, k_scales[g])
            V = fp8.dequantize(vs, v_scales[g])
            for h in range(g * G, (g + 1) * G):
                out[b, h] = attend(qf[b, h], K, V, scale)
    return out


def decode_step_fp8(k_pool8, v_pool8, q, k, v, block_table, context_lens, block_size,
                    theta, k_scales, v_scales, scale=None):
    """write_decode_kv_fp8 followed by paged_gqa_decode_fp8.
    Returns (out_f64, k_pool_new, v_pool_new, q_rot_bits)."""
    k_new, v_new, q_rot_bits, _ = write_decode_kv_fp8(
        k_pool8, v_pool8, q, k, v, block_table, context_lens, block_size, theta,
        k_scales, v_scales)
    out = paged_gqa_decode_fp8(q_rot_bits, k_new, v_new, block_table, context_lens,
                               block_size, k_scales, v_scales, scale)
    return out, k_new, v_new, q_rot_bits


# -------------------------------------------------------------------- prefill
# mini-infer README, "Project overview": prefill runs as its own forward for a
# request's prompt before the request joins the batched decode steps; course
# project section 2.1: the inference loop is a prefill stage then a decode
# stage, with the KV cache appended as tokens are processed. A prefill chunk
# of sequence b holds n_b new tokens at positions ctx_b .. ctx_b + n_b - 1
# (ctx_b tokens already cached; 0 for a fresh prompt). The new tokens are
# packed over the batch: token i of sequence b is row cu[b] + i of q, k, v
# (cu = prefix sums of n_b). Each new token's K/V is written like a decode
# step's, and each new token attends causally over positions 0 .. its own.

def _prefill_rows(context_lens, cu_seqlens):
    """(row, sequence, position) of every packed new token."""
    out = []
    for b in range(len(context_lens)):
        for i in range(int(cu_seqlens[b]), int(cu_seqlens[b + 1])):
            out.append((i, b, int(context_lens[b]) + i - int(cu_seqlens[b])))
    return out


def write_prefill_kv(k_pool, v_pool, q, k, v, block_table, context_lens, cu_seqlens,
                     block_size, theta):
    """Append every new token's rotated K and its V at its position; rotate q.

    q : uint16 [T, Hq, D];  k, v : uint16 [T, Hkv, D]  (packed rows)
    Returns (k_pool_new, v_pool_new, q_rot_bits [T, Hq, D])."""
    k_new = np.array(k_pool, dtype=np.uint16, copy=True)
    v_new = np.array(v_pool, dtype=np.uint16, copy=True)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    q_rot = np.empty((T, Hq, D), dtype=np.float64)
    for i, b, pos in _prefill_rows(context_lens, cu_seqlens):
        blk, off = paged.slot(block_table[b], pos, block_size)
        for g in range(Hkv):
            k_new[blk, g, off, :] = bf16.encode(rope.apply(bf16.decode(k[i, g]), pos, theta))
            v_new[blk, g, off, :] = v[i, g]
        for h in range(Hq):
            q_rot[i, h] = rope.apply(bf16.decode(q[i, h]), pos, theta)
    return k_new, v_new, bf16.encode(q_rot)


def paged_prefill_attention(q_rot, k_pool, v_pool, block_table, context_lens, cu_seqlens,
                            block_size, scale=None):
    """Causal paged GQA attention of the packed new tokens: the token at
    position p of sequence b attends over positions 0 .. p of its sequence
    (cached prefix and the new tokens, already written). Returns float64
    [T, Hq, D]."""
    qf = bf16.decode(q_rot)
    T, Hq, D = qf.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(np.float64(D))
    out = np.empty((T, Hq, D), dtype=np.float64)
    for b in range(len(context_lens)):
        lo, hi = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        if hi == lo:
            continue
        last = int(context_lens[b]) + hi - lo          # keys of the last new token
        for g in range(Hkv):
            ks, vs = gather_kv(k_pool, v_pool, block_table, block_size, b, g, last)
            K, V = bf16.decode(ks), bf16.decode(vs)
            for i in range(lo, hi):
                L = int(context_lens[b]) + i - lo + 1
                for h in range(g * G, (g + 1) * G):
                    out[i, h] = attend(qf[i, h], K[:L], V[:L], scale)
    return out


def prefill_step(k_pool, v_pool, q, k, v, block_table, context_lens, cu_seqlens, block_size,
                 theta, scale=None):
    """write_prefill_kv followed by paged_prefill_attention.
    Returns (out_f64, k_pool_new, v_pool_new, q_rot_bits)."""
    k_new, v_new, q_rot_bits = write_prefill_kv(k_pool, v_pool, q, k, v, block_table,
                                                context_lens, cu_seqlens, block_size, theta)
    out = paged_prefill_attention(q_rot_bits, k_new, v_new, block_table, context_lens,
                                  cu_seqlens, block_size, scale)
    return out, k_new, v_new, q_rot_bits


def write_prefill_kv_fp8(k_pool8, v_pool8, q, k, v, block_table, context_lens, cu_seqlens,
                         block_size, theta, k_scales, v_scales):
    """write_prefill_kv into an 8-bit cache: every new token's bf16 K (rotated)
    and V are quantised with their KV head's scales, as in
    write_decode_kv_fp8. Returns (k_pool_new, v_pool_new, q_rot_bits)."""
    k_new = np.array(k_pool8, dtype=np.uint8, copy=True)
    v_new = np.array(v_pool8, dtype=np.uint8, copy=True)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    q_rot = np.empty((T, Hq, D), dtype=np.float64)
    for i, b, pos in _prefill_rows(context_lens, cu_seqlens):
        blk, off = paged.slot(block_table[b], pos, block_size)
        for g in range(Hkv):
            k_rot = bf16.decode(bf16.encode(rope.apply(bf16.decode(k[i, g]), pos, theta)))
            k_new[blk, g, off, :] = fp8.quantize(k_rot, k_scales[g])
            v_new[blk, g, off, :] = fp8.quantize(bf16.decode(v[i, g]), v_scales[g])
        for h in range(Hq):
            q_rot[i, h] = rope.apply(bf16.decode(q[i, h]), pos, theta)
    return k_new, v_new, bf16.encode(q_rot)


def paged_prefill_attention_fp8(q_rot, k_pool8, v_pool8, block_table, context_lens, cu_seqlens,
                                block_size, k_scales, v_scales, scale=None):
    """Causal prefill attention over an 8-bit cache: the codes gathered through
    the block table are dequantised with their head's scales, then the same
    causal attention as paged_prefill_attention. Returns float64 [T, Hq, D]."""
    qf = bf16.decode(q_rot)
    T, Hq, D = qf.shape
    Hkv = k_pool8.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(np.float64(D))
    out = np.empty((T, Hq, D), dtype=np.float64)
    for b in range(len(context_lens)):
        lo, hi = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        if hi == lo:
            continue
        last = int(context_lens[b]) + hi - lo
        for g in range(Hkv):
            ks, vs = gather_kv(k_pool8, v_pool8, block_table, block_size, b, g, last)
            K, V = fp8.dequantize(ks, k_scales[g]), fp8.dequantize(vs, v_scales[g])
            for i in range(lo, hi):
                L = int(context_lens[b]) + i - lo + 1
                for h in range(g * G, (g + 1) * G):
                    out[i, h] = attend(qf[i, h], K[:L], V[:L], scale)
    return out


def prefill_step_fp8(k_pool8, v_pool8, q, k, v, block_table, context_lens, cu_seqlens,
                     block_size, theta, k_scales, v_scales, scale=None):
    """write_prefill_kv_fp8 followed by paged_prefill_attention_fp8.
    Returns (out_f64, k_pool_new, v_pool_new, q_rot_bits)."""
    k_new, v_new, q_rot_bits = write_prefill_kv_fp8(k_pool8, v_pool8, q, k, v, block_table,
                                                    context_lens, cu_seqlens, block_size, theta,
                                                    k_scales, v_scales)
    out = paged_prefill_attention_fp8(q_rot_bits, k_new, v_new, block_table, context_lens,
                                      cu_seqlens, block_size, k_scales, v_scales, scale)
    return out, k_new, v_new, q_rot_bits
