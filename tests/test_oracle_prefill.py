"""Pins for the oracle's prefill (CPU only): a chunk of one token per
sequence is a decode step (pinned separately); a whole prompt matches torch's
causal scaled_dot_product_attention in float64 on the contiguous K/V; a
prefill split into chunks equals the corresponding rows of one unsplit
prefill; block relabelling, placement and NaN-poison invariants."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from oracle import attention, bf16, paged

CFG = workloads.DecodeConfig("pf", batch=3, num_q_heads=6, num_kv_heads=2, head_dim=32,
                             block_size=16, num_blocks=64, rope_theta=1e4, ctx_draw="fixed",
                             seed=71)


def _prefill(case):
    return attention.prefill_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                  case.block_table, case.context_lens, case.cu_seqlens, 16,
                                  case.cfg.rope_theta)


def test_single_token_chunks_equal_the_decode_step():
    case = workloads.make_prefill_case(CFG, (0, 17, 40), (1, 1, 1))
    out, kn, vn, qb = _prefill(case)
    ref, kd, vd, qd = attention.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                            case.block_table, case.context_lens, 16,
                                            CFG.rope_theta)
    assert np.array_equal(out, ref)
    assert np.array_equal(kn, kd) and np.array_equal(vn, vd) and np.array_equal(qb, qd)


def test_whole_prompt_matches_torch_causal_sdpa():
    case = workloads.make_prefill_case(CFG, (0, 0, 0), (37, 16, 5))
    out, kn, vn, qb = _prefill(case)
    G = CFG.num_q_heads // CFG.num_kv_heads
    for b in range(3):
        lo, hi = case.cu_seqlens[b], case.cu_seqlens[b + 1]
        n = hi - lo
        K = np.stack([bf16.decode(attention.gather_kv(kn, vn, case.block_table, 16, b, g, n)[0])
                      for g in range(CFG.num_kv_heads)])
        V = np.stack([bf16.decode(attention.gather_kv(kn, vn, case.block_table, 16, b, g, n)[1])
                      for g in range(CFG.num_kv_heads)])
        Q = bf16.decode(qb[lo:hi]).transpose(1, 0, 2)             # [Hq, n, D]
        t = F.scaled_dot_product_attention(torch.from_numpy(Q)[None], torch.from_numpy(K)[None],
                                           torch.from_numpy(V)[None], is_causal=True,
                                           enable_gqa=True)[0].numpy()
        assert np.abs(t.transpose(1, 0, 2) - out[lo:hi]).max() < 1e-12
    assert G == 3


def test_chunked_prefill_equals_rows_of_one_unsplit_prefill():
    full = workloads.make_prefill_case(CFG, (0, 0, 0), (45, 20, 33), seed=5)
    out_full, kf, vf, _ = _prefill(full)
    # the same prompts split at 30 / 7 / 16 tokens: first chunk, then the rest
    split = (30, 7, 16)
    rows1, rows2 = [], []
    for b in range(3):
        lo = full.cu_seqlens[b]
        rows1 += list(range(lo, lo + split[b]))
        rows2 += list(range(lo + split[b], full.cu_seqlens[b + 1]))
    n1 = np.array(split, np.int32)
    n2 = full.new_lens - n1
    cu1 = np.concatenate([[0], np.cumsum(n1)]).astype(np.int32)
    cu2 = np.concatenate([[0], np.cumsum(n2)]).astype(np.int32)
    o1, k1, v1, _ = attention.prefill_step(full.k_pool, full.v_pool, full.q[rows1], full.k[rows1],
                                           full.v[rows1], full.block_table,
                                           np.zeros(3, np.int32), cu1, 16, CFG.rope_theta)
    o2, k2, v2, _ = attention.prefill_step(k1, v1, full.q[rows2], full.k[rows2], full.v[rows2],
                                           full.block_table, n1, cu2, 16, CFG.rope_theta)
    assert np.array_equal(o1, out_full[rows1])
    assert np.array_equal(o2, out_full[rows2])
    assert np.array_equal(k2, kf) and np.array_equal(v2, vf)


def test_prefill_writes_exactly_the_new_slots():
    case = workloads.make_prefill_case(CFG, (3, 16, 40), (20, 9, 1))
    _, kn, vn, _ = _prefill(case)
    changed = np.zeros(case.k_pool.shape[:3], bool)
    for b in range(3):
        for p in range(case.context_lens[b], case.context_lens[b] + case.new_lens[b]):
            blk, off = paged.slot(case.block_table[b], p, 16)
            changed[blk, :, off] = True
    same_k = (kn == case.k_pool) | (np.isnan(bf16.decode(kn)) & np.isnan(bf16.decode(case.k_pool)))
    assert np.all(same_k[~changed])
    assert not np.any(np.isnan(bf16.decode(kn[changed])))
    assert int(changed.sum()) == int(case.new_lens.sum()) * CFG.num_kv_heads


def test_prefill_v_bits_land_at_their_positions():
    case = workloads.make_prefill_case(CFG, (3, 16, 40), (20, 9, 1))
    _, kn, vn, _ = _prefill(case)
    for b in range(3):
        for j in range(case.new_lens[b]):
            p = case.context_lens[b] + j
            blk, off = paged.slot(case.block_table[b], p, 16)
            assert np.array_equal(vn[blk, :, off], case.v[case.cu_seqlens[b] + j])


def test_prefill_block_permutation_invariance_and_no_nan():
    case = workloads.make_prefill_case(CFG, (3, 16, 40), (20, 9, 30))
    out, kn, vn, qb = _prefill(case)
    assert np.all(np.isfinite(out))
    pi = np.random.default_rng(1).permutation(case.num_blocks)
    k2, v2 = np.empty_like(kn), np.empty_like(vn)
    k2[pi], v2[pi] = kn, vn
    t2 = np.where(case.block_table >= 0, pi[np.maximum(case.block_table, 0)], -1)
    out2 = attention.paged_prefill_attention(qb, k2, v2, t2, case.context_lens, case.cu_seqlens, 16)
    assert np.array_equal(out, out2)


def test_prefill_flops_closed_form():
    # one sequence, no prefix, n tokens: sum_{p<n} (p+1) = n(n+1)/2 key visits
    assert workloads.prefill_flops([0], [4], 2, 8) == 4 * 8 * 2 * 10
    assert workloads.prefill_flops([3], [2], 1, 1) == 4 * (4 + 5)


def test_fp8_prefill_composes_the_pinned_pieces():
    """8-bit prefill: single-token chunks equal the pinned 8-bit decode step;
    the attention over codes equals the pinned bf16 prefill attention over
    their decoded values (scales as exact multipliers)."""
    from oracle import fp8
    ks = np.array([0.5, 2.0], np.float32)
    vs = np.array([4.0, 0.25], np.float32)
    one = workloads.make_prefill_case(CFG, (0, 17, 40), (1, 1, 1), kv_format="fp8")
    out, kn, vn, qb = attention.prefill_step_fp8(one.k_pool, one.v_pool, one.q, one.k, one.v,
                                                 one.block_table, one.context_lens, one.cu_seqlens,
                                                 16, CFG.rope_theta, ks, vs)
    ref, kd, vd, qd = attention.decode_step_fp8(one.k_pool, one.v_pool, one.q, one.k, one.v,
                                                one.block_table, one.context_lens, 16,
                                                CFG.rope_theta, ks, vs)
    assert np.array_equal(out, ref) and np.array_equal(kn, kd) and np.array_equal(vn, vd)
    case = workloads.make_prefill_case(CFG, (3, 16, 40), (20, 9, 30), kv_format="fp8", seed=4)
    out, kn, vn, qb = attention.prefill_step_fp8(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                                 case.block_table, case.context_lens,
                                                 case.cu_seqlens, 16, CFG.rope_theta, ks, vs)
    assert np.all(np.isfinite(out))
    kb = bf16.encode(fp8.decode(kn) * ks[None, :, None, None].astype(np.float64))
    vb = bf16.encode(fp8.decode(vn) * vs[None, :, None, None].astype(np.float64))
    ref = attention.paged_prefill_attention(qb, kb, vb, case.block_table, case.context_lens,
                                            case.cu_seqlens, 16)
    assert np.array_equal(out, ref)
