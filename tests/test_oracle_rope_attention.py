"""Pins for the oracle's RoPE, write_decode_kv and paged GQA attention (CPU only).

None of these re-types the oracle's formula: each checks a closed form, an
invariant, brute force with math.fsum, or an independent library routine
(torch's scaled_dot_product_attention with enable_gqa, the routine the course
project names for grouped-query attention).
"""
import cmath
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from oracle import attention, bf16, paged, rope


# ----------------------------------------------------------------------- RoPE
def test_rope_identity_at_position_zero_bit_exact():
    x = np.random.default_rng(0).standard_normal((5, 128))
    assert np.array_equal(rope.apply(x, 0, 1e6), x)


@pytest.mark.parametrize("D,theta", [(64, 1e4), (128, 1e6)])
def test_rope_preserves_norm(D, theta):
    rng = np.random.default_rng(D)
    x = rng.standard_normal((50, D))
    for pos in [1, 17, 1000, 16384]:
        y = rope.apply(x, pos, theta)
        assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13, atol=0)


def test_rope_pair_zero_rotates_by_position():
    # inv_freq_0 = theta^0 = 1, so pair (0, D/2) turns by exactly `pos` radians
    x = np.zeros(128)
    x[0] = 1.0
    for pos in [1, 3, 100, 16384]:
        y = rope.apply(x, pos, 1e6)
        assert y[0] == math.cos(pos) and y[64] == math.sin(pos)


def test_rope_inverse_frequencies_closed_form():
    f = rope.inv_freq(128, 1e6)
    assert f[0] == 1.0
    assert abs(f[1] - 1e6 ** (-2 / 128)) < 1e-16
    assert abs(f[-1] - 1e6 ** (-126 / 128)) <= 1e-16 * 1e6 ** (-126 / 128) * 4


def test_rope_equals_complex_rotation():
    """Independent formulation: z_i = x_i + 1j*x_{i+D/2} times e^{1j*pos*theta^(-2i/D)}."""
    rng = np.random.default_rng(2)
    D, theta = 64, 1e4
    x = rng.standard_normal(D)
    for pos in [0, 5, 37, 100, 4097]:
        y = rope.apply(x, pos, theta)
        for i in range(D // 2):
            z = complex(x[i], x[i + D // 2]) * cmath.exp(1j * pos * theta ** (-2.0 * i / D))
            assert abs(y[i] - z.real) < 1e-12 and abs(y[i + D // 2] - z.imag) < 1e-12


def test_rope_relative_position_property():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n in [(10, 3), (1000, 999), (16384, 5)]:
        lhs = rope.apply(q, m, 1e6) @ rope.apply(k, n, 1e6)
        rhs = rope.apply(q, m - n, 1e6) @ k
        assert abs(lhs - rhs) < 1e-10 * (1 + abs(rhs))


def test_rope_matches_rotate_half_form_in_torch():
    """The rotate_half formulation (cat(-x2, x1)) evaluated by torch in fp64."""
    rng = np.random.default_rng(4)
    D, theta, pos = 128, 1e6, 1234
    x = torch.from_numpy(rng.standard_normal((3, D)))
    inv = 1.0 / (theta ** (torch.arange(0, D, 2, dtype=torch.float64) / D))
    emb = torch.cat([pos * inv, pos * inv])
    rot = torch.cat([-x[:, D // 2:], x[:, : D // 2]], dim=-1)
    ref = x * emb.cos() + rot * emb.sin()
    assert np.allclose(rope.apply(x.numpy(), pos, theta), ref.numpy(), rtol=0, atol=1e-12)


# -------------------------------------------------------------- write_decode_kv
def test_write_decode_kv_touches_exactly_the_new_slots():
    case = workloads.make_decode_case(workloads.CONFIGS["tiny"], pool="poison")
    cfg = case.cfg
    kn, vn, qrot_bits, qrot = attention.write_decode_kv(
        case.k_pool, case.v_pool, case.q, case.k, case.v, case.block_table,
        case.context_lens, cfg.block_size, cfg.rope_theta)
    changed = np.zeros(case.k_pool.shape[:3], dtype=bool)
    flat = kn.reshape(-1, cfg.head_dim) != case.k_pool.reshape(-1, cfg.head_dim)
    changed_k = flat.any(-1).reshape(changed.shape)
    expect = np.zeros_like(changed)
    for b, ctx in enumerate(case.context_lens):
        # closed form: logical block ctx // bs, offset ctx % bs
        blk = case.block_table[b, ctx // cfg.block_size]
        expect[blk, :, ctx % cfg.block_size] = True
    assert np.array_equal(changed_k, expect)       # every poisoned write slot is overwritten
    # V is a bit copy, every other byte untouched
    for b, ctx in enumerate(case.context_lens):
        blk = case.block_table[b, ctx // cfg.block_size]
        assert np.array_equal(vn[blk, :, ctx % cfg.block_size], case.v[b])
        assert np.array_equal(kn[blk, :, ctx % cfg.block_size],
                              bf16.encode(np.stack([rope.apply(bf16.decode(case.k[b, g]), int(ctx), cfg.rope_theta)
                                                    for g in range(cfg.num_kv_heads)])))
    mask = ~expect[..., None].repeat(cfg.head_dim, -1)
    assert np.array_equal(kn[mask], case.k_pool[mask])
    assert np.array_equal(vn[mask], case.v_pool[mask])
    assert qrot_bits.shape == case.q.shape


def test_write_decode_kv_at_position_zero_stores_k_unchanged():
    cfg = workloads.CONFIGS["tiny"]
    case = workloads.make_decode_case(cfg, pool="poison", context_lens=[0, 16])
    kn, vn, qrot_bits, _ = attention.write_decode_kv(
        case.k_pool, case.v_pool, case.q, case.k, case.v, case.block_table,
        case.context_lens, cfg.block_size, cfg.rope_theta)
    blk = case.block_table[0, 0]
    assert np.array_equal(kn[blk, :, 0], case.k[0])      # RoPE(pos 0) = identity, bf16 exact
    assert np.array_equal(qrot_bits[0], case.q[0])


# ------------------------------------------------------------------- attention
def _scatter_contiguous(K, V, table, bs, Hkv, D, N):
    """Place contiguous per-sequence K/V [B][Hkv, L, D] into pools by flat index arithmetic."""
    kp = np.full((N, Hkv, bs, D), workloads.NAN_BF16, dtype=np.uint16)
    vp = kp.copy()
    kf, vf = kp.reshape(-1), vp.reshape(-1)
    for b in range(len(K)):
        L = K[b].shape[1]
        for p in range(L):
            blk = table[b][p // bs]
            for g in range(Hkv):
                base = ((blk * Hkv + g) * bs + p % bs) * D
                kf[base: base + D] = K[b][g, p]
                vf[base: base + D] = V[b][g, p]
    return kp, vp


def _contig_case(seed=0, B=3, Hq=8, Hkv=2, D=32, bs=16, lens=(1, 16, 45), N=64):
    rng = np.random.default_rng(seed)
    K = [workloads.bf16_normal(rng, (Hkv, L, D)) for L in lens]
    V = [workloads.bf16_normal(rng, (Hkv, L, D)) for L in lens]
    table, _ = workloads.make_block_table(rng, [L - 1 for L in lens], bs, N, "shuffled")
    kp, vp = _scatter_contiguous(K, V, table, bs, Hkv, D, N)
    q = workloads.bf16_normal(rng, (B, Hq, D))
    ctx = np.array([L - 1 for L in lens], dtype=np.int32)
    return q, K, V, kp, vp, table, ctx


def test_paged_equals_contiguous_sdpa_fp64():
    """Paged attention == dense attention on the contiguous copy, via torch's
    scaled_dot_product_attention(enable_gqa=True) in float64."""
    q, K, V, kp, vp, table, ctx = _contig_case()
    B, Hq, D = q.shape
    out = attention.paged_gqa_decode(q, kp, vp, table, ctx, 16)
    for b in range(B):
        qt = torch.from_numpy(bf16.decode(q[b]))[None, :, None, :]          # [1,Hq,1,D]
        kt = torch.from_numpy(bf16.decode(K[b]))[None]                       # [1,Hkv,L,D]
        vt = torch.from_numpy(bf16.decode(V[b]))[None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, enable_gqa=True)[0, :, 0, :]
        assert np.allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)


def test_gqa_equals_repeat_interleave_mha_bit_exact():
    q, K, V, kp, vp, table, ctx = _contig_case(seed=1)
    G = q.shape[1] // kp.shape[1]
    out = attention.paged_gqa_decode(q, kp, vp, table, ctx, 16)
    out_mha = attention.paged_gqa_decode(q, np.repeat(kp, G, axis=1), np.repeat(vp, G, axis=1),
                                         table, ctx, 16)
    assert np.array_equal(out, out_mha)


def test_block_table_permutation_invariance_bit_exact():
    case = workloads.make_decode_case(workloads.CONFIGS["tiny"], pool="poison")
    cfg = case.cfg
    kn, vn, qb, _ = attention.write_decode_kv(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                              case.block_table, case.context_lens,
                                              cfg.block_size, cfg.rope_theta)
    out = attention.paged_gqa_decode(qb, kn, vn, case.block_table, case.context_lens, 16)
    pi = np.random.default_rng(9).permutation(case.num_blocks)
    kp2, vp2 = np.empty_like(kn), np.empty_like(vn)
    kp2[pi] = kn
    vp2[pi] = vn
    t2 = np.where(case.block_table >= 0, pi[np.maximum(case.block_table, 0)], -1)
    out2 = attention.paged_gqa_decode(qb, kp2, vp2, t2, case.context_lens, 16)
    assert np.array_equal(out, out2)


def test_softmax_weights_sum_to_one():
    """With V = one-hot rows the output IS the probability vector."""
    rng = np.random.default_rng(5)
    for L in [1, 2, 17, 64]:
        K = rng.standard_normal((L, 64)) * 3
        V = np.eye(64)[:L]
        p = attention.attend(rng.standard_normal(64), K, V, 1 / 8)
        assert np.all(p[:L] >= 0) and np.all(p[L:] == 0)
        assert abs(p.sum() - 1.0) <= 1e-15 * L


def test_attention_closed_forms():
    rng = np.random.default_rng(6)
    K = rng.standard_normal((40, 64))
    V = rng.standard_normal((40, 64))
    # L = 1: the single value vector, exactly
    assert np.array_equal(attention.attend(rng.standard_normal(64), K[:1], V[:1], 0.125), V[0])
    # q = 0: uniform weights, the mean of V
    assert np.allclose(attention.attend(np.zeros(64), K, V, 0.125), V.mean(0), rtol=0, atol=1e-15)
    # constant V rows: output is that constant
    c = rng.standard_normal(64)
    assert np.allclose(attention.attend(rng.standard_normal(64), K, np.tile(c, (40, 1)), 0.125),
                       c, rtol=0, atol=1e-14)
    # q = lambda * k_t* with large lambda: attention collapses onto V_t*
    t = 17
    Kn = K / np.linalg.norm(K, axis=1, keepdims=True)
    out = attention.attend(1e4 * Kn[t], Kn, V, 1.0)
    assert np.allclose(out, V[t], rtol=0, atol=1e-12)
    # huge scores do not overflow (stable form)
    out = attention.attend(np.full(64, 1e3), K, V, 1.0)
    assert np.all(np.isfinite(out))


def test_attention_brute_force_tiny_config():
    """Pure-Python loops with math.fsum over the tiny workload, <= 1e-13."""
    cfg = workloads.CONFIGS["tiny"]
    case = workloads.make_decode_case(cfg, pool="poison")
    out, kn, vn, qb = attention.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                            case.block_table, case.context_lens,
                                            cfg.block_size, cfg.rope_theta)
    D, bs, G = cfg.head_dim, cfg.block_size, cfg.group
    qf = bf16.decode(qb)
    for b in range(cfg.batch):
        L = int(case.context_lens[b]) + 1
        for h in range(cfg.num_q_heads):
            g = h // G
            keys, vals = [], []
            for p in range(L):
                blk = int(case.block_table[b, p // bs])
                keys.append([float(x) for x in bf16.decode(kn[blk, g, p % bs])])
                vals.append([float(x) for x in bf16.decode(vn[blk, g, p % bs])])
            s = [math.fsum(qf[b, h, d] * keys[t][d] for d in range(D)) / math.sqrt(D) for t in range(L)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            for d in range(D):
                ref = math.fsum(w[t] * vals[t][d] for t in range(L)) / z
                assert abs(out[b, h, d] - ref) <= 1e-13


def test_tail_and_unallocated_nan_never_reach_the_output():
    cfg = workloads.CONFIGS["tiny"]
    case = workloads.make_decode_case(cfg, pool="poison")
    out, *_ = attention.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                    case.block_table, case.context_lens, cfg.block_size,
                                    cfg.rope_theta)
    assert np.all(np.isfinite(out))


def test_torch_sdpa_gqa_on_the_tiny_workload():
    """Whole decode step vs torch sdpa(enable_gqa=True) on the gathered, written cache."""
    cfg = workloads.CONFIGS["tiny"]
    case = workloads.make_decode_case(cfg, pool="poison")
    out, kn, vn, qb = attention.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                            case.block_table, case.context_lens,
                                            cfg.block_size, cfg.rope_theta)
    for b in range(cfg.batch):
        L = int(case.context_lens[b]) + 1
        idx = [(int(case.block_table[b, p // 16]), p % 16) for p in range(L)]
        K = np.stack([kn[blk, :, off] for blk, off in idx], axis=1)     # [Hkv, L, D]
        V = np.stack([vn[blk, :, off] for blk, off in idx], axis=1)
        qt = torch.from_numpy(bf16.decode(qb[b]))[None, :, None, :]
        ref = F.scaled_dot_product_attention(qt, torch.from_numpy(bf16.decode(K))[None],
                                             torch.from_numpy(bf16.decode(V))[None],
                                             enable_gqa=True)[0, :, 0, :].numpy()
        assert np.allclose(out[b], ref, rtol=0, atol=1e-12)


def test_planted_mistakes_are_caught():
    """A wrong KV-head mapping (h mod Hkv) or a dropped scale fails the sdpa pin."""
    q, K, V, kp, vp, table, ctx = _contig_case(seed=7)
    b = 2
    qt = torch.from_numpy(bf16.decode(q[b]))[None, :, None, :]
    ref = F.scaled_dot_product_attention(qt, torch.from_numpy(bf16.decode(K[b]))[None],
                                         torch.from_numpy(bf16.decode(V[b]))[None],
                                         enable_gqa=True)[0, :, 0, :].numpy()
    good = attention.paged_gqa_decode(q, kp, vp, table, ctx, 16)[b]
    assert np.allclose(good, ref, atol=1e-12)
    noscale = attention.paged_gqa_decode(q, kp, vp, table, ctx, 16, scale=1.0)[b]
    assert not np.allclose(noscale, ref, atol=1e-3)
    Hkv = kp.shape[1]
    wrong = np.stack([attention.attend(bf16.decode(q[b, h]), bf16.decode(K[b][h % Hkv]),
                                       bf16.decode(V[b][h % Hkv]), 1 / np.sqrt(32))
                      for h in range(q.shape[1])])
    assert not np.allclose(wrong, ref, atol=1e-3)
