"""Seeded generators: determinism, shapes and structure of each workload (CPU)."""
import numpy as np
import pytest

import workloads
from oracle import paged


@pytest.mark.parametrize("name", ["tiny", "qwen3_1p7b", "qwen2p5_7b_b1", "qwen2p5_7b_b4",
                                  "qwen2p5_7b_b8"])
def test_generator_is_deterministic_and_well_formed(name):
    cfg = workloads.CONFIGS[name]
    a = workloads.make_decode_case(cfg, pool="poison")
    b = workloads.make_decode_case(cfg, pool="poison")
    for f in ["context_lens", "block_table", "q", "k", "v", "k_pool", "v_pool"]:
        assert np.array_equal(getattr(a, f), getattr(b, f))
    B = cfg.batch
    assert a.q.shape == (B, cfg.num_q_heads, cfg.head_dim)
    assert a.k.shape == (B, cfg.num_kv_heads, cfg.head_dim)
    assert a.k_pool.shape == (a.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim)
    used = []
    for bb in range(B):
        n = paged.blocks_needed(int(a.context_lens[bb]) + 1, cfg.block_size)
        row = a.block_table[bb]
        assert np.all(row[:n] >= 0) and np.all(row[:n] < a.num_blocks)
        assert np.all(row[n:] == -1)
        used.extend(row[:n].tolist())
    assert len(set(used)) == len(used)              # distinct physical blocks
    if cfg.table == "every_other":
        assert all(u % 2 == 0 for u in used)
    if cfg.ctx_draw == "uniform":
        assert np.all(a.context_lens >= cfg.ctx_lo) and np.all(a.context_lens <= cfg.ctx_hi)


def test_poison_layout():
    cfg = workloads.CONFIGS["tiny"]
    c = workloads.make_decode_case(cfg, pool="poison")
    nan = workloads.NAN_BF16
    for b, ctx in enumerate(c.context_lens):
        for p in range(int(ctx)):
            blk = c.block_table[b, p // 16]
            assert not np.any(c.k_pool[blk, :, p % 16] == nan)
        blk = c.block_table[b, ctx // 16]
        assert np.all(c.k_pool[blk, :, ctx % 16:] == nan)
        assert np.all(c.v_pool[blk, :, ctx % 16:] == nan)
    used = set(c.block_table[c.block_table >= 0].tolist())
    for blk in range(c.num_blocks):
        if blk not in used:
            assert np.all(c.k_pool[blk] == nan)


def test_loguniform_contexts_in_range():
    cfg = workloads.CONFIGS["qwen3_8b_long"]
    rng = np.random.default_rng(cfg.seed)
    ctx = workloads.draw_context_lens(cfg, rng)
    assert ctx.shape == (32,)
    assert np.all(ctx >= 1024) and np.all(ctx <= 16384)


def test_byte_counts_agree_with_oracle_formula():
    for name in ["tiny", "qwen3_1p7b"]:
        cfg = workloads.CONFIGS[name]
        c = workloads.make_decode_case(cfg, pool="bench")
        assert workloads.attention_bytes(c.context_lens, cfg.num_q_heads, cfg.num_kv_heads,
                                         cfg.head_dim, cfg.block_size) == \
            paged.expected_algorithmic_bytes_attention(c.context_lens, cfg.num_q_heads,
                                                       cfg.num_kv_heads, cfg.head_dim,
                                                       cfg.block_size)


def test_bf16_rounding_of_draws():
    f = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-39], dtype=np.float32)
    bits = workloads.f32_to_bf16_bits(f)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0021]
