"""Seeded synthetic workloads for the paged-KV GQA decode step.

Shared by the tests, the benchmark and the smoke check. This module only draws
random inputs of the right shapes and structure and counts bytes for the
measurement; it holds none of the method's arithmetic and imports neither the
oracle nor the GPU library.

The shapes follow the Qwen-family models the pages run (Qwen3-1.7B and
Qwen3-8B in the on-device inference course project, Qwen2.5-7B-Instruct in the
mini-infer README), with 16-token KV blocks. Values are bf16 draws of N(0, 1)
(weights N(0, 0.02)); no dataset or trained weight is involved.

bf16 values are carried as uint16 bit patterns. The float32 -> bf16 rounding
here (round to nearest, ties to even, on the integer bit pattern) only turns
random draws into bf16 inputs.
"""
import math
from dataclasses import dataclass, field

import numpy as np

NAN_BF16 = np.uint16(0x7FC0)
NAN_FP8 = np.uint8(0x7F)


def f32_to_bf16_bits(a):
    """float32 array -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rnd = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rnd) >> 16).astype(np.uint16)


def bf16_normal(rng, shape, std=1.0):
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a)


def fp8_normal_like(rng, shape):
    """Random 8-bit E4M3 bit patterns with N(0, 1)-like magnitudes: the exponent
    field is floor(log2|x|) + 7 of a normal draw x (clipped to 0..15, field 0
    being the subnormal range), the 3 significand bits are uniform and the
    sign is that of x. Plain bit construction -- no rounding of values -- and
    the NaN patterns 0x7F / 0xFF are never drawn."""
    x = rng.standard_normal(shape, dtype=np.float32)
    e = np.clip(np.floor(np.log2(np.maximum(np.abs(x), np.float32(1e-30)))).astype(np.int64) + 7, 0, 15)
    m = rng.integers(0, 8, shape)
    m = np.where((e == 15) & (m == 7), 6, m)
    s = (x < 0).astype(np.int64) << 7
    return (s | (e << 3) | m).astype(np.uint8)


@dataclass
class DecodeConfig:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int          # 0 -> derived from the draw (fragmented tables)
    rope_theta: float
    ctx_draw: str            # "fixed" | "uniform" | "loguniform"
    ctx_lo: int = 0
    ctx_hi: int = 0
    ctx_fixed: tuple = ()
    table: str = "shuffled"  # "shuffled" | "every_other"
    seed: int = 0
    # full-layer extras
    hidden: int = 0
    intermediate: int = 0
    rms_eps: float = 1e-6

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads


CONFIGS = {
    "tiny": DecodeConfig(
        "tiny", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
        num_blocks=32, rope_theta=1e4, ctx_draw="fixed", ctx_fixed=(37, 100), seed=1),
    "qwen3_1p7b": DecodeConfig(
        "qwen3_1p7b", batch=8, num_q_heads=16, num_kv_heads=8, head_dim=128,
        block_size=16, num_blocks=4096, rope_theta=1e6, ctx_draw="uniform",
        ctx_lo=128, ctx_hi=2048, seed=2),
    "qwen2p5_7b_b1": DecodeConfig(
        "qwen2p5_7b_b1", batch=1, num_q_heads=28, num_kv_heads=4, head_dim=128,
        block_size=16, num_blocks=0, rope_theta=1e6, ctx_draw="uniform",
        ctx_lo=256, ctx_hi=1024, table="every_other", seed=301),
    "qwen2p5_7b_b4": DecodeConfig(
        "qwen2p5_7b_b4", batch=4, num_q_heads=28, num_kv_heads=4, head_dim=128,
        block_size=16, num_blocks=0, rope_theta=1e6, ctx_draw="uniform",
        ctx_lo=256, ctx_hi=1024, table="every_other", seed=304),
    "qwen2p5_7b_b8": DecodeConfig(
        "qwen2p5_7b_b8", batch=8, num_q_heads=28, num_kv_heads=4, head_dim=128,
        block_size=16, num_blocks=0, rope_theta=1e6, ctx_draw="uniform",
        ctx_lo=256, ctx_hi=1024, table="every_other", seed=308),
    "qwen3_8b_long": DecodeConfig(
        "qwen3_8b_long", batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, num_blocks=40000, rope_theta=1e6, ctx_draw="loguniform",
        ctx_lo=1024, ctx_hi=16384, seed=4),
    "qwen3_8b_layer": DecodeConfig(
        "qwen3_8b_layer", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, num_blocks=4096, rope_theta=1e6, ctx_draw="uniform",
        ctx_lo=512, ctx_hi=4096, seed=5, hidden=4096, intermediate=12288,
        rms_eps=1e-6),
}


def draw_context_lens(cfg, rng):
    if cfg.ctx_draw == "fixed":
        return np.asarray(cfg.ctx_fixed, dtype=np.int32)
    if cfg.ctx_draw == "uniform":
        return rng.integers(cfg.ctx_lo, cfg.ctx_hi + 1, cfg.batch).astype(np.int32)
    if cfg.ctx_draw == "loguniform":
        u = rng.uniform(math.log(cfg.ctx_lo), math.log(cfg.ctx_hi), cfg.batch)
        return np.floor(np.exp(u)).astype(np.int32)
    raise ValueError(cfg.ctx_draw)


def nblocks(n_tokens, bs):
    return -(-int(n_tokens) // bs)


@dataclass
class DecodeCase:
    """One decode step's inputs. bf16 tensors are uint16 bit patterns."""
    cfg: DecodeConfig
    context_lens: np.ndarray      # int32 [B], tokens cached before the step
    block_table: np.ndarray       # int32 [B, MB], -1 padded
    num_blocks: int
    q: np.ndarray                 # [B, Hq, D]
    k: np.ndarray                 # [B, Hkv, D]
    v: np.ndarray                 # [B, Hkv, D]
    k_pool: np.ndarray            # [N, Hkv, bs, D]
    v_pool: np.ndarray
    extras: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self):
        return self.block_table.shape[1]


def make_block_table(rng, ctx, bs, num_blocks, mode):
    need = [nblocks(c + 1, bs) for c in ctx]
    mb = max(need) if need else 1
    table = np.full((len(ctx), max(mb, 1)), -1, dtype=np.int32)
    if mode == "shuffled":
        perm = rng.permutation(num_blocks).astype(np.int32)
        pos = 0
        for b, n in enumerate(need):
            table[b, :n] = perm[pos:pos + n]
            pos += n
        if pos > num_blocks:
            raise ValueError("pool too small for the drawn contexts")
    elif mode == "every_other":
        nxt = 0
        for b, n in enumerate(need):
            table[b, :n] = np.arange(nxt, nxt + 2 * n, 2, dtype=np.int32)
            nxt += 2 * n
    else:
        raise ValueError(mode)
    return table, need


def make_decode_case(cfg, pool="poison", seed=None, context_lens=None, num_blocks=None,
                     table_mode=None, kv_format="bf16"):
    """Draw one decode step.

    pool = "poison": cached slots [0, ctx) hold N(0,1); the write slot, the tail
           slots of the last block and every unallocated block hold NaN.
    pool = "bench":  every slot of every allocated block holds N(0,1);
           unallocated blocks are zero (never read).
    pool = "full":   every element of the pool holds N(0,1).
    kv_format = "bf16": pools of bf16 bits; "fp8": pools of E4M3 codes drawn by
           fp8_normal_like (q, k, v stay bf16).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    ctx = (np.asarray(context_lens, dtype=np.int32) if context_lens is not None
           else draw_context_lens(cfg, rng))
    B, Hq, Hkv, D, bs = len(ctx), cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    mode = table_mode or cfg.table
    need = [nblocks(c + 1, bs) for c in ctx]
    N = num_blocks or cfg.num_blocks
    if not N:
        N = 64 * -(-(2 * sum(need)) // 64)
    table, need = make_block_table(rng, ctx, bs, N, mode)
    q = bf16_normal(rng, (B, Hq, D))
    k = bf16_normal(rng, (B, Hkv, D))
    v = bf16_normal(rng, (B, Hkv, D))

    shape = (N, Hkv, bs, D)
    if kv_format == "bf16":
        draw, nan, dt = bf16_normal, NAN_BF16, np.uint16
    elif kv_format == "fp8":
        draw, nan, dt = fp8_normal_like, NAN_FP8, np.uint8
    else:
        raise ValueError(kv_format)
    if pool == "full":
        k_pool = draw(rng, shape)
        v_pool = draw(rng, shape)
    else:
        ids = np.concatenate([table[b, :need[b]] for b in range(B)]) if B else np.zeros(0, np.int32)
        fill = nan if pool == "poison" else dt(0)
        k_pool = np.full(shape, fill, dtype=dt)
        v_pool = np.full(shape, fill, dtype=dt)
        k_pool[ids] = draw(rng, (len(ids), Hkv, bs, D))
        v_pool[ids] = draw(rng, (len(ids), Hkv, bs, D))
    if pool == "poison":
        for b in range(B):
            last = table[b, need[b] - 1]
            first_bad = int(ctx[b]) % bs       # write slot, then the tail
            k_pool[last, :, first_bad:, :] = nan
            v_pool[last, :, first_bad:, :] = nan
    return DecodeCase(cfg, ctx, table, N, q, k, v, k_pool, v_pool)


def make_layer_weights(cfg, seed=None, std=0.02):
    """bf16 weights of one decoder layer (nn.Linear layout), N(0, std), unit gains."""
    rng = np.random.default_rng((cfg.seed if seed is None else seed) + 1000)
    H, I, D = cfg.hidden, cfg.intermediate, cfg.head_dim
    Hq, Hkv = cfg.num_q_heads, cfg.num_kv_heads
    one = np.uint16(0x3F80)
    return {
        "ln1_w": np.full(H, one, dtype=np.uint16),
        "w_qkv": bf16_normal(rng, ((Hq + 2 * Hkv) * D, H), std),
        "w_o": bf16_normal(rng, (H, Hq * D), std),
        "ln2_w": np.full(H, one, dtype=np.uint16),
        "w_gate": bf16_normal(rng, (I, H), std),
        "w_up": bf16_normal(rng, (I, H), std),
        "w_down": bf16_normal(rng, (H, I), std),
    }


def make_layer_input(cfg, seed=None):
    rng = np.random.default_rng((cfg.seed if seed is None else seed) + 2000)
    return bf16_normal(rng, (cfg.batch, cfg.hidden))


# ---------------------------------------------------------------- byte counts
def attention_bytes(context_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                    kv_elem_bytes=2):
    """Algorithmic HBM bytes of one paged decode attention call: K and V of the
    L = ctx + 1 attended tokens once per (sequence, kv head) at kv_elem_bytes
    per element (2 for bf16, 1 for an 8-bit cache, which adds its two fp32
    scales per kv head), bf16 q in and out once, the used block-table entries
    and the lengths."""
    L = np.asarray(context_lens, dtype=np.int64) + 1
    kv = 2 * kv_elem_bytes * num_kv_heads * head_dim * int(L.sum())
    qo = 2 * 2 * len(L) * num_q_heads * head_dim
    table = 4 * int(sum(nblocks(x, block_size) for x in L))
    scales = 8 * num_kv_heads if kv_elem_bytes == 1 else 0
    return kv + qo + table + 4 * len(L) + scales


def write_bytes(batch, num_q_heads, num_kv_heads, head_dim, kv_elem_bytes=2):
    """Algorithmic bytes of write_decode_kv: bf16 q in and q_rot out, bf16 k
    and v in, the new K and V rows out at kv_elem_bytes per element, one
    table entry and one length per sequence."""
    return (2 * 2 * batch * head_dim * (num_q_heads + num_kv_heads)
            + 2 * kv_elem_bytes * batch * head_dim * num_kv_heads + 8 * batch)


def layer_weight_bytes(cfg):
    H, I, D = cfg.hidden, cfg.intermediate, cfg.head_dim
    Hq, Hkv = cfg.num_q_heads, cfg.num_kv_heads
    n = H * (Hq + 2 * Hkv) * D + Hq * D * H + 3 * H * I
    return 2 * n + 2 * 2 * H


def layer_bytes(cfg, context_lens):
    """Algorithmic bytes of one full-layer decode step: weights once, the
    activations in and out, plus the write and the attention."""
    B = len(context_lens)
    return (layer_weight_bytes(cfg) + 2 * 2 * B * cfg.hidden
            + write_bytes(B, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim)
            + attention_bytes(context_lens, cfg.num_q_heads, cfg.num_kv_heads,
                              cfg.head_dim, cfg.block_size))


def layer_flops(cfg, context_lens):
    H, I, D = cfg.hidden, cfg.intermediate, cfg.head_dim
    Hq, Hkv = cfg.num_q_heads, cfg.num_kv_heads
    B = len(context_lens)
    gemm = 2 * B * (H * (Hq + 2 * Hkv) * D + Hq * D * H + 3 * H * I)
    L = np.asarray(context_lens, dtype=np.int64) + 1
    return gemm + 4 * Hq * D * int(L.sum())


# -------------------------------------------------------------------- prefill
@dataclass
class PrefillCase:
    """One prefill chunk per sequence: n_b new tokens after ctx_b cached ones.
    q, k, v are packed over the batch ([T, H, D], rows cu[b] .. cu[b+1])."""
    cfg: DecodeConfig
    context_lens: np.ndarray      # int32 [B], tokens cached before the chunk
    new_lens: np.ndarray          # int32 [B]
    cu_seqlens: np.ndarray        # int32 [B + 1]
    block_table: np.ndarray       # int32 [B, MB], -1 padded
    num_blocks: int
    q: np.ndarray                 # [T, Hq, D]
    k: np.ndarray                 # [T, Hkv, D]
    v: np.ndarray
    k_pool: np.ndarray            # [N, Hkv, bs, D]
    v_pool: np.ndarray


PREFILL_CONFIGS = {
    "prefill_small": (DecodeConfig("prefill_small", batch=4, num_q_heads=8, num_kv_heads=2,
                                   head_dim=64, block_size=16, num_blocks=64, rope_theta=1e4,
                                   ctx_draw="fixed", seed=61),
                      (0, 5, 40, 16), (37, 1, 16, 50)),
    "qwen3_8b_prefill": (DecodeConfig("qwen3_8b_prefill", batch=4, num_q_heads=32,
                                      num_kv_heads=8, head_dim=128, block_size=16,
                                      num_blocks=4096, rope_theta=1e6, ctx_draw="fixed",
                                      seed=62),
                         None, None),
}


def make_prefill_case(cfg, context_lens, new_lens, pool="poison", seed=None, reserve=0,
                      kv_format="bf16"):
    """Draw a prefill chunk. pool = "poison": cached slots [0, ctx) hold N(0,1);
    the slots the chunk will write, the tail and unallocated blocks hold NaN.
    pool = "bench": every slot of the allocated blocks holds N(0,1). The block
    tables cover ctx + n + reserve tokens (reserve: room for decode steps).
    kv_format "fp8": pools of E4M3 codes (fp8_normal_like), poison 0x7F."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    ctx = np.asarray(context_lens, dtype=np.int32)
    n = np.asarray(new_lens, dtype=np.int32)
    B, Hq, Hkv, D, bs = len(ctx), cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(n)
    T = int(cu[-1])
    total = ctx + n + int(reserve)
    need = [nblocks(t, bs) for t in total]
    N = cfg.num_blocks
    table = np.full((B, max(max(need), 1)), -1, dtype=np.int32)
    perm = rng.permutation(N).astype(np.int32)
    pos = 0
    for b, m in enumerate(need):
        table[b, :m] = perm[pos:pos + m]
        pos += m
    if pos > N:
        raise ValueError("pool too small for the drawn contexts")
    q = bf16_normal(rng, (T, Hq, D))
    k = bf16_normal(rng, (T, Hkv, D))
    v = bf16_normal(rng, (T, Hkv, D))
    shape = (N, Hkv, bs, D)
    if kv_format == "bf16":
        draw, nan, dt = bf16_normal, NAN_BF16, np.uint16
    elif kv_format == "fp8":
        draw, nan, dt = fp8_normal_like, NAN_FP8, np.uint8
    else:
        raise ValueError(kv_format)
    fill = nan if pool == "poison" else dt(0)
    k_pool = np.full(shape, fill, dtype=dt)
    v_pool = np.full(shape, fill, dtype=dt)
    ids = np.concatenate([table[b, :need[b]] for b in range(B)])
    k_pool[ids] = draw(rng, (len(ids), Hkv, bs, D))
    v_pool[ids] = draw(rng, (len(ids), Hkv, bs, D))
    if pool == "poison":
        for b in range(B):
            for p in range(int(ctx[b]), need[b] * bs):
                blk = table[b, p // bs]
                k_pool[blk, :, p % bs, :] = nan
                v_pool[blk, :, p % bs, :] = nan
    return PrefillCase(cfg, ctx, n, cu, table, N, q, k, v, k_pool, v_pool)


def prefill_flops(context_lens, new_lens, num_q_heads, head_dim):
    """Multiply-add flops of the causal attention of a prefill chunk: each new
    token at position p scores and weights p + 1 keys (2 * 2 * D per key and
    query head)."""
    tot = 0
    for c, n in zip(context_lens, new_lens):
        c, n = int(c), int(n)
        tot += n * c + n * (n + 1) // 2          # sum over new tokens of (p + 1)
    return 4 * head_dim * num_q_heads * tot


def prefill_attention_bytes(context_lens, new_lens, num_q_heads, num_kv_heads, head_dim,
                            block_size):
    """Minimum HBM bytes of the prefill attention: each sequence's K and V of
    its ctx + n tokens once per kv head, q in and out once, table entries."""
    tot = 0
    for c, n in zip(context_lens, new_lens):
        L = int(c) + int(n)
        tot += 4 * num_kv_heads * head_dim * L + 4 * int(n) * num_q_heads * head_dim
        tot += 4 * nblocks(L, block_size)
    return tot + 8 * len(context_lens)
