"""GPU parity of the prefill chunk (prompt KV write + causal paged attention)
against the fp64 oracle, through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_246_amd as mk
import workloads
from oracle import attention as oatt
from oracle import bf16 as obf16
from tests.gpu_harness import (DEV, bits_to_dev, check_tolerance, codes_to_dev, dev_to_bits,
                               ulp_diff_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mk.lib()


def _say(*a):
    print(*a, flush=True)


class PrefillOnDevice:
    def __init__(self, case, k_scales=None, v_scales=None):
        cfg = case.cfg
        self.case = case
        self.fp8 = case.k_pool.dtype == np.uint8
        self.B = len(case.context_lens)
        self.T = int(case.cu_seqlens[-1])
        self.Hq, self.Hkv, self.D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
        to_dev = codes_to_dev if self.fp8 else bits_to_dev
        self.k_pool, self.v_pool = to_dev(case.k_pool), to_dev(case.v_pool)
        self.q, self.k, self.v = bits_to_dev(case.q), bits_to_dev(case.k), bits_to_dev(case.v)
        self.q_rot = torch.empty_like(self.q)
        self.out = torch.empty_like(self.q)
        self.table = torch.from_numpy(case.block_table).to(DEV)
        self.ctx = torch.from_numpy(case.context_lens).to(DEV)
        self.cu = torch.from_numpy(case.cu_seqlens).to(DEV)
        self.mbps = case.block_table.shape[1]
        self.max_new = int(case.new_lens.max())
        self.pool = mk.mi_kv_pool_init(case.num_blocks, 16, self.Hkv, self.D, self.k_pool,
                                       self.v_pool, flags=mk.MI_POOL_KV_FP8 if self.fp8 else 0)
        if self.fp8:
            mk.mi_kv_pool_set_scales(self.pool, k_scales, v_scales)

    def run(self):
        mk.mi_write_prefill_kv(self.pool, self.q, self.k, self.v, self.q_rot, self.table, self.mbps,
                               self.ctx, self.cu, self.B, self.T, self.Hq, self.case.cfg.rope_theta)
        mk.mi_paged_prefill_attention(self.pool, self.q_rot, self.out, self.table, self.mbps,
                                      self.ctx, self.cu, self.B, self.T, self.max_new, self.Hq)
        torch.cuda.synchronize()

    def close(self):
        if self.pool:
            mk.mi_kv_pool_destroy(self.pool)
            self.pool = None


def _check_write(case, dev, kn, vn, qb):
    gk, gv = dev_to_bits(dev.k_pool), dev_to_bits(dev.v_pool)
    assert np.array_equal(gv, vn)
    changed = np.zeros(case.k_pool.shape[:3], bool)
    for b in range(len(case.context_lens)):
        for p in range(case.context_lens[b], case.context_lens[b] + case.new_lens[b]):
            changed[case.block_table[b, p // 16], :, p % 16] = True
    assert np.array_equal(gk[~changed], kn[~changed])
    assert ulp_diff_bf16(gk[changed], kn[changed]).max() <= 1
    assert ulp_diff_bf16(dev_to_bits(dev.q_rot), qb).max() <= 1


def _full_check(case, label):
    ref, kn, vn, qb = oatt.prefill_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                        case.block_table, case.context_lens, case.cu_seqlens, 16,
                                        case.cfg.rope_theta)
    dev = PrefillOnDevice(case)
    try:
        dev.run()
        _check_write(case, dev, kn, vn, qb)
        mx, rel = check_tolerance(dev_to_bits(dev.out), ref, label)
        _say("  %s max|d| %.3g relL2 %.3g" % (label, mx, rel))
        assert mk.mi_kv_pool_check_errors(dev.pool) == 0
    finally:
        dev.close()


def test_prefill_small_mixed_chunks():
    cfg, ctx, n = workloads.PREFILL_CONFIGS["prefill_small"]
    _full_check(workloads.make_prefill_case(cfg, ctx, n), "prefill_small")


GROUPS = [(1, 1), (3, 1), (4, 2), (7, 1), (8, 1)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", GROUPS)
def test_prefill_groups_head_dims_and_diagonals(D, Hq, Hkv):
    """Chunks starting on and off block boundaries (the causal diagonal spans
    one or two key tiles), single-token chunks and a partial last query block."""
    cfg = workloads.DecodeConfig("pfg", batch=5, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                 block_size=16, num_blocks=96, rope_theta=1e4, ctx_draw="fixed",
                                 seed=D * 3 + Hq)
    case = workloads.make_prefill_case(cfg, (0, 7, 16, 33, 100), (33, 17, 1, 48, 5))
    _full_check(case, "G=%d D=%d" % (Hq // Hkv, D))


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_score_far_above_the_first_tile_takes_the_rescaling_pass(D):
    """The prefill kernel's first pass fixes each query's softmax reference at
    the largest score of the first key tile; every query here is the same
    vector u and token 40's key is 30 u, so for the queries at and after
    position 40 one score lies hundreds of log2 units above that reference
    (its weight would overflow float32). Those waves must repeat the chunk
    with the online rescaling form and still match the oracle; the other
    waves keep their first-pass results."""
    cfg = workloads.DecodeConfig("pf_far", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=D,
                                 block_size=16, num_blocks=32, rope_theta=1e4, ctx_draw="fixed",
                                 seed=40 + D)
    case = workloads.make_prefill_case(cfg, (0, 20), (100, 60))
    u = case.q[0, 0].copy()
    case.q[:] = u
    big = obf16.encode(30.0 * obf16.decode(u))
    case.k[40] = big                       # sequence 0, position 40
    case.k[case.cu_seqlens[1] + 30] = big  # sequence 1, position 50 (after 20 cached)
    ref, kn, vn, qb = oatt.prefill_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                        case.block_table, case.context_lens, case.cu_seqlens, 16,
                                        case.cfg.rope_theta)
    dev = PrefillOnDevice(case)
    try:
        # three calls on one pool: each call has its own generation number in
        # the pool's redo word, so every call repeats and none reads a stale one
        for call in range(3):
            dev.out.fill_(0)
            dev.run()
            _check_write(case, dev, kn, vn, qb)
            check_tolerance(dev_to_bits(dev.out), ref, "far scores D=%d call %d" % (D, call))
        assert mk.mi_kv_pool_check_errors(dev.pool) == 0
    finally:
        dev.close()


def test_prefill_rescaling_pass_at_qwen3_8b_heads():
    """The rescaling launch at Qwen3-8B-shaped heads (32/8, D 128) with
    chunks of 700, 300 and 50 tokens after 0, 100 and 16 cached: 15 query
    blocks x 32 heads x 3 sequences = 1,440 waves. A key of 30 u in every
    sequence (all queries u) sends the call through that launch, and the whole
    output must match the oracle on two calls in a row."""
    cfg = workloads.PREFILL_CONFIGS["qwen3_8b_prefill"][0]
    case = workloads.make_prefill_case(cfg, (0, 100, 16), (700, 300, 50))
    u = case.q[0, 0].copy()
    case.q[:] = u
    big = obf16.encode(30.0 * obf16.decode(u))
    for b, pos in enumerate((5, 60, 10)):   # new-token index of the large key
        case.k[case.cu_seqlens[b] + pos] = big
    ref, kn, vn, qb = oatt.prefill_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                        case.block_table, case.context_lens, case.cu_seqlens, 16,
                                        case.cfg.rope_theta)
    dev = PrefillOnDevice(case)
    try:
        for call in range(2):
            dev.out.fill_(0)
            dev.run()
            _check_write(case, dev, kn, vn, qb)
            check_tolerance(dev_to_bits(dev.out), ref, "qwen3_8b rescaling call %d" % call)
        assert mk.mi_kv_pool_check_errors(dev.pool) == 0
    finally:
        dev.close()


def test_prefill_qwen3_8b_shape_full():
    """Qwen3-8B-shaped chunk (32/8 heads, D 128): a 1000-token prompt, a 700-token
    chunk after 600 cached tokens and a 64-token chunk after 3000; the whole
    written cache and q_rot, then every (token, head) output against the
    oracle."""
    cfg = workloads.PREFILL_CONFIGS["qwen3_8b_prefill"][0]
    case = workloads.make_prefill_case(cfg, (0, 600, 3000), (1000, 700, 64))
    _full_check(case, "qwen3_8b mixed chunk")


def test_prefill_benchmark_chunk_one_head_per_kv_head():
    """The benchmark's chunk (4 fresh prompts of 2048 tokens, 32/8 heads) in
    its launch configuration: the whole written cache and q_rot against the
    oracle, then every query row of the first query head of each KV head
    (8 of 32 heads, 65,536 rows) against the oracle row by row."""
    cfg = workloads.PREFILL_CONFIGS["qwen3_8b_prefill"][0]
    case = workloads.make_prefill_case(cfg, (0, 0, 0, 0), (2048, 2048, 2048, 2048))
    kn, vn, qb = oatt.write_prefill_kv(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                       case.block_table, case.context_lens, case.cu_seqlens, 16,
                                       cfg.rope_theta)
    dev = PrefillOnDevice(case)
    try:
        dev.run()
        assert mk.mi_kv_pool_check_errors(dev.pool) == 0
        _check_write(case, dev, kn, vn, qb)
        out = dev_to_bits(dev.out)
    finally:
        dev.close()
    G = cfg.num_q_heads // cfg.num_kv_heads
    heads = list(range(0, cfg.num_q_heads, G))
    scale = 1.0 / np.sqrt(float(cfg.head_dim))
    ref = np.empty((out.shape[0], len(heads), cfg.head_dim))
    for b in range(len(case.context_lens)):
        lo, hi = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        last = int(case.context_lens[b]) + hi - lo
        for j, h in enumerate(heads):
            ks, vs = oatt.gather_kv(kn, vn, case.block_table, 16, b, h // G, last)
            K, V = obf16.decode(ks), obf16.decode(vs)
            for i in range(lo, hi):
                L = int(case.context_lens[b]) + i - lo + 1
                ref[i, j] = oatt.attend(obf16.decode(qb[i, h]), K[:L], V[:L], scale)
    mx, rel = check_tolerance(out[:, heads], ref, "prefill 4 x 2048")
    _say("  max|d| %.3g relL2 %.3g over %d outputs" % (mx, rel, ref.size))


def test_prefill_then_decode_step():
    """A prompt prefilled on the GPU, then one decode step on the same pool:
    the decode output matches the oracle's prefill + decode."""
    cfg, _, _ = workloads.PREFILL_CONFIGS["prefill_small"]
    case = workloads.make_prefill_case(cfg, (0, 0, 0, 0), (37, 16, 1, 60), seed=9, reserve=1)
    _, kn, vn, _ = oatt.prefill_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                     case.block_table, case.context_lens, case.cu_seqlens, 16,
                                     cfg.rope_theta)
    ctx2 = case.new_lens.astype(np.int32)
    rng = np.random.default_rng(2)
    B = len(ctx2)
    q2 = workloads.bf16_normal(rng, (B, cfg.num_q_heads, cfg.head_dim))
    k2 = workloads.bf16_normal(rng, (B, cfg.num_kv_heads, cfg.head_dim))
    v2 = workloads.bf16_normal(rng, (B, cfg.num_kv_heads, cfg.head_dim))
    ref, _, _, _ = oatt.decode_step(kn, vn, q2, k2, v2, case.block_table, ctx2, 16, cfg.rope_theta)
    dev = PrefillOnDevice(case)
    try:
        dev.run()
        qd, kd, vd = bits_to_dev(q2), bits_to_dev(k2), bits_to_dev(v2)
        qr, out = torch.empty_like(qd), torch.empty_like(qd)
        ctxd = torch.from_numpy(ctx2).to(DEV)
        mk.mi_write_decode_kv(dev.pool, qd, kd, vd, qr, dev.table, dev.mbps, ctxd, B,
                              cfg.num_q_heads, cfg.rope_theta)
        need = mk.mi_paged_gqa_decode_workspace_bytes(dev.pool, B, cfg.num_q_heads, int(ctx2.max()))
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        mk.mi_paged_gqa_decode(dev.pool, qr, out, dev.table, dev.mbps, ctxd, B, cfg.num_q_heads,
                               0.0, int(ctx2.max()), ws, need)
        torch.cuda.synchronize()
        check_tolerance(dev_to_bits(out), ref, "prefill then decode")
        assert mk.mi_kv_pool_check_errors(dev.pool) == 0
    finally:
        dev.close()


def test_prefill_past_the_ranked_batch_limit():
    """More than 64 sequences: the query blocks are taken in plain block-index
    order instead of the longest-first ranking; both must cover every block."""
    rng = np.random.default_rng(246)
    B = 300
    ctx = tuple(int(x) for x in rng.integers(0, 48, B))
    n = tuple(int(x) for x in rng.integers(1, 70, B))
    cfg = workloads.DecodeConfig("pfb", batch=B, num_q_heads=4, num_kv_heads=2, head_dim=64,
                                 block_size=16, num_blocks=B * 8 + 8, rope_theta=1e4,
                                 ctx_draw="fixed", seed=17)
    _full_check(workloads.make_prefill_case(cfg, ctx, n), "B=300")


def test_prefill_errors_and_faults():
    cfg, ctx, n = workloads.PREFILL_CONFIGS["prefill_small"]
    case = workloads.make_prefill_case(cfg, ctx, n)
    dev = PrefillOnDevice(case)
    try:
        with pytest.raises(mk.MikvError) as e:        # output aliases input
            mk.mi_paged_prefill_attention(dev.pool, dev.q_rot, dev.q_rot, dev.table, dev.mbps,
                                          dev.ctx, dev.cu, dev.B, dev.T, dev.max_new, dev.Hq)
        assert e.value.status == mk.MI_ERR_INVALID_ARG
        with pytest.raises(mk.MikvError) as e:        # unsupported group
            mk.mi_paged_prefill_attention(dev.pool, dev.q_rot, dev.out, dev.table, dev.mbps,
                                          dev.ctx, dev.cu, dev.B, dev.T, dev.max_new, 3)
        assert e.value.status == mk.MI_ERR_UNSUPPORTED
        # a chunk longer than max_new_tokens is a recorded fault, not an access
        dev.run()
        mk.mi_paged_prefill_attention(dev.pool, dev.q_rot, dev.out, dev.table, dev.mbps,
                                      dev.ctx, dev.cu, dev.B, dev.T, 16, dev.Hq)
        assert mk.mi_kv_pool_check_errors(dev.pool) & mk.MI_FAULT_CONTEXT_LEN
    finally:
        dev.close()


@pytest.mark.parametrize("D,Hq,Hkv", [(64, 8, 2), (128, 32, 8), (128, 7, 1)])
def test_prefill_over_an_8bit_cache(D, Hq, Hkv):
    """Prefill chunks over an E4M3 pool with per-head scales: written V codes
    bit-exact, K codes within one code, outputs within tolerance of the
    oracle's dequantise-then-attend."""
    from oracle import fp8 as ofp8
    cfg = workloads.DecodeConfig("pf8", batch=4, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                 block_size=16, num_blocks=128, rope_theta=1e6, ctx_draw="fixed",
                                 seed=D + Hq)
    case = workloads.make_prefill_case(cfg, (0, 7, 40, 300), (70, 1, 33, 96), kv_format="fp8")
    rng = np.random.default_rng(D)
    ks = rng.uniform(0.3, 3.0, Hkv).astype(np.float32)
    vs = rng.uniform(0.3, 3.0, Hkv).astype(np.float32)
    ref, kn, vn, qb = oatt.prefill_step_fp8(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                            case.block_table, case.context_lens, case.cu_seqlens,
                                            16, cfg.rope_theta, ks, vs)
    dev = PrefillOnDevice(case, ks, vs)
    try:
        dev.run()
        assert mk.mi_kv_pool_check_errors(dev.pool) == 0
        gk, gv = dev.k_pool.cpu().numpy(), dev.v_pool.cpu().numpy()
        assert np.array_equal(gv, vn)
        def ordered(x):                 # E4M3 codes in value order
            x = x.astype(np.int64)
            return np.where(x & 0x80, -(x & 0x7F), x & 0x7F)
        changed = gk != kn
        assert np.abs(ordered(gk[changed]) - ordered(kn[changed])).max(initial=0) <= 1
        assert not np.isnan(ofp8.decode(gk[changed])).any()
        assert ulp_diff_bf16(dev_to_bits(dev.q_rot), qb).max() <= 1
        mx, rel = check_tolerance(dev_to_bits(dev.out), ref, "fp8 prefill D=%d G=%d" % (D, Hq // Hkv))
        _say("  max|d| %.3g relL2 %.3g, K codes differing: %d" % (mx, rel, int(changed.sum())))
    finally:
        dev.close()
