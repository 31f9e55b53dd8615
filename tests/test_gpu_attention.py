"""GPU parity of write_decode_kv, the gather and paged GQA decode attention
against the fp64 oracle, through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_246_amd as mk
import workloads
from oracle import attention as oatt
from tests.gpu_harness import (DEV, DeviceCase, bf16_bits_to_f64, bits_to_dev, check_decode_write,
                               check_tolerance, dev_to_bits, oracle_decode_step)

pytestmark = pytest.mark.gpu

SMALL_CONFIGS = ["tiny", "qwen3_1p7b", "qwen2p5_7b_b1", "qwen2p5_7b_b4", "qwen2p5_7b_b8"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mk.lib()       # fail loudly if the library is missing


def _say(*a):
    print(*a, flush=True)


def _custom_cfg(Hq, Hkv, D, theta=1e4, seed=0):
    return workloads.DecodeConfig("custom", batch=0, num_q_heads=Hq, num_kv_heads=Hkv,
                                  head_dim=D, block_size=16, num_blocks=0, rope_theta=theta,
                                  ctx_draw="fixed", seed=seed)


def _check_write(case, dc):
    """Pools after the GPU write vs the oracle's write: bit-exact placement and V,
    K and q_rot within one bf16 ulp; every other byte untouched."""
    cfg = case.cfg
    kn, vn, qrot_bits, _ = oatt.write_decode_kv(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                                case.block_table, case.context_lens,
                                                cfg.block_size, cfg.rope_theta)
    return check_decode_write(case, dev_to_bits(dc.k_pool), dev_to_bits(dc.v_pool),
                              dev_to_bits(dc.q_rot), kn, vn, qrot_bits)


@pytest.mark.parametrize("name", SMALL_CONFIGS)
def test_write_decode_kv_parity(name):
    case = workloads.make_decode_case(workloads.CONFIGS[name], pool="poison")
    _say("write_decode_kv", name, "B", len(case.context_lens))
    dc = DeviceCase(case)
    try:
        dc.write()
        torch.cuda.synchronize()
        off = _check_write(case, dc)
        _say("  elements differing by one ulp:", off)
        assert dc.faults() == 0
    finally:
        dc.close()


def test_write_decode_kv_in_place_q():
    case = workloads.make_decode_case(workloads.CONFIGS["qwen3_1p7b"], pool="poison")
    dc = DeviceCase(case)
    try:
        dc.write()
        expect = dev_to_bits(dc.q_rot)
        dc.k_pool.copy_(bits_to_dev(case.k_pool))
        dc.v_pool.copy_(bits_to_dev(case.v_pool))
        mk.mi_write_decode_kv(dc.pool, dc.q, dc.k, dc.v, dc.q, dc.table, dc.mbps, dc.ctx, dc.B,
                              dc.Hq, case.cfg.rope_theta)
        assert np.array_equal(dev_to_bits(dc.q), expect)
    finally:
        dc.close()


@pytest.mark.parametrize("name", SMALL_CONFIGS)
def test_decode_step_parity(name):
    cfg = workloads.CONFIGS[name]
    case = workloads.make_decode_case(cfg, pool="poison")
    _say("decode step", name)
    ref, _, _, _ = oatt.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                    case.block_table, case.context_lens, cfg.block_size,
                                    cfg.rope_theta)
    dc = DeviceCase(case)
    try:
        dc.write()
        dc.attend()
        torch.cuda.synchronize()
        mx, rel = check_tolerance(dev_to_bits(dc.out), ref, name)
        _say("  max|d| %.3g  relL2 %.3g" % (mx, rel))
        assert dc.faults() == 0
    finally:
        dc.close()


@pytest.mark.parametrize("split", [16, 64, 256, 1024])
def test_split_sizes_all_within_tolerance_and_permutation_invariant(split):
    cfg = workloads.CONFIGS["qwen3_1p7b"]
    case = workloads.make_decode_case(cfg, pool="poison")
    _say("split", split)
    ref, kn, vn, qb = oatt.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                       case.block_table, case.context_lens, 16, cfg.rope_theta)
    dc = DeviceCase(case)
    try:
        dc.write()
        dc.attend(split_tokens=split)
        torch.cuda.synchronize()
        out1 = dev_to_bits(dc.out)
        check_tolerance(out1, ref, "split %d" % split)
        # relabel physical blocks by a random permutation and move their contents
        pi = np.random.default_rng(split).permutation(case.num_blocks)
        kp, vp = dev_to_bits(dc.k_pool), dev_to_bits(dc.v_pool)
        kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
        kp2[pi] = kp
        vp2[pi] = vp
        t2 = np.where(case.block_table >= 0, pi[np.maximum(case.block_table, 0)], -1).astype(np.int32)
        dc.k_pool.copy_(bits_to_dev(kp2))
        dc.v_pool.copy_(bits_to_dev(vp2))
        dc.table.copy_(torch.from_numpy(t2))
        dc.attend(split_tokens=split)
        torch.cuda.synchronize()
        assert np.array_equal(dev_to_bits(dc.out), out1)
    finally:
        dc.close()


def test_repeated_calls_with_other_splits_in_between_are_bit_identical():
    """A call with many cut segments (16-token shares), one with few, then the
    first again on the same pool: the repeats are bit-identical, so no state
    of one call (partials, merge bookkeeping) leaks into the next."""
    cfg = workloads.CONFIGS["qwen3_1p7b"]
    case = workloads.make_decode_case(cfg, pool="poison")
    ref, _, _, _ = oatt.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                    case.block_table, case.context_lens, 16, cfg.rope_theta)
    dc = DeviceCase(case)
    try:
        dc.write()
        outs = []
        for split in (16, 1024, 16, 1024):
            dc.attend(split_tokens=split)
            torch.cuda.synchronize()
            outs.append(dev_to_bits(dc.out))
            check_tolerance(outs[-1], ref, "split %d" % split)
        assert np.array_equal(outs[0], outs[2])
        assert np.array_equal(outs[1], outs[3])
        assert dc.faults() == 0
    finally:
        dc.close()


@pytest.mark.parametrize("name,len_extra", [("tiny", 1), ("qwen3_1p7b", 0), ("qwen3_1p7b", 1)])
def test_gather_bit_exact(name, len_extra):
    cfg = workloads.CONFIGS[name]
    case = workloads.make_decode_case(cfg, pool="poison")
    dc = DeviceCase(case)
    try:
        if len_extra:
            dc.write()
        l_max = int(case.context_lens.max()) + 1
        ko = torch.full((dc.B, dc.Hkv, l_max, dc.D), 0x5555, dtype=torch.int16, device=DEV)
        vo = ko.clone()
        mk.mi_gather_kv(dc.pool, dc.table, dc.mbps, dc.ctx, dc.B, len_extra, ko, vo, l_max)
        torch.cuda.synchronize()
        ko, vo = dev_to_bits(ko), dev_to_bits(vo)
        kp, vp = dev_to_bits(dc.k_pool), dev_to_bits(dc.v_pool)
        for b in range(dc.B):
            n = int(case.context_lens[b]) + len_extra
            for g in range(dc.Hkv):
                ks, vs = oatt.gather_kv(kp, vp, case.block_table, 16, b, g, n)
                assert np.array_equal(ko[b, g, :n], ks)
                assert np.array_equal(vo[b, g, :n], vs)
                assert np.all(ko[b, g, n:] == 0x5555)
        assert dc.faults() == 0
    finally:
        dc.close()


GROUPS = [(1, 1), (2, 1), (3, 1), (4, 2), (10, 2), (6, 1), (14, 2), (8, 1)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", GROUPS)
def test_group_sizes_head_dims_and_block_boundaries(D, Hq, Hkv):
    """Every supported group size at both head dims, with contexts on and
    around block boundaries (ctx = 0, 15, 16, 17, 31, 32, 33, 47, 100)."""
    cfg = _custom_cfg(Hq, Hkv, D, seed=D + Hq)
    ctx = [0, 15, 16, 17, 31, 32, 33, 47, 100]
    case = workloads.make_decode_case(cfg, pool="poison", context_lens=ctx, num_blocks=96)
    _say("groups", Hq, Hkv, "D", D)
    ref, _, _, _ = oatt.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                    case.block_table, case.context_lens, 16, cfg.rope_theta)
    dc = DeviceCase(case)
    try:
        dc.write()
        _check_write(case, dc)
        for split in (0, 16, 32):
            dc.attend(split_tokens=split)
            torch.cuda.synchronize()
            check_tolerance(dev_to_bits(dc.out), ref, "G=%d D=%d split=%d" % (Hq // Hkv, D, split))
        # ctx = 0 attends to its own new token only: output = v (bf16 bits)
        G = Hq // Hkv
        out0 = dev_to_bits(dc.out)[0]
        for h in range(Hq):
            assert np.array_equal(out0[h], case.v[0, h // G])
        assert dc.faults() == 0
    finally:
        dc.close()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("top", [383, 384])
def test_per_segment_form_at_its_length_limit(top, fmt):
    """With the library's split, contexts whose longest segment has at most 24
    tiles (L = ctx + 1 <= 384) take the one-launch per-segment kernel (eight
    waves per (sequence, KV head), merged in LDS); one token more takes the
    stream-K kernel and the combine. Both sides of the limit, and the same
    inputs through an explicit split (always stream-K), against the oracle."""
    cfg = _custom_cfg(32, 8, 128, theta=1e6, seed=top)
    ctx = [top, 0, 15, 16, 17, 200, top - 1, 100]
    case = workloads.make_decode_case(cfg, pool="poison", context_lens=ctx, num_blocks=256,
                                      kv_format=fmt)
    if fmt == "fp8":
        ks = np.array([1.0, 0.37, 2.0, 0.8125, 3.3, 0.5, 1.7, 0.25], np.float32)
        vs = ks[::-1].copy()
        ref = oatt.decode_step_fp8(case.k_pool, case.v_pool, case.q, case.k, case.v, case.block_table,
                                   case.context_lens, 16, cfg.rope_theta, ks, vs)[0]
        dc = DeviceCase(case, ks, vs)
    else:
        ref = oatt.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v, case.block_table,
                               case.context_lens, 16, cfg.rope_theta)[0]
        dc = DeviceCase(case)
    try:
        dc.write()
        for split in (0, 32):
            dc.attend(split_tokens=split)
            torch.cuda.synchronize()
            mx, rel = check_tolerance(dev_to_bits(dc.out), ref, "top=%d %s split=%d" % (top, fmt, split))
            _say("  top %d %s split %d: max|d| %.3g relL2 %.3g" % (top, fmt, split, mx, rel))
        assert dc.faults() == 0
    finally:
        dc.close()


@pytest.mark.parametrize("B,ctx_hi", [(65, 40), (130, 200), (1024, 300)])
def test_batches_past_one_prefix_chunk_and_at_the_maximum(B, ctx_hi):
    """The kernels build the tile prefix over the batch 64 sequences at a time
    with a carry: batches of 65 and 130 cross one and two chunk boundaries,
    1024 is the largest batch a call accepts. Write and attention against the
    oracle, two split sizes."""
    cfg = workloads.DecodeConfig("big_batch", batch=B, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                 block_size=16, num_blocks=0, rope_theta=1e4, ctx_draw="uniform",
                                 ctx_lo=0, ctx_hi=ctx_hi, seed=B)
    case = workloads.make_decode_case(cfg, pool="poison")
    _say("batch", B, "tokens", int(case.context_lens.sum()) + B)
    ref, _, _, _ = oatt.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                    case.block_table, case.context_lens, 16, cfg.rope_theta)
    dc = DeviceCase(case)
    try:
        dc.write()
        _check_write(case, dc)
        for split in (0, 64):
            dc.attend(split_tokens=split)
            torch.cuda.synchronize()
            check_tolerance(dev_to_bits(dc.out), ref, "B=%d split=%d" % (B, split))
        assert dc.faults() == 0
    finally:
        dc.close()


def test_long_context_config_full_size():
    """Qwen3-8B-shaped long-context workload at full size in the benchmark's
    launch configuration, every output against the oracle: the whole K and V
    pools and q_rot after the write (V bit-exact, K and q_rot within one ulp,
    every other element bit-identical), then all B x Hq x D attention outputs."""
    cfg = workloads.CONFIGS["qwen3_8b_long"]
    case = workloads.make_decode_case(cfg, pool="poison")
    _say("qwen3_8b_long: tokens", int(case.context_lens.sum()) + len(case.context_lens))
    dc = DeviceCase(case)
    try:
        dc.write()
        dc.attend()
        torch.cuda.synchronize()
        out = dev_to_bits(dc.out)
        gk, gv, gq = dev_to_bits(dc.k_pool), dev_to_bits(dc.v_pool), dev_to_bits(dc.q_rot)
        assert dc.faults() == 0
    finally:
        dc.close()
    ref, kn, vn, qb = oracle_decode_step(case, "qwen3_8b_long")
    off = check_decode_write(case, gk, gv, gq, kn, vn, qb)
    mx, rel = check_tolerance(out, ref, "qwen3_8b_long")
    _say("  one ulp off: %d; max|d| %.3g relL2 %.3g over %d outputs" % (off, mx, rel, out.size))


def test_empty_batch_is_a_no_op():
    case = workloads.make_decode_case(workloads.CONFIGS["tiny"], pool="poison")
    dc = DeviceCase(case)
    try:
        mk.mi_write_decode_kv(dc.pool, dc.q, dc.k, dc.v, dc.q_rot, dc.table, dc.mbps, dc.ctx, 0,
                              dc.Hq, 1e4)
        ws = torch.empty(256, dtype=torch.uint8, device=DEV)
        mk.mi_paged_gqa_decode(dc.pool, dc.q_rot, dc.out, dc.table, dc.mbps, dc.ctx, 0, dc.Hq,
                               0.0, 0, ws, 256)
        torch.cuda.synchronize()
        assert np.array_equal(dev_to_bits(dc.k_pool), case.k_pool)
    finally:
        dc.close()


def test_device_faults_are_recorded_not_fatal():
    """Out-of-range block ids and lengths, planted from the host, are caught by
    the kernels' own range checks: no access happens, the error word says so."""
    cfg = workloads.CONFIGS["tiny"]
    case = workloads.make_decode_case(cfg, pool="poison")
    dc = DeviceCase(case)
    try:
        bad = case.block_table.copy()
        bad[1, 2] = case.num_blocks + 5
        dc.table.copy_(torch.from_numpy(bad))
        dc.write()
        dc.attend()
        bits = dc.faults()
        assert bits & mk.MI_FAULT_BLOCK_ID
        dc.table.copy_(torch.from_numpy(case.block_table))
        assert dc.faults() == 0                        # the read clears the word
        # a length beyond max_context_len: recorded, output of that row is NaN
        dc.attend(max_ctx=int(case.context_lens.min()))
        bits = dc.faults()
        assert bits & mk.MI_FAULT_CONTEXT_LEN
        out = bf16_bits_to_f64(dev_to_bits(dc.out))
        b_long = int(np.argmax(case.context_lens))
        assert np.all(np.isnan(out[b_long]))
    finally:
        dc.close()


def test_argument_errors():
    case = workloads.make_decode_case(workloads.CONFIGS["tiny"], pool="poison")
    dc = DeviceCase(case)
    try:
        need = mk.mi_paged_gqa_decode_workspace_bytes(dc.pool, dc.B, dc.Hq, dc.max_ctx)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        with pytest.raises(mk.MikvError) as e:
            mk.mi_paged_gqa_decode(dc.pool, dc.q_rot, dc.out, dc.table, dc.mbps, dc.ctx, dc.B,
                                   dc.Hq, 0.0, dc.max_ctx, ws, need - 1)
        assert e.value.status == mk.MI_ERR_WORKSPACE_TOO_SMALL
        with pytest.raises(mk.MikvError) as e:
            mk.mi_paged_gqa_decode(dc.pool, dc.q_rot, dc.out, dc.table, dc.mbps, dc.ctx, dc.B,
                                   3, 0.0, dc.max_ctx, ws, need)
        assert e.value.status == mk.MI_ERR_UNSUPPORTED
        with pytest.raises(mk.MikvError) as e:
            mk.mi_paged_gqa_decode(dc.pool, dc.q_rot, dc.q_rot, dc.table, dc.mbps, dc.ctx, dc.B,
                                   dc.Hq, 0.0, dc.max_ctx, ws, need)
        assert e.value.status == mk.MI_ERR_INVALID_ARG
    finally:
        dc.close()
