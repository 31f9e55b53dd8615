"""GPU parity of the one-launch decode step (mi_paged_gqa_decode_step): the
cache after it and q_rot equal, bit for bit, those of the two calls it
stands for (mi_write_decode_kv, then mi_paged_gqa_decode) on identical copies
of the inputs; its outputs meet the fp64 oracle's tolerance and stay within
a few bf16 steps of the two-call outputs (its attention rotates the query
heads in float32) (needs an MI355X)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_246_amd as mk
import workloads
from oracle import attention as oatt
from tests.gpu_harness import (DEV, DeviceCase, bf16_bits_to_f64, check_decode_write,
                               check_tolerance, dev_to_bits, oracle_decode_step)

pytestmark = pytest.mark.gpu

SMALL_CONFIGS = ["tiny", "qwen3_1p7b", "qwen2p5_7b_b1", "qwen2p5_7b_b4", "qwen2p5_7b_b8"]
GROUPS = [(1, 1), (2, 1), (3, 1), (4, 2), (10, 2), (6, 1), (14, 2), (8, 1)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mk.lib()       # fail loudly if the library is missing


def _say(*a):
    print(*a, flush=True)


def _step(dc, with_q_rot=True):
    ws_bytes = mk.mi_paged_gqa_decode_workspace_bytes(dc.pool, dc.B, dc.Hq, dc.max_ctx)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    mk.mi_paged_gqa_decode_step(dc.pool, dc.q, dc.k, dc.v, dc.q_rot if with_q_rot else None,
                                dc.out, dc.table, dc.mbps, dc.ctx, dc.B, dc.Hq,
                                dc.case.cfg.rope_theta, 0.0, dc.max_ctx, ws, ws_bytes)


def _against_two_calls(case, ref, label, k_scales=None, v_scales=None, with_q_rot=True):
    """Both paths on separate device copies: pools and q_rot bit-identical,
    outputs within tolerance of the oracle and close to the two-call path."""
    two = DeviceCase(case, k_scales, v_scales)
    one = DeviceCase(case, k_scales, v_scales)
    try:
        two.write()
        two.attend()
        one.q_rot.fill_(0x5555)
        _step(one, with_q_rot)
        torch.cuda.synchronize()
        assert torch.equal(one.k_pool, two.k_pool), "K cache differs"
        assert torch.equal(one.v_pool, two.v_pool), "V cache differs"
        if with_q_rot:
            assert torch.equal(one.q_rot, two.q_rot), "q_rot differs"
        else:
            assert bool((one.q_rot == 0x5555).all()), "q_rot written although not asked for"
        assert one.faults() == 0 and two.faults() == 0
        out1, out2 = dev_to_bits(one.out), dev_to_bits(two.out)
        mx, rel = check_tolerance(out1, ref, label)
        d = np.abs(bf16_bits_to_f64(out1) - bf16_bits_to_f64(out2))
        assert d.max() <= 4e-3 + 2.0 ** -7 * np.abs(bf16_bits_to_f64(out2)).max(), d.max()
        _say("  %s max|d| %.3g relL2 %.3g, vs two calls %.3g (%d of %d differ)"
             % (label, mx, rel, d.max(), int((out1 != out2).sum()), out1.size))
        return out1
    finally:
        one.close()
        two.close()


def _custom_cfg(Hq, Hkv, D, theta=1e4, seed=0):
    return workloads.DecodeConfig("custom", batch=0, num_q_heads=Hq, num_kv_heads=Hkv,
                                  head_dim=D, block_size=16, num_blocks=0, rope_theta=theta,
                                  ctx_draw="fixed", seed=seed)


def _ref(case):
    ref, _, _, _ = oatt.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                    case.block_table, case.context_lens, 16, case.cfg.rope_theta)
    return ref


@pytest.mark.parametrize("name", SMALL_CONFIGS)
def test_step_equals_write_then_attention(name):
    case = workloads.make_decode_case(workloads.CONFIGS[name], pool="poison")
    _say("step", name)
    _against_two_calls(case, _ref(case), name)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", GROUPS)
def test_step_group_sizes_head_dims_and_block_boundaries(D, Hq, Hkv):
    """Every group size at both head dims, contexts on and around block
    boundaries; ctx = 0 attends to its own new token only (output = v)."""
    cfg = _custom_cfg(Hq, Hkv, D, seed=3 * D + Hq)
    ctx = [0, 15, 16, 17, 31, 32, 33, 47, 100]
    case = workloads.make_decode_case(cfg, pool="poison", context_lens=ctx, num_blocks=96)
    _say("step groups", Hq, Hkv, "D", D)
    out = _against_two_calls(case, _ref(case), "G=%d D=%d" % (Hq // Hkv, D))
    G = Hq // Hkv
    for h in range(Hq):
        assert np.array_equal(out[0, h], case.v[0, h // G])


@pytest.mark.parametrize("name", ["tiny", "qwen3_1p7b", "qwen2p5_7b_b8"])
def test_step_over_an_8bit_cache(name):
    cfg = workloads.CONFIGS[name]
    case = workloads.make_decode_case(cfg, pool="poison", kv_format="fp8")
    rng = np.random.default_rng(7)
    ks = rng.choice([0.5, 1.0, 2.0, 0.37, 1.6], cfg.num_kv_heads).astype(np.float32)
    vs = rng.choice([0.25, 1.0, 0.8, 3.0], cfg.num_kv_heads).astype(np.float32)
    ref, _, _, _ = oatt.decode_step_fp8(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                        case.block_table, case.context_lens, 16, cfg.rope_theta,
                                        ks, vs)
    _say("step fp8", name)
    _against_two_calls(case, ref, "fp8 " + name, ks, vs)


def test_step_without_q_rot_output():
    case = workloads.make_decode_case(workloads.CONFIGS["qwen3_1p7b"], pool="poison")
    _against_two_calls(case, _ref(case), "no q_rot", with_q_rot=False)


def test_step_long_context_full_size():
    """The Qwen3-8B-shaped long-context workload at full size: the whole cache
    and q_rot equal the two-call path's bit for bit (and so the oracle's write,
    checked with the two-call path), and every output is within tolerance of
    the oracle and close to the two-call path's."""
    cfg = workloads.CONFIGS["qwen3_8b_long"]
    case = workloads.make_decode_case(cfg, pool="poison")
    _say("step qwen3_8b_long")
    two, one = DeviceCase(case), DeviceCase(case)
    try:
        two.write()
        two.attend()
        _step(one)
        torch.cuda.synchronize()
        assert torch.equal(one.k_pool, two.k_pool) and torch.equal(one.v_pool, two.v_pool)
        assert torch.equal(one.q_rot, two.q_rot)
        out1, out2 = dev_to_bits(one.out), dev_to_bits(two.out)
        gk, gv, gq = dev_to_bits(one.k_pool), dev_to_bits(one.v_pool), dev_to_bits(one.q_rot)
        assert one.faults() == 0 and two.faults() == 0
    finally:
        one.close()
        two.close()
    ref, kn, vn, qb = oracle_decode_step(case, "qwen3_8b_long")
    check_decode_write(case, gk, gv, gq, kn, vn, qb)
    mx, rel = check_tolerance(out1, ref, "step qwen3_8b_long")
    d = np.abs(bf16_bits_to_f64(out1) - bf16_bits_to_f64(out2))
    assert d.max() <= 1e-2, d.max()
    _say("  max|d| %.3g relL2 %.3g over %d outputs, vs two calls %.3g" % (mx, rel, out1.size, d.max()))


def test_step_argument_errors():
    case = workloads.make_decode_case(workloads.CONFIGS["tiny"], pool="poison")
    dc = DeviceCase(case)
    try:
        ws_bytes = mk.mi_paged_gqa_decode_workspace_bytes(dc.pool, dc.B, dc.Hq, dc.max_ctx)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
        theta = case.cfg.rope_theta
        for kw in [dict(q_rot=dc.q), dict(q_rot=dc.out), dict(out=dc.q), dict(ws_bytes=ws_bytes - 1),
                   dict(theta=0.0)]:
            a = dict(q_rot=dc.q_rot, out=dc.out, ws_bytes=ws_bytes, theta=theta)
            a.update(kw)
            with pytest.raises(mk.MikvError):
                mk.mi_paged_gqa_decode_step(dc.pool, dc.q, dc.k, dc.v, a["q_rot"], a["out"], dc.table,
                                            dc.mbps, dc.ctx, dc.B, dc.Hq, a["theta"], 0.0, dc.max_ctx,
                                            ws, a["ws_bytes"])
        mk.mi_paged_gqa_decode_step(dc.pool, dc.q, dc.k, dc.v, dc.q_rot, dc.out, dc.table, dc.mbps,
                                    dc.ctx, 0, dc.Hq, theta, 0.0, dc.max_ctx, ws, ws_bytes)
        torch.cuda.synchronize()
        assert dc.faults() == 0
    finally:
        dc.close()


def test_step_faults_are_recorded_not_fatal():
    """A bad block id planted from the host: recorded, and the cache ends as
    after the two calls with the same table. A length beyond max_context_len:
    recorded, that sequence gets NaN outputs and no cache write."""
    case = workloads.make_decode_case(workloads.CONFIGS["tiny"], pool="poison")
    ctx = case.context_lens
    bad = case.block_table.copy()
    bad[1, int(ctx[1]) // 16] = case.num_blocks + 5          # the slot's own block
    bad[0, 0] = -3                                           # a block read, not written
    two, one = DeviceCase(case), DeviceCase(case)
    try:
        for dc in (two, one):
            dc.table.copy_(torch.from_numpy(bad.astype(np.int32)))
        two.write()
        two.attend()
        _step(one)
        torch.cuda.synchronize()
        assert two.faults() & mk.MI_FAULT_BLOCK_ID
        assert one.faults() & mk.MI_FAULT_BLOCK_ID
        assert torch.equal(one.k_pool, two.k_pool) and torch.equal(one.v_pool, two.v_pool)
        assert one.faults() == 0                             # the read clears the word
    finally:
        one.close()
        two.close()

    dc = DeviceCase(case)
    try:
        k0, v0 = dc.k_pool.clone(), dc.v_pool.clone()
        b_long = int(np.argmax(ctx))
        dc.max_ctx = int(ctx.min())
        _step(dc)
        torch.cuda.synchronize()
        assert dc.faults() & mk.MI_FAULT_CONTEXT_LEN
        out = bf16_bits_to_f64(dev_to_bits(dc.out))
        assert np.all(np.isnan(out[b_long]))
        blk, off = int(case.block_table[b_long, int(ctx[b_long]) // 16]), int(ctx[b_long]) % 16
        assert torch.equal(dc.k_pool[blk, :, off], k0[blk, :, off])
        assert torch.equal(dc.v_pool[blk, :, off], v0[blk, :, off])
        b_short = int(np.argmin(ctx))
        assert np.all(np.isfinite(out[b_short]))
    finally:
        dc.close()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (3, 1), (8, 1), (10, 2)])
def test_step_8bit_group_sizes_head_dims(D, Hq, Hkv):
    """The 8-bit cache's query-slice layout at both head dims and several
    group sizes, contexts on and around block boundaries, per-head scales."""
    cfg = _custom_cfg(Hq, Hkv, D, seed=7 * D + Hq)
    ctx = [0, 15, 16, 17, 33, 64, 100]
    case = workloads.make_decode_case(cfg, pool="poison", context_lens=ctx, num_blocks=96,
                                      kv_format="fp8")
    ks = np.linspace(0.5, 1.5, Hkv).astype(np.float32)
    vs = np.linspace(2.0, 0.75, Hkv).astype(np.float32)
    ref, _, _, _ = oatt.decode_step_fp8(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                        case.block_table, case.context_lens, 16, cfg.rope_theta,
                                        ks, vs)
    _say("step fp8 groups", Hq, Hkv, "D", D)
    _against_two_calls(case, ref, "fp8 G=%d D=%d" % (Hq // Hkv, D), ks, vs)
