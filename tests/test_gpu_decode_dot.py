"""GPU parity of the dot-product decode attention (pool flag
MI_POOL_DECODE_DOT: q.k and the weighted V sum on the vector ALUs) against the
fp64 oracle, through the C ABI, over bf16 and 8-bit caches (needs an MI355X).
Same cases and tolerance as the matrix-core kernel's tests."""
import numpy as np
import pytest
import torch

import paged_kv_cache_246_amd as mk
import workloads
from oracle import attention as oatt
from tests.gpu_harness import (DeviceCase, check_tolerance, dev_to_bits, drop_oracle,
                               oracle_decode_step)

pytestmark = pytest.mark.gpu

CONFIGS = ["tiny", "qwen3_1p7b", "qwen2p5_7b_b1", "qwen2p5_7b_b4", "qwen2p5_7b_b8"]
GROUPS = [(1, 1), (3, 1), (4, 2), (14, 2), (8, 1)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mk.lib()       # fail loudly if the library is missing


def _say(*a):
    print(*a, flush=True)


def _scales(Hkv, seed):
    rng = np.random.default_rng(seed)
    base = np.array([1.0, 0.37, 2.0, 0.8125, 3.3, 0.5, 1.7, 0.25], np.float32)
    return (base[rng.permutation(8)[:Hkv] % 8].astype(np.float32),
            base[rng.permutation(8)[:Hkv] % 8].astype(np.float32))


def _run(case, ref, label, ks=None, vs=None, splits=(0,)):
    dc = DeviceCase(case, ks, vs, extra_flags=mk.MI_POOL_DECODE_DOT)
    try:
        dc.write()
        for split in splits:
            dc.attend(split_tokens=split)
            torch.cuda.synchronize()
            mx, rel = check_tolerance(dev_to_bits(dc.out), ref, "%s split=%d" % (label, split))
            _say("  %s split %d: max|d| %.3g relL2 %.3g" % (label, split, mx, rel))
        assert dc.faults() == 0
    finally:
        dc.close()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("name", CONFIGS)
def test_dot_decode_parity(name, fmt):
    cfg = workloads.CONFIGS[name]
    case = workloads.make_decode_case(cfg, pool="poison", kv_format=fmt)
    _say("dot decode", name, fmt)
    if fmt == "fp8":
        ks, vs = _scales(cfg.num_kv_heads, len(name))
        ref = oatt.decode_step_fp8(case.k_pool, case.v_pool, case.q, case.k, case.v, case.block_table,
                                   case.context_lens, 16, cfg.rope_theta, ks, vs)[0]
        _run(case, ref, name, ks, vs, splits=(0, 64))
    else:
        ref = oatt.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v, case.block_table,
                               case.context_lens, 16, cfg.rope_theta)[0]
        _run(case, ref, name, splits=(0, 16, 256))


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", GROUPS)
def test_dot_group_sizes_head_dims_and_block_boundaries(Hq, Hkv, D, fmt):
    """Every lane split (8 or 16 lanes per key row) and prefetch depth the
    kernel is built with, contexts on and around block boundaries."""
    cfg = workloads.DecodeConfig("custom", batch=0, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                 block_size=16, num_blocks=0, rope_theta=1e4, ctx_draw="fixed",
                                 seed=D + Hq)
    ctx = [0, 15, 16, 17, 31, 32, 33, 47, 100]
    case = workloads.make_decode_case(cfg, pool="poison", context_lens=ctx, num_blocks=96, kv_format=fmt)
    label = "G=%d D=%d %s" % (Hq // Hkv, D, fmt)
    if fmt == "fp8":
        ks, vs = _scales(Hkv, D + Hq)
        ref = oatt.decode_step_fp8(case.k_pool, case.v_pool, case.q, case.k, case.v, case.block_table,
                                   case.context_lens, 16, cfg.rope_theta, ks, vs)[0]
        _run(case, ref, label, ks, vs, splits=(0, 16))
    else:
        ref = oatt.decode_step(case.k_pool, case.v_pool, case.q, case.k, case.v, case.block_table,
                               case.context_lens, 16, cfg.rope_theta)[0]
        _run(case, ref, label, splits=(0, 16, 32))


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_dot_long_context_full_size(fmt):
    """The Qwen3-8B-shaped long-context workload at full size: all
    B x Hq x D outputs of the dot-product form against the oracle."""
    cfg = workloads.CONFIGS["qwen3_8b_long"]
    case = workloads.make_decode_case(cfg, pool="poison", kv_format=fmt)
    _say("dot qwen3_8b_long", fmt)
    if fmt == "fp8":
        ks, vs = _scales(cfg.num_kv_heads, 45)
        ref = oracle_decode_step(case, "qwen3_8b_long_fp8", ks, vs)[0]
        _run(case, ref, "qwen3_8b_long fp8", ks, vs)
        drop_oracle("qwen3_8b_long_fp8")
    else:
        ref = oracle_decode_step(case, "qwen3_8b_long")[0]
        _run(case, ref, "qwen3_8b_long")
