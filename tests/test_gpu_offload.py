"""KV offload on the GPU: block copies between the pool and page-locked host
swap space (bit-exact), and the planner-driven loop in swap mode against the
oracle running the same plans (needs an MI355X)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_246_amd as mk
import workloads
from oracle import attention as oatt
from tests.gpu_harness import DEV, bits_to_dev, check_tolerance, codes_to_dev, dev_to_bits, ulp_diff_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mk.lib()


@pytest.mark.parametrize("staging", [True, False], ids=["staged", "per_block"])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_swap_out_then_in_moves_blocks_bit_exactly(fmt, staging):
    """Pairs in runs of consecutive slots over consecutive and over scattered
    device blocks, on a pool with a staging buffer (scattered runs packed into
    one transfer) and on one without (one transfer per block)."""
    N, Hkv, D, S = 48, 4, 128, 40
    rng = np.random.default_rng(5)
    if fmt == "bf16":
        kp = workloads.bf16_normal(rng, (N, Hkv, 16, D))
        vp = workloads.bf16_normal(rng, (N, Hkv, 16, D))
        kd, vd = bits_to_dev(kp), bits_to_dev(vp)
        hk = torch.zeros((S, Hkv, 16, D), dtype=torch.int16, pin_memory=True)
        flags = 0
    else:
        kp = workloads.fp8_normal_like(rng, (N, Hkv, 16, D))
        vp = workloads.fp8_normal_like(rng, (N, Hkv, 16, D))
        kd, vd = codes_to_dev(kp), codes_to_dev(vp)
        hk = torch.zeros((S, Hkv, 16, D), dtype=torch.uint8, pin_memory=True)
        flags = mk.MI_POOL_KV_FP8
    hv = torch.zeros_like(hk)
    if staging:
        flags |= mk.MI_POOL_SWAP_STAGING
    pool = mk.mi_kv_pool_init(N, 16, Hkv, D, kd, vd, flags=flags)
    try:
        # a run of consecutive pairs (merged into one transfer) and scattered ones
        out_pairs = np.array([[3, 10], [4, 11], [5, 12], [40, 0], [7, 39], [0, 5]], np.int32)
        mk.mi_kv_swap_out(pool, hk, hv, S, out_pairs)
        torch.cuda.synchronize()
        hkn, hvn = hk.numpy(), hv.numpy()
        as_u = (lambda a: a.view(np.uint16)) if fmt == "bf16" else (lambda a: a)
        for d, h in out_pairs:
            assert np.array_equal(as_u(hkn[h]), kp[d]) and np.array_equal(as_u(hvn[h]), vp[d])
        in_pairs = np.array([[10, 20], [11, 21], [12, 22], [0, 47], [39, 1], [5, 6]], np.int32)
        mk.mi_kv_swap_in(pool, hk, hv, S, in_pairs)
        torch.cuda.synchronize()
        gk = dev_to_bits(kd) if fmt == "bf16" else kd.cpu().numpy()
        gv = dev_to_bits(vd) if fmt == "bf16" else vd.cpu().numpy()
        ek, ev = kp.copy(), vp.copy()
        for (d, h), (h2, d2) in zip(out_pairs, in_pairs):
            assert h == h2
            ek[d2], ev[d2] = kp[d], vp[d]
        assert np.array_equal(gk, ek) and np.array_equal(gv, ev)
        # consecutive slots holding scattered blocks (packed through the staging
        # buffer when the pool has one)
        before_k = gk.copy()
        out2 = np.array([[9, 20], [2, 21], [30, 22], [17, 23], [44, 24]], np.int32)
        mk.mi_kv_swap_out(pool, hk, hv, S, out2)
        in2 = np.array([[24, 33], [20, 34], [21, 35], [22, 36], [23, 37]], np.int32)
        mk.mi_kv_swap_in(pool, hk, hv, S, in2)
        torch.cuda.synchronize()
        gk2 = dev_to_bits(kd) if fmt == "bf16" else kd.cpu().numpy()
        gv2 = dev_to_bits(vd) if fmt == "bf16" else vd.cpu().numpy()
        hkn, hvn = hk.numpy(), hv.numpy()
        for d, h in out2:
            assert np.array_equal(as_u(hkn[h]), ek[d]) and np.array_equal(as_u(hvn[h]), ev[d])
        ek2, ev2 = ek.copy(), ev.copy()
        src = {h: d for d, h in out2}
        for h, d in in2:
            ek2[d], ev2[d] = ek[src[h]], ev[src[h]]
        assert np.array_equal(gk2, ek2) and np.array_equal(gv2, ev2)
        assert not np.array_equal(gk2, before_k)
        with pytest.raises(mk.MikvError):           # one slot named twice
            mk.mi_kv_swap_out(pool, hk, hv, S, np.array([[1, 2], [3, 2]], np.int32))
        with pytest.raises(mk.MikvError):           # a slot past the swap space: nothing copied
            mk.mi_kv_swap_out(pool, hk, hv, S, np.array([[1, 2], [2, S]], np.int32))
        with pytest.raises(mk.MikvError):           # a block past the pool
            mk.mi_kv_swap_in(pool, hk, hv, S, np.array([[1, N]], np.int32))
    finally:
        mk.mi_kv_pool_destroy(pool)


@pytest.mark.parametrize("evict", [mk.MI_EVICT_LIFO, mk.MI_EVICT_FIFO, mk.MI_EVICT_LRU],
                         ids=["lifo", "fifo", "lru"])
def test_planner_loop_with_kv_offload(evict):
    """Tight pool with a host swap space, under each eviction policy: requests
    are swapped out and back while decoding; every step's outputs and the
    final cache match the oracle executing the same plans (copies included)."""
    Hq, Hkv, D, theta = 8, 2, 64, 1e4
    N, mbps, R, S = 14, 12, 4, 24
    rng = np.random.default_rng(78)
    kp = np.zeros((N, Hkv, 16, D), np.uint16)
    vp = np.zeros_like(kp)
    hkp = np.zeros((S, Hkv, 16, D), np.uint16)
    hvp = np.zeros_like(hkp)
    kd, vd = bits_to_dev(kp), bits_to_dev(vp)
    hk = torch.zeros((S, Hkv, 16, D), dtype=torch.int16, pin_memory=True)
    hv = torch.zeros_like(hk)
    pool = mk.mi_kv_pool_init(N, 16, Hkv, D, kd, vd, flags=mk.MI_POOL_SWAP_STAGING)
    s = mk.Scheduler(pool, mbps, R, host_slots=S, evict=evict)
    reqs = [(0, 0, 40, 30), (0, 1, 70, 24), (1, 2, 17, 40), (2, 3, 100, 8), (3, 4, 5, 35),
            (6, 5, 33, 9)]
    pending = sorted(reqs)
    swaps = 0
    try:
        for t in range(400):
            while pending and pending[0][0] <= t:
                _, rid, p, n = pending.pop(0)
                s.submit(rid, p, n)
            plan = s.step()
            if len(plan["swap_out"]):
                mk.mi_kv_swap_out(pool, hk, hv, S, plan["swap_out"])
                for d, h in plan["swap_out"]:
                    hkp[h], hvp[h] = kp[d], vp[d]
                swaps += len(plan["swap_out"])
            if len(plan["swap_in"]):
                mk.mi_kv_swap_in(pool, hk, hv, S, plan["swap_in"])
                for h, d in plan["swap_in"]:
                    kp[d], vp[d] = hkp[h], hvp[h]
            npf, ndc = plan["num_prefill"], plan["num_decode"]
            if npf:
                ctx = plan["context_lens"][:npf]
                n = plan["new_tokens"][:npf]
                cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
                T = int(cu[-1])
                table = np.ascontiguousarray(plan["block_table"][:npf])
                q = workloads.bf16_normal(rng, (T, Hq, D))
                k = workloads.bf16_normal(rng, (T, Hkv, D))
                v = workloads.bf16_normal(rng, (T, Hkv, D))
                ref, kp, vp, _ = oatt.prefill_step(kp, vp, q, k, v, table, ctx, cu, 16, theta)
                qd = bits_to_dev(q)
                qr, out = torch.empty_like(qd), torch.empty_like(qd)
                td, cd, cud = (torch.from_numpy(a).to(DEV) for a in (table, ctx, cu))
                mk.mi_write_prefill_kv(pool, qd, bits_to_dev(k), bits_to_dev(v), qr, td, mbps, cd,
                                       cud, npf, T, Hq, theta)
                mk.mi_paged_prefill_attention(pool, qr, out, td, mbps, cd, cud, npf, T,
                                              int(n.max()), Hq)
                torch.cuda.synchronize()
                check_tolerance(dev_to_bits(out), ref, "step %d prefill" % t)
            if ndc:
                ctx = np.ascontiguousarray(plan["context_lens"][npf:npf + ndc])
                table = np.ascontiguousarray(plan["block_table"][npf:npf + ndc])
                q = workloads.bf16_normal(rng, (ndc, Hq, D))
                k = workloads.bf16_normal(rng, (ndc, Hkv, D))
                v = workloads.bf16_normal(rng, (ndc, Hkv, D))
                ref, kp, vp, _ = oatt.decode_step(kp, vp, q, k, v, table, ctx, 16, theta)
                qd = bits_to_dev(q)
                qr, out = torch.empty_like(qd), torch.empty_like(qd)
                td, cd = torch.from_numpy(table).to(DEV), torch.from_numpy(ctx).to(DEV)
                mx = int(ctx.max())
                mk.mi_write_decode_kv(pool, qd, bits_to_dev(k), bits_to_dev(v), qr, td, mbps, cd,
                                      ndc, Hq, theta)
                need = mk.mi_paged_gqa_decode_workspace_bytes(pool, ndc, Hq, mx)
                ws = torch.empty(need, dtype=torch.uint8, device=DEV)
                mk.mi_paged_gqa_decode(pool, qr, out, td, mbps, cd, ndc, Hq, 0.0, mx, ws, need)
                torch.cuda.synchronize()
                check_tolerance(dev_to_bits(out), ref, "step %d decode" % t)
            assert mk.mi_kv_pool_check_errors(pool) == 0
            if not pending and s.num_waiting() == 0 and s.num_running() == 0 and s.num_swapped() == 0:
                break
    finally:
        s.close()
    torch.cuda.synchronize()
    gk, gv = dev_to_bits(kd), dev_to_bits(vd)
    mk.mi_kv_pool_destroy(pool)
    assert swaps > 0
    assert np.array_equal(gv, vp)
    assert ulp_diff_bf16(gk, kp).max() <= 1
    print("block copies out", swaps, flush=True)
