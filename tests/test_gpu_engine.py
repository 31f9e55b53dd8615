"""A continuous-batching loop on the GPU: the library's step planner admits,
grows, preempts and retires requests; each step runs the prefill rows
(mi_write_prefill_kv + mi_paged_prefill_attention) and the decode rows
(mi_write_decode_kv + mi_paged_gqa_decode) on the device. The oracle runs
the same plans on its own copy of the cache; every step's attention outputs
and, at the end, the cache must agree (needs an MI355X)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_246_amd as mk
import workloads
from oracle import attention as oatt
from tests.gpu_harness import DEV, bits_to_dev, check_tolerance, dev_to_bits, ulp_diff_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mk.lib()


def test_planner_driven_prefill_and_decode_steps():
    Hq, Hkv, D, theta = 8, 2, 64, 1e4
    N, mbps, R = 14, 12, 4          # tight pool: soft and hard brakes and one preemption
    rng = np.random.default_rng(77)
    kp = np.zeros((N, Hkv, 16, D), np.uint16)
    vp = np.zeros_like(kp)
    kd, vd = bits_to_dev(kp), bits_to_dev(vp)
    pool = mk.mi_kv_pool_init(N, 16, Hkv, D, kd, vd)
    s = mk.Scheduler(pool, mbps, R)
    reqs = [(0, 0, 40, 30), (0, 1, 70, 24), (1, 2, 17, 40), (2, 3, 100, 8), (3, 4, 5, 35),
            (6, 5, 33, 9)]
    pending = sorted(reqs)
    steps = prefills = decodes = 0
    saw_brake = set()
    preempted = 0
    try:
        for t in range(400):
            while pending and pending[0][0] <= t:
                _, rid, p, n = pending.pop(0)
                s.submit(rid, p, n)
            plan = s.step()
            saw_brake.add(plan["brake"])
            preempted += len(plan["preempted"])
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
                td = torch.from_numpy(table).to(DEV)
                cd = torch.from_numpy(ctx).to(DEV)
                cud = torch.from_numpy(cu).to(DEV)
                mk.mi_write_prefill_kv(pool, qd, bits_to_dev(k), bits_to_dev(v), qr, td, mbps, cd,
                                       cud, npf, T, Hq, theta)
                mk.mi_paged_prefill_attention(pool, qr, out, td, mbps, cd, cud, npf, T,
                                              int(n.max()), Hq)
                torch.cuda.synchronize()
                check_tolerance(dev_to_bits(out), ref, "step %d prefill" % t)
                prefills += npf
            if ndc:
                ctx = np.ascontiguousarray(plan["context_lens"][npf:npf + ndc])
                table = np.ascontiguousarray(plan["block_table"][npf:npf + ndc])
                q = workloads.bf16_normal(rng, (ndc, Hq, D))
                k = workloads.bf16_normal(rng, (ndc, Hkv, D))
                v = workloads.bf16_normal(rng, (ndc, Hkv, D))
                ref, kp, vp, _ = oatt.decode_step(kp, vp, q, k, v, table, ctx, 16, theta)
                qd = bits_to_dev(q)
                qr, out = torch.empty_like(qd), torch.empty_like(qd)
                td = torch.from_numpy(table).to(DEV)
                cd = torch.from_numpy(ctx).to(DEV)
                mx = int(ctx.max())
                mk.mi_write_decode_kv(pool, qd, bits_to_dev(k), bits_to_dev(v), qr, td, mbps, cd,
                                      ndc, Hq, theta)
                need = mk.mi_paged_gqa_decode_workspace_bytes(pool, ndc, Hq, mx)
                ws = torch.empty(need, dtype=torch.uint8, device=DEV)
                mk.mi_paged_gqa_decode(pool, qr, out, td, mbps, cd, ndc, Hq, 0.0, mx, ws, need)
                torch.cuda.synchronize()
                check_tolerance(dev_to_bits(out), ref, "step %d decode" % t)
                decodes += ndc
            steps += 1
            assert mk.mi_kv_pool_check_errors(pool) == 0
            if not pending and s.num_waiting() == 0 and s.num_running() == 0:
                break
    finally:
        s.close()
    gk, gv = dev_to_bits(kd), dev_to_bits(vd)
    mk.mi_kv_pool_destroy(pool)
    assert prefills >= len(reqs) and decodes > 20
    assert saw_brake == {mk.MI_BRAKE_PROCEED, mk.MI_BRAKE_SOFT, mk.MI_BRAKE_HARD} and preempted >= 1
    assert np.array_equal(gv, vp)
    assert ulp_diff_bf16(gk, kp).max() <= 1
    print("steps", steps, "prefill rows", prefills, "decode rows", decodes, "brakes", saw_brake,
          flush=True)
