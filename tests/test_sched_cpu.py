"""The library's step planner (host code, no GPU) against the oracle model,
step by step: every plan (ids, contexts, token counts, block-table rows,
preemptions, retirements, brake state) equal, on hand-made and random
request streams."""
import numpy as np
import pytest

import paged_kv_cache_246_amd as mk
from oracle import paged, sched


def _compare(plan, ref, mbps):
    rows = [(r[0], r[1], r[2], r[3]) for r in ref.prefill] + \
           [(r[0], r[1], 1, r[2]) for r in ref.decode]
    assert plan["num_prefill"] == len(ref.prefill) and plan["num_decode"] == len(ref.decode)
    assert plan["brake"] == ref.brake
    assert list(plan["preempted"]) == ref.preempted
    assert list(plan["finished"]) == ref.finished
    assert list(plan["swapped_out"]) == ref.swapped_out
    assert [tuple(x) for x in plan["swap_out"]] == ref.swap_out
    assert [tuple(x) for x in plan["swap_in"]] == ref.swap_in
    for i, (rid, ctx, n, blocks) in enumerate(rows):
        assert plan["ids"][i] == rid and plan["context_lens"][i] == ctx and plan["new_tokens"][i] == n
        want = np.full(mbps, -1, np.int32)
        want[:len(blocks)] = blocks
        assert np.array_equal(plan["block_table"][i], want)


def _run(N, mbps, max_running, requests, hard=0.10, soft=0.30, max_steps=5000, host_slots=0,
         evict=sched.EVICT_LIFO):
    """requests: list of (arrival_step, rid, prompt, max_new)."""
    pool = mk.mi_kv_pool_init(N, 16, 2, 64, flags=mk.MI_POOL_HOST_ONLY)
    s = mk.Scheduler(pool, mbps, max_running, hard, soft, host_slots=host_slots, evict=evict)
    ref = sched.Scheduler(N, max_running=max_running, hard=hard, soft=soft, max_blocks_per_seq=mbps,
                          host_slots=host_slots, evict=evict)
    try:
        pending = sorted(requests)
        brakes = set()
        for t in range(max_steps):
            while pending and pending[0][0] <= t:
                _, rid, p, n = pending.pop(0)
                s.submit(rid, p, n)
                ref.submit(rid, p, n)
            plan = s.step()
            r = ref.step()
            _compare(plan, r, mbps)
            assert plan["free_blocks"] == ref.pool.num_free() == mk.mi_kv_num_free_blocks(pool)
            brakes.add(plan["brake"])
            if not pending and ref.idle():
                break
        assert ref.idle() and s.num_waiting() == 0 and s.num_running() == 0
        assert s.num_swapped() == 0
        assert mk.mi_kv_num_free_blocks(pool) == N
        return brakes
    finally:
        s.close()
        mk.mi_kv_pool_destroy(pool)


def test_hand_made_stream_hits_every_brake():
    reqs = [(0, 0, 1120, 10), (0, 1, 16, 10), (1, 2, 16, 10), (2, 3, 90 * 16 - 1200, 5),
            (3, 4, 300, 40), (5, 5, 16, 3)]
    brakes = _run(100, 100, 8, reqs)
    assert mk.MI_BRAKE_SOFT in brakes


@pytest.mark.parametrize("evict", [mk.MI_EVICT_LIFO, mk.MI_EVICT_FIFO])
@pytest.mark.parametrize("seed", range(6))
def test_random_streams_match_the_oracle(seed, evict):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(30, 300))
    mbps = int(rng.integers(8, 40))
    reqs = []
    for rid in range(int(rng.integers(20, 80))):
        prompt = int(rng.integers(1, 16 * mbps // 2))
        new = int(rng.integers(1, 16 * mbps - prompt + 1))
        if paged.blocks_needed(prompt + new, 16) > min(N, mbps):
            continue
        reqs.append((int(rng.integers(0, 200)), rid, prompt, new))
    _run(N, mbps, int(rng.integers(1, 12)), reqs, hard=float(rng.choice([0.0, 0.1, 0.2])),
         soft=float(rng.choice([0.0, 0.3, 0.5])), evict=evict)


def test_submit_refuses_requests_that_can_never_fit():
    pool = mk.mi_kv_pool_init(10, 16, 2, 64, flags=mk.MI_POOL_HOST_ONLY)
    s = mk.Scheduler(pool, 8, 4)
    try:
        with pytest.raises(mk.MikvError) as e:
            s.submit(1, 8 * 16, 1)                    # 9 blocks > row of 8
        assert e.value.status == mk.MI_ERR_UNSUPPORTED
        with pytest.raises(mk.MikvError) as e:
            s.submit(2, 0, 5)
        assert e.value.status == mk.MI_ERR_INVALID_ARG
        s.submit(3, 16, 16)
        p = s.step()
        assert p["num_prefill"] == 1 and mk.mi_kv_num_free_blocks(pool) == 9
    finally:
        s.close()
        assert mk.mi_kv_num_free_blocks(pool) == 10  # destroy returned the blocks
        mk.mi_kv_pool_destroy(pool)


@pytest.mark.parametrize("evict", [mk.MI_EVICT_LIFO, mk.MI_EVICT_FIFO, mk.MI_EVICT_LRU])
@pytest.mark.parametrize("seed", range(6))
def test_random_swap_streams_match_the_oracle(seed, evict):
    rng = np.random.default_rng(200 + seed)
    N = int(rng.integers(16, 80))
    mbps = int(rng.integers(6, 30))
    reqs = []
    for rid in range(int(rng.integers(20, 60))):
        prompt = int(rng.integers(1, 16 * mbps // 2))
        new = int(rng.integers(1, 16 * mbps - prompt + 1))
        if paged.blocks_needed(prompt + new, 16) > min(N, mbps):
            continue
        reqs.append((int(rng.integers(0, 100)), rid, prompt, new))
    _run(N, mbps, int(rng.integers(2, 8)), reqs, hard=float(rng.choice([0.0, 0.1])),
         soft=float(rng.choice([0.0, 0.3])), host_slots=int(rng.integers(0, 3 * N)), evict=evict)


def test_eviction_policy_argument():
    pool = mk.mi_kv_pool_init(10, 16, 2, 64, flags=mk.MI_POOL_HOST_ONLY)
    s = mk.Scheduler(pool, 8, 4)
    try:
        assert mk.lib().mi_sched_set_eviction(s.h, 3) == mk.MI_ERR_INVALID_ARG
        assert mk.lib().mi_sched_set_eviction(s.h, mk.MI_EVICT_FIFO) == mk.MI_OK
    finally:
        s.close()
        mk.mi_kv_pool_destroy(pool)
