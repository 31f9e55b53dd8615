"""Pins for the oracle's step planner (CPU only): brake decisions in scenarios
worked out by hand from the serving-framework report's rules (hard: free <
10 %; soft: decodes running and free < 30 %), the block counts of the paged
cache (ceil(tokens / 16)), recompute preemption order, and lifecycle
invariants over random request streams."""
import numpy as np
import pytest

from oracle import paged, sched


def _tables_disjoint_and_complete(s):
    held = [b for r in s.running for b in r.blocks]
    assert len(held) == len(set(held))
    assert len(held) + s.pool.num_free() == s.N


def test_fresh_system_admits_until_capacity_ignoring_the_soft_brake():
    # 100 blocks, prompts of 480 tokens = 30 blocks: no decode is running when
    # admission starts, so only capacity and the hard brake apply.
    s = sched.Scheduler(100, max_running=8)
    for i in range(5):
        s.submit(i, 480, 4)
    p = s.step()
    assert [x[0] for x in p.prefill] == [0, 1, 2]            # 4th needs 30, 10 free
    assert p.brake == sched.PROCEED and s.pool.num_free() == 10
    assert all(len(x[3]) == 30 for x in p.prefill)
    # next step: 3 decodes at ctx 480 need block 31 each -> 7 free (7 %): hard
    p = s.step()
    assert p.brake == sched.HARD and p.prefill == []
    assert [x[1] for x in p.decode] == [480, 480, 480]
    assert s.pool.num_free() == 7


def test_soft_brake_needs_running_decodes_and_is_strict():
    # 100 blocks. Request A: 70 blocks (1120 tokens) -> 30 free: 30 % is not
    # below 30 %, so B (1 block) is admitted in the same step.
    s = sched.Scheduler(100, max_running=8)
    s.submit(0, 1120, 10)
    s.submit(1, 16, 10)
    p = s.step()
    assert [x[0] for x in p.prefill] == [0, 1]
    # step 2: A grows to 71 blocks (ctx 1120 -> needs 71), B to 2: 27 free
    # with decodes running -> soft brake: C waits
    s.submit(2, 16, 10)
    p = s.step()
    assert s.pool.num_free() == 27
    assert p.brake == sched.SOFT and p.prefill == []
    assert [x[0] for x in p.decode] == [0, 1]


def test_hard_brake_threshold_is_strict():
    # 10 of 100 free is not below 10 %: admission proceeds when decodes are
    # idle; at 9 free it is a hard brake.
    s = sched.Scheduler(100, max_running=8)
    s.submit(0, 90 * 16, 3)
    s.submit(1, 16, 3)
    p = s.step()
    assert [x[0] for x in p.prefill] == [0, 1] and s.pool.num_free() == 9
    s.submit(2, 16, 3)
    p = s.step()                               # growth: ctx 1440 -> 91 blocks, 8 free
    assert p.brake == sched.HARD and p.prefill == []


def test_block_counts_follow_ceil_of_tokens():
    s = sched.Scheduler(64, max_running=4)
    s.submit(0, 17, 40)
    p = s.step()
    assert len(p.prefill[0][3]) == paged.blocks_needed(17, 16) == 2
    for step in range(40):
        p = s.step()
        if not p.decode:
            break
        rid, ctx, blocks = p.decode[0]
        assert len(blocks) == paged.blocks_needed(ctx + 1, 16)


def test_recompute_preemption_takes_the_latest_admitted():
    # 8 blocks. A (prompt 48 = 3 blocks) and B (prompt 64 = 4 blocks): 1 free.
    s = sched.Scheduler(8, max_running=4, hard=0.0, soft=0.0)
    s.submit(0, 48, 40)
    s.submit(1, 64, 40)
    p = s.step()
    assert [x[0] for x in p.prefill] == [0, 1] and s.pool.num_free() == 1
    # A at ctx 48 needs a 4th block (takes the last free one); B at ctx 64 needs
    # a 5th: pool empty -> B (latest) is preempted and re-queued
    p = s.step()
    assert p.preempted == [1] and [x[0] for x in p.decode] == [0]
    assert s.waiting[0].rid == 1 and s.waiting[0].prompt == 65 and s.waiting[0].max_new == 39
    _tables_disjoint_and_complete(s)


def test_fifo_recompute_preemption_takes_the_earliest_admitted():
    # The same pool as above under FIFO eviction. Step 2: A (entered first)
    # takes the last free block for position 48; B at ctx 64 needs a 5th: the
    # pool is empty, so A is preempted (its 4 blocks return), and B retries
    # and gets one of them.
    s = sched.Scheduler(8, max_running=4, hard=0.0, soft=0.0, evict=sched.EVICT_FIFO)
    s.submit(0, 48, 40)
    s.submit(1, 64, 40)
    s.step()
    p = s.step()
    assert p.preempted == [0] and [x[0] for x in p.decode] == [1]
    assert p.decode[0][1] == 64 and len(p.decode[0][2]) == 5
    assert s.waiting[0].rid == 0 and s.waiting[0].prompt == 49 and s.waiting[0].max_new == 39
    assert s.pool.num_free() == 3
    _tables_disjoint_and_complete(s)


def test_fifo_swap_out_moves_the_earliest_admitted():
    # Blocks come off the LIFO free stack 0, 1, 2, ...: A holds 0-2, B 3-6; at
    # step 2 A takes 7 for position 48, B needs a 5th block: A (first in) goes
    # to host slots 0-3 in block order; its blocks return in that order, so
    # B's 5th block is 7 (the last one pushed).
    s = sched.Scheduler(8, max_running=4, hard=0.0, soft=0.0, host_slots=16,
                        evict=sched.EVICT_FIFO)
    s.submit(0, 48, 6)
    s.submit(1, 64, 40)
    s.step()
    p = s.step()
    assert p.swapped_out == [0] and p.preempted == []
    assert p.swap_out == [(0, 0), (1, 1), (2, 2), (7, 3)]
    assert [(x[0], x[1], x[2]) for x in p.decode] == [(1, 64, [3, 4, 5, 6, 7])]
    # A (ctx 48, 4 host blocks) needs 4 device blocks to come back: with 3
    # free it waits while B decodes; B retires after 39 decodes at 7 blocks
    # (positions up to 103), then A returns in the same step with its old context
    while True:
        p = s.step()
        if p.swap_in:
            break
        assert [x[0] for x in p.decode] == [1]
    assert p.finished == [1] and [x[0] for x in p.swap_in] == [0, 1, 2, 3]
    assert [(x[0], x[1]) for x in p.decode] == [(0, 48)]


def test_lru_gives_the_fifo_plans():
    """Every running request is read at every step, so the least recently used
    one is the one holding its blocks longest: the FIFO victim. Same random
    streams (with host swap space) under both names, plan for plan."""
    for seed in range(4):
        plans = []
        for evict in (sched.EVICT_FIFO, sched.EVICT_LRU):
            rng = np.random.default_rng(90 + seed)
            N = int(rng.integers(16, 60))
            s = sched.Scheduler(N, max_running=int(rng.integers(2, 6)), hard=0.02, soft=0.05,
                                host_slots=int(rng.integers(0, 40)), evict=evict)
            out = []
            rid = 0
            for t in range(1500):
                if rid < 30 and rng.random() < 0.3:
                    prompt, new = int(rng.integers(1, 200)), int(rng.integers(1, 80))
                    if paged.blocks_needed(prompt + new, 16) <= N:
                        s.submit(rid, prompt, new)
                        rid += 1
                out.append(s.step())
            plans.append(out)
        assert plans[0] == plans[1]


def test_unknown_eviction_policy_is_refused():
    with pytest.raises(ValueError):
        sched.Scheduler(8, evict=3)


@pytest.mark.parametrize("evict", [sched.EVICT_LIFO, sched.EVICT_FIFO])
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_streams_keep_invariants_and_finish(seed, evict):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(40, 200))
    s = sched.Scheduler(N, max_running=int(rng.integers(2, 9)), evict=evict)
    produced = {}
    want = {}
    rid = 0
    for t in range(4000):
        if rid < 60 and rng.random() < 0.3:
            prompt, new = int(rng.integers(1, 300)), int(rng.integers(1, 60))
            if paged.blocks_needed(prompt + new, 16) <= N:
                s.submit(rid, prompt, new)
                want[rid] = new
                rid += 1
        p = s.step()
        for x in p.prefill + p.decode:
            produced[x[0]] = produced.get(x[0], 0) + 1
        _tables_disjoint_and_complete(s)
        if rid >= 60 and s.idle():
            break
    assert s.idle() and s.pool.num_free() == N
    assert produced == want                       # every request made exactly its tokens


# ------------------------------------------------------------ KV offload
def test_swap_preemption_keeps_context_and_resumes_first():
    s = sched.Scheduler(8, max_running=4, hard=0.0, soft=0.0, host_slots=16)
    s.submit(0, 48, 6)
    s.submit(1, 64, 40)
    s.step()
    p = s.step()
    # B (latest) swapped out: its 4 blocks to host slots 0..3 in block order
    assert p.swapped_out == [1] and p.preempted == []
    assert p.swap_out == [(3, 0), (4, 1), (5, 2), (6, 3)]
    assert [x[0] for x in p.decode] == [0]
    s.submit(2, 16, 3)                       # a new request must not overtake B
    while True:
        p = s.step()
        if p.swap_in:
            break
        assert p.prefill == []
    # A finished: B comes back with its 4 blocks + the block for position 64,
    # decodes at its old context, then C is admitted behind it
    assert [x[0] for x in p.swap_in] == [0, 1, 2, 3]
    dec = {x[0]: x for x in p.decode}
    assert dec[1][1] == 64 and len(dec[1][2]) == 5
    assert [x[0] for x in p.prefill] == [2]


def test_small_host_space_falls_back_to_recompute():
    s = sched.Scheduler(8, max_running=4, hard=0.0, soft=0.0, host_slots=3)
    s.submit(0, 48, 40)
    s.submit(1, 64, 40)
    s.step()
    p = s.step()
    assert p.swapped_out == [] and p.preempted == [1]


@pytest.mark.parametrize("evict", [sched.EVICT_LIFO, sched.EVICT_FIFO])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_swap_streams_preserve_every_block_content(seed, evict):
    """Tag every logical block (request, index) as it is written, move tags with
    the plan's swap-out / swap-in pairs, and check that every running request
    reads its own tags in order after every step."""
    rng = np.random.default_rng(50 + seed)
    N = int(rng.integers(16, 60))
    s = sched.Scheduler(N, max_running=int(rng.integers(2, 6)), hard=0.0, soft=0.0,
                        host_slots=int(rng.integers(8, 40)), evict=evict)
    dev, host = {}, {}
    want, produced = {}, {}
    rid = 0
    for t in range(3000):
        if rid < 40 and rng.random() < 0.3:
            prompt, new = int(rng.integers(1, 200)), int(rng.integers(1, 80))
            if paged.blocks_needed(prompt + new, 16) <= N:
                s.submit(rid, prompt, new)
                want[rid] = new
                rid += 1
        p = s.step()
        for d, h in p.swap_out:
            host[h] = dev.pop(d)
        for h, d in p.swap_in:
            dev[d] = host.pop(h)
        for r_id, ctx, n, blocks in p.prefill:          # prompt writes blocks 0..
            for j in range(paged.blocks_needed(n, 16)):
                dev[blocks[j]] = (r_id, j)
        for r_id, ctx, blocks in p.decode:              # decode writes block ctx // 16
            j = ctx // 16
            if ctx % 16 == 0:
                dev[blocks[j]] = (r_id, j)
            for i in range(j + 1):
                assert dev[blocks[i]] == (r_id, i)
        for x in p.prefill + p.decode:
            produced[x[0]] = produced.get(x[0], 0) + 1
        if rid >= 40 and s.idle():
            break
    assert s.idle() and s.pool.num_free() == N and s.host.num_free() == s.host.num_blocks
    assert produced == want
