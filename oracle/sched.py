"""Continuous-batching step planner over the paged KV pool: block lifecycle and
admission with the KV-protection brakes (test infrastructure only).

Pages followed:

* mini-infer README, "Project overview" and "Architecture": a scheduler keeps
  waiting and running queues; prefill runs as its own forward and the request
  then joins the batched decode steps; requests are admitted dynamically at
  every step (continuous batching); the KV cache manager hands out blocks from
  a free-block pool and each request owns a BlockTable.
* nxmr.cn inference-techniques article, section 2.1: a request of n tokens
  holds ceil(n / page_size) pages, popped from the free list.
* vLLM-based inference-framework project report, "SLO-aware, KV-cache
  protecting scheduler": before admitting a new prefill it looks at the free
  KV-cache space. Hard brake: free space below a critical threshold (10 %) ->
  no new prefill is admitted. Soft brake: decode work is running and free
  space is below a safety threshold (30 %) -> no new prefill is admitted.
  Otherwise new requests proceed.

Readings where the pages are silent (the same in the library):

* Free space = free blocks / pool blocks, measured when the admission is
  considered (after this step's decode growth and after earlier admissions
  in the same step); "below" is strict (<).
* A step: (1) retire running requests that have produced max_new_tokens and
  return their blocks; (2) give every running request the block its decode
  write needs (position ctx, i.e. ceil((ctx + 1) / 16) blocks), in arrival
  order; if the pool is empty, preempt the running request the eviction
  policy picks (below; by default the most recently admitted one): its
  blocks return to the pool; it goes back to the head of the waiting queue
  and will be prefilled again over prompt + generated tokens (vLLM's
  recompute preemption); then retry; (3) admit waiting requests in FIFO
  order while a running slot is free, no brake holds and the pool has the
  ceil(prompt / 16) blocks of the prompt; the first request that cannot be
  admitted stops admission (no overtaking); (4) emit the plan: the admitted
  prefills (context 0, n = prompt tokens) and the running decodes (context =
  tokens cached), then advance: a prefill produces the request's first token,
  a decode one more.
* The brake state reported for a step is the one the first admission check
  saw (0 proceed, 1 soft, 2 hard); with nothing waiting it is evaluated
  anyway.
* Blocks come from the pool's LIFO free stack (oracle.paged.FreeBlockStack).
* A request whose full length (prompt + max_new_tokens) needs more blocks
  than its table row or the whole pool is refused at submission.

KV offload (course project, optional task 3 "KV Cache Offloading": move
inactive KV blocks out to CPU memory and bring them back when needed, with
an eviction policy). Reading for a paged cache: the inactive blocks are those
of a preempted request. With a host swap space of S block slots (a LIFO
stack like the device pool), a preemption victim whose blocks fit the free
host slots is swapped out instead of recomputed: its device blocks are
copied to host slots (emitted as (device id, host slot) pairs, to run before
anything else in the step) and returned to the pool; it keeps its context
and generated count and joins the swapped queue. The victim is the one the
eviction policy below picks.
Swapped requests come back first, in the order they were swapped out,
regardless of the brakes (they are not new prefills), and while any request
remains swapped out no new request is admitted: a swap-in needs the request's blocks plus the block its decode
write needs; the device blocks are allocated in block order and paired with
the host slots (emitted as (host slot, device id) pairs, run after the
swap-outs), the host slots are freed, and the request decodes in this same
step after the requests already running. Without host space (or when the
victim's blocks do not fit) preemption recomputes as above.

Eviction policy (the same page: "design an eviction policy -- LRU / FIFO /
by layer / by token segment"). It picks the victim among the running
requests, for swap-out and for recompute preemption alike:

* LIFO (the default): the most recently admitted running request (vLLM's
  preemption order);
* FIFO: the running request that entered the running set first (admitted,
  or swapped back in, earliest) -- first in, first out;
* LRU: the least recently used running request. Every step reads the KV of
  every running request (each one decodes), so the last use of all of them
  is the previous step and recency cannot separate them; ties go to the one
  that has held its blocks longest, which makes LRU pick the FIFO victim.
  LRU is accepted as a name for that policy (the tests check that the two
  give identical plans).

Pinned by tests/test_oracle_sched.py against scenarios whose decisions follow
from the stated rules by hand, and by invariants (no block in two tables,
every block returned at the end).
"""
from dataclasses import dataclass, field

from . import paged

PROCEED, SOFT, HARD = 0, 1, 2
EVICT_LIFO, EVICT_FIFO, EVICT_LRU = 0, 1, 2


@dataclass
class Request:
    rid: int
    prompt: int
    max_new: int
    generated: int = 0
    ctx: int = 0                  # tokens cached
    blocks: list = field(default_factory=list)
    host_slots: list = field(default_factory=list)


@dataclass
class Plan:
    prefill: list                 # (rid, ctx, n, blocks)
    decode: list                  # (rid, ctx, blocks)
    preempted: list               # recomputed
    finished: list
    brake: int
    swapped_out: list = field(default_factory=list)   # rids
    swap_out: list = field(default_factory=list)      # (device id, host slot)
    swap_in: list = field(default_factory=list)       # (host slot, device id)


class Scheduler:
    def __init__(self, num_blocks, block_size=16, max_running=64, hard=0.10, soft=0.30,
                 max_blocks_per_seq=None, host_slots=0, evict=EVICT_LIFO):
        self.pool = paged.FreeBlockStack(num_blocks)
        self.host = paged.FreeBlockStack(host_slots) if host_slots > 0 else None
        self.swapped = []
        self.N = num_blocks
        self.bs = block_size
        self.max_running = max_running
        self.hard = hard
        self.soft = soft
        self.mbps = max_blocks_per_seq
        self.waiting = []
        self.running = []               # in the order they entered the running set
        if evict not in (EVICT_LIFO, EVICT_FIFO, EVICT_LRU):
            raise ValueError("unknown eviction policy")
        self.evict = evict

    def submit(self, rid, prompt, max_new):
        """Queue a request; refused (ValueError) if its full length could never
        fit its block-table row or the pool."""
        need = paged.blocks_needed(prompt + max_new, self.bs)
        if prompt < 1 or max_new < 1 or need > self.N or (self.mbps is not None and need > self.mbps):
            raise ValueError("request can never be scheduled")
        self.waiting.append(Request(rid, prompt, max_new))

    def _alloc(self, n):
        try:
            return self.pool.alloc(n)
        except MemoryError:
            return None

    def _free_frac(self):
        return self.pool.num_free() / self.N

    def _brake(self, decodes_running):
        f = self._free_frac()
        if f < self.hard:
            return HARD
        if decodes_running and f < self.soft:
            return SOFT
        return PROCEED

    def _victim_index(self):
        """Index in self.running (entry order) of the request to evict."""
        return len(self.running) - 1 if self.evict == EVICT_LIFO else 0

    def _release(self, r):
        self.pool.free(r.blocks)
        r.blocks = []

    def step(self):
        # (1) retire
        finished = []
        keep = []
        for r in self.running:
            if r.generated >= r.max_new:
                self._release(r)
                finished.append(r.rid)
            else:
                keep.append(r)
        self.running = keep
        # (2) decode growth, evicting a running request on exhaustion
        preempted = []
        swapped_out, swap_out = [], []
        i = 0
        while i < len(self.running):
            r = self.running[i]
            need = paged.blocks_needed(r.ctx + 1, self.bs)
            if len(r.blocks) >= need:
                i += 1
                continue
            ids = self._alloc(1)
            if ids is not None:
                r.blocks += ids
                i += 1
                continue
            vi = self._victim_index()
            victim = self.running.pop(vi)
            if self.host is not None and self.host.num_free() >= len(victim.blocks):
                slots = self.host.alloc(len(victim.blocks))
                swap_out += list(zip(victim.blocks, slots))
                self._release(victim)
                victim.host_slots = slots
                self.swapped.append(victim)
                swapped_out.append(victim.rid)
                if vi < i:
                    i -= 1
                continue
            self._release(victim)
            victim.prompt = victim.prompt + victim.generated
            victim.max_new = victim.max_new - victim.generated
            victim.generated = 0
            victim.ctx = 0
            self.waiting.insert(0, victim)
            preempted.append(victim.rid)
            # i unchanged: if the victim was r itself the loop ends; if it
            # stood before r, r moved down one place
            if vi < i:
                i -= 1
        # (3') swap-ins first, oldest swapped first, regardless of the brakes
        swap_in = []
        while self.swapped and len(self.running) < self.max_running:
            r = self.swapped[0]
            nb = len(r.host_slots)
            need = max(nb, paged.blocks_needed(r.ctx + 1, self.bs))
            ids = self._alloc(need)
            if ids is None:
                break
            self.swapped.pop(0)
            swap_in += list(zip(r.host_slots, ids[:nb]))
            self.host.free(r.host_slots)
            r.host_slots = []
            r.blocks = list(ids)
            self.running.append(r)
        # (3) admission
        decoding = len(self.running) > 0
        brake = self._brake(decoding)
        admitted = []
        while (self.waiting and not self.swapped
               and len(self.running) + len(admitted) < self.max_running):
            if self._brake(decoding) != PROCEED:
                break
            r = self.waiting[0]
            need = paged.blocks_needed(r.prompt, self.bs)
            ids = self._alloc(need)
            if ids is None:
                break
            self.waiting.pop(0)
            r.blocks = list(ids)
            admitted.append(r)
        # (4) plan, then advance
        plan = Plan(prefill=[(r.rid, 0, r.prompt, list(r.blocks)) for r in admitted],
                    decode=[(r.rid, r.ctx, list(r.blocks)) for r in self.running],
                    preempted=preempted, finished=finished, brake=brake,
                    swapped_out=swapped_out, swap_out=swap_out, swap_in=swap_in)
        for r in self.running:
            r.ctx += 1
            r.generated += 1
        for r in admitted:
            r.ctx = r.prompt
            r.generated = 1
        self.running += admitted
        return plan

    def idle(self):
        return not self.waiting and not self.running and not self.swapped
