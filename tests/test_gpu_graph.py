"""HIP graph capture (torch.cuda.CUDAGraph) of the decode step, as two calls
(mi_write_decode_kv + mi_paged_gqa_decode) and as one launch
(mi_paged_gqa_decode_step), of the full decoder layer and of a prefill
chunk (with and without the rescaling repeat). Each graph is captured
once and replayed several times (the decode step and the layer on new
inputs written into the captured buffers), with eager work and
synchronisations between replays; every replay must equal, bit for bit, the
same call run eagerly on a second copy of the inputs (needs an MI355X)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_246_amd as mk
import workloads
from oracle import bf16 as obf16
from tests.gpu_harness import DEV, DeviceCase, bits_to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mk.lib()       # fail loudly if the library is missing


def _make_step(dc, one_launch, stream):
    theta = dc.case.cfg.rope_theta
    ws_bytes = mk.mi_paged_gqa_decode_workspace_bytes(dc.pool, dc.B, dc.Hq, dc.max_ctx)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)

    def step():
        st = stream.cuda_stream
        if one_launch:
            mk.mi_paged_gqa_decode_step(dc.pool, dc.q, dc.k, dc.v, dc.q_rot, dc.out, dc.table,
                                        dc.mbps, dc.ctx, dc.B, dc.Hq, theta, 0.0, dc.max_ctx, ws,
                                        ws_bytes, st)
        else:
            mk.mi_write_decode_kv(dc.pool, dc.q, dc.k, dc.v, dc.q_rot, dc.table, dc.mbps, dc.ctx,
                                  dc.B, dc.Hq, theta, st)
            mk.mi_paged_gqa_decode(dc.pool, dc.q_rot, dc.out, dc.table, dc.mbps, dc.ctx, dc.B,
                                   dc.Hq, 0.0, dc.max_ctx, ws, ws_bytes, st)
    return step, ws


@pytest.mark.parametrize("one_launch", [False, True])
@pytest.mark.parametrize("name,fmt", [("qwen3_1p7b", "bf16"), ("qwen2p5_7b_b8", "bf16"),
                                      ("qwen3_1p7b", "fp8")])
def test_decode_step_graph_replays(name, fmt, one_launch):
    print("graph", name, fmt, "one launch" if one_launch else "two calls", flush=True)
    case = workloads.make_decode_case(workloads.CONFIGS[name], pool="poison", kv_format=fmt)
    rng = np.random.default_rng(11)
    qs = [rng.standard_normal(case.q.shape).astype(np.float32) for _ in range(4)]
    qs = [(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)).to(DEV) for x in qs]
    eager, graphed = DeviceCase(case), DeviceCase(case)
    try:
        side = torch.cuda.Stream()
        step_e, ws_e = _make_step(eager, one_launch, torch.cuda.current_stream())
        step_g, ws_g = _make_step(graphed, one_launch, side)
        with torch.cuda.stream(side):
            step_g()                                # first call outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step_g()
        torch.cuda.synchronize()
        for i, qi in enumerate(qs):
            eager.q.copy_(qi)
            graphed.q.copy_(qi)
            torch.cuda.synchronize()
            step_e()                                # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(graphed.out, eager.out), "replay %d: outputs differ" % i
            assert torch.equal(graphed.q_rot, eager.q_rot), "replay %d: q_rot differs" % i
            assert torch.equal(graphed.k_pool, eager.k_pool), "replay %d: K cache differs" % i
            assert torch.equal(graphed.v_pool, eager.v_pool), "replay %d: V cache differs" % i
        assert eager.faults() == 0 and graphed.faults() == 0
        del g
    finally:
        eager.close()
        graphed.close()


@pytest.mark.parametrize("one_launch", [False, True])
def test_decode_step_graph_replays_with_growing_contexts(one_launch):
    """The serving use of a captured step: the graph is captured once with a
    max_context_len that leaves room for 20 more tokens, and before each
    replay every sequence's length grows by one on the device (a new block
    id entered in its table row whenever the new token starts a block), with
    new q, k and v. Every replay equals the eager step on a second copy bit
    for bit, and the oracle's step from the pools as they were before it:
    the write (V bit-exact, K and q_rot within one ulp, nothing else moved)
    and the outputs (within tolerance)."""
    from oracle import attention as oatt
    from tests.gpu_harness import check_decode_write, check_tolerance, dev_to_bits
    steps = 20
    cfg = workloads.CONFIGS["qwen3_1p7b"]
    case = workloads.make_decode_case(cfg, pool="poison")
    B = len(case.context_lens)
    old = case.block_table
    used = set(old[old >= 0].tolist())
    free = [i for i in range(case.num_blocks) if i not in used]
    mb = max(old.shape[1], max(workloads.nblocks(c + 1 + steps, 16) for c in case.context_lens))
    case.block_table = np.full((B, mb), -1, np.int32)
    case.block_table[:, :old.shape[1]] = old
    print("graph growing contexts", "one launch" if one_launch else "two calls", flush=True)
    eager, graphed = DeviceCase(case), DeviceCase(case)
    try:
        for dc in (eager, graphed):
            dc.max_ctx = int(case.context_lens.max()) + steps
        side = torch.cuda.Stream()
        step_e, _ = _make_step(eager, one_launch, torch.cuda.current_stream())
        step_g, _ = _make_step(graphed, one_launch, side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step_g()
        torch.cuda.synchronize()
        ctx = case.context_lens.copy()
        table = case.block_table.copy()
        rng = np.random.default_rng(12)
        crossed = 0
        for i in range(steps):
            if i:
                ctx += 1                                # the previous step's token is cached
            for b in range(B):
                if ctx[b] % 16 == 0 and table[b, ctx[b] // 16] < 0:
                    table[b, ctx[b] // 16] = free.pop()
                    crossed += 1
            q = workloads.bf16_normal(rng, case.q.shape)
            k = workloads.bf16_normal(rng, case.k.shape)
            v = workloads.bf16_normal(rng, case.v.shape)
            kp0, vp0 = dev_to_bits(eager.k_pool), dev_to_bits(eager.v_pool)
            for dc in (eager, graphed):
                dc.ctx.copy_(torch.from_numpy(ctx))
                dc.table.copy_(torch.from_numpy(table))
                dc.q.copy_(bits_to_dev(q))
                dc.k.copy_(bits_to_dev(k))
                dc.v.copy_(bits_to_dev(v))
            torch.cuda.synchronize()
            step_e()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(graphed.out, eager.out), "replay %d: outputs differ" % i
            assert torch.equal(graphed.q_rot, eager.q_rot), "replay %d: q_rot differs" % i
            assert torch.equal(graphed.k_pool, eager.k_pool), "replay %d: K cache differs" % i
            assert torch.equal(graphed.v_pool, eager.v_pool), "replay %d: V cache differs" % i
            ref, kn, vn, qb = oatt.decode_step(kp0, vp0, q, k, v, table, ctx, 16, cfg.rope_theta)
            check_decode_write(workloads.DecodeCase(cfg, ctx, table, case.num_blocks, q, k, v, kp0, vp0),
                               dev_to_bits(graphed.k_pool), dev_to_bits(graphed.v_pool),
                               dev_to_bits(graphed.q_rot), kn, vn, qb)
            check_tolerance(dev_to_bits(graphed.out), ref, "replay %d" % i)
        assert crossed >= B, crossed                    # every sequence entered a new block
        assert eager.faults() == 0 and graphed.faults() == 0
        del g
    finally:
        eager.close()
        graphed.close()


LAYER = workloads.DecodeConfig(
    "graph_layer", batch=12, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
    num_blocks=256, rope_theta=1e6, ctx_draw="uniform", ctx_lo=0, ctx_hi=150, seed=21,
    hidden=768, intermediate=1536, rms_eps=1e-6)


class _LayerSetup:
    """One decoder layer over its own pool copy, callable on a given stream."""

    def __init__(self, cfg, case, w):
        self.B = len(case.context_lens)
        self.kp, self.vp = bits_to_dev(case.k_pool), bits_to_dev(case.v_pool)
        self.wd = {n: bits_to_dev(a) for n, a in w.items()}
        self.x = torch.empty((self.B, cfg.hidden), dtype=torch.int16, device=DEV)
        self.xo = torch.empty_like(self.x)
        self.table = torch.from_numpy(case.block_table).to(DEV)
        self.ctx = torch.from_numpy(case.context_lens).to(DEV)
        self.mbps, self.max_ctx = case.block_table.shape[1], int(case.context_lens.max())
        self.pool = mk.mi_kv_pool_init(case.num_blocks, 16, cfg.num_kv_heads, cfg.head_dim,
                                       self.kp, self.vp)
        self.lc = mk.layer_config(cfg.hidden, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                  cfg.intermediate, cfg.rms_eps, cfg.rope_theta)
        self.lw = mk.layer_weights(**self.wd)
        self.need = mk.mi_decoder_layer_workspace_bytes(self.lc, self.pool, self.B, self.max_ctx)
        self.ws = torch.empty(self.need, dtype=torch.uint8, device=DEV)

    def __call__(self, stream):
        mk.mi_decoder_layer_decode(self.pool, self.lc, self.lw, self.x, self.xo, self.table,
                                   self.mbps, self.ctx, self.B, self.max_ctx, self.ws, self.need,
                                   stream.cuda_stream)

    def close(self):
        if self.pool:
            mk.mi_kv_pool_destroy(self.pool)
            self.pool = None


def test_decoder_layer_graph_replays():
    """The full decoder-layer decode step captured once and replayed on four
    new hidden-state batches equals the eager layer bit for bit."""
    print("graph layer", flush=True)
    cfg = LAYER
    case = workloads.make_decode_case(cfg, pool="poison")
    w = workloads.make_layer_weights(cfg, std=0.03)
    xs = [workloads.make_layer_input(workloads.DecodeConfig(**{**cfg.__dict__, "seed": 30 + i}))
          for i in range(4)]
    eager, graphed = _LayerSetup(cfg, case, w), _LayerSetup(cfg, case, w)
    try:
        side = torch.cuda.Stream()
        graphed.x.copy_(bits_to_dev(xs[0]))
        with torch.cuda.stream(side):
            graphed(side)                               # first call outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            graphed(side)
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream()
        eager.x.copy_(bits_to_dev(xs[0]))
        eager(cur)                                      # the same first call, eagerly
        torch.cuda.synchronize()
        for i, xi in enumerate(xs):
            xdev = bits_to_dev(xi)
            eager.x.copy_(xdev)
            graphed.x.copy_(xdev)
            torch.cuda.synchronize()
            eager(cur)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(graphed.xo, eager.xo), "replay %d: outputs differ" % i
            assert torch.equal(graphed.kp, eager.kp), "replay %d: K cache differs" % i
            assert torch.equal(graphed.vp, eager.vp), "replay %d: V cache differs" % i
        assert mk.mi_kv_pool_check_errors(eager.pool) == 0
        assert mk.mi_kv_pool_check_errors(graphed.pool) == 0
        del g
    finally:
        eager.close()
        graphed.close()


def _prefill_call(dev, stream):
    st = stream.cuda_stream
    mk.mi_write_prefill_kv(dev.pool, dev.q, dev.k, dev.v, dev.q_rot, dev.table, dev.mbps, dev.ctx,
                           dev.cu, dev.B, dev.T, dev.Hq, dev.case.cfg.rope_theta, st)
    mk.mi_paged_prefill_attention(dev.pool, dev.q_rot, dev.out, dev.table, dev.mbps, dev.ctx,
                                  dev.cu, dev.B, dev.T, dev.max_new, dev.Hq, 0.0, st)


def _far_case(D):
    """Every query the same vector u, one key 30 u: later queries score far
    above their first key tile, so the attention repeats the chunk with the
    rescaling launch."""
    cfg = workloads.DecodeConfig("pf_far_graph", batch=2, num_q_heads=4, num_kv_heads=2,
                                 head_dim=D, block_size=16, num_blocks=32, rope_theta=1e4,
                                 ctx_draw="fixed", seed=50 + D)
    case = workloads.make_prefill_case(cfg, (0, 20), (100, 60))
    u = case.q[0, 0].copy()
    case.q[:] = u
    case.k[40] = obf16.encode(30.0 * obf16.decode(u))        # sequence 0, position 40
    return case


@pytest.mark.parametrize("kind", ["mixed", "far"])
def test_prefill_graph_replays(kind):
    """Prefill (KV write + causal attention) captured once and replayed three
    times, eager prefill calls between replays: every replay equals the eager
    call bit for bit, also when the chunk needs the rescaling repeat (then the
    captured call repeats on every replay)."""
    from tests.test_gpu_prefill import PrefillOnDevice
    print("graph prefill", kind, flush=True)
    if kind == "mixed":
        cfg = workloads.DecodeConfig("pf_graph", batch=3, num_q_heads=8, num_kv_heads=2,
                                     head_dim=128, block_size=16, num_blocks=64, rope_theta=1e6,
                                     ctx_draw="fixed", seed=60)
        case = workloads.make_prefill_case(cfg, (0, 37, 16), (50, 9, 33))
    else:
        case = _far_case(128)
    eager, graphed = PrefillOnDevice(case), PrefillOnDevice(case)
    try:
        side = torch.cuda.Stream()
        cur = torch.cuda.current_stream()
        _prefill_call(graphed, side)                    # first call outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            _prefill_call(graphed, side)
        torch.cuda.synchronize()
        for i in range(3):
            eager.out.fill_(0)
            graphed.out.fill_(0)
            torch.cuda.synchronize()
            _prefill_call(eager, cur)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(graphed.out, eager.out), "replay %d: outputs differ" % i
            assert torch.equal(graphed.q_rot, eager.q_rot), "replay %d: q_rot differs" % i
            assert torch.equal(graphed.k_pool, eager.k_pool), "replay %d: K cache differs" % i
            assert torch.equal(graphed.v_pool, eager.v_pool), "replay %d: V cache differs" % i
            assert bool(torch.isfinite(graphed.out.view(torch.bfloat16).float()).all())
        assert mk.mi_kv_pool_check_errors(eager.pool) == 0
        assert mk.mi_kv_pool_check_errors(graphed.pool) == 0
        del g
    finally:
        eager.close()
        graphed.close()
