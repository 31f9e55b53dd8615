"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
as two calls (mi_write_decode_kv + mi_paged_gqa_decode) and as one launch
(mi_paged_gqa_decode_step). Each replay runs on new query values written
into the captured buffers, with eager steps and synchronisations between
replays, and must equal, bit for bit, the same step run eagerly on a second
copy of the inputs (needs an MI355X)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_246_amd as mk
import workloads
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
@pytest.mark.parametrize("name", ["qwen3_1p7b", "qwen2p5_7b_b8"])
def test_decode_step_graph_replays(name, one_launch):
    print("graph", name, "one launch" if one_launch else "two calls", flush=True)
    case = workloads.make_decode_case(workloads.CONFIGS[name], pool="poison")
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
