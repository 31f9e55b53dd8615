"""Benchmark of the paged-KV GQA decode step on one MI355X.

A step is one pass of the hot path over one batch: write_decode_kv (RoPE,
append) then paged GQA decode attention, on the Qwen3-8B-shaped long-context
workload (batch 32, 32 query / 8 KV heads, head_dim 128, 16-token blocks,
contexts log-uniform in [1024, 16384], 40000-block pool). Inputs are seeded
synthetic bf16 N(0, 1) draws, resident in HBM before timing starts. The full
decoder-layer step (Qwen3-8B-shaped, batch 8) is timed in the same run and
reported as layer-step tokens/s.

Prints ONE JSON line. `value` = algorithmic bytes of the step / step time.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
METRIC = "paged GQA decode attention: KV GB/s & % HBM peak; layer-step tokens/s"


def recorded_traffic():
    """HBM bytes per attention launch from the committed counter summary, if it
    was taken on the current kernel source (else None)."""
    import hashlib
    src = os.path.join(ROOT, "paged_kv_cache_246_amd", "csrc", "attention.hip")
    summ = os.path.join(ROOT, "profiles", "attention_qwen3_8b_long_hbm_counters.md")
    try:
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        fields = dict(ln.split(": ", 1) for ln in open(summ).read().splitlines() if ": " in ln)
        if fields.get("source_sha256_prefix", "").strip() == sha:
            return int(fields["traffic_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        pass
    return None


def _dev(a, torch, dev):
    if a.dtype == np.uint8:                    # E4M3 codes of an 8-bit cache
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)


FLUSH_BYTES = 512 << 20          # > the 256 MB last-level cache and the L2s
FLUSHED_REPS = 20


def _pct(xs):
    return {"p10": round(float(np.percentile(xs, 10)), 5),
            "p50": round(float(np.percentile(xs, 50)), 5),
            "p90": round(float(np.percentile(xs, 90)), 5)}


def time_step(torch, stream, fn, steps, warmup, flush=None):
    """Warm: `warmup` untimed calls, then `steps` back-to-back calls with one
    HIP event pair (on `stream`) around all of them: ms_per_step = total /
    steps; then `steps` more calls with an event pair around each, for the
    p10/p50/p90 of single calls (kept apart so that the per-call event
    packets do not enter the back-to-back figure).
    Flushed (if `flush`, a device buffer of FLUSH_BYTES, is given): the median
    (and p10/p90) of FLUSHED_REPS single calls, each after an untimed fill of
    the buffer on the same stream, which evicts the L2s and the last-level
    cache."""
    E = lambda: torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):         # graph replays launch on the current stream
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = E(), E()
        t0.record(stream)
        for _ in range(steps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        evs = [(E(), E()) for _ in range(steps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) for a, b in evs]
        res = {"ms_per_step": round(t0.elapsed_time(t1) / steps, 5), "warm_ms": _pct(per)}
        if flush is not None:
            cold = []
            for i in range(FLUSHED_REPS):
                flush.fill_(i & 255)
                a, b = E(), E()
                a.record(stream)
                fn()
                b.record(stream)
                torch.cuda.synchronize()
                cold.append(a.elapsed_time(b))
            res["flushed_ms"] = _pct(cold)
    return res


def graph_of(torch, fn, reps):
    """A HIP graph (torch.cuda.CUDAGraph) holding `reps` calls of fn, captured
    on a side stream after one eager call there; returns (graph, stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(reps):
            fn(side)
    torch.cuda.synchronize()
    return g, side


CALIB_BLOCKS = 4096     # cache blocks (65,536 tokens) the 8-bit scales are calibrated on


def run_attention_bench(args, torch, mk, workloads, kv_format="bf16", dot=False):
    """The long-context decode step (write + attention) over a bf16 cache or an
    8-bit (E4M3) cache of the same workload. The 8-bit cache is the bf16 one
    quantised under per-head scales calibrated on its first CALIB_BLOCKS blocks
    (mi_kv_pool_calibrate_scales, margin 1), and the step's output is compared
    with the same step over the bf16 cache. dot: the pool takes
    MI_POOL_DECODE_DOT (the attention on vector-ALU dot products); the
    one-launch and flushed forms are then left out."""
    dev = "cuda:0"
    cfg = workloads.CONFIGS["qwen3_8b_long"]
    case = workloads.make_decode_case(cfg, pool="bench", kv_format="bf16")
    fp8 = kv_format == "fp8"
    kv_elem = 1 if fp8 else 2
    B, Hq, Hkv, D = len(case.context_lens), cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    kp16, vp16 = _dev(case.k_pool, torch, dev), _dev(case.v_pool, torch, dev)
    q, k, v = _dev(case.q, torch, dev), _dev(case.k, torch, dev), _dev(case.v, torch, dev)
    q_rot, out = torch.empty_like(q), torch.empty_like(q)
    table = torch.from_numpy(case.block_table).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    mbps, max_ctx = case.block_table.shape[1], int(case.context_lens.max())
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream
    out16, calib = None, None
    if fp8:
        # the same step over the bf16 cache, for the 8-bit output's error
        out16 = torch.empty_like(q)
        p16 = mk.mi_kv_pool_init(case.num_blocks, 16, Hkv, D, kp16, vp16)
        try:
            w16 = mk.mi_paged_gqa_decode_workspace_bytes(p16, B, Hq, max_ctx)
            ws16 = torch.empty(w16, dtype=torch.uint8, device=dev)
            mk.mi_write_decode_kv(p16, q, k, v, q_rot, table, mbps, ctx, B, Hq, cfg.rope_theta, st)
            mk.mi_paged_gqa_decode(p16, q_rot, out16, table, mbps, ctx, B, Hq, 0.0, max_ctx, ws16, w16, st)
            torch.cuda.synchronize()
        finally:
            mk.mi_kv_pool_destroy(p16)
        kp = torch.zeros(kp16.shape, dtype=torch.uint8, device=dev)
        vp = torch.zeros_like(kp)
    else:
        kp, vp = kp16, vp16
    flags = (mk.MI_POOL_KV_FP8 if fp8 else 0) | (mk.MI_POOL_DECODE_DOT if dot else 0)
    pool = mk.mi_kv_pool_init(case.num_blocks, 16, Hkv, D, kp, vp, flags=flags)
    if fp8:
        nb = min(case.num_blocks, CALIB_BLOCKS)
        rows_k = kp16[:nb].permute(0, 2, 1, 3).reshape(nb * 16, Hkv, D).contiguous()
        rows_v = vp16[:nb].permute(0, 2, 1, 3).reshape(nb * 16, Hkv, D).contiguous()
        mk.mi_kv_pool_calibrate_scales(pool, rows_k, rows_v, nb * 16, 1.0, st)
        mk.mi_kv_pool_quantize(pool, kp16, vp16, st)
        torch.cuda.synchronize()
        ks, vs = mk.mi_kv_pool_get_scales(pool)
        calib = {"sample_tokens": nb * 16, "k_scales": [round(min(ks), 6), round(max(ks), 6)],
                 "v_scales": [round(min(vs), 6), round(max(vs), 6)]}
        del rows_k, rows_v, kp16, vp16
    ws_bytes = mk.mi_paged_gqa_decode_split_workspace_bytes(pool, B, Hq, max_ctx, args.split)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step(ev=None):
        mk.mi_write_decode_kv(pool, q, k, v, q_rot, table, mbps, ctx, B, Hq, cfg.rope_theta, st)
        if ev is not None:
            ev[0].record(stream)
        mk.mi_paged_gqa_decode_split(pool, q_rot, out, table, mbps, ctx, B, Hq, 0.0, max_ctx,
                                     args.split, ws, ws_bytes, st)
        if ev is not None:
            ev[1].record(stream)

    # Back-to-back steps with one event pair around all of them (the step
    # rate), then as many steps again with an event pair around each
    # attention call (its launch times; kept apart so that the event packets
    # do not enter the step rate).
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    attn_ms = [a.elapsed_time(b) for a, b in evs]

    # The same step as one launch (mi_paged_gqa_decode_step), timed alike.
    ms_one = None
    if not args.split and not dot:
        ws1_bytes = mk.mi_paged_gqa_decode_workspace_bytes(pool, B, Hq, max_ctx)
        ws1 = torch.empty(ws1_bytes, dtype=torch.uint8, device=dev)

        def one():
            mk.mi_paged_gqa_decode_step(pool, q, k, v, q_rot, out, table, mbps, ctx, B, Hq,
                                        cfg.rope_theta, 0.0, max_ctx, ws1, ws1_bytes, st)

        for _ in range(args.warmup):
            one()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(args.steps):
            one()
        t1.record(stream)
        torch.cuda.synchronize()
        ms_one = t0.elapsed_time(t1) / args.steps
    # The two calls replayed from a HIP graph of 20 captured steps, the way a
    # serving loop launches its decode steps.
    ms_graph = None
    if not dot:
        def step_on(s):
            mk.mi_write_decode_kv(pool, q, k, v, q_rot, table, mbps, ctx, B, Hq, cfg.rope_theta,
                                  s.cuda_stream)
            mk.mi_paged_gqa_decode_split(pool, q_rot, out, table, mbps, ctx, B, Hq, 0.0, max_ctx,
                                         args.split, ws, ws_bytes, s.cuda_stream)

        g, side = graph_of(torch, step_on, 20)
        tg = time_step(torch, side, g.replay, max(3, args.steps // 20), 2)
        ms_graph = tg["ms_per_step"] / 20
        del g
    # Flushed: single steps (write + attention), each after a fill that evicts
    # the caches; the attention launch is timed on its own inside the step.
    flushed = None
    if not args.no_flushed and not dot:
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        cold_step, cold_attn = [], []
        for i in range(FLUSHED_REPS):
            flush.fill_(i & 255)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            a.record(stream)
            step(ev)
            b.record(stream)
            torch.cuda.synchronize()
            cold_step.append(a.elapsed_time(b))
            cold_attn.append(ev[0].elapsed_time(ev[1]))
        del flush
        flushed = {"step_ms": _pct(cold_step), "attention_ms": _pct(cold_attn)}
    faults = mk.mi_kv_pool_check_errors(pool)
    mk.mi_kv_pool_destroy(pool)
    if faults:
        raise RuntimeError("device fault bits %#x during the benchmark" % faults)
    vs_bf16 = None
    if out16 is not None:
        a = out.view(torch.bfloat16).float()
        b = out16.view(torch.bfloat16).float()
        vs_bf16 = {"max_abs": round(float((a - b).abs().max()), 5),
                   "rel_l2": round(float((a - b).norm() / b.norm()), 5)}

    ctx_np = case.context_lens
    attn_bytes = workloads.attention_bytes(ctx_np, Hq, Hkv, D, 16, kv_elem_bytes=kv_elem)
    write_bytes = workloads.write_bytes(B, Hq, Hkv, D, kv_elem_bytes=kv_elem)
    return dict(
        case=case, cfg=cfg, ms_step=ms_step, ms_one=ms_one, ms_graph=ms_graph, wall=wall, attn_ms=attn_ms,
        flushed=flushed,
        attn_bytes=attn_bytes, step_bytes=attn_bytes + write_bytes,
        tokens=int(ctx_np.sum()) + B,
        split=args.split or None,
        calib=calib, vs_bf16=vs_bf16,
    )


def run_dot_compare(args, torch, mk, workloads):
    """The long-context step's attention in its two forms, bf16 and 8-bit
    caches: the matrix-core kernel (default) against the dot-product kernel
    (MI_POOL_DECODE_DOT), mean launch time and algorithmic GB/s of each."""
    res = {"workload": "qwen3-8b-shaped long-context decode attention (mi_paged_gqa_decode)"}
    for fmt in ("bf16", "fp8"):
        row = {}
        for name, dot in (("mfma", False), ("dot", True)):
            r = run_attention_bench(args, torch, mk, workloads, kv_format=fmt, dot=dot)
            ms = float(np.mean(r["attn_ms"]))
            row[name] = {"attention_avg_launch_ms": round(ms, 5),
                         "GBps": round(r["attn_bytes"] / (ms * 1e-3) / 1e9, 1),
                         "hbm_frac": round(r["attn_bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        row["dot_over_mfma_time"] = round(row["dot"]["attention_avg_launch_ms"]
                                          / row["mfma"]["attention_avg_launch_ms"], 3)
        res[fmt] = row
    return res


def run_prefill_bench(args, torch, mk, workloads, cached=False):
    """Prefill chunk on a Qwen3-8B-shaped layer: 4 prompts of 2048 new tokens
    (packed, 8192 rows): mi_write_prefill_kv + mi_paged_prefill_attention.
    Fresh prompts, or (cached) chunks after 4000/6000/2000/8000 cached tokens
    (chunked prefill). The causal attention is a dense contraction: reported
    against the bf16 MFMA peak."""
    dev = "cuda:0"
    cfg = workloads.PREFILL_CONFIGS["qwen3_8b_prefill"][0]
    ctx_l = (4000, 6000, 2000, 8000) if cached else (0, 0, 0, 0)
    new_l = (2048, 2048, 2048, 2048)
    case = workloads.make_prefill_case(cfg, ctx_l, new_l, pool="bench")
    B, T = len(ctx_l), int(case.cu_seqlens[-1])
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    kp, vp = _dev(case.k_pool, torch, dev), _dev(case.v_pool, torch, dev)
    q, k, v = _dev(case.q, torch, dev), _dev(case.k, torch, dev), _dev(case.v, torch, dev)
    q_rot, out = torch.empty_like(q), torch.empty_like(q)
    table = torch.from_numpy(case.block_table).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    cu = torch.from_numpy(case.cu_seqlens).to(dev)
    mbps, max_new = case.block_table.shape[1], int(case.new_lens.max())
    pool = mk.mi_kv_pool_init(case.num_blocks, 16, Hkv, D, kp, vp)
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream

    def write():
        mk.mi_write_prefill_kv(pool, q, k, v, q_rot, table, mbps, ctx, cu, B, T, Hq,
                               cfg.rope_theta, st)

    def attention():
        mk.mi_paged_prefill_attention(pool, q_rot, out, table, mbps, ctx, cu, B, T, max_new, Hq,
                                      0.0, st)

    def step():
        write()
        attention()

    # The step (write + attention) back to back; then the attention alone:
    # back to back under one event pair (its average launch duration, the
    # roofline's) and with an event pair per call (percentiles). The calls
    # repeat the same work on the same inputs.
    steps = max(1, args.steps // 5)
    warm = max(1, args.warmup // 2)
    t_step = time_step(torch, stream, step, steps, warm)
    t_attn = time_step(torch, stream, attention, steps, warm)
    t_write = time_step(torch, stream, write, steps, warm)
    ms = t_step["ms_per_step"]
    attn_ms = t_attn["ms_per_step"]
    faults = mk.mi_kv_pool_check_errors(pool)
    mk.mi_kv_pool_destroy(pool)
    if faults:
        raise RuntimeError("device fault bits %#x during the prefill benchmark" % faults)
    flops = workloads.prefill_flops(case.context_lens, case.new_lens, Hq, D)
    tflops = flops / (attn_ms * 1e-3) / 1e12
    return {
        "workload": ("qwen3-8b-shaped prefill, 4 chunks x 2048 tokens after 4000/6000/2000/8000 "
                     "cached tokens (32/8 heads, D 128)" if cached else
                     "qwen3-8b-shaped prefill, 4 fresh prompts x 2048 tokens (32/8 heads, D 128)"),
        "steps": steps,
        "ms_per_step": round(ms, 5),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "attention_avg_launch_ms": round(attn_ms, 5),
        "attention_per_call_ms": t_attn["warm_ms"],
        "write_avg_launch_ms": t_write["ms_per_step"],
        "attention_flops": int(flops),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4)},
    }


def run_offload_bench(args, torch, mk, workloads):
    """KV offload path: 2048 blocks of a Qwen3-8B-shaped pool (8 KV heads,
    D 128: 32 KiB per block per cache, 128 MiB in all) swapped out to
    page-locked host memory and back, once as one run of consecutive blocks
    and slots and once as scattered pairs (a shuffled block table). PCIe GB/s
    per direction, K and V bytes."""
    dev = "cuda:0"
    N, Hkv, D, n = 4096, 8, 128, 2048
    kd = torch.zeros((N, Hkv, 16, D), dtype=torch.int16, device=dev)
    vd = torch.zeros_like(kd)
    hk = torch.zeros((n, Hkv, 16, D), dtype=torch.int16, pin_memory=True)
    hv = torch.zeros_like(hk)
    pool = mk.mi_kv_pool_init(N, 16, Hkv, D, kd, vd, flags=mk.MI_POOL_SWAP_STAGING)
    rng = np.random.default_rng(7)
    res = {}
    nbytes = 2 * n * Hkv * 16 * D * 2
    try:
        for name, ids in (("contiguous", np.arange(n, dtype=np.int32)),
                          ("scattered", rng.permutation(N)[:n].astype(np.int32))):
            out_pairs = np.stack([ids, np.arange(n, dtype=np.int32)], 1)
            in_pairs = np.stack([np.arange(n, dtype=np.int32), ids], 1)
            for _ in range(2):
                mk.mi_kv_swap_out(pool, hk, hv, n, out_pairs)
                mk.mi_kv_swap_in(pool, hk, hv, n, in_pairs)
            torch.cuda.synchronize()
            times = {}
            for label, fn, pairs in (("out", mk.mi_kv_swap_out, out_pairs),
                                     ("in", mk.mi_kv_swap_in, in_pairs)):
                t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 5
                t0.record()
                for _ in range(reps):
                    fn(pool, hk, hv, n, pairs)
                t1.record()
                torch.cuda.synchronize()
                times[label] = t0.elapsed_time(t1) / reps
            res[name] = {"swap_out_ms": round(times["out"], 3), "swap_in_ms": round(times["in"], 3),
                         "swap_out_GBps": round(nbytes / (times["out"] * 1e-3) / 1e9, 1),
                         "swap_in_GBps": round(nbytes / (times["in"] * 1e-3) / 1e9, 1)}
    finally:
        mk.mi_kv_pool_destroy(pool)
    res["bytes_per_direction"] = nbytes
    return res


def run_serving_offload_bench(args, torch, mk, evict):
    """KV offload as a second workload (the course project's optional task: long
    contexts, prompts >= 4K and >= 1K generated tokens; report decode tokens/s
    and peak memory): the library's step planner serving 16 requests with
    prompts U[4096, 8192] and U[1024, 1280] new tokens (seed 9) on a
    Qwen3-8B-shaped cache (32/8 heads, D 128) of 2048 blocks (128 MiB of K
    and V, far below the requests' demand), 8 running at most, tight KV
    brakes (2 % / 5 %), a 4096-slot page-locked host swap space and the given
    eviction policy, so decode growth forces swap-outs and later swap-ins.
    Every step runs the plan through the C ABI: swaps, then prefill rows
    (write + causal attention), then decode rows (write + attention); q, k, v
    are fresh N(0, 1) draws on the device. GPU time per phase from HIP
    events, planner host time per step, peak device memory (device memory in
    use from hipMemGetInfo, sampled every 8 steps) and the peak KV held on
    the device and in all."""
    import time
    dev = "cuda:0"
    N, Hq, Hkv, D, theta, R, S = 2048, 32, 8, 128, 1e6, 8, 4096
    mbps = (8192 + 1280 + 15) // 16 + 1
    rng = np.random.default_rng(9)
    reqs = [(i, int(rng.integers(4096, 8193)), int(rng.integers(1024, 1281))) for i in range(16)]
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free0, total = torch.cuda.mem_get_info()
    kd = torch.zeros((N, Hkv, 16, D), dtype=torch.int16, device=dev)
    vd = torch.zeros_like(kd)
    hk = torch.zeros((S, Hkv, 16, D), dtype=torch.int16, pin_memory=True)
    hv = torch.zeros_like(hk)
    pool = mk.mi_kv_pool_init(N, 16, Hkv, D, kd, vd, flags=mk.MI_POOL_SWAP_STAGING)
    sch = mk.Scheduler(pool, mbps, R, hard=0.02, soft=0.05, host_slots=S, evict=evict)
    ws_bytes = mk.mi_paged_gqa_decode_workspace_bytes(pool, R, Hq, mbps * 16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    rnd = lambda *shape: torch.randn(shape, dtype=torch.bfloat16, device=dev, generator=gen).view(torch.int16)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    phases = {"swap": [], "prefill": [], "decode": []}
    plan_s, steps = 0.0, 0
    tok = {"prefill": 0, "decode": 0, "swap_blocks_out": 0, "swap_blocks_in": 0}
    held = {}                                   # request -> blocks it holds (device or host)
    peak_dev_blocks, peak_all_blocks, peak_used = 0, 0, total - free0
    try:
        for rid, prompt, new in reqs:
            sch.submit(rid, prompt, new)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        while sch.num_waiting() or sch.num_running() or sch.num_swapped():
            t0 = time.perf_counter()
            plan = sch.step()
            plan_s += time.perf_counter() - t0
            steps += 1
            so, si = plan["swap_out"], plan["swap_in"]
            if len(so) or len(si):
                a, b = ev(), ev()
                a.record()
                if len(so):
                    mk.mi_kv_swap_out(pool, hk, hv, S, so)
                if len(si):
                    mk.mi_kv_swap_in(pool, hk, hv, S, si)
                b.record()
                phases["swap"].append((a, b))
                tok["swap_blocks_out"] += len(so)
                tok["swap_blocks_in"] += len(si)
            npf, ndc = plan["num_prefill"], plan["num_decode"]
            for rid in plan["finished"]:
                held.pop(int(rid), None)
            for rid in plan["preempted"]:
                held.pop(int(rid), None)
            for i in range(npf + ndc):
                held[int(plan["ids"][i])] = int((plan["block_table"][i] >= 0).sum())
            peak_dev_blocks = max(peak_dev_blocks, N - plan["free_blocks"])
            peak_all_blocks = max(peak_all_blocks, sum(held.values()))
            if npf:
                ctx = plan["context_lens"][:npf]
                n = plan["new_tokens"][:npf]
                cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
                T = int(cu[-1])
                q, k, v = rnd(T, Hq, D), rnd(T, Hkv, D), rnd(T, Hkv, D)
                qr, out = torch.empty_like(q), torch.empty_like(q)
                td = torch.from_numpy(np.ascontiguousarray(plan["block_table"][:npf])).to(dev)
                cd, cud = torch.from_numpy(ctx).to(dev), torch.from_numpy(cu).to(dev)
                a, b = ev(), ev()
                a.record()
                mk.mi_write_prefill_kv(pool, q, k, v, qr, td, mbps, cd, cud, npf, T, Hq, theta)
                mk.mi_paged_prefill_attention(pool, qr, out, td, mbps, cd, cud, npf, T, int(n.max()), Hq)
                b.record()
                phases["prefill"].append((a, b))
                tok["prefill"] += T
            if ndc:
                ctx = np.ascontiguousarray(plan["context_lens"][npf:npf + ndc])
                q, k, v = rnd(ndc, Hq, D), rnd(ndc, Hkv, D), rnd(ndc, Hkv, D)
                qr, out = torch.empty_like(q), torch.empty_like(q)
                td = torch.from_numpy(np.ascontiguousarray(plan["block_table"][npf:npf + ndc])).to(dev)
                cd = torch.from_numpy(ctx).to(dev)
                a, b = ev(), ev()
                a.record()
                mk.mi_write_decode_kv(pool, q, k, v, qr, td, mbps, cd, ndc, Hq, theta)
                mk.mi_paged_gqa_decode(pool, qr, out, td, mbps, cd, ndc, Hq, 0.0, int(ctx.max()), ws,
                                       ws_bytes)
                b.record()
                phases["decode"].append((a, b))
                tok["decode"] += ndc
            if steps % 8 == 0:
                f, _ = torch.cuda.mem_get_info()
                peak_used = max(peak_used, total - f)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        f, _ = torch.cuda.mem_get_info()
        peak_used = max(peak_used, total - f)
        faults = mk.mi_kv_pool_check_errors(pool)
    finally:
        sch.close()
        mk.mi_kv_pool_destroy(pool)
    if faults:
        raise RuntimeError("device fault bits %#x during the serving benchmark" % faults)
    ms = {k: sum(a.elapsed_time(b) for a, b in v) for k, v in phases.items()}
    block_bytes = 2 * Hkv * 16 * D * 2
    swapped = (tok["swap_blocks_out"] + tok["swap_blocks_in"]) * block_bytes
    name = {mk.MI_EVICT_LIFO: "lifo", mk.MI_EVICT_FIFO: "fifo", mk.MI_EVICT_LRU: "lru"}[evict]
    return {
        "workload": "step planner over 16 Qwen3-8B-shaped requests, prompts U[4096, 8192], "
                    "U[1024, 1280] new tokens, 2048-block pool, 8 running, brakes 2 %/5 %, "
                    "4096 host slots",
        "eviction": name,
        "steps": steps,
        "prefill_tokens": tok["prefill"], "decode_tokens": tok["decode"],
        "swap_blocks_out": tok["swap_blocks_out"], "swap_blocks_in": tok["swap_blocks_in"],
        "gpu_ms": {k: round(v, 3) for k, v in ms.items()},
        "prefill_tokens_per_s_gpu": round(tok["prefill"] / (ms["prefill"] * 1e-3), 1) if ms["prefill"] else None,
        "decode_tokens_per_s_gpu": round(tok["decode"] / (ms["decode"] * 1e-3), 1) if ms["decode"] else None,
        "decode_tokens_per_s_wall": round(tok["decode"] / wall, 1),
        "swap_GBps": round(swapped / (ms["swap"] * 1e-3) / 1e9, 2) if ms["swap"] else None,
        "planner_us_per_step": round(plan_s / steps * 1e6, 2),
        "wall_s": round(wall, 3),
        "kv_pool_bytes": N * block_bytes,
        "peak_kv_bytes_on_device": peak_dev_blocks * block_bytes,
        "peak_kv_bytes_held": peak_all_blocks * block_bytes,
        "peak_device_bytes_in_use": int(peak_used),
        "device_bytes_in_use_before": int(total - free0),
    }


def run_small_workloads(args, torch, mk, workloads):
    """Decode step on the other decode workloads: step time, algorithmic GB/s
    and fraction of the HBM peak (they are launch-latency bound). Each is
    timed in four forms -- the two calls (mi_write_decode_kv +
    mi_paged_gqa_decode) and the one-launch step (mi_paged_gqa_decode_step),
    each called eagerly and replayed from a HIP graph of 20 captured steps --
    warm (back to back) and flushed (single steps after a 512 MiB fill that
    evicts the caches; these workloads fit the 256 MB last-level cache)."""
    dev = "cuda:0"
    res = {}
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    G_REPS = 20
    for name in ["tiny", "qwen3_1p7b", "qwen2p5_7b_b1", "qwen2p5_7b_b4", "qwen2p5_7b_b8"]:
        cfg = workloads.CONFIGS[name]
        case = workloads.make_decode_case(cfg, pool="bench")
        B, Hq, Hkv, D = len(case.context_lens), cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
        kp, vp = _dev(case.k_pool, torch, dev), _dev(case.v_pool, torch, dev)
        q, k, v = _dev(case.q, torch, dev), _dev(case.k, torch, dev), _dev(case.v, torch, dev)
        q_rot, out = torch.empty_like(q), torch.empty_like(q)
        table = torch.from_numpy(case.block_table).to(dev)
        ctx = torch.from_numpy(case.context_lens).to(dev)
        mbps, max_ctx = case.block_table.shape[1], int(case.context_lens.max())
        pool = mk.mi_kv_pool_init(case.num_blocks, 16, Hkv, D, kp, vp)
        ws_bytes = mk.mi_paged_gqa_decode_workspace_bytes(pool, B, Hq, max_ctx)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream()

        def two_calls(s=stream):
            mk.mi_write_decode_kv(pool, q, k, v, q_rot, table, mbps, ctx, B, Hq, cfg.rope_theta,
                                  s.cuda_stream)
            mk.mi_paged_gqa_decode(pool, q_rot, out, table, mbps, ctx, B, Hq, 0.0, max_ctx, ws,
                                   ws_bytes, s.cuda_stream)

        def one_launch(s=stream):
            mk.mi_paged_gqa_decode_step(pool, q, k, v, q_rot, out, table, mbps, ctx, B, Hq,
                                        cfg.rope_theta, 0.0, max_ctx, ws, ws_bytes, s.cuda_stream)

        nbytes = (workloads.attention_bytes(case.context_lens, Hq, Hkv, D, 16)
                  + workloads.write_bytes(B, Hq, Hkv, D))
        entry = {"algorithmic_bytes": int(nbytes)}
        for form, fn in (("two_calls", two_calls), ("one_launch", one_launch)):
            t = time_step(torch, stream, fn, args.steps, args.warmup, flush)
            g, side = graph_of(torch, fn, G_REPS)
            g1, side1 = graph_of(torch, fn, 1)
            tg = time_step(torch, side, g.replay, max(3, args.steps // G_REPS), 2)
            tg1 = time_step(torch, side1, g1.replay, 1, 1, flush)
            ms_graph = tg["ms_per_step"] / G_REPS
            entry[form] = {
                "ms_per_step": t["ms_per_step"], "warm_ms": t["warm_ms"],
                "flushed_ms": t["flushed_ms"],
                "graph_ms_per_step": round(ms_graph, 5),
                "graph_flushed_ms": tg1["flushed_ms"],
            }
            del g, g1
        best = min(entry["two_calls"]["graph_ms_per_step"], entry["one_launch"]["graph_ms_per_step"])
        ms = entry["two_calls"]["ms_per_step"]
        entry.update({
            "ms_per_step": ms,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "tokens_per_s": round(B / (ms * 1e-3), 1),
            "best_graph_ms_per_step": round(best, 5),
            "best_graph_GBps": round(nbytes / (best * 1e-3) / 1e9, 1),
            "best_graph_hbm_frac": round(nbytes / (best * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        })
        faults = mk.mi_kv_pool_check_errors(pool)
        mk.mi_kv_pool_destroy(pool)
        if faults:
            raise RuntimeError("device fault bits %#x on %s" % (faults, name))
        res[name] = entry
    return res


def run_layer_bench(args, torch, mk, workloads):
    dev = "cuda:0"
    cfg = workloads.CONFIGS["qwen3_8b_layer"]
    case = workloads.make_decode_case(cfg, pool="bench")
    w = workloads.make_layer_weights(cfg)
    x = workloads.make_layer_input(cfg)
    B = len(case.context_lens)
    kp, vp = _dev(case.k_pool, torch, dev), _dev(case.v_pool, torch, dev)
    wd = {n: _dev(a, torch, dev) for n, a in w.items()}
    xd = _dev(x, torch, dev)
    xo = torch.empty_like(xd)
    table = torch.from_numpy(case.block_table).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    mbps, max_ctx = case.block_table.shape[1], int(case.context_lens.max())
    pool = mk.mi_kv_pool_init(case.num_blocks, 16, cfg.num_kv_heads, cfg.head_dim, kp, vp)
    lc = mk.layer_config(cfg.hidden, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                         cfg.intermediate, cfg.rms_eps, cfg.rope_theta)
    lw = mk.layer_weights(**wd)
    ws_bytes = mk.mi_decoder_layer_workspace_bytes(lc, pool, B, max_ctx)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(s=stream):
        mk.mi_decoder_layer_decode(pool, lc, lw, xd, xo, table, mbps, ctx, B, max_ctx, ws,
                                   ws_bytes, s.cuda_stream)

    flush = None if args.no_flushed else torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    t = time_step(torch, stream, step, args.steps, args.warmup, flush)
    g, side = graph_of(torch, step, 20)
    tg = time_step(torch, side, g.replay, 3, 1)
    del g, flush
    ms = t["ms_per_step"]
    faults = mk.mi_kv_pool_check_errors(pool)
    mk.mi_kv_pool_destroy(pool)
    if faults:
        raise RuntimeError("device fault bits %#x during the layer benchmark" % faults)
    nbytes = workloads.layer_bytes(cfg, case.context_lens)
    flops = workloads.layer_flops(cfg, case.context_lens)
    return {
        "workload": "qwen3-8b-shaped decoder layer, batch 8, H 4096, I 12288, ctx U[512,4096]",
        "ms_per_step": round(ms, 5),
        "tokens_per_s": round(B / (ms * 1e-3), 1),
        "algorithmic_bytes": int(nbytes),
        "achieved_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "achieved_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
        "warm_ms": t["warm_ms"],
        "flushed_ms": t.get("flushed_ms"),
        "flushed_hbm_frac": None if "flushed_ms" not in t else round(
            nbytes / (t["flushed_ms"]["p50"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "graph_ms_per_step": round(tg["ms_per_step"] / 20, 5),
    }


def run_stream_read(torch, mk):
    """Streaming-read bandwidth of the part (mi_hbm_stream_read): 1 GiB read
    by 512 workgroups of 256 threads, one contiguous chunk each, non-temporal
    16-byte loads; a 512 MiB fill between timed reads evicts the caches.
    Median of 10 reads."""
    dev = "cuda:0"
    n, wgs = 1 << 30, 512
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(3)
    sink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        mk.mi_hbm_stream_read(src, n, sink, wgs, stream.cuda_stream)
    ms = []
    for i in range(10):
        flush.fill_(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        mk.mi_hbm_stream_read(src, n, sink, wgs, stream.cuda_stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    med = float(np.median(ms))
    return {"bytes": n, "workgroups": wgs, "median_ms": round(med, 5),
            "GBps": round(n / (med * 1e-3) / 1e9, 1)}


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_threads():
    """Threads the oracle's numpy/BLAS may use: the CPUs this process may run
    on, capped by OMP_NUM_THREADS when the environment sets it (a GPU machine's
    CPU share)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(cap)) if cap.isdigit() and int(cap) > 0 else n


def _oracle_long_context(case, cfg, workloads, budget_s):
    """The oracle on the long-context workload: whole sequences (write then
    attention, each over a compact pool of its own blocks), pass after pass
    over the batch until about budget_s seconds of oracle time."""
    from oracle import attention as oatt
    B = len(case.context_lens)
    done_bytes, done_tokens, t_total, n = 0, 0, 0.0, 0
    while t_total < budget_s:
        for b in range(B):
            ctx = case.context_lens[b:b + 1]
            need = -(-(int(ctx[0]) + 1) // 16)
            ids = case.block_table[b, :need]
            kp = case.k_pool[ids]
            vp = case.v_pool[ids]
            table = np.arange(need, dtype=np.int32)[None, :]
            t0 = time.perf_counter()
            oatt.decode_step(kp, vp, case.q[b:b + 1], case.k[b:b + 1], case.v[b:b + 1], table,
                             ctx, 16, cfg.rope_theta)
            t_total += time.perf_counter() - t0
            n += 1
            done_tokens += int(ctx[0]) + 1
            done_bytes += (workloads.attention_bytes(ctx, cfg.num_q_heads, cfg.num_kv_heads,
                                                     cfg.head_dim, 16)
                           + workloads.write_bytes(1, cfg.num_q_heads, cfg.num_kv_heads,
                                                   cfg.head_dim))
            if t_total >= budget_s:
                break
    return done_bytes, t_total, n, done_tokens


def _oracle_step_seconds(fn, reps):
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_baseline(case, cfg, workloads, budget_s):
    """The fp64 oracle as it stands, timed on the host cores with
    time.perf_counter (input generation excluded), once with numpy/BLAS
    limited to N threads (threadpoolctl) and once to 1 thread:
     - the long-context workload (the line's `value`): whole sequences until
       about budget_s seconds of oracle time at each thread count;
     - the other decode workloads: the whole step, median of 5;
     - the Qwen3-8B-shaped decoder layer: the whole layer, 1 rep.
    GB/s = the same algorithmic bytes as the GPU figures / oracle time."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as oatt
    from oracle import layer as olayer

    N = _oracle_threads()
    per = {}
    head = {}
    for threads in (N, 1):
        with threadpool_limits(limits=threads):
            nbytes, t, n, tokens = _oracle_long_context(case, cfg, workloads, budget_s)
            head[threads] = (nbytes, t, n, tokens)
            for name in ["tiny", "qwen3_1p7b", "qwen2p5_7b_b1", "qwen2p5_7b_b4", "qwen2p5_7b_b8"]:
                c = workloads.CONFIGS[name]
                dc = workloads.make_decode_case(c, pool="bench")
                sec = _oracle_step_seconds(lambda: oatt.decode_step(
                    dc.k_pool, dc.v_pool, dc.q, dc.k, dc.v, dc.block_table, dc.context_lens, 16,
                    c.rope_theta), 5)
                nb = (workloads.attention_bytes(dc.context_lens, c.num_q_heads, c.num_kv_heads,
                                                c.head_dim, 16)
                      + workloads.write_bytes(len(dc.context_lens), c.num_q_heads, c.num_kv_heads,
                                              c.head_dim))
                per.setdefault(name, {})["threads_%d" % threads] = {
                    "s_per_step": round(sec, 5), "GBps": round(nb / sec / 1e9, 4)}
            lc = workloads.CONFIGS["qwen3_8b_layer"]
            lcase = workloads.make_decode_case(lc, pool="bench")
            w = workloads.make_layer_weights(lc)
            x = workloads.make_layer_input(lc)
            sec = _oracle_step_seconds(lambda: olayer.decoder_layer_decode(
                x, w, lcase.k_pool, lcase.v_pool, lcase.block_table, lcase.context_lens, 16,
                lc.num_q_heads, lc.num_kv_heads, lc.head_dim, lc.rms_eps, lc.rope_theta), 1)
            nb = workloads.layer_bytes(lc, lcase.context_lens)
            per.setdefault("qwen3_8b_layer", {})["threads_%d" % threads] = {
                "s_per_step": round(sec, 4), "GBps": round(nb / sec / 1e9, 4),
                "tokens_per_s": round(len(lcase.context_lens) / sec, 3)}
    nbytes, t, n, tokens = head[N]
    nb1, t1, _, _ = head[1]
    B = len(case.context_lens)
    per["qwen3_8b_long"] = {"threads_%d" % N: {"GBps": round(nbytes / t / 1e9, 4)},
                            "threads_1": {"GBps": round(nb1 / t1 / 1e9, 4)}}
    return {
        "value": round(nbytes / t / 1e9, 4),
        "unit": "GB/s",
        "cores": N,
        "kind": "oracle",
        "sample": "%d sequence steps (%.2f passes over the %d sequences, %d tokens, write + "
                  "attention, fp64 numpy, numpy/BLAS limited to %d threads), %.1f s"
                  % (n, n / B, B, tokens, N, t),
        "cpu_model": _cpu_model(),
        "cpus_available": len(os.sched_getaffinity(0)),
        "one_thread_value": round(nb1 / t1 / 1e9, 4),
        "per_workload": per,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--split", type=int, default=0, help="split-K tokens (0: library default)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-layer", action="store_true", help="skip the full-layer step")
    ap.add_argument("--no-small", action="store_true", help="skip the smaller decode workloads")
    ap.add_argument("--no-fp8", action="store_true", help="skip the 8-bit cache variant of the step")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill chunk")
    ap.add_argument("--no-offload", action="store_true", help="skip the KV swap measurement")
    ap.add_argument("--no-serving", action="store_true",
                    help="skip the planner-driven serving run with KV offload")
    ap.add_argument("--layer-only", action="store_true",
                    help="time only the full-layer step (for its kernel profile)")
    ap.add_argument("--small-only", action="store_true",
                    help="time only the smaller decode workloads (for their kernel profile)")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle time on the long-context workload per thread count")
    ap.add_argument("--no-flushed", action="store_true",
                    help="skip the cache-flushed timings of the long-context step and the layer")
    ap.add_argument("--no-stream-read", action="store_true",
                    help="skip the streaming-read bandwidth measurement")
    ap.add_argument("--no-dot", action="store_true",
                    help="skip the dot-product form of the attention (MI_POOL_DECODE_DOT)")
    ap.add_argument("--dot-only", action="store_true",
                    help="time only the two attention forms, bf16 and 8-bit (for their kernel profile)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill chunks (for their kernel profile)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the paged decode path is single-GPU "
              "(no collectives); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_246_amd as mk
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        # A plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it
        # scales the counters taken on the attention kernel.
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return
    mk.lib()

    if args.layer_only:
        lay = run_layer_bench(args, torch, mk, workloads)
        print(json.dumps({"metric": "layer-step tokens/s", "value": lay["tokens_per_s"],
                          "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "layer_step": lay}), flush=True)
        return

    if args.dot_only:
        print(json.dumps({"metric": "decode attention, matrix-core and dot-product forms",
                          "steps": args.steps, "warmup": args.warmup,
                          "decode_dot_form": run_dot_compare(args, torch, mk, workloads)}), flush=True)
        return

    if args.prefill_only:
        print(json.dumps({"metric": "prefill chunk attention", "steps": args.steps, "warmup": args.warmup,
                          "prefill": run_prefill_bench(args, torch, mk, workloads),
                          "prefill_cached_prefix": run_prefill_bench(args, torch, mk, workloads,
                                                                     cached=True)}), flush=True)
        return

    if args.small_only:
        print(json.dumps({"metric": "decode step time, smaller workloads", "steps": args.steps,
                          "warmup": args.warmup,
                          "other_workloads": run_small_workloads(args, torch, mk, workloads)}),
              flush=True)
        return

    r = run_attention_bench(args, torch, mk, workloads)
    ms = r["ms_step"]
    value = r["step_bytes"] / (ms * 1e-3) / 1e9
    attn_ms = float(np.mean(r["attn_ms"]))
    achieved = r["attn_bytes"] / (attn_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 N(0,1) K/V, q, k, v; no dataset)",
        "config": {
            "workload": "qwen3-8b-shaped long-context paged GQA decode step "
                        "(write_decode_kv + attention)",
            "batch": len(r["case"].context_lens),
            "num_q_heads": r["cfg"].num_q_heads,
            "num_kv_heads": r["cfg"].num_kv_heads,
            "head_dim": r["cfg"].head_dim,
            "block_size": 16,
            "context_lens": "log-uniform [1024, 16384], seed 4",
            "tokens_attended": r["tokens"],
            "pool_blocks": r["case"].num_blocks,
            "split_tokens": r["split"],
        },
        "hbm_frac": round(value / PEAK_HBM_GBPS, 4),
        "layer_step_tokens_per_s_attention_only": round(len(r["case"].context_lens) / (ms * 1e-3), 1),
        "roofline": {
            "kernel": "mi_paged_gqa_decode (attention partial kernel + combine kernel)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "avg_launch_ms": round(attn_ms, 5),
            "algorithmic_bytes": int(r["attn_bytes"]),
            "traffic": recorded_traffic(),
        },
        "decode_step_one_launch": None if r["ms_one"] is None else {
            "entry_point": "mi_paged_gqa_decode_step",
            "ms_per_step": round(r["ms_one"], 5),
            "GBps": round(r["step_bytes"] / (r["ms_one"] * 1e-3) / 1e9, 1),
        },
        "decode_step_graph": None if r["ms_graph"] is None else {
            "what": "the two calls replayed from a HIP graph of 20 captured steps",
            "ms_per_step": round(r["ms_graph"], 5),
            "GBps": round(r["step_bytes"] / (r["ms_graph"] * 1e-3) / 1e9, 1),
        },
        "attention_launch_ms": _pct(r["attn_ms"]),
    }
    if r["flushed"] is not None:
        fs, fa = r["flushed"]["step_ms"], r["flushed"]["attention_ms"]
        line["flushed"] = {
            "what": "median and p10/p90 of %d single steps, each after an untimed 512 MiB fill "
                    "that evicts the L2s and the last-level cache" % FLUSHED_REPS,
            "step_ms": fs, "attention_ms": fa,
            "step_GBps": round(r["step_bytes"] / (fs["p50"] * 1e-3) / 1e9, 1),
            "attention_GBps": round(r["attn_bytes"] / (fa["p50"] * 1e-3) / 1e9, 1),
            "attention_hbm_frac": round(r["attn_bytes"] / (fa["p50"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        }
    if not args.no_stream_read:
        sr = run_stream_read(torch, mk)
        line["hbm_stream_read"] = sr
        line["roofline"]["frac_of_stream_read"] = round(achieved / sr["GBps"], 4)
    if not args.no_fp8:
        r8 = run_attention_bench(args, torch, mk, workloads, kv_format="fp8")
        ms8 = r8["ms_step"]
        attn8 = float(np.mean(r8["attn_ms"]))
        line["kv_fp8"] = {
            "workload": ("same step over an 8-bit E4M3 cache: the bf16 cache quantised under "
                         "per-head scales calibrated on its first %d tokens" % r8["calib"]["sample_tokens"]),
            "calibrated_scales_min_max": {"k": r8["calib"]["k_scales"], "v": r8["calib"]["v_scales"]},
            "output_vs_bf16_cache": r8["vs_bf16"],
            "ms_per_step": round(ms8, 5),
            "algorithmic_bytes_per_step": int(r8["step_bytes"]),
            "GBps": round(r8["step_bytes"] / (ms8 * 1e-3) / 1e9, 1),
            "hbm_frac": round(r8["step_bytes"] / (ms8 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "attention_avg_launch_ms": round(attn8, 5),
            "attention_GBps": round(r8["attn_bytes"] / (attn8 * 1e-3) / 1e9, 1),
            "attention_hbm_frac": round(r8["attn_bytes"] / (attn8 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "step_speedup_vs_bf16": round(ms / ms8, 3),
            "one_launch_ms_per_step": None if r8["ms_one"] is None else round(r8["ms_one"], 5),
            "graph_ms_per_step": None if r8["ms_graph"] is None else round(r8["ms_graph"], 5),
        }
    if not args.no_dot:
        line["decode_dot_form"] = run_dot_compare(args, torch, mk, workloads)
    if not args.no_prefill:
        line["prefill"] = run_prefill_bench(args, torch, mk, workloads)
        line["prefill_cached_prefix"] = run_prefill_bench(args, torch, mk, workloads, cached=True)
    if not args.no_offload:
        line["kv_offload"] = run_offload_bench(args, torch, mk, workloads)
    if not args.no_serving:
        line["serving_offload"] = [run_serving_offload_bench(args, torch, mk, e)
                                   for e in (mk.MI_EVICT_LIFO, mk.MI_EVICT_FIFO)]
    if not args.no_layer:
        try:
            line["layer_step"] = run_layer_bench(args, torch, mk, workloads)
        except mk.MikvError as e:
            line["layer_step"] = {"error": str(e)}
    if not args.no_small:
        line["other_workloads"] = run_small_workloads(args, torch, mk, workloads)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(r["case"], r["cfg"], workloads, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
