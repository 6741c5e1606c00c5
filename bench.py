"""Benchmark: DeFT tree attention, one decode step, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--chunk-tokens C]

A step is one pass of the hot path over one synthetic batch: partial
attention (every KV chunk streamed once per KV head for its query group) and
the log-sum-exp merge, as the library's default call runs them, in one
launch (deft_tree_attention_fused: the partial work-groups and then merge
work-groups that take each (query, head) row once its partials are in),
with the plan's device image, Q and the paged KV pool already resident in
HBM.  The same step as two launches (partial kernel, then merge kernel;
deft_tree_attention, bitwise the same output) is timed beside it.  The host
planner and the plan upload (a PCIe copy) are timed separately and reported
as extra fields.

Cold caches without flushes in the timed region: the tree's KV pages are
placed R times at disjoint positions of one pool, with one block table per
copy, and consecutive steps cycle through the copies (and through R copies of
Q and of the output), so R * KV bytes (>= 512 MB) evicts the 256 MB Infinity
Cache and the L2s between reuses of a copy.

The chunk size is the library's rule (deft_plan_auto_chunk_tokens) unless
--chunk-tokens gives one; the workload's hand-tuned size is timed beside it
when they differ.  Besides the graph-timed steps: per-step latency
distributions (median, p10, p90) cold (after a 1 GiB write that evicts the
Infinity Cache and the L2s) and warm; a 1 GiB streaming-read calibration
(libdeft_bench) giving the achievable HBM bandwidth, the second roofline
fraction; the oracle on the host cores (all threads, and one thread for the
three smallest workloads).

Prints ONE JSON line.  `value` is the step latency in microseconds.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-attn latency (us) + achieved HBM GB/s, 4K prefix / 64-node tree, bf16"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
VALU_F32_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 << 20


def source_hash() -> str:
    h = hashlib.sha1()
    for f in ("deft_attention.hip", "deft_plan.cpp", "deft_internal.h"):
        with open(os.path.join(ROOT, "tree_structured_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def path_lengths(parents, seg_lens, query_nodes, query_lens=None):
    """Tokens each query attends to (its own node cut to query_lens if given)."""
    out = []
    for i, x in enumerate(query_nodes):
        t = 0 if query_lens is None else int(query_lens[i]) - int(seg_lens[x])
        while x >= 0:
            t += int(seg_lens[x])
            x = int(parents[x])
        out.append(t)
    return out


def placements(wl, copies, rng):
    """R block tables placing the tree's pages at disjoint pool positions."""
    import numpy as np
    n_lp = wl.block_table.shape[0]
    if wl.num_pages >= copies * n_lp * 4:      # a big pool: random distinct positions
        pages = rng.choice(wl.num_pages, size=copies * n_lp, replace=False).astype(np.int32)
        return wl.num_pages, [pages[r * n_lp:(r + 1) * n_lp] for r in range(copies)]
    # a pool sized to the tree: stack R copies of the generator's own placement
    base = wl.block_table.astype(np.int64)
    span = int(base.max()) + 1
    return span * copies, [(base + r * span).astype(np.int32) for r in range(copies)]


def cpu_baseline(wl, budget_s: float, threads=None):
    """The fp64 oracle on the host cores: whole workload or a query sample,
    repeated for about `budget_s` seconds; returns per-step microseconds.
    threads=1 limits the BLAS pools to one thread for the run."""
    import contextlib
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # noqa: BLE001
        threadpool_info = threadpool_limits = None
    ctx = threadpool_limits(limits=threads) if (threads and threadpool_limits) else contextlib.nullcontext()
    with ctx:
        return _cpu_baseline(wl, budget_s, threadpool_info)


def _cpu_baseline(wl, budget_s, threadpool_info):
    import numpy as np
    from oracle import attention as OA
    from tree_structured_decode_amd import workloads as W
    try:
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = 1
    ids, kp, vp = W.compact_pool(wl, poison=False)
    nq = wl.num_queries
    t0 = time.perf_counter()
    OA.tree_attention(wl.q, kp, vp, wl.block_table, wl.parents, wl.seg_lens, wl.query_nodes,
                      page_ids=ids, queries=[0], query_lens=wl.query_lens)
    one = time.perf_counter() - t0
    nsamp = int(max(1, min(nq, budget_s / max(one, 1e-6))))
    sample = list(np.linspace(0, nq - 1, nsamp).round().astype(int))
    reps, elapsed = 0, 0.0
    t0 = time.perf_counter()
    while True:
        OA.tree_attention(wl.q, kp, vp, wl.block_table, wl.parents, wl.seg_lens, wl.query_nodes,
                          page_ids=ids, queries=sample, query_lens=wl.query_lens)
        reps += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s or (nsamp < nq and reps >= 1):
            break
    per_query = elapsed / (reps * len(sample))
    return {
        "value": per_query * nq * 1e6,
        "unit": "us",
        "cores": int(blas),
        "kind": "oracle",
        "sample": (f"{len(sample)} of {nq} queries x {reps} repetitions ({elapsed:.1f} s), "
                   f"scaled to all {nq} queries; host cpu_count {os.cpu_count()}, "
                   f"affinity {len(os.sched_getaffinity(0))}, BLAS threads {blas}"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--chunk-tokens", type=int, default=0,
                    help="chunk size; 0 (default) takes the library's rule (deft_plan_auto_chunk_tokens)")
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--dist-iters", type=int, default=100,
                    help="timed iterations of the per-step latency distributions (cold and warm)")
    ap.add_argument("--profile-run", action="store_true",
                    help="eager steps only (for rocprofv3 kernel traces and counters)")
    ap.add_argument("--profile-graph", action="store_true",
                    help="with --profile-run: replay the timed graph of K steps instead")
    ap.add_argument("--profile-two-dispatch", action="store_true",
                    help="with --profile-run: eager steps as two launches (partial kernel, merge kernel)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run a plain elementwise copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the tree-attention path runs on a single GPU "
              "(it has no multi-GPU sharding); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from tree_structured_decode_amd import deft as D
    from tree_structured_decode_amd import workloads as W

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n,
                          "launches": 5}), flush=True)
        return
    pool_pages = None
    if args.workload == 5:
        pool_pages = W.hbm_pool_pages(torch.cuda.get_device_properties(0).total_memory)
    wl = W.standard_workload(args.workload, pool_pages=pool_pages)
    hand_chunk = wl.chunk_tokens            # the size tuned by hand for this workload
    if args.chunk_tokens:
        wl.chunk_tokens, chunk_rule = args.chunk_tokens, "given"
    else:
        ad = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
        wl.chunk_tokens = D.deft_plan_auto_chunk_tokens(wl.parents, wl.seg_lens, wl.query_nodes, ad,
                                                        query_lens=wl.query_lens)
        chunk_rule = "auto"
    eb = wl.k_tokens.element_size()
    T, hq, hkv, d, nq = wl.total_tokens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_queries
    kv_bytes = T * 2 * hkv * d * eb
    q_bytes = nq * hq * d * eb
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / kv_bytes))
    rng = np.random.default_rng(12345)
    n_pages, tables = placements(wl, copies, rng)

    # KV pool with R placements of the tree's tokens; everything else NaN.
    shape = (n_pages, wl.page_size, hkv, d)
    kc = torch.full(shape, float("nan"), dtype=wl.dtype, device=dev)
    vc = torch.full(shape, float("nan"), dtype=wl.dtype, device=dev)
    t_idx = np.arange(T)
    kt, vt = wl.k_tokens.to(dev), wl.v_tokens.to(dev)
    for bt in tables:
        pi = torch.from_numpy(bt[t_idx // 16].astype(np.int64)).to(dev)
        ri = torch.from_numpy((t_idx % 16).astype(np.int64)).to(dev)
        kc[pi, ri] = kt
        vc[pi, ri] = vt
    del kt, vt
    bts = [torch.from_numpy(bt).to(dev) for bt in tables]
    qs = [wl.q.to(dev).clone() for _ in range(copies)]
    outs = [torch.empty_like(qs[0]) for _ in range(copies)]

    desc = D.make_desc(wl.dtype, hq, hkv, d, n_pages)
    # host planner timing (a1-a6), then the device image (a7)
    plan_times = []
    for _ in range(20):
        t0 = time.perf_counter()
        if wl.query_lens is None:
            plan = D.deft_plan_create(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens)
        else:
            plan = D.deft_plan_create_multi_token(wl.parents, wl.seg_lens, wl.query_nodes, wl.query_lens,
                                                  wl.chunk_tokens)
        plan_times.append(time.perf_counter() - t0)
    plan_bytes, ws_bytes = D.deft_plan_device_bytes(plan, desc)
    dev_plan = torch.empty(plan_bytes, dtype=torch.uint8, device=dev)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    view = D.deft_plan_export(plan)
    S = view["num_slots"]
    # separate partial buffers for timing the two kernels alone, in the format
    # deft_tree_attention uses internally
    bf16 = wl.dtype == torch.bfloat16
    fmt = D.DEFT_PARTIAL_BF16_NORM if bf16 else D.DEFT_PARTIAL_F32
    part_o = torch.empty((S, hq, d), dtype=torch.bfloat16 if bf16 else torch.float32, device=dev)
    part_m = torch.empty((S, hq), dtype=torch.float32, device=dev)
    part_l = torch.empty((S, hq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    up0, up1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    up0.record()
    D.deft_plan_upload(plan, desc, dev_plan)
    up1.record()
    torch.cuda.synchronize()
    upload_us = up0.elapsed_time(up1) * 1e3

    def step(i, what="step"):
        """One step: the library's default call (a single dispatch: partial
        and merge work-groups in one grid), or one of its legs."""
        r = i % copies
        if what == "step":
            D.deft_tree_attention_fused(qs[r], kc, vc, bts[r], plan, outs[r], desc, workspace)
        elif what == "two":
            D.deft_tree_attention(qs[r], kc, vc, bts[r], plan, outs[r], desc, workspace)
        elif what == "partial":
            D.deft_partial_attention(qs[r], kc, vc, bts[r], plan, desc, part_o, part_m, part_l, fmt)
        else:
            D.deft_lse_merge(plan, desc, part_o, part_m, part_l, outs[r], fmt)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.profile_run:
        if args.profile_graph:
            # the timed leg as bench.py runs it: a graph of K steps over the
            # cold copies, replayed 1 + 5 times
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.graph(g, stream=s):
                for i in range(args.steps):
                    step(i)
            torch.cuda.synchronize()
            for _ in range(6):
                g.replay()
                torch.cuda.synchronize()
        else:
            for i in range(args.steps):
                step(i, "two" if args.profile_two_dispatch else "step")
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": wl.name, "chunk_tokens": wl.chunk_tokens, "steps": args.steps,
                          "copies": copies, "kv_bytes": kv_bytes, "q_bytes": q_bytes,
                          "partial_bytes": S * hq * (d * (2 if bf16 else 4) + 8), "source_hash": source_hash()}),
              flush=True)
        return
    for i in range(copies):          # an eager pass over every copy is the reference
        step(i)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]

    def capture(what, first, n):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=s):
            for i in range(first, first + n):
                step(i, what)
        torch.cuda.synchronize()
        return g

    def timed(g):
        """Replay three times to warm (caches, and the clocks after the host-side
        checks left the GPU idle), then time one replay: (wall s, event ms)."""
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1)

    g_step = capture("step", 0, args.steps)
    # every replay must reproduce the eager result (eager work between replays)
    for _ in range(2):
        for o in outs:
            o.fill_(float("nan"))
        g_step.replay()
        torch.cuda.synchronize()
        for r in range(min(copies, args.steps)):
            assert torch.equal(outs[r], eager[r]), f"graph replay differs from eager run (copy {r})"
        step(0)
        torch.cuda.synchronize()
    wall, ev_ms = timed(g_step)

    def timed_median(g, reps=5):
        """Per-kernel legs: median event time of `reps` timed replays."""
        return sorted(timed(g)[1] for _ in range(reps))[reps // 2]

    step_ms_median = timed_median(g_step)
    g_part = capture("partial", 0, args.steps)
    part_ms = timed_median(g_part)
    g_merge = capture("merge", 0, args.steps)
    merge_ms = timed_median(g_merge)
    # the partial kernel then the merge kernel (deft_tree_attention): same
    # results bit for bit, timed the same way
    g_two = capture("two", 0, args.steps)
    for o in outs:
        o.fill_(float("nan"))
    two_ms = timed_median(g_two)
    for r in range(min(copies, args.steps)):
        assert torch.equal(outs[r], eager[r]), f"two-dispatch path differs from the single dispatch (copy {r})"
    del g_two
    # the merge graph leaves outs[] holding merge-only results; restore the reference state
    for i in range(copies):
        step(i)
    torch.cuda.synchronize()
    # The same step with fp32 partials in the workspace (desc.f32_partials):
    # bf16 inputs only (fp32 inputs use fp32 partials already).
    f32p = None
    if bf16:
        desc32 = D.make_desc(wl.dtype, hq, hkv, d, n_pages, f32_partials=True)
        _, wb32 = D.deft_plan_device_bytes(plan, desc32)
        ws32 = torch.empty(wb32, dtype=torch.uint8, device=dev)
        outs32 = [torch.empty_like(o) for o in outs]

        def step32(i):
            r = i % copies
            D.deft_tree_attention_fused(qs[r], kc, vc, bts[r], plan, outs32[r], desc32, ws32)

        for i in range(copies):
            step32(i)
        torch.cuda.synchronize()
        err32 = max(float((outs32[r].float() - eager[r].float()).abs().max()) for r in range(copies))
        g32 = torch.cuda.CUDAGraph()
        s32 = torch.cuda.Stream()
        s32.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g32, stream=s32):
            for i in range(args.steps):
                step32(i)
        torch.cuda.synchronize()
        f32p = {"step_us": timed_median(g32) * 1e3 / args.steps, "max_abs_diff_vs_default": err32,
                "partial_bytes": S * hq * (d * 4 + 8)}
        del g32, ws32, outs32
    def alt_plan_leg(create):
        """Another plan of the same tree on the same kernels, inputs and
        copies, timed the same way; returns (step us, max |diff| vs DeFT)."""
        plan2 = create(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens)
        pb2, wb2 = D.deft_plan_device_bytes(plan2, desc)
        dev2 = torch.empty(max(pb2, 256), dtype=torch.uint8, device=dev)
        ws2 = torch.empty(max(wb2, 256), dtype=torch.uint8, device=dev)
        D.deft_plan_upload(plan2, desc, dev2)
        outs2 = [torch.empty_like(o) for o in outs]

        def step2(i):
            r = i % copies
            D.deft_tree_attention_fused(qs[r], kc, vc, bts[r], plan2, outs2[r], desc, ws2)

        for i in range(copies):
            step2(i)
        torch.cuda.synchronize()
        err = max(float((outs2[r].float() - eager[r].float()).abs().max()) for r in range(copies))
        g2 = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g2, stream=s2):
            for i in range(args.steps):
                step2(i)
        torch.cuda.synchronize()
        _, ms2 = timed(g2)
        del g2
        return ms2 * 1e3 / args.steps, err, D.deft_plan_export(plan2)

    # Query-centric baseline: every query streams its own root-to-node path
    # (no KV-Guided Grouping).  Node granularity: chunks never cross a node.
    # (Both take whole nodes only, so multi-token query nodes skip them.)
    alt = wl.query_lens is None
    qc_us, qc_err, _ = alt_plan_leg(D.deft_plan_create_query_centric) if alt else (None, None, None)
    nc_us, nc_err, nc_info = alt_plan_leg(D.deft_plan_create_node_chunks) if alt else (None, None, None)
    copies_saved = copies
    copies = 1                        # warm: the same copy every step, labelled as such
    g_warm = capture("step", 0, args.steps)
    _, warm_ms = timed(g_warm)
    copies = copies_saved
    del g_step, g_part, g_merge, g_warm

    # The workload's hand-tuned chunk size, timed the same way, when the
    # library's rule chose another one.
    hand_us = None
    if hand_chunk != wl.chunk_tokens:
        def hand_plan(p, s_, q_, c_):
            if wl.query_lens is None:
                return D.deft_plan_create(p, s_, q_, hand_chunk)
            return D.deft_plan_create_multi_token(p, s_, q_, wl.query_lens, hand_chunk)
        hand_us, _, _ = alt_plan_leg(hand_plan)

    # Per-step latency distributions: each step bracketed by events on the
    # launch stream, eagerly launched behind GPU work that lets the host run
    # ahead: cold = after a 1 GiB write that evicts the Infinity Cache and the
    # L2s (and the step cycles through the cold copies), warm = the same copy
    # every step behind an idle spin.
    def step_distribution(cold, n_iter, n_warm=10):
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if cold else None
        pairs = []
        for i in range(n_warm + n_iter):
            if cold:
                flush.fill_(i & 255)
            else:
                torch.cuda._sleep(200000)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step(i if cold else 0)
            e1.record()
            if i >= n_warm:
                pairs.append((e0, e1))
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
        del flush
        return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
                "p90": float(np.percentile(t, 90)), "iters": n_iter}

    lat_cold = step_distribution(True, args.dist_iters)
    lat_warm = step_distribution(False, args.dist_iters)

    # Achievable HBM read bandwidth on this device: a plain 1 GiB streaming
    # read (libdeft_bench), median of 10 timed launches.
    import ctypes
    blib = ctypes.CDLL(os.path.join(ROOT, "tree_structured_decode_amd", "libdeft_bench.so"))
    blib.deft_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    blib.deft_bench_stream_read_sink_floats.restype = ctypes.c_size_t
    cal_bytes = 1 << 30
    cal_src = torch.ones(cal_bytes // 4, dtype=torch.float32, device=dev)
    cal_sink = torch.empty(int(blib.deft_bench_stream_read_sink_floats()), dtype=torch.float32, device=dev)
    cal_stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cal_t = []
    for i in range(13):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = blib.deft_bench_stream_read(ctypes.c_void_p(cal_src.data_ptr()), cal_bytes,
                                         ctypes.c_void_p(cal_sink.data_ptr()), cal_stream)
        e1.record()
        assert rc == 0, "stream-read calibration launch failed"
        if i >= 3:
            cal_t.append((e0, e1))
    torch.cuda.synchronize()
    assert abs(float(cal_sink.double().sum()) - cal_bytes // 4) < 1.0, "stream read checksum"
    cal_gbs = cal_bytes / (float(np.median([a.elapsed_time(b) for a, b in cal_t])) * 1e-3) / 1e9
    del cal_src, cal_sink
    assert torch.isfinite(outs[0].float()).all(), "non-finite output"

    ms_per_step = wall / args.steps * 1e3
    latency_us = ms_per_step * 1e3
    paths = path_lengths(wl.parents, wl.seg_lens, wl.query_nodes, wl.query_lens)
    flops = 4.0 * d * hq * float(sum(paths))
    naive_kv = float(sum(paths)) * 2 * hkv * d * eb
    part_bytes = S * hq * (d * (2 if wl.dtype == torch.bfloat16 else 4) + 8)
    algo_step = kv_bytes + 2 * q_bytes
    mean_step = step_ms_median * 1e3 / args.steps     # a step is one launch
    mean_part = part_ms * 1e3 / args.steps
    mean_merge = merge_ms * 1e3 / args.steps
    # The step's one kernel (partial_attention with its merge work-groups):
    # KV and Q read, out written.  The bound whose time floor is larger:
    # matrix-core flops or HBM bytes.
    algo_launch = kv_bytes + 2 * q_bytes
    mfma_bound = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > algo_launch / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": flops / (mean_step * 1e-6) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": algo_launch / (mean_step * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["kernel"] = "partial_attention (single dispatch: partial and merge work-groups)"
    roof["algorithmic_bytes_per_launch"] = algo_launch
    roof["frac"] = roof["achieved"] / roof["peak"]
    if roof["unit"] == "GB/s":
        roof["frac_of_achievable"] = roof["achieved"] / cal_gbs
    roof["launch_us_mean"] = mean_step
    # the partial kernel alone, as the two-dispatch path launches it
    roof_partial = {"kernel": "partial_attention (partials only)", "launch_us_mean": mean_part,
                    "algorithmic_bytes_per_launch": kv_bytes + q_bytes,
                    "achieved_gbs": (kv_bytes + q_bytes) / (mean_part * 1e-6) / 1e9}
    roof_partial["frac"] = roof_partial["achieved_gbs"] / HBM_PEAK_GBS
    roof["traffic"] = None
    counters = os.path.join(ROOT, "profiles", "hbm_counters.json")
    if os.path.exists(counters):
        with open(counters) as f:
            cj = json.load(f)
        key = f"{wl.name}/C{wl.chunk_tokens}"
        ent = cj.get(key)
        if ent and ent.get("source_hash") == source_hash():
            roof["traffic"] = ent["bytes_per_launch"]
            roof["traffic_detail"] = ent

    line = {
        "metric": METRIC if args.workload == 2 else f"tree-attn latency (us) + achieved HBM GB/s, {wl.name}",
        "value": latency_us,
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "chunk_tokens": wl.chunk_tokens, "num_queries": nq,
            "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d, "total_tokens": T,
            "page_size": wl.page_size, "cold_copies": copies, "pool_pages": n_pages,
        },
        "achieved_hbm_gbs": algo_step / (latency_us * 1e-6) / 1e9,
        "achieved_hbm_frac": algo_step / (latency_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "queries_per_s": nq / (latency_us * 1e-6),
        "timing": ("a step is the library's default call, one launch (deft_tree_attention_fused: partial and "
                   "merge work-groups in one grid); hipGraph of the K steps, replayed three times untimed then "
                   "once timed (value, step_us_events); the legs (the single dispatch again, the partial kernel, "
                   "the merge kernel, the two-dispatch deft_tree_attention) are the median of 5 timed "
                   "replays of K launches"),
        "step_us_events": ev_ms * 1e3 / args.steps,
        "single_dispatch_step_us_median": mean_step,
        "two_dispatch_step_us": two_ms * 1e3 / args.steps,
        "partial_kernel_us_mean": mean_part,
        "merge_kernel_us_mean": mean_merge,
        "f32_partials": f32p,
        "query_centric_baseline": None if qc_us is None else {
            "step_us": qc_us,
            "kv_bytes_read_ideal": naive_kv,
            "deft_speedup": qc_us / (ev_ms * 1e3 / args.steps),
            "max_abs_diff_vs_deft": qc_err,
        },
        "node_granularity": None if nc_us is None else {
            "step_us": nc_us,
            "num_chunks": nc_info["num_chunks"],
            "deft_speedup": nc_us / (ev_ms * 1e3 / args.steps),
            "max_abs_diff_vs_deft": nc_err,
        },
        "warm_step_us": warm_ms * 1e3 / args.steps,
        "chunk_rule": chunk_rule,
        "hand_picked_chunk_tokens": hand_chunk,
        "hand_picked_step_us": hand_us,
        "step_latency_us": {
            "cold": lat_cold, "warm": lat_warm,
            "method": ("each step bracketed by HIP events on the launch stream, eager launches; cold: after a "
                       "1 GiB write evicting the Infinity Cache and the L2s; warm: the same inputs every step"),
        },
        "hbm_calibration": {"stream_read_gbs": cal_gbs, "bytes": cal_bytes, "launches": 10,
                            "kernel": "deft_bench_stream_read (libdeft_bench.so)"},
        "planner_host_us_median": float(np.median(plan_times) * 1e6),
        "plan_upload_us": upload_us,
        "plan_device_bytes": plan_bytes,
        "algorithmic_bytes": {"kv_unique": kv_bytes, "q": q_bytes, "out": q_bytes,
                              "naive_per_query_kv": naive_kv,
                              "kv_io_saved_frac": 1.0 - kv_bytes / naive_kv,
                              "partials_written": part_bytes},
        "flops": flops,
        "partial_mfma_tflops": flops / (mean_part * 1e-6) / 1e12,
        "roofline": roof,
        "roofline_partial_kernel": roof_partial,
        "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
        if args.workload in (1, 2, 3):
            line["cpu_baseline_1thread"] = cpu_baseline(wl, args.cpu_budget * 0.75, threads=1)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
