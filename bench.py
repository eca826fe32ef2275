"""Decode-attention benchmark: KV GB/s, fraction of the 8 TB/s HBM peak and
microseconds per batch on the skewed variable-length workload (one sequence of
131072 tokens and 31 of 256; GQA 32 query / 8 KV heads, head dim 128, bf16,
paged KV with 16-token pages and a shuffled block table).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload skewed_gqa]

One step = one call of the decode (plan already on the device, inputs resident
in HBM).  Before every timed step a 1 GiB scratch buffer is read through, which
evicts the KV from the 256 MB last-level cache without leaving dirty lines
behind (a write-based flush would leave write-back traffic running into the
timed step), so each step reads its KV from HBM; the flush is outside the
timed region.  The same box's plain streaming-read ceiling (1 GiB, the
library's read probe, same flush) is reported beside the result.

Each step is timed with a pair of HIP events that the library records through
hipExtLaunchKernel at the start of the call's first kernel and the end of its
last (cc_debug_kernel_events), on the stream the kernels run on: the interval
rocprofv3 traces for the kernel.  Events recorded as ordinary markers around
the call add about 6 us of queue handling per step (a tiny kernel measures
6.4 us that way); that time is reported beside the result.  The two comparison
launches of the same computation (one
workgroup per (sequence, KV head); split + separate combine kernel) are timed
the same way beside it, and the fp64 CPU oracle is timed on the host cores.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_DENSE_PEAK_TFLOPS = 2500.0
METRIC = "decode-attn KV GB/s & fraction of 8 TB/s HBM peak; \u00b5s/batch on skewed varlen"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="skewed_gqa")
    ap.add_argument("--layout", choices=["nhd", "hnd"], default="hnd",
                    help="page layout of the GQA K/V caches: head-major [Hkv][P][d] (default) or token-major [P][Hkv][d]")
    ap.add_argument("--variant-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time back-to-back calls eagerly and replayed from a captured HIP graph")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="also time the MFMA ceiling probe (dense bf16, register operands)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a 256 MiB fill and a 1 GiB read of known size (scales profiler byte counters)")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def time_steps(torch, run, steps, warmup, flush=None, kernel_events=None):
    """Per-step event timings (ms) of run(); flush() runs untimed before each step.

    With kernel_events (the binding's debug_kernel_events) the library records
    each step's events at its kernels' start and end; otherwise the events are
    recorded on the stream around run().

    Python's garbage collector is paused while steps are enqueued: a collection
    between a step's two events would show up as GPU idle time inside it."""
    import gc
    gc.collect()
    gc.disable()
    try:
        return _time_steps(torch, run, steps, warmup, flush, kernel_events)
    finally:
        gc.enable()


def _time_steps(torch, run, steps, warmup, flush, kernel_events):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        if flush:
            flush()
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    if kernel_events:
        for a, b in ev:  # torch creates an event at its first record
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
    for a, b in ev:
        if flush:
            flush()
        if kernel_events:
            kernel_events(a, b)
            run()
            kernel_events(None, None)  # the next flush must not record into them
        else:
            a.record(stream)
            run()
            b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def time_interleaved(torch, runs, steps, warmup, flush, kernel_events):
    """Kernel-timed steps of several launches in alternating rounds: round i
    runs every launch once (the order rotated each round), each after the
    flush, so a slow drift of the shader clock over the run (the MFMA-bound
    kernels show one) reaches every launch alike.  runs: {name: (fn, steps)};
    a launch with fewer steps than the others takes part in the first rounds
    only.  Returns {name: ms array}."""
    import gc
    gc.collect()
    gc.disable()
    try:
        stream = torch.cuda.current_stream()
        names = list(runs)
        for _ in range(warmup):
            for n in names:
                if flush:
                    flush()
                runs[n][0]()
        torch.cuda.synchronize()
        ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(runs[n][1])] for n in names}
        for n in names:
            for a, b in ev[n]:
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        rounds = max(runs[n][1] for n in names)
        for i in range(rounds):
            for j in range(len(names)):
                n = names[(i + j) % len(names)]
                if i >= runs[n][1]:
                    continue
                a, b = ev[n][i]
                if flush:
                    flush()
                kernel_events(a, b)
                runs[n][0]()
                kernel_events(None, None)
            if i % 16 == 15:
                torch.cuda.synchronize()  # bounded queue of pending launches
        torch.cuda.synchronize()
        return {n: np.array([a.elapsed_time(b) for a, b in ev[n]]) for n in names}
    finally:
        gc.enable()


def stats(ms):
    return dict(mean_us=float(ms.mean() * 1e3), median_us=float(np.median(ms) * 1e3),
                p10_us=float(np.percentile(ms, 10) * 1e3), p90_us=float(np.percentile(ms, 90) * 1e3))


def graph_pass(torch, s, calls=100, reps=5):
    """Warm back-to-back decode calls: host-launched one by one, then replayed
    from a HIP graph that holds the same calls (what a launch-bound caller does).
    Per-call time between two stream events around all the calls."""
    stream = torch.cuda.current_stream()

    def timed(fn):
        best = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            best.append(a.elapsed_time(b) * 1e3 / calls)
        return float(np.median(best))

    def eager():
        for _ in range(calls):
            s.run()

    eager()
    torch.cuda.synchronize()
    eager_us = timed(eager)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        s.run()
    stream.wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            s.run()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    graph_us = timed(g.replay)
    return {"calls": calls, "eager_us_per_call": eager_us, "graph_us_per_call": graph_us}


def timeline_pass(torch, B, s, workers, xcds, flush):
    """One cold decode with the in-kernel timeline on: CU busy fraction and XCD placement."""
    buf = torch.zeros(8 * workers, dtype=torch.int64, device="cuda")
    B.debug_timeline(buf)
    flush()
    s.run()
    torch.cuda.synchronize()
    B.debug_timeline(None)
    t = buf.view(workers, 8).cpu().numpy().astype(np.int64)
    start, stream_end, merged, arrived, end, xcc = t[:, 0], t[:, 1], t[:, 2], t[:, 3], t[:, 4], t[:, 5]
    listed, weighed = t[:, 6], t[:, 7]   # GQA: after the slot lists, after the per-row max and sum
    t0 = start.min()
    span = float(end.max() - t0)                      # 100 MHz ticks
    busy = float((end - start).sum()) / (workers * span) if span > 0 else 0.0
    to_us = 1e-2
    return {"makespan_us": span * to_us, "cu_busy_frac": busy,
            "start_spread_us": float(start.max() - t0) * to_us,
            "stream_end_us": [float(np.percentile(stream_end - t0, q)) * to_us for q in (0, 50, 100)],
            "end_us": [float(np.percentile(end - t0, q)) * to_us for q in (0, 50, 100)],
            "post_stream_us_median_max": [float(np.median(end - stream_end)) * to_us,
                                          float((end - stream_end).max()) * to_us],
            "piece_merge_us_median": float(np.median(merged - stream_end)) * to_us,
            "piece_merge_steps_us_median": ([float(np.median(listed - stream_end)) * to_us,
                                             float(np.median(weighed - listed)) * to_us,
                                             float(np.median(merged - weighed)) * to_us] if listed.any() else None),
            "arrival_us_median": float(np.median(arrived - merged)) * to_us,
            "unit_merge_us_max": float((end - arrived).max()) * to_us,
            "xcd_is_w_mod_x": bool(np.all(xcc == np.arange(workers) % xcds)),
            "xcd_ids_seen": sorted(set(int(x) for x in xcc))}


KERNEL_SOURCES = {"gqa_decode_kernel": ("decode_gqa.hip", "merge.h", "launch.h", "plan.h"),
                  "mla_decode_kernel": ("decode_mla.hip", "merge.h", "launch.h", "plan.h"),
                  "moe_gemm_kernel": ("moe.hip", "launch.h", "plan.h")}


def kernel_name(mode):
    return "gqa_decode_kernel" if mode == 0 else "mla_decode_kernel"


def source_hash(kernel):
    """sha256[:16] of the sources the decode kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, "cross_cu_load_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel, workload, layout=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if the
    kernel's sources are unchanged since it was taken (else None)."""
    import re
    name = f"{kernel}_{workload}_{layout}.md" if layout else f"{kernel}_{workload}.md"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_sha256_16: (\w+)", text)
    m_tr = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    if not m_src or not m_tr or m_src.group(1) != source_hash(kernel):
        return None
    return int(m_tr.group(1))


def mfma_flops(wl):
    """Dense contraction flops of one decode: 2 (dk + dv) per (query head, key)."""
    c = wl.cfg
    keys = c.topk * c.q_tokens * c.batch if wl.indices is not None else int(wl.seqlens.sum()) * c.q_tokens
    return 2.0 * (c.head_dim_qk + c.head_dim_v) * c.num_q_heads * keys


def indexer_pass(torch, B, W, wl, flush, ke, steps, warmup):
    """The indexer that produces the sparse workload's index sets (paged score
    + top-k over each request's cached tokens), kernel-timed like the decode."""
    c = wl.cfg
    ix = W.make_indexer_inputs(wl)
    p = B.indexer_problem(c.batch, c.q_tokens, W.INDEXER_DIM, c.page_size, wl.max_pages, wl.num_pages, c.topk)

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()

    q, k, bt = dev(ix.q), dev(ix.k_cache), dev(wl.block_table)
    scratch = torch.empty(B.indexer_scratch_size(p, wl.seqlens), dtype=torch.uint8, device="cuda")
    out = torch.empty((c.batch, c.q_tokens, c.topk), dtype=torch.int32, device="cuda")
    ms = time_steps(torch, lambda: B.indexer_topk(p, wl.seqlens, q, k, bt, scratch, out), steps, warmup, flush, ke)
    key_bytes = int(wl.seqlens.astype(np.int64).sum()) * W.INDEXER_DIM * 2
    st = stats(ms)
    return {"us_mean": st["mean_us"], "us_median": st["median_us"], "key_bytes": key_bytes,
            "key_gbs": key_bytes / (st["mean_us"] * 1e-6) / 1e9, "selected_per_token": c.topk}, ix


def indexer_cpu_baseline(wl, ix):
    """The indexer oracle on the host: the whole batch once."""
    from oracle import indexer as I
    t0 = time.perf_counter()
    I.indexer_topk(ix.q, ix.k_cache, wl.block_table, wl.seqlens, wl.cfg.topk)
    return (time.perf_counter() - t0) * 1e6


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def cpu_baseline(wl, args, min_seconds=10.0, max_reps=8):
    """The fp64 oracle, as it stands, on the host cores: the whole workload,
    repeated until about ten seconds of CPU work have run (at most 8 times).
    ``cores`` is the number of threads the oracle's BLAS actually ran with
    (bounded by the cores this process may run on)."""
    from oracle import attention as A
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    reps = 0
    t0 = time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        A.decode_attention_wl(wl)
        reps += 1
    total = time.perf_counter() - t0
    dt = total / reps
    return {"value": wl.unique_kv_bytes() / dt / 1e9, "unit": "GB/s", "cores": int(min(blas, affinity)), "kind": "oracle",
            "sample": f"the whole {wl.cfg.name} batch, {reps} times ({total:.1f} s, {dt * 1e6:.0f} us/batch)",
            "us_per_batch": dt * 1e6, "affinity_cores": affinity, "blas_threads": int(blas),
            "cpu_model": cpu_model()}


MOE_METRIC = "MoE grouped GEMM TFLOP/s & fraction of 2.5 PFLOP/s bf16 dense MFMA peak"


def mfma_probe_pass(torch, B, cus, ke):
    """The practical dense bf16 MFMA ceiling: TFLOP/s of register-operand
    MFMA chains with one and two waves per SIMD."""
    out = {}
    for waves in (4, 8):
        sink = torch.empty(cus * waves * 64, dtype=torch.int32, device="cuda")
        flops = B.probe_mfma(cus, waves, 4096, sink)
        ms = time_steps(torch, lambda: B.probe_mfma(cus, waves, 4096, sink), 10, 2, None, ke)
        out[f"waves_per_simd_{waves // 4}"] = flops / (float(np.median(ms)) * 1e-3) / 1e12
    return out


def bench_moe(args, torch, B, W, cus, xcds, flush, ke):
    """The varlen MoE grouped GEMM: all experts in one persistent launch."""
    cfg = W.MOE_BY_NAME[args.workload]
    wl = W.make_moe_workload(cfg)
    prob = B.moe_problem(cfg.num_experts, cfg.hidden, cfg.out_dim)
    log(args, f"workload {cfg.name}: {cfg.num_experts} experts, rows {int(wl.expert_tokens.sum())} "
              f"(max {int(wl.expert_tokens.max())}, min {int(wl.expert_tokens.min())}), K {cfg.hidden}, N {cfg.out_dim}")
    t0 = time.perf_counter()
    workers = cus * B.MOE_WORKGROUPS_PER_CU   # the resident workgroups of one wave
    for _ in range(20):
        plan = B.moe_plan(prob, wl.expert_tokens, num_cus=workers, num_xcds=xcds)
    plan_us = (time.perf_counter() - t0) / 20 * 1e6
    s = B.moe_session(wl, plan)
    # the fused launch and the comparison launches in alternating rounds: this
    # kernel is bound by on-chip work, and the shader clock drifts over a run
    runs = {"fused": (s.run, args.steps)}
    if not args.no_variants:
        v1_plan = B.moe_plan(prob, wl.expert_tokens, num_cus=workers, num_xcds=xcds, policy=B.POLICY_PER_UNIT)
        v1 = B.moe_session(wl, v1_plan)
        v2 = B.moe_session(wl, plan)
        runs["per_tile_workgroup"] = (v1.run, args.variant_steps)
        runs["split_then_combine"] = (lambda: v2.run(B.REDUCE_SPLIT_COMBINE), args.variant_steps)
        # the plain Stream-K split (contiguous equal chunks, every chunk boundary
        # inside a tile), for what the data-parallel rounds save or cost
        v3_plan = B.moe_plan(prob, wl.expert_tokens, num_cus=workers, num_xcds=xcds, policy=B.POLICY_STREAMK)
        v3 = B.moe_session(wl, v3_plan)
        runs["streamk_contiguous"] = (v3.run, args.variant_steps)
    timed = time_interleaved(torch, runs, args.steps, args.warmup, flush, ke)
    ms = timed["fused"]
    ms_markers = time_steps(torch, s.run, args.steps, args.warmup, flush)
    st = stats(ms)
    dirty, flags = B.workspace_check(plan, s.workspace)
    assert dirty == 0 and flags == 0, "workspace left dirty"
    workers = int(plan.view(np.int32)[11])
    tline = timeline_pass(torch, B, s, workers, xcds, flush)
    variants = {k: stats(v) for k, v in timed.items() if k != "fused"}
    for v in variants.values():
        v["tflops"] = wl.flops() / (v["mean_us"] * 1e-6) / 1e12
    tflops = wl.flops() / (st["mean_us"] * 1e-6) / 1e12
    result = {
        "metric": MOE_METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": st["mean_us"] / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "experts": cfg.num_experts, "hidden": cfg.hidden, "out_dim": cfg.out_dim,
                   "tokens": cfg.tokens, "top_k": cfg.top_k, "rows": int(wl.expert_tokens.sum()),
                   "rows_max_min": [int(wl.expert_tokens.max()), int(wl.expert_tokens.min())],
                   "tile": [256, 256, 64], "num_cus": cus, "num_xcds": xcds, "workers": workers,
                   "plan_policy": (f"streamk_dp: whole tiles round-robin; a last round under 3/4 full split in "
                                   f"equal cost chunks (1 per k tile + {int(plan.view(np.int32)[23])} per tile)"),
                   "partial_slots": int(plan.view(np.int32)[18])},
        "us_per_batch": st["mean_us"], "us_per_batch_median": st["median_us"],
        "us_p10_p90": [st["p10_us"], st["p90_us"]],
        "timing": ("kernel start to end (hipExtLaunchKernel events), cold, per step; the comparison launches "
                   "in alternating rounds with it"),
        "us_per_batch_event_markers": stats(ms_markers),
        "plan_host_us": plan_us,
        "min_bytes": wl.bytes_min(), "min_bytes_gbs": wl.bytes_min() / (st["mean_us"] * 1e-6) / 1e9,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_DENSE_PEAK_TFLOPS,
                     "traffic": profiled_traffic("moe_gemm_kernel", cfg.name)},
        "variants": variants,
        "timeline": tline,
    }
    if variants:
        result["speedup_vs_variants"] = {k: v["mean_us"] / st["mean_us"] for k, v in variants.items()}
    if args.mfma_probe:
        result["mfma_probe_tflops"] = mfma_probe_pass(torch, B, cus, ke)
    if not args.no_cpu_baseline:
        from oracle import moe as M
        t0 = time.perf_counter()
        M.grouped_gemm(wl.x, wl.w, wl.offsets)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": wl.flops() / dt / 1e12, "unit": "TFLOP/s",
                                  "cores": min(len(os.sched_getaffinity(0)), _blas_threads()), "kind": "oracle",
                                  "sample": f"the whole {cfg.name} batch once ({dt:.1f} s, fp64)",
                                  "cpu_model": cpu_model()}
    print(json.dumps(result), flush=True)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode path has no "
              f"multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch

    from cross_cu_load_amd import binding as B
    from cross_cu_load_amd import workloads as W

    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cus, xcds = B.device_query(0)
    if args.calibrate:   # kernels of known traffic for the profiler's byte counters
        cal = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        for _ in range(2):
            B.workspace_init(cal)          # writes exactly 256 MiB
        torch.cuda.synchronize()
        del cal
    if args.workload in W.MOE_BY_NAME:
        scratch = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        sink = torch.empty(1024 * 512, dtype=torch.int32, device="cuda")
        bench_moe(args, torch, B, W, cus, xcds, lambda: B.probe_read(scratch, 0, 1024, sink), B.debug_kernel_events)
        return
    cfg = W.CONFIG_BY_NAME[args.workload]
    if cfg.mode == W.MODE_GQA:
        cfg = dataclasses.replace(cfg, kv_layout=W.KV_HND if args.layout == "hnd" else W.KV_NHD)
    wl = W.make_workload(cfg)
    shared = wl.prefix_group is not None
    # algorithmic bytes: every distinct K/V row the batch attends over once (a
    # shared prefix once per group)
    kv = wl.unique_kv_bytes()
    prob = B.problem_for(wl)
    log(args, f"workload {cfg.name}: batch {cfg.batch}, sum L {int(wl.seqlens.sum())}, KV {kv / 1e6:.1f} MB, "
              f"CUs {cus}, XCDs {xcds}")

    # host plan, timed on its own
    def make_plan():
        if shared:
            return B.plan_prefix(prob, wl.seqlens, wl.prefix_group, wl.prefix_len, wl.block_table, num_cus=cus,
                                 num_xcds=xcds)
        return B.plan(prob, wl.seqlens, wl.block_table, num_cus=cus, num_xcds=xcds)

    t0 = time.perf_counter()
    for _ in range(20):
        plan = make_plan()
    plan_us = (time.perf_counter() - t0) / 20 * 1e6
    s = B.session(wl, plan)
    scratch = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1024 * 512, dtype=torch.int32, device="cuda")

    def flush():
        B.probe_read(scratch, 0, 1024, sink)

    ke = B.debug_kernel_events

    # practical ceiling: a plain 1 GiB streaming read, same flush; plain loads
    # (method 0) and the non-temporal loads the kernels use (method 3)
    probe_buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    probe_by_method = {}
    for m in (0, 3):
        pms = time_steps(torch, lambda: B.probe_read(probe_buf, m, 1024, sink), 20, 3, flush, ke)
        probe_by_method[m] = (1 << 30) / (float(np.median(pms)) * 1e-3) / 1e9
    probe_gbs = max(probe_by_method.values())
    del probe_buf
    log(args, f"read probe ceiling: {probe_gbs:.0f} GB/s (plain {probe_by_method[0]:.0f}, nt {probe_by_method[3]:.0f})")

    ms = time_steps(torch, s.run, args.steps, args.warmup, flush, ke)
    ms_markers = time_steps(torch, s.run, args.steps, args.warmup, flush)
    warm = time_steps(torch, s.run, args.steps, args.warmup, None, ke)
    st = stats(ms)
    dirty, flags = B.workspace_check(plan, s.workspace)
    assert dirty == 0 and flags == 0, "workspace left dirty"
    log(args, f"stream-k fused: {st}")
    workers = int(plan.view(np.int32)[11])  # plan header: worker (chunk) count
    tline = timeline_pass(torch, B, s, workers, xcds, flush)
    log(args, f"timeline: {tline}")

    variants = {}
    if not args.no_variants:
        v1_plan = B.plan(prob, wl.seqlens, wl.block_table, num_cus=cus, num_xcds=xcds, policy=B.POLICY_PER_UNIT)
        v1 = B.session(wl, v1_plan)
        variants["per_unit_workgroup"] = stats(time_steps(torch, v1.run, args.variant_steps, 3, flush, ke))
        del v1
        v2 = B.session(wl, plan)
        variants["split_then_combine"] = stats(time_steps(
            torch, lambda: v2.run(B.REDUCE_SPLIT_COMBINE), args.variant_steps, 3, flush, ke))
        del v2
        if shared:   # the same batch with every sequence reading its own copy of the prefix
            plain = B.plan(prob, wl.seqlens, wl.block_table, num_cus=cus, num_xcds=xcds)
            v3 = B.session(wl, plain)
            variants["no_prefix_sharing"] = stats(time_steps(torch, v3.run, args.variant_steps, 3, flush, ke))
            del v3
        for k, v in variants.items():
            v["kv_gbs"] = kv / (v["mean_us"] * 1e-6) / 1e9
            log(args, f"{k}: {v}")

    mean_s = st["mean_us"] * 1e-6
    gbs = kv / mean_s / 1e9
    layout_name = args.layout if cfg.mode == W.MODE_GQA else "latent"
    result = {
        "metric": METRIC,
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": st["mean_us"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seqlens_sum": int(wl.seqlens.sum()),
                   "seqlen_max": int(wl.seqlens.max()), "num_q_heads": cfg.num_q_heads,
                   "num_kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim_qk, "page_size": cfg.page_size,
                   "num_cus": cus, "num_xcds": xcds, "tile_tokens": 32, "kv_bytes": kv,
                   "plan_policy": f"streamk, equal cost chunks: 1 per tile + {int(plan.view(np.int32)[23])} per unit",
                   "kv_layout": layout_name},
        "us_per_batch": st["mean_us"],
        **({"shared_prefix": {"prefix_len": int(cfg.prefix_len), "prefix_units": int(plan.view(np.int32)[26]),
                              "unique_kv_bytes": kv, "kv_bytes_without_sharing": wl.kv_bytes()}} if shared else {}),
        "us_per_batch_median": st["median_us"],
        "us_p10_p90": [st["p10_us"], st["p90_us"]],
        "warm_us_median": stats(warm)["median_us"],
        "timing": "kernel start to end (hipExtLaunchKernel events), cold, per step",
        "us_per_batch_event_markers": stats(ms_markers),
        "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
        "read_probe_ceiling_gbs": probe_gbs,
        "read_probe_gbs_plain_nt": [probe_by_method[0], probe_by_method[3]],
        "frac_of_read_probe": gbs / probe_gbs,
        "plan_host_us": plan_us,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": profiled_traffic(kernel_name(cfg.mode), cfg.name, layout_name)},
        "mfma_tflops": mfma_flops(wl) / mean_s / 1e12,
        "mfma_frac_of_bf16_dense_peak": mfma_flops(wl) / mean_s / 1e12 / BF16_DENSE_PEAK_TFLOPS,
        "variants": variants,
        "timeline": tline,
    }
    if cfg.mode == W.MODE_MLA_SPARSE:
        result["indexer"], ix = indexer_pass(torch, B, W, wl, flush, ke, args.steps, args.warmup)
        if not args.no_cpu_baseline:
            result["indexer"]["cpu_oracle_us"] = indexer_cpu_baseline(wl, ix)
        log(args, f"indexer: {result['indexer']}")
    if args.mfma_probe:
        result["mfma_probe_tflops"] = mfma_probe_pass(torch, B, cus, ke)
    if args.graph:
        result["graph"] = graph_pass(torch, s)
        log(args, f"graph: {result['graph']}")
    if variants:
        result["speedup_vs_variants"] = {k: v["mean_us"] / st["mean_us"] for k, v in variants.items()}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
