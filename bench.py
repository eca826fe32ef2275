"""Decode-attention benchmark: KV GB/s, fraction of the 8 TB/s HBM peak and
microseconds per batch on the skewed variable-length workload (one sequence of
131072 tokens and 31 of 256; GQA 32 query / 8 KV heads, head dim 128, bf16,
paged KV with 16-token pages and a shuffled block table).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload skewed_gqa]

One step = one call of the decode (plan already on the device, inputs resident
in HBM).  Before every timed step a 1 GiB scratch write evicts the 256 MB
last-level cache, so each step reads its KV from HBM; the write is outside the
timed region.  Each step is timed with HIP events recorded on the stream the
kernels run on.  The two comparison launches of the same computation (one
workgroup per (sequence, KV head); split + separate combine kernel) are timed
the same way beside it, and the fp64 CPU oracle is timed on the host cores.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="skewed_gqa")
    ap.add_argument("--variant-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def time_steps(torch, run, steps, warmup, flush=None):
    """Per-step event timings (ms) of run(); flush() runs untimed before each step."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        if flush:
            flush()
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        if flush:
            flush()
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def stats(ms):
    return dict(mean_us=float(ms.mean() * 1e3), median_us=float(np.median(ms) * 1e3),
                p10_us=float(np.percentile(ms, 10) * 1e3), p90_us=float(np.percentile(ms, 90) * 1e3))


def cpu_baseline(wl, args):
    """The fp64 oracle, as it stands, on the host cores: the whole workload once."""
    from oracle import attention as A
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    t0 = time.perf_counter()
    A.decode_attention_wl(wl)
    dt = time.perf_counter() - t0
    return {"value": wl.kv_bytes() / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the whole {wl.cfg.name} batch once ({dt:.2f} s, {dt * 1e6:.0f} us/batch)",
            "us_per_batch": dt * 1e6}


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
    cfg = W.CONFIG_BY_NAME[args.workload]
    wl = W.make_workload(cfg)
    kv = wl.kv_bytes()
    prob = B.problem_for(wl)
    log(args, f"workload {cfg.name}: batch {cfg.batch}, sum L {int(wl.seqlens.sum())}, KV {kv / 1e6:.1f} MB, "
              f"CUs {cus}, XCDs {xcds}")

    # host plan, timed on its own
    t0 = time.perf_counter()
    for _ in range(20):
        plan = B.plan(prob, wl.seqlens, wl.block_table, num_cus=cus, num_xcds=xcds)
    plan_us = (time.perf_counter() - t0) / 20 * 1e6
    s = B.session(wl, plan)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def flush():
        scratch.fill_(1)

    ms = time_steps(torch, s.run, args.steps, args.warmup, flush)
    warm = time_steps(torch, s.run, args.steps, args.warmup)
    st = stats(ms)
    dirty, flags = B.workspace_check(plan, s.workspace)
    assert dirty == 0 and flags == 0, "workspace left dirty"
    log(args, f"stream-k fused: {st}")

    variants = {}
    if not args.no_variants:
        v1_plan = B.plan(prob, wl.seqlens, wl.block_table, num_cus=cus, num_xcds=xcds, policy=B.POLICY_PER_UNIT)
        v1 = B.session(wl, v1_plan)
        variants["per_unit_workgroup"] = stats(time_steps(torch, v1.run, args.variant_steps, 3, flush))
        del v1
        v2 = B.session(wl, plan)
        variants["split_then_combine"] = stats(time_steps(
            torch, lambda: v2.run(B.REDUCE_SPLIT_COMBINE), args.variant_steps, 3, flush))
        del v2
        for k, v in variants.items():
            v["kv_gbs"] = kv / (v["mean_us"] * 1e-6) / 1e9
            log(args, f"{k}: {v}")

    mean_s = st["mean_us"] * 1e-6
    gbs = kv / mean_s / 1e9
    result = {
        "metric": "decode-attn KV GB/s & fraction of 8 TB/s HBM peak; us/batch on skewed varlen",
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
                   "num_cus": cus, "num_xcds": xcds, "tile_tokens": 32, "kv_bytes": kv},
        "us_per_batch": st["mean_us"],
        "us_per_batch_median": st["median_us"],
        "us_p10_p90": [st["p10_us"], st["p90_us"]],
        "warm_us_median": stats(warm)["median_us"],
        "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
        "plan_host_us": plan_us,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "variants": variants,
    }
    if variants:
        result["speedup_vs_variants"] = {k: v["mean_us"] / st["mean_us"] for k, v in variants.items()}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
