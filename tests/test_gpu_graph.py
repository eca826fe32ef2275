"""Decode calls captured in a HIP graph replay to the eager result.

A launch-bound caller (the tiny and index-sparse configurations, where a
decode takes a few microseconds of GPU time) captures its decode calls in a
HIP graph and replays them.  The library launches kernels only: it records no
memset and allocates nothing per call, and the arrival counters are reset by
the kernels themselves, so every replay starts from the state the previous one
left.  Each replay here runs between eager work on the same buffers (the
outputs are overwritten with NaN eagerly, then replayed) and must match the
eager result bit for bit; the workspace must be clean afterwards.  The plan
upload (pinned host to device) can be captured with the decode calls as well.
"""
import dataclasses

import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W

from gpu_helpers import clean, compare, run

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    ("tiny_gqa", dict()),
    ("skewed_gqa", dict(batch=8, seqlen_hi=20000)),
    ("deepseek_mla", dict(batch=4, seqlen_hi=3000)),
    ("sparse_mla", dict(batch=2, seqlen_hi=2000)),
]


@pytest.mark.parametrize("reduce", [B.REDUCE_FUSED, B.REDUCE_SPLIT_COMBINE])
@pytest.mark.parametrize("name,small", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(dev, name, small, reduce):
    cfg = W.CONFIG_BY_NAME[name]
    if small:
        cfg = W.small_variant(cfg, **small)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, reduce=reduce, tag=f"graph {name}")
    compare(s, wl)
    out0, lse0 = s.out.clone(), s.lse.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s.run(reduce)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            s.run(reduce)
    torch.cuda.synchronize()
    for rep in range(4):
        s.out.fill_(float("nan"))
        s.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(s.out, out0) and torch.equal(s.lse, lse0), f"replay {rep}"
        s.run(reduce)  # eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(s.out, out0)
    clean(s, plan)


@pytest.mark.parametrize("name,small", [c for c in CASES if c[0] in ("tiny_gqa", "sparse_mla")],
                         ids=["tiny_gqa", "sparse_mla"])
def test_graph_with_plan_upload(dev, name, small):
    """The plan upload (pinned host -> device copy) captured with the decode:
    the device plan is wiped eagerly before every replay, so each replay's
    result shows that the captured copy wrote the plan again first."""
    cfg = W.CONFIG_BY_NAME[name]
    if small:
        cfg = W.small_variant(cfg, **small)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag=f"graph+upload {name}")
    compare(s, wl)
    out0, lse0 = s.out.clone(), s.lse.clone()
    pinned = torch.from_numpy(plan.copy()).pin_memory()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s.plan_dev.copy_(pinned, non_blocking=True)
        s.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s.plan_dev.copy_(pinned, non_blocking=True)
        s.run()
    torch.cuda.synchronize()
    for rep in range(4):
        s.plan_dev.zero_()
        s.out.fill_(float("nan"))
        s.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(s.plan_dev.cpu(), pinned), f"replay {rep}: plan not uploaded"
        assert torch.equal(s.out, out0) and torch.equal(s.lse, lse0), f"replay {rep}"
    clean(s, plan)
