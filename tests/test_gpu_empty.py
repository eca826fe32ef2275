"""GPU results for sequences with no cached tokens (through the C ABI).

Such a sequence gets no piece in the plan; cc_decode writes out = 0 and
lse = -inf for it, the neutral element of the log-sum-exp merge (the oracle's
reading of an empty key set).  The other sequences of the batch keep the usual
bars against the fp64 oracle, for every plan policy and both reductions, and
the workspace is left clean.
"""
import dataclasses

import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W

from gpu_helpers import clean, compare, run

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [("skewed_gqa", W.KV_NHD), ("skewed_gqa", W.KV_HND), ("deepseek_mla", W.KV_NHD)]


@pytest.mark.parametrize("reduce", [B.REDUCE_FUSED, B.REDUCE_SPLIT_COMBINE])
@pytest.mark.parametrize("policy,unit_cost", [(B.POLICY_STREAMK, None), (B.POLICY_STREAMK, 0),
                                              (B.POLICY_PER_UNIT, 0)])
@pytest.mark.parametrize("name,layout", CASES)
def test_empty_sequences_in_a_batch(dev, name, layout, policy, unit_cost, reduce):
    cfg = dataclasses.replace(W.small_variant(W.CONFIG_BY_NAME[name], batch=6, seqlen_hi=5000, seed_offset=21),
                              kv_layout=layout)
    sl = np.array([0, 300, 0, 4000, 17, 0], np.int32)
    wl = W.make_workload(cfg, seqlens=sl)
    s, plan = run(wl, *dev, policy=policy, unit_cost=unit_cost, reduce=reduce, tag=f"empty {name} layout={layout}")
    compare(s, wl)
    clean(s, plan)


@pytest.mark.parametrize("name", ["skewed_gqa", "deepseek_mla"])
def test_every_sequence_empty(dev, name):
    cfg = W.small_variant(W.CONFIG_BY_NAME[name], batch=3, seqlen_hi=100, seed_offset=22)
    # a one-page cache to point at; the plan and the device see lengths 0
    wl = W.make_workload(cfg, seqlens=np.array([1, 0, 0], np.int32))
    wl = dataclasses.replace(wl, seqlens=np.zeros(3, np.int32))
    s, plan = run(wl, *dev, tag=f"all-empty {name}")
    assert int(plan.view(np.int32)[17]) == 0, "no work item"
    s.out.fill_(float("nan"))
    s.lse.fill_(float("nan"))
    s.run()
    torch.cuda.synchronize()
    assert bool(torch.all(s.out == 0)) and bool(torch.all(s.lse == float("-inf")))
    clean(s, plan)


@pytest.mark.parametrize("reduce", [B.REDUCE_FUSED, B.REDUCE_SPLIT_COMBINE])
def test_kernel_events_bracket_a_call_with_empty_sequences(dev, reduce):
    """With empty sequences the call's first kernel is the output fill: the
    debug kernel events still bracket the whole call (about as long as the
    same call between ordinary event records, not just the fill), the outputs
    do not change, and a call after clearing them records nothing."""
    cfg = W.small_variant(W.CONFIG_BY_NAME["skewed_gqa"], batch=6, seqlen_hi=8000, seed_offset=23)
    wl = W.make_workload(cfg, seqlens=np.array([0, 3000, 0, 7000, 40, 0], np.int32))
    s, plan = run(wl, *dev, reduce=reduce, tag="empty kernel-events")
    o0, l0 = s.out.clone(), s.lse.clone()
    stream = torch.cuda.current_stream()
    a, b, c, d = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    for e in (a, b, c, d):
        e.record(stream)
    torch.cuda.synchronize()
    kernel_ms, marker_ms = [], []
    for _ in range(5):
        B.debug_kernel_events(a, b)
        s.run(reduce)
        B.debug_kernel_events(None, None)
        c.record(stream)
        s.run(reduce)
        d.record(stream)
        torch.cuda.synchronize()
        kernel_ms.append(a.elapsed_time(b))
        marker_ms.append(c.elapsed_time(d))
        s.run(reduce)
        torch.cuda.synchronize()
        assert a.elapsed_time(b) == kernel_ms[-1]
    assert torch.equal(s.out, o0) and torch.equal(s.lse, l0)
    # the interval covers the decode, not just the short fill kernel, and is no
    # longer than the marker-bracketed call beyond timing noise
    km, mk = float(np.median(kernel_ms)), float(np.median(marker_ms))
    assert 0.5 * mk <= km <= 1.1 * mk + 0.005
    compare(s, wl)
    clean(s, plan)
