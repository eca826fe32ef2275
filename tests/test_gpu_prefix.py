"""GPU parity of shared-prefix decode (cc_plan_prefix + cc_decode) against the
fp64 oracle, through the C ABI.

The oracle is the plain definition read through each sequence's block table:
it neither knows nor needs the sharing, so the check is that reading a
shared prefix once for up to 16 / G members, and merging it as one more split
of each member, gives every sequence its own attention result.  Cases cover
one and several groups, members whose whole sequence is the prefix, sequences
in no group (and empty ones), both page layouts, head dims 64 and 128, CU
counts from 1 to 1024 (prefix pieces shared by waves, whole in one wave, and
split across compute units), both unit costs, the split + combine launch,
repeat runs, poisoned partial slots, a stale plan, and the full-size
shared-prefix workload (64 sequences, one 4096-token prefix).
"""
import dataclasses

import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W
from oracle import attention as A

from gpu_helpers import TOL_LSE, TOL_OUT, clean, compare, full_oracle, full_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SP = W.CONFIG_BY_NAME["shared_prefix_gqa"]


def run_prefix(wl, cus, xcds, unit_cost=None, reduce=B.REDUCE_FUSED, tag=""):
    print(f"[gpu] prefix {tag} B={wl.cfg.batch} groups={list(wl.prefix_len)} C={cus} unit_cost={unit_cost} "
          f"reduce={reduce}", flush=True)
    plan = B.plan_prefix(B.problem_for(wl), wl.seqlens, wl.prefix_group, wl.prefix_len, wl.block_table,
                         num_cus=cus, num_xcds=xcds, unit_cost=unit_cost)
    assert int(plan.view(np.int32)[26]) > 0 or not (wl.prefix_len > 0).any(), "the plan shares a prefix"
    s = B.session(wl, plan)
    s.run(reduce)
    torch.cuda.synchronize()
    return s, plan


def grouped(cfg, seqlens, groups, plens, seed_offset=0):
    cfg = dataclasses.replace(cfg, batch=len(seqlens), seed=cfg.seed + 200 + seed_offset)
    return W.make_grouped_workload(cfg, seqlens, groups, plens)


BASE = dataclasses.replace(SP, prefix_len=0)


@pytest.mark.parametrize("layout", [W.KV_NHD, W.KV_HND])
@pytest.mark.parametrize("cus", [1, 8, 64, 256, 1024])
def test_one_group(dev, cus, layout):
    rng = np.random.default_rng(cus)
    Lp = 512
    sl = (Lp + rng.integers(0, 900, size=9)).astype(np.int32)
    sl[3] = Lp                                   # a member that is all prefix
    wl = grouped(dataclasses.replace(BASE, kv_layout=layout), sl, np.zeros(9, np.int32), [Lp], cus)
    s, plan = run_prefix(wl, cus, dev[1], tag="one-group")
    compare(s, wl, label=f"prefix one group C={cus}")
    clean(s, plan)


def test_waves_with_more_arrivals_than_their_list(dev):
    """One workgroup (C = 1) over 40 members of a group: each wave finishes
    far more whole split pieces than its list of put-off arrivals holds, so it
    arrives and merges the rest itself; every output meets the oracle bars."""
    rng = np.random.default_rng(40)
    Lp = 256
    sl = (Lp + rng.integers(0, 300, size=40)).astype(np.int32)
    wl = grouped(BASE, sl, np.zeros(40, np.int32), [Lp], 40)
    s, plan = run_prefix(wl, 1, dev[1], tag="arrival-overflow")
    compare(s, wl, label="prefix C=1 40 members")
    clean(s, plan)
    # the members merged by their wave and those merged after the stream give
    # the same bits from run to run
    o0, l0 = s.out.clone(), s.lse.clone()
    for _ in range(5):
        s.out.fill_(float("nan"))
        s.run()
    torch.cuda.synchronize()
    assert torch.equal(s.out, o0) and torch.equal(s.lse, l0)


@pytest.mark.parametrize("unit_cost", [0, None])
@pytest.mark.parametrize("cus", [7, 64, 256])
def test_several_groups_and_loners(dev, cus, unit_cost):
    """Three groups (prefixes of 1, 4 and 40 pages, one group of a single
    member), sequences in no group, an empty one."""
    sl = np.array([16 + 5, 16, 16 + 300, 64 + 1, 64 + 64, 0, 777, 640 + 3, 640 + 900, 640, 640 + 33, 640 + 1,
                   33, 640 + 640, 64 + 2000], np.int32)
    grp = np.array([0, 0, 0, 1, 1, -1, -1, 2, 2, 2, 2, 2, -1, 2, 1], np.int32)
    wl = grouped(BASE, sl, grp, [16, 64, 640], cus)
    s, plan = run_prefix(wl, cus, dev[1], unit_cost=unit_cost, tag="groups")
    compare(s, wl, label=f"prefix groups C={cus} unit_cost={unit_cost}")
    clean(s, plan)


@pytest.mark.parametrize("hkv,hq,d", [(8, 32, 64), (2, 32, 128), (4, 8, 128), (1, 16, 64), (8, 8, 128)])
def test_group_sizes_and_head_dims(dev, hkv, hq, d):
    """G = 4, 16, 2, 16, 1: prefix units of 4, 1, 8, 1 and 16 members."""
    cfg = dataclasses.replace(BASE, num_q_heads=hq, num_kv_heads=hkv, head_dim_qk=d, head_dim_v=d,
                              softmax_scale=1 / np.sqrt(d))
    rng = np.random.default_rng(hq * 7 + hkv)
    Lp = 256
    sl = (Lp + rng.integers(0, 600, size=20)).astype(np.int32)
    grp = np.where(np.arange(20) % 5 == 4, -1, 0).astype(np.int32)
    wl = grouped(cfg, sl, grp, [Lp], hq)
    s, plan = run_prefix(wl, 256, dev[1], tag=f"G={hq // hkv} d={d}")
    compare(s, wl, label=f"prefix G={hq // hkv} d={d}")
    clean(s, plan)


def test_split_combine_launch(dev):
    sl = np.array([1100, 1500, 1100, 2500, 1024, 1800], np.int32)
    wl = grouped(BASE, sl, np.zeros(6, np.int32), [1024], 5)
    s, plan = run_prefix(wl, dev[0], dev[1], reduce=B.REDUCE_SPLIT_COMBINE, tag="v2")
    compare(s, wl, label="prefix split_combine")
    clean(s, plan)


def test_repeat_runs_and_poisoned_partials(dev):
    sl = np.array([3000, 2600, 2100, 4096, 2050, 2200, 2049, 3333], np.int32)
    wl = grouped(BASE, sl, np.zeros(8, np.int32), [2048], 6)
    s, plan = run_prefix(wl, dev[0], dev[1], tag="repeat")
    o0, l0 = s.out.clone(), s.lse.clone()
    units = int(plan.view(np.int32)[15])
    partials_off = -(-(256 + 128 * units) // 256) * 256
    assert int(plan.view(np.int32)[18]) > 0
    for i in range(10):
        s.out.fill_(float("nan"))
        if i % 2:
            s.workspace[partials_off:].view(torch.float32).fill_(float("nan"))
        s.run()
    torch.cuda.synchronize()
    assert torch.equal(s.out, o0) and torch.equal(s.lse, l0)
    clean(s, plan)
    compare(s, wl, label="prefix repeat")


def test_stale_prefix_plan(dev):
    """A member that grew since the plan: flagged, and its output is NaN."""
    sl = np.array([600, 700, 512, 900], np.int32)
    wl = grouped(BASE, sl, np.zeros(4, np.int32), [512], 7)
    planned = sl.copy()
    planned[2] = 520                   # the plan thinks member 2 has 8 own tokens; it has none
    wl2 = W.make_grouped_workload(wl.cfg, planned, wl.prefix_group, wl.prefix_len)
    plan = B.plan_prefix(B.problem_for(wl2), planned, wl2.prefix_group, wl2.prefix_len, wl2.block_table,
                         num_cus=dev[0], num_xcds=dev[1])
    wl2.seqlens = sl.copy()
    s = B.session(wl2, plan)
    s.run()
    dirty, flags = B.workspace_check(plan, s.workspace)
    assert dirty == 0 and flags & 1
    assert np.all(np.isnan(s.lse.cpu().numpy()[2]))


def test_full_size_shared_prefix_workload(dev):
    """64 sequences sharing a 4096-token prefix, each output against the oracle;
    and the same batch planned without sharing gives the same answers."""
    wl = full_workload("shared_prefix_gqa", W.KV_HND)
    ref = full_oracle("shared_prefix_gqa", W.KV_HND)
    s, plan = run_prefix(wl, dev[0], dev[1], tag="full")
    compare(s, wl, ref=ref, label="shared_prefix_gqa fused prefix plan HND")
    clean(s, plan)
    plain = B.plan(B.problem_for(wl), wl.seqlens, wl.block_table, num_cus=dev[0], num_xcds=dev[1])
    s2 = B.session(wl, plain)
    s2.run()
    torch.cuda.synchronize()
    compare(s2, wl, ref=ref, label="shared_prefix_gqa fused plain plan HND")
    clean(s2, plain)
    assert float((s.out - s2.out).abs().max()) <= 2 * TOL_OUT
