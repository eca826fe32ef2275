"""GPU parity of the MLA and index-sparse MLA decode paths against the fp64
oracle (through the C ABI).

Bars as for GQA: max|out - oracle| <= 1e-2, max|lse - oracle| <= 1e-3, no
NaN/Inf.  The full-size dense workload (64 sequences of 1024..16384 tokens)
and the full-size sparse workload (2 requests x 8 query tokens, 2048 indices
each) run in the launch configuration the benchmark times and are checked on
every output, for the fused path and for both comparison launches.
"""
import dataclasses

import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W
from oracle import attention as A
from oracle import planner as PL

from gpu_helpers import clean, compare, full_oracle, full_workload, run

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MLA = W.CONFIG_BY_NAME["deepseek_mla"]
SPARSE = W.CONFIG_BY_NAME["sparse_mla"]


def v_row(wl, b, j):
    """V row (first dv columns of the latent row) of token j of sequence b, as float32."""
    P = wl.cfg.page_size
    page = wl.block_table[b, j // P]
    return A.bf16_to_f64(wl.k_cache[page, j % P, 0, :wl.cfg.head_dim_v]).astype(np.float32)


@pytest.mark.parametrize("page", [32, 64, 256])
def test_mla_small_all_outputs(dev, page):
    cfg = dataclasses.replace(W.small_variant(MLA, batch=6, seqlen_hi=3000, seed_offset=page), page_size=page)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag=f"mla-small P={page}")
    compare(s, wl)
    clean(s, plan)


def test_mla_ragged_and_single_token(dev):
    sl = np.array([1, 2, 31, 32, 33, 63, 64, 65, 127, 1, 4097, 700], np.int32)
    cfg = W.small_variant(MLA, batch=len(sl), seqlen_hi=5000)
    wl = W.make_workload(cfg, seqlens=sl)
    s, plan = run(wl, *dev, tag="mla-ragged")
    compare(s, wl)
    clean(s, plan)
    out = s.out.cpu().numpy()
    for b in np.nonzero(sl == 1)[0]:   # one key: p = 1, the output is that token's V row exactly
        v = v_row(wl, b, 0)
        for h in range(cfg.num_q_heads):
            assert np.array_equal(out[b, 0, h], v)


@pytest.mark.parametrize("unit_cost", [0, None])
def test_mla_full_size_all_outputs(dev, unit_cost):
    wl = full_workload("deepseek_mla")
    s, plan = run(wl, *dev, unit_cost=unit_cost, tag="mla-full")
    ref = PL.plan_for(wl, num_cus=dev[0], num_xcds=dev[1], heads_per_unit=128,
                      unit_cost=B.default_unit_cost(B.MODE_MLA) if unit_cost is None else unit_cost)
    assert plan.tobytes() == ref["blob"]
    compare(s, wl, ref=full_oracle("deepseek_mla"), label=f"deepseek_mla fused unit_cost={unit_cost}")
    clean(s, plan)


@pytest.mark.parametrize("variant", ["per_unit", "split_combine"])
@pytest.mark.parametrize("name", ["deepseek_mla", "sparse_mla"])
def test_mla_full_size_comparison_variants(dev, name, variant):
    wl = full_workload(name)
    policy, reduce = ((B.POLICY_PER_UNIT, B.REDUCE_FUSED) if variant == "per_unit"
                      else (B.POLICY_STREAMK, B.REDUCE_SPLIT_COMBINE))
    s, plan = run(wl, *dev, policy=policy, reduce=reduce, tag=f"{name}-{variant}")
    compare(s, wl, ref=full_oracle(name), label=f"{name} {variant}")
    clean(s, plan)


@pytest.mark.parametrize("L,topk", [(300, 300), (300, 45), (64, 33), (1, 1), (2048, 2048)])
def test_sparse_small_all_outputs(dev, L, topk):
    cfg = dataclasses.replace(W.small_variant(SPARSE, batch=2, seqlen_hi=L, seed_offset=topk), topk=topk)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag=f"sparse L={L} topk={topk}")
    compare(s, wl)
    clean(s, plan)
    if topk == 1:    # one index: the output is that token's V row exactly
        out = s.out.cpu().numpy()
        for b in range(cfg.batch):
            for t in range(cfg.q_tokens):
                v = v_row(wl, b, int(wl.indices[b, t, 0]))
                for h in range(cfg.num_q_heads):
                    assert np.array_equal(out[b, t, h], v)


@pytest.mark.parametrize("page", [16, 32, 128, 256])
def test_sparse_page_sizes(dev, page):
    """Index-sparse gathers at pages of 16 to 256 tokens (the workload uses 64),
    every output."""
    cfg = dataclasses.replace(W.small_variant(SPARSE, batch=2, seqlen_hi=1500, seed_offset=page),
                              topk=200, page_size=page)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag=f"sparse page={page}")
    compare(s, wl, label=f"sparse page {page}")
    clean(s, plan)


def test_sparse_full_size_all_outputs(dev):
    wl = full_workload("sparse_mla")
    s, plan = run(wl, *dev, tag="sparse-full")
    compare(s, wl, ref=full_oracle("sparse_mla"), label="sparse_mla fused")
    clean(s, plan)


def test_sparse_index_order_irrelevant(dev):
    """The same index sets in another order give the same result (to rounding)."""
    cfg = W.small_variant(SPARSE, batch=2, seqlen_hi=1000, seed_offset=9)
    cfg = dataclasses.replace(cfg, topk=500)
    wl = W.make_workload(cfg)
    s, _ = run(wl, *dev, tag="sparse-order-a")
    idx2 = wl.indices[:, :, ::-1].copy()
    wl2 = W.Workload(wl.cfg, wl.seqlens, wl.block_table, wl.q, wl.k_cache, None, idx2)
    s2, _ = run(wl2, *dev, tag="sparse-order-b")
    assert torch.allclose(s.out, s2.out, atol=2e-2, rtol=0)
    assert torch.allclose(s.lse, s2.lse, atol=2e-3, rtol=0)
    compare(s2, wl2)


@pytest.mark.parametrize("policy,reduce", [(B.POLICY_PER_UNIT, B.REDUCE_FUSED),
                                           (B.POLICY_STREAMK, B.REDUCE_SPLIT_COMBINE)])
@pytest.mark.parametrize("name", ["deepseek_mla", "sparse_mla"])
def test_mla_comparison_variants(dev, policy, reduce, name):
    cfg = W.CONFIG_BY_NAME[name]
    cfg = W.small_variant(cfg, batch=4, seqlen_hi=3000 if name == "deepseek_mla" else 2000)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, policy=policy, reduce=reduce, tag="mla-variant")
    compare(s, wl)
    clean(s, plan)


@pytest.mark.parametrize("unit_cost", [0, None])
@pytest.mark.parametrize("cus", [1, 7, 64, 256, 1024])
def test_mla_split_points_move_with_cu_count(dev, cus, unit_cost):
    cfg = W.small_variant(MLA, batch=3, seqlen_hi=4000, seed_offset=cus)
    wl = W.make_workload(cfg)
    s, plan = run(wl, cus, dev[1], unit_cost=unit_cost, tag="mla-cus")
    compare(s, wl)
    clean(s, plan)


def test_mla_repeat_runs_bitwise_identical(dev):
    cfg = W.small_variant(MLA, batch=8, seqlen_hi=16000, seed_offset=3)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag="mla-repeat")
    o0, l0 = s.out.clone(), s.lse.clone()
    for _ in range(10):
        s.out.fill_(float("nan"))
        s.run()
    torch.cuda.synchronize()
    assert torch.equal(s.out, o0) and torch.equal(s.lse, l0)
    clean(s, plan)


@pytest.mark.parametrize("polls", [0, 1])
@pytest.mark.parametrize("name", ["deepseek_mla", "sparse_mla"])
def test_mla_merge_when_pieces_stop_waiting(dev, name, polls):
    """The in-kernel merge with finished pieces that stop polling at once (poll
    limit forced low from the host): their head slices fall to the pieces still
    there, the last arriver never waits, so the output is bitwise the same and
    the arrival counters and claim masks are left zeroed."""
    cfg = W.CONFIG_BY_NAME[name]
    cfg = W.small_variant(cfg, batch=6, seqlen_hi=6000, seed_offset=11) if name == "deepseek_mla" else \
        W.small_variant(cfg, batch=2, seqlen_hi=4096, seed_offset=11)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag=f"mla-merge-polls {name}")
    assert int(plan.view(np.int32)[18]) > 0, "the case must split some unit"
    o0, l0 = s.out.clone(), s.lse.clone()
    try:
        B.debug_merge_poll_limit(polls)
        for _ in range(3):
            s.out.fill_(float("nan"))
            s.run()
        torch.cuda.synchronize()
    finally:
        B.debug_merge_poll_limit(-1)
    assert torch.equal(s.out, o0) and torch.equal(s.lse, l0)
    clean(s, plan)
    compare(s, wl)
