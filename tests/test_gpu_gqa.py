"""GPU parity of the GQA decode path against the fp64 oracle (through the C ABI).

Bars: max|out - oracle| <= 1e-2 and max|lse - oracle| <= 1e-3 (absolute), no
NaN/Inf, for bf16 inputs with fp32 accumulation.  Full-size workloads run in
the launch configuration the benchmark times (one chunk per compute unit,
32-token tiles, the device's XCD count) and are checked on every output, for
the fused path and for both comparison launches.
"""
import dataclasses

import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W
from oracle import attention as A

from gpu_helpers import clean, compare, full_oracle, full_workload, run

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", ["fused", "per_unit", "split_combine"])
def test_tiny_gqa_config(dev, variant):
    wl = full_workload("tiny_gqa")
    policy, reduce = {"fused": (B.POLICY_STREAMK, B.REDUCE_FUSED),
                      "per_unit": (B.POLICY_PER_UNIT, B.REDUCE_FUSED),
                      "split_combine": (B.POLICY_STREAMK, B.REDUCE_SPLIT_COMBINE)}[variant]
    s, plan = run(wl, *dev, policy=policy, reduce=reduce, tag="tiny")
    compare(s, wl, ref=full_oracle("tiny_gqa"), label=f"tiny_gqa {variant}")
    clean(s, plan)


@pytest.mark.parametrize("layout", [W.KV_NHD, W.KV_HND])
@pytest.mark.parametrize("name,batch,hi", [("llama3_8b_gqa", 8, 3000), ("skewed_gqa", 6, 5000),
                                           ("tiny_gqa", 3, 100)])
def test_small_workloads_all_outputs(dev, name, batch, hi, layout):
    cfg = W.small_variant(W.CONFIG_BY_NAME[name], batch=batch, seqlen_hi=hi)
    cfg = dataclasses.replace(cfg, kv_layout=layout)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag="small")
    compare(s, wl)
    clean(s, plan)


def test_ragged_and_single_token_sequences(dev):
    cfg = W.CONFIG_BY_NAME["skewed_gqa"]
    sl = np.array([1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 1, 4097, 1, 999, 1], np.int32)
    cfg = W.small_variant(cfg, batch=len(sl), seqlen_hi=5000)
    wl = W.make_workload(cfg, seqlens=sl)
    s, plan = run(wl, *dev, tag="ragged")
    compare(s, wl)
    clean(s, plan)
    # a one-token sequence returns its V row: p = 1, l = 1, bf16 -> fp32 is exact
    out = s.out.cpu().numpy()
    G, P = cfg.group, cfg.page_size
    for b in np.nonzero(sl == 1)[0]:
        page = wl.block_table[b, 0]
        for h in range(cfg.num_q_heads):
            v = A.bf16_to_f64(wl.v_cache[page, 0, h // G]).astype(np.float32)
            assert np.array_equal(out[b, 0, h], v)


@pytest.mark.parametrize("unit_cost", [0, None])
@pytest.mark.parametrize("layout", [W.KV_NHD, W.KV_HND])
def test_skewed_full_size_all_outputs(dev, layout, unit_cost):
    """Every output of the skewed workload (one 131072-token sequence and 31 of
    256), for the pages' equal tile split (unit cost 0) and the measured
    default unit cost."""
    wl = full_workload("skewed_gqa", layout)
    s, plan = run(wl, *dev, unit_cost=unit_cost, tag="skewed-full")
    compare(s, wl, ref=full_oracle("skewed_gqa"),
            label=f"skewed_gqa fused {'HND' if layout else 'NHD'} unit_cost={unit_cost}")
    clean(s, plan)


@pytest.mark.parametrize("layout", [W.KV_NHD, W.KV_HND])
def test_llama_full_size_all_outputs(dev, layout):
    """Every output of the Llama-3-8B-shaped workload (64 sequences, log-uniform
    lengths in [128, 32768])."""
    wl = full_workload("llama3_8b_gqa", layout)
    s, plan = run(wl, *dev, tag="llama-full")
    compare(s, wl, ref=full_oracle("llama3_8b_gqa"), label=f"llama3_8b_gqa fused {'HND' if layout else 'NHD'}")
    clean(s, plan)


@pytest.mark.parametrize("variant", ["per_unit", "split_combine"])
@pytest.mark.parametrize("name", ["skewed_gqa", "llama3_8b_gqa"])
def test_full_size_comparison_variants(dev, name, variant):
    """The two comparison launches at full size, in the page layout the
    benchmark times, on every output."""
    wl = full_workload(name, W.KV_HND)
    policy, reduce = ((B.POLICY_PER_UNIT, B.REDUCE_FUSED) if variant == "per_unit"
                      else (B.POLICY_STREAMK, B.REDUCE_SPLIT_COMBINE))
    s, plan = run(wl, *dev, policy=policy, reduce=reduce, tag=f"{name}-{variant}")
    compare(s, wl, ref=full_oracle(name), label=f"{name} {variant} HND")
    clean(s, plan)


@pytest.mark.parametrize("policy,reduce", [(B.POLICY_PER_UNIT, B.REDUCE_FUSED),
                                           (B.POLICY_STREAMK, B.REDUCE_SPLIT_COMBINE)])
@pytest.mark.parametrize("name", ["tiny_gqa", "skewed_gqa"])
def test_comparison_variants(dev, policy, reduce, name):
    cfg = W.CONFIG_BY_NAME[name]
    if name == "skewed_gqa":
        cfg = W.small_variant(cfg, batch=6, seqlen_hi=5000)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, policy=policy, reduce=reduce, tag="variant")
    compare(s, wl)
    clean(s, plan)


@pytest.mark.parametrize("unit_cost", [0, None])
@pytest.mark.parametrize("cus", [1, 8, 64, 255, 256, 1024])
def test_split_points_move_with_cu_count(dev, cus, unit_cost):
    cfg = W.small_variant(W.CONFIG_BY_NAME["skewed_gqa"], batch=5, seqlen_hi=4000, seed_offset=cus)
    wl = W.make_workload(cfg)
    s, plan = run(wl, cus, dev[1], unit_cost=unit_cost, tag="cus")
    compare(s, wl)
    clean(s, plan)


def test_repeat_runs_bitwise_identical_and_counters_reset(dev):
    cfg = W.small_variant(W.CONFIG_BY_NAME["skewed_gqa"], batch=8, seqlen_hi=20000)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag="repeat")
    o0, l0 = s.out.clone(), s.lse.clone()
    for i in range(20):
        s.out.fill_(float("nan"))
        s.run()
    torch.cuda.synchronize()
    assert torch.equal(s.out, o0) and torch.equal(s.lse, l0)
    clean(s, plan)


def test_stale_partials_do_not_leak(dev):
    """Partial slots pre-filled with NaN: every slot a merge reads is written first."""
    cfg = W.small_variant(W.CONFIG_BY_NAME["skewed_gqa"], batch=6, seqlen_hi=8000)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag="nan-poison")
    o0, l0 = s.out.clone(), s.lse.clone()
    units = int(plan.view(np.int32)[15])
    partials_off = -(-(256 + 128 * units) // 256) * 256
    assert int(plan.view(np.int32)[18]) > 0, "the case must split some unit"
    s.workspace[partials_off:].view(torch.float32).fill_(float("nan"))
    s.run()
    torch.cuda.synchronize()
    assert torch.equal(s.out, o0) and torch.equal(s.lse, l0)
    clean(s, plan)


def test_page_placement_is_bitwise_irrelevant(dev):
    cfg = W.small_variant(W.CONFIG_BY_NAME["llama3_8b_gqa"], batch=6, seqlen_hi=4000)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag="placement-a")
    o_a = s.out.clone()
    # re-place every page at a different physical slot, same logical content
    perm = np.random.default_rng(3).permutation(wl.num_pages)
    k2 = np.empty_like(wl.k_cache)
    v2 = np.empty_like(wl.v_cache)
    k2[perm] = wl.k_cache
    v2[perm] = wl.v_cache
    bt2 = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    wl2 = W.Workload(wl.cfg, wl.seqlens, bt2, wl.q, k2, v2, None)
    s2, _ = run(wl2, *dev, tag="placement-b")
    assert torch.equal(s2.out, o_a) and torch.equal(s2.lse, s.lse)


@pytest.mark.parametrize("reduce", [B.REDUCE_FUSED, B.REDUCE_SPLIT_COMBINE])
def test_kernel_events_bracket_the_call(dev, reduce):
    """Events set with cc_debug_kernel_events are recorded at the start of the
    call's first kernel and the end of its last: their interval is positive and
    shorter than the same call bracketed by ordinary event records; outputs are
    unchanged; after clearing them a call records nothing."""
    cfg = W.small_variant(W.CONFIG_BY_NAME["skewed_gqa"], batch=8, seqlen_hi=20000)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, reduce=reduce, tag="kernel-events")
    o0 = s.out.clone()
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
        s.run(reduce)  # cleared: must not move a or b
        torch.cuda.synchronize()
        assert a.elapsed_time(b) == kernel_ms[-1]
    assert torch.equal(s.out, o0)
    # the kernel interval is not longer than the marker interval beyond noise
    assert 0 < np.median(kernel_ms) <= 1.05 * np.median(marker_ms)
    clean(s, plan)


@pytest.mark.parametrize("reduce", [B.REDUCE_FUSED, B.REDUCE_SPLIT_COMBINE])
@pytest.mark.parametrize("hkv,hq,d", [(8, 8, 128), (4, 8, 64), (4, 32, 128), (1, 16, 64), (2, 32, 128)])
def test_group_sizes_and_head_dims(dev, hkv, hq, d, reduce):
    """G = 1 (MHA), 2, 8 and 16 at head dims 64 and 128 on ragged batches, every
    output (the workloads themselves all have G = 4)."""
    base = W.small_variant(W.CONFIG_BY_NAME["llama3_8b_gqa"], batch=10, seqlen_hi=2500, seed_offset=hq + hkv + d)
    cfg = dataclasses.replace(base, num_q_heads=hq, num_kv_heads=hkv, head_dim_qk=d, head_dim_v=d,
                              softmax_scale=1 / np.sqrt(d))
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, reduce=reduce, tag=f"G={hq // hkv} d={d}")
    compare(s, wl, label=f"gqa G={hq // hkv} d={d}")
    clean(s, plan)


@pytest.mark.parametrize("layout", [W.KV_NHD, W.KV_HND])
@pytest.mark.parametrize("page", [32, 64, 256, 1024])
def test_page_sizes(dev, page, layout):
    """Pages of 32 to 1024 tokens (the workloads use 16 and one 512-token page):
    32-token blocks lie inside a page or cover several, every output."""
    cfg = dataclasses.replace(W.small_variant(W.CONFIG_BY_NAME["llama3_8b_gqa"], batch=9, seqlen_hi=3000,
                                              seed_offset=page + layout), page_size=page, kv_layout=layout)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, tag=f"gqa page={page} layout={layout}")
    compare(s, wl, label=f"gqa page {page} {'HND' if layout else 'NHD'}")
    clean(s, plan)
