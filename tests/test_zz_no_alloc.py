"""cc_decode_noalloc (the library's own scratch array instead of a caller
workspace) against cc_decode with a workspace, through the C ABI.

The two entry points run the same kernels on the same plan, so their out and
lse must agree bit for bit (the merges combine splits in a fixed order).  Each
case makes two no-allocation calls in a row, the second on a smaller input
(fewer sequences, so a smaller plan and workspace): the scratch array keeps
the first call's contents, and the second must not see them.  A plan whose
workspace exceeds the array is refused on the host.
"""
import dataclasses

import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W

from gpu_helpers import TOL_LSE, TOL_OUT, compare

torch = pytest.importorskip("torch")


def _noalloc(s, stream=None):
    B.decode_noalloc(s.prob, s.plan_host, s.plan_dev, s.q, s.k, s.v, s.block_table, s.seqlens, s.indices,
                     s.out, s.lse, stream)


def _session(cfg, dev):
    wl = W.make_workload(cfg)
    plan = B.plan(B.problem_for(wl), wl.seqlens, wl.block_table, num_cus=dev[0], num_xcds=dev[1])
    assert B.workspace_size(plan) <= B.NOALLOC_WORKSPACE_BYTES
    return wl, plan, B.session(wl, plan)


CASES = [
    ("skewed_gqa", dict(batch=12, seqlen_hi=20000), dict(batch=5, seqlen_hi=3000)),
    ("llama3_8b_gqa", None, dict(batch=9, seqlen_hi=4000)),
    ("deepseek_mla", None, dict(batch=6, seqlen_hi=5000)),
    ("sparse_mla", None, dict(batch=1, seqlen_hi=3000)),
    ("tiny_gqa", None, dict(batch=2, seqlen_hi=300)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,first,second", CASES)
def test_noalloc_matches_cc_decode_on_two_calls(dev, name, first, second):
    base = W.CONFIG_BY_NAME[name]
    if name in ("skewed_gqa", "llama3_8b_gqa"):
        base = dataclasses.replace(base, kv_layout=W.KV_HND)
    cfg1 = base if first is None else W.small_variant(base, seed_offset=41, **first)
    cfg2 = W.small_variant(base, seed_offset=42, **second)
    sizes = []
    for i, cfg in enumerate((cfg1, cfg2)):
        wl, plan, s = _session(cfg, dev)
        sizes.append(B.workspace_size(plan))
        print(f"[gpu] noalloc {name} call {i}: batch {cfg.batch}, workspace {sizes[-1]} B", flush=True)
        s.run()
        torch.cuda.synchronize()
        ref_o, ref_l = s.out.clone(), s.lse.clone()
        s.out.fill_(float("nan"))
        s.lse.fill_(float("nan"))
        _noalloc(s)
        torch.cuda.synchronize()
        assert torch.equal(s.out, ref_o) and torch.equal(s.lse, ref_l)
        if i == 1:   # the smaller call also meets the oracle bars
            compare(s, wl, label=f"{name} noalloc second call")
    assert sizes[1] < sizes[0]


@pytest.mark.gpu
def test_noalloc_after_a_plan_with_fewer_units(dev):
    """A plan with 96 units (its partials right after their counters in a
    plan-sized workspace), then one with 512: in the scratch array the second
    plan's counters must still start at zero, wherever the first kept its
    partials."""
    small = W.small_variant(dataclasses.replace(W.CONFIG_BY_NAME["skewed_gqa"], kv_layout=W.KV_HND),
                            batch=12, seqlen_hi=20000, seed_offset=44)
    big = dataclasses.replace(W.CONFIG_BY_NAME["llama3_8b_gqa"], kv_layout=W.KV_HND)
    for cfg in (small, big, small):
        wl, plan, s = _session(cfg, dev)
        print(f"[gpu] noalloc growing plans: {cfg.name} units {int(plan.view(np.int32)[15])}", flush=True)
        s.run()
        torch.cuda.synchronize()
        ref_o, ref_l = s.out.clone(), s.lse.clone()
        s.out.fill_(float("nan"))
        _noalloc(s)
        torch.cuda.synchronize()
        assert torch.equal(s.out, ref_o) and torch.equal(s.lse, ref_l)


@pytest.mark.gpu
def test_noalloc_repeated_calls_stay_identical(dev):
    """Counters left by one call are what the next starts from: ten calls in a
    row on one stream give the same bits."""
    cfg = W.small_variant(W.CONFIG_BY_NAME["deepseek_mla"], batch=8, seqlen_hi=9000, seed_offset=43)
    wl, plan, s = _session(cfg, dev)
    _noalloc(s)
    torch.cuda.synchronize()
    o0, l0 = s.out.clone(), s.lse.clone()
    for _ in range(10):
        s.out.fill_(float("nan"))
        _noalloc(s)
    torch.cuda.synchronize()
    assert torch.equal(s.out, o0) and torch.equal(s.lse, l0)


def test_noalloc_refuses_a_plan_larger_than_its_array(lib):
    """Host check, before any device work: 1024 chunks over 64 MLA sequences of
    16K tokens need ~136 MB of partials."""
    import ctypes
    sl = np.full(64, 16384, np.int32)
    prob = B.problem(B.MODE_MLA, 64, 1, 128, 1, 576, 512, 64, 256, 64 * 256, 0, 1 / 192 ** 0.5)
    plan = B.plan(prob, sl, None, num_cus=1024, num_xcds=8)
    assert B.workspace_size(plan) > B.NOALLOC_WORKSPACE_BYTES
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the size check fails first
    rc = lib.cc_decode_noalloc(ctypes.byref(prob), plan.ctypes.data_as(ctypes.c_void_p), fake, fake, fake, None,
                               fake, fake, None, fake, fake, None)
    assert rc == B.CC_ERR_BUFFER
    assert b"scratch array" in lib.cc_last_error()
