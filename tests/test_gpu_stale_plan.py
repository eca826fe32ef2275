"""A plan used with sequence lengths it was not built for (through the C ABI).

cc_plan_check refuses such a plan on the host (the plan's header holds a hash
of the lengths it was built for).  cc_decode takes its lengths in device
memory, so its kernels check instead: a piece ending past its sequence, or a
unit's last piece ending before it, sets bit 0 of the workspace error word
and the affected sequences come out NaN — never a plausible wrong answer.
Cases: the plan built for a shorter and for a longer sequence, for an empty
sequence that now has tokens, and for a non-empty one that is now empty.
In the GQA kernel only the mismatching sequence is poisoned, so the other
sequences still meet the oracle bars; the MLA kernel poisons every unit of a
workgroup that holds a mismatching piece.
"""
import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W
from oracle import attention as A

from gpu_helpers import TOL_LSE, TOL_OUT

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SEQ = np.array([3000, 700, 45, 5000, 129, 2048], np.int32)


def _plan_lengths(kind):
    """(actual lengths, lengths the plan is built for, the stale sequence)."""
    actual, planned = SEQ.copy(), SEQ.copy()
    if kind == "shorter":          # the sequence grew by a token since the plan
        planned[1] -= 1
        b = 1
    elif kind == "shorter_tiles":  # ... by several tiles
        planned[3] -= 100
        b = 3
    elif kind == "longer":         # the plan covers tokens the sequence does not have
        planned[2] += 3
        b = 2
    elif kind == "was_empty":      # planned as empty, has tokens now
        planned[4] = 0
        b = 4
    else:                          # "now_empty": planned with tokens, empty now
        actual[5] = 0
        b = 5
    return actual, planned, b


@pytest.mark.parametrize("kind", ["shorter", "shorter_tiles", "longer", "was_empty", "now_empty"])
@pytest.mark.parametrize("name", ["skewed_gqa", "deepseek_mla"])
def test_stale_plan_is_flagged_and_poisoned(dev, name, kind):
    actual, planned, b = _plan_lengths(kind)
    cfg = W.small_variant(W.CONFIG_BY_NAME[name], batch=len(SEQ), seqlen_hi=6000, seed_offset=31)
    # the cache holds pages for the longer of the two lengths of every sequence
    wl = W.make_workload(cfg, seqlens=np.maximum(actual, planned))
    wl.seqlens = actual.copy()
    prob = B.problem_for(wl)
    print(f"[gpu] stale plan {name} {kind}: sequence {b} planned {planned[b]} actual {actual[b]}", flush=True)
    plan = B.plan(prob, planned, None, num_cus=dev[0], num_xcds=dev[1])
    with pytest.raises(B.CrossCUError) as ei:
        B.plan_check(plan, prob, actual)
    assert ei.value.code == B.CC_ERR_PLAN
    B.plan_check(plan, prob, planned)
    s = B.session(wl, plan)
    s.run()
    dirty, flags = B.workspace_check(plan, s.workspace)
    assert dirty == 0
    assert flags & 1, "the seqlen bit of the error word"
    out = s.out.cpu().numpy()
    lse = s.lse.cpu().numpy()
    assert np.all(np.isnan(out[b])) and np.all(np.isnan(lse[b]))
    if cfg.mode == W.MODE_GQA:     # the other sequences are untouched
        ref_o, ref_l = A.decode_attention_wl(wl)
        keep = np.arange(len(SEQ)) != b
        assert np.max(np.abs(out[keep] - ref_o[keep])) <= TOL_OUT
        assert np.max(np.abs(lse[keep] - ref_l[keep])) <= TOL_LSE
    # the same workspace with a plan for the actual lengths: clean again, right answer
    good = B.plan(prob, actual, wl.block_table, num_cus=dev[0], num_xcds=dev[1])
    s2 = B.session(wl, good)
    s2.run()
    dirty, flags = B.workspace_check(good, s2.workspace)
    assert dirty == 0 and flags == 0
    ref_o, ref_l = A.decode_attention_wl(wl)
    o2, l2 = s2.out.cpu().numpy(), s2.lse.cpu().numpy()
    empty = ref_l == -np.inf
    assert np.all(o2[empty] == 0) and np.all(l2[empty] == -np.inf)
    assert np.max(np.abs(o2[~empty] - ref_o[~empty])) <= TOL_OUT
    assert np.max(np.abs(l2[~empty] - ref_l[~empty])) <= TOL_LSE
