"""Determinism: 100 calls in a row give the same bits, call by call.

The merge of a split unit combines its partials in split-index order whichever
piece arrives last, and every other sum runs in a fixed order, so repeated
calls on the same inputs and plan must agree bitwise with the first one, not
only at the end of a run of calls.  Each call overwrites the outputs with NaN
first; the comparison with the first call's bits runs on the device after
every call and is read back once.  Full-size workloads in the benchmark's
launch configuration, for both reductions of the decode kernels (the fused
merge and split + combine) and for the MoE grouped GEMM.  The workspace is
clean afterwards (every arrival counter back at zero, no data flag).
"""
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W

from gpu_helpers import clean, full_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CALLS = 100


def _repeat(run, outs):
    """Run `run` CALLS times; count, per call, the outputs whose bits differ from the first call's."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    bad = torch.zeros((), dtype=torch.int64, device=outs[0].device)
    for _ in range(CALLS):
        for o in outs:
            o.fill_(float("nan"))
        run()
        for o, r in zip(outs, ref):
            # bitwise: the same bytes (NaN would differ from itself under ==)
            bad += (o.view(torch.int32) != r.view(torch.int32)).any().to(torch.int64)
    return int(bad.item())


@pytest.mark.parametrize("name", ["skewed_gqa", "deepseek_mla", "sparse_mla", "shared_prefix_gqa"])
@pytest.mark.parametrize("reduce", [B.REDUCE_FUSED, B.REDUCE_SPLIT_COMBINE])
def test_decode_100_calls_bitwise(dev, name, reduce):
    cus, xcds = dev
    print(f"[gpu] determinism {name} reduce={reduce} x{CALLS}", flush=True)
    if name == W.SHARED_PREFIX.name:   # the prefix plan: prefix units shared by their groups
        wl = W.make_workload(W.SHARED_PREFIX)
        plan = B.plan_prefix(B.problem_for(wl), wl.seqlens, wl.prefix_group, wl.prefix_len, wl.block_table,
                             num_cus=cus, num_xcds=xcds)
    else:
        wl = full_workload(name)
        plan = B.plan(B.problem_for(wl), wl.seqlens, wl.block_table, num_cus=cus, num_xcds=xcds)
    s = B.session(wl, plan)
    assert _repeat(lambda: s.run(reduce), [s.out, s.lse]) == 0
    clean(s, plan)


def test_moe_100_calls_bitwise(dev):
    wl = W.make_moe_workload(W.MOE_BY_NAME["moe_grouped_gemm"])
    c = wl.cfg
    cus, xcds = dev
    print(f"[gpu] determinism moe x{CALLS}", flush=True)
    plan = B.moe_plan(B.moe_problem(c.num_experts, c.hidden, c.out_dim), wl.expert_tokens, num_cus=cus,
                      num_xcds=xcds, policy=B.POLICY_STREAMK_DP)
    s = B.moe_session(wl, plan)
    assert _repeat(lambda: s.run(), [s.y]) == 0
    dirty, flags = B.workspace_check(plan, s.workspace)
    assert dirty == 0 and flags == 0
