"""GPU parity of the MoE grouped GEMM (cc_moe_plan + cc_moe_gemm) against the
fp64 oracle, through the C ABI.

Bar: bf16 products are exact in fp32 and the GPU adds K of them (and up to a
few split partials) in fp32 in some order, so |y - oracle| <= 2 gamma_K S per
element, S = sum_k |x_k w_k| (Higham, "Accuracy and Stability of Numerical
Algorithms", section 3.1; the factor 2 covers the partial sums of a split
tile), and no NaN/Inf.  Cases: several expert counts (empty experts, experts
whose rows do not fill a tile, one row), hidden and output sizes, 1 to 1024
chunks, both unit costs, one workgroup per tile, split + combine, repeat runs
with poisoned partial slots, and the full-size 64-expert workload on every
output.
"""
import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W
from oracle import moe as M

from gpu_helpers import MARGINS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CFG = W.MOE_BY_NAME["moe_grouped_gemm"]
_FULL = {}


def run(wl, cus, xcds, policy=B.POLICY_STREAMK_DP, unit_cost=None, reduce=B.REDUCE_FUSED, tag=""):
    c = wl.cfg
    print(f"[gpu] moe {tag} E={c.num_experts} K={c.hidden} N={c.out_dim} rows={int(wl.expert_tokens.sum())} C={cus} "
          f"policy={policy} unit_cost={unit_cost} reduce={reduce}", flush=True)
    plan = B.moe_plan(B.moe_problem(c.num_experts, c.hidden, c.out_dim), wl.expert_tokens, num_cus=cus,
                      num_xcds=xcds, policy=policy, unit_cost=unit_cost)
    s = B.moe_session(wl, plan)
    s.y.fill_(float("nan"))
    s.run(reduce)
    torch.cuda.synchronize()
    return s, plan


def check(s, wl, ref=None, label=None):
    if ref is None:
        ref = (M.grouped_gemm(wl.x, wl.w, wl.offsets), M.abs_product_sums(wl.x, wl.w, wl.offsets))
    y = s.y.cpu().numpy().astype(np.float64)
    want, scale = ref
    assert np.all(np.isfinite(y))
    err = np.abs(y - want)
    bound = 2 * M.gamma(wl.cfg.hidden) * scale
    ratio = float((err / np.maximum(bound, 1e-300)).max())
    print(f"       max|dy|={err.max():.3e}  max|dy|/bound={ratio:.3f}", flush=True)
    MARGINS.append({"case": label or wl.cfg.name, "max_dy": float(err.max()), "max_dy_over_bound": ratio,
                    "outputs": int(y.size)})
    assert np.all(err <= bound)


def clean(s, plan):
    dirty, flags = B.workspace_check(plan, s.workspace)
    assert dirty == 0 and flags == 0


@pytest.mark.parametrize("policy", [B.POLICY_STREAMK, B.POLICY_STREAMK_DP])
@pytest.mark.parametrize("cus", [1, 8, 64, 256, 1024])
@pytest.mark.parametrize("counts", [[300, 0, 5, 1000, 128, 129, 1], [40], [0, 0, 257, 0]])
def test_small_expert_mixes(dev, counts, cus, policy):
    cfg = W.small_moe(CFG, num_experts=len(counts), hidden=512, out_dim=512, tokens=2048, top_k=1,
                      seed_offset=len(counts) + cus)
    wl = W.make_moe_workload(cfg, expert_tokens=counts)
    s, plan = run(wl, cus, dev[1], policy=policy, tag="mix")
    check(s, wl)
    clean(s, plan)


@pytest.mark.parametrize("K,N", [(64, 256), (1024, 512), (4096, 256)])
@pytest.mark.parametrize("unit_cost", [0, None])
def test_shapes_and_unit_costs(dev, K, N, unit_cost):
    cfg = W.small_moe(CFG, num_experts=8, hidden=K, out_dim=N, tokens=512, top_k=2, seed_offset=K + N)
    wl = W.make_moe_workload(cfg)
    s, plan = run(wl, dev[0], dev[1], unit_cost=unit_cost, tag="shape")
    check(s, wl)
    clean(s, plan)


@pytest.mark.parametrize("policy,reduce", [(B.POLICY_PER_UNIT, B.REDUCE_FUSED),
                                           (B.POLICY_STREAMK, B.REDUCE_SPLIT_COMBINE)])
def test_comparison_launches(dev, policy, reduce):
    cfg = W.small_moe(CFG, num_experts=16, hidden=1024, out_dim=512, tokens=1024, top_k=4, seed_offset=3)
    wl = W.make_moe_workload(cfg)
    s, plan = run(wl, dev[0], dev[1], policy=policy, reduce=reduce, tag="variant")
    check(s, wl)
    clean(s, plan)


def test_repeat_runs_and_poisoned_partials(dev):
    cfg = W.small_moe(CFG, num_experts=16, hidden=2048, out_dim=512, tokens=1024, top_k=4, seed_offset=4)
    wl = W.make_moe_workload(cfg)
    s, plan = run(wl, dev[0], dev[1], tag="repeat")
    assert int(plan.view(np.int32)[18]) > 0, "the case must split some tile"
    y0 = s.y.clone()
    units = int(plan.view(np.int32)[15])
    partials_off = -(-(256 + 128 * units) // 256) * 256
    for i in range(10):
        s.y.fill_(float("nan"))
        if i % 2:
            s.workspace[partials_off:].view(torch.float32).fill_(float("nan"))
        s.run()
    torch.cuda.synchronize()
    assert torch.equal(s.y, y0)
    clean(s, plan)


def _full():
    if not _FULL:
        wl = W.make_moe_workload(CFG)
        _FULL["wl"] = wl
        _FULL["ref"] = (M.grouped_gemm(wl.x, wl.w, wl.offsets), M.abs_product_sums(wl.x, wl.w, wl.offsets))
    return _FULL["wl"], _FULL["ref"]


@pytest.mark.parametrize("variant", ["fused", "fused_contiguous", "per_unit", "split_combine"])
def test_full_size_every_output(dev, variant):
    """64 experts, hidden 4096, output 2048, 32768 routed rows (Zipf-skewed),
    in the launch configuration the benchmark times (one workgroup per
    compute unit)."""
    wl, ref = _full()
    policy, reduce = {"fused": (B.POLICY_STREAMK_DP, B.REDUCE_FUSED),
                      "fused_contiguous": (B.POLICY_STREAMK, B.REDUCE_FUSED),
                      "per_unit": (B.POLICY_PER_UNIT, B.REDUCE_FUSED),
                      "split_combine": (B.POLICY_STREAMK_DP, B.REDUCE_SPLIT_COMBINE)}[variant]
    s, plan = run(wl, dev[0] * B.MOE_WORKGROUPS_PER_CU, dev[1], policy=policy, reduce=reduce, tag=f"full {variant}")
    check(s, wl, ref, label=f"moe_grouped_gemm {variant}")
    clean(s, plan)
