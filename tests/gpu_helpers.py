"""Shared helpers of the GPU parity tests: run a plan through the C ABI and
compare out / lse with the fp64 oracle.

Bars: max|out - oracle| <= 1e-2 and max|lse - oracle| <= 1e-3 (absolute), no
NaN/Inf, for bf16 inputs with fp32 accumulation; a sequence with no cached
tokens must give exactly out = 0 and lse = -inf.

Every comparison's margins (max|dout|, max|dlse|, outputs compared) are
collected in MARGINS; when the environment names a file in CC_PARITY_LOG the
session writes them there as JSON at its end (tests/conftest.py).
"""
import numpy as np

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W
from oracle import attention as A

TOL_OUT, TOL_LSE = 1e-2, 1e-3
MARGINS = []

# full-size workloads and their oracle results, built once per session
_WL, _REF = {}, {}


def full_workload(name, layout=None):
    """The full-size workload `name` (optionally with another page layout), cached."""
    import dataclasses
    key = (name, layout)
    if key not in _WL:
        cfg = W.CONFIG_BY_NAME[name]
        if layout is not None:
            cfg = dataclasses.replace(cfg, kv_layout=layout)
        _WL[key] = W.make_workload(cfg)
    return _WL[key]


def full_oracle(name, layout=None):
    """fp64 oracle (out, lse) of every output of the full-size workload `name`,
    cached (the page layouts hold the same logical values, so one result
    serves both)."""
    if name not in _REF:
        _REF[name] = A.decode_attention_wl(full_workload(name, layout))
    return _REF[name]


def run(wl, cus, xcds, tile=32, policy=B.POLICY_STREAMK, unit_cost=None, reduce=B.REDUCE_FUSED, tag=""):
    import torch
    print(f"[gpu] {tag} cfg={wl.cfg.name} B={wl.cfg.batch} C={cus} X={xcds} T={tile} policy={policy} "
          f"unit_cost={unit_cost} reduce={reduce}", flush=True)
    plan = B.plan(B.problem_for(wl), wl.seqlens, wl.block_table, num_cus=cus, num_xcds=xcds,
                  tile_tokens=tile, policy=policy, unit_cost=unit_cost)
    s = B.session(wl, plan)
    s.run(reduce)
    torch.cuda.synchronize()
    return s, plan


def compare(s, wl, only=None, ref=None, label=None):
    """Element-wise comparison with the oracle; ``only`` = (b, t, kv_head) units to check.

    ``ref`` = a precomputed oracle (out, lse) of every output; ``label`` names
    the case in MARGINS."""
    if ref is None:
        ref_o, ref_l = A.decode_attention_wl(wl, only=only)
    else:
        ref_o, ref_l = ref
    out = s.out.cpu().numpy().astype(np.float64)
    lse = s.lse.cpu().numpy().astype(np.float64)
    if only is not None:
        G = wl.cfg.group
        mask = np.zeros(lse.shape, bool)
        for (b, t, g) in only:
            mask[b, t, g * G:(g + 1) * G] = True
        out, ref_o = out[mask], ref_o[mask]
        lse, ref_l = lse[mask], ref_l[mask]
    # sequences with no cached tokens: exactly out = 0, lse = -inf
    empty = ref_l == -np.inf
    assert np.all(out[empty] == 0) and np.all(lse[empty] == -np.inf)
    out, ref_o, lse, ref_l = out[~empty], ref_o[~empty], lse[~empty], ref_l[~empty]
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    if lse.size == 0:
        return 0.0, 0.0
    do = float(np.max(np.abs(out - ref_o)))
    dl = float(np.max(np.abs(lse - ref_l)))
    print(f"       max|dout|={do:.3e} max|dlse|={dl:.3e} over {out.size} outputs", flush=True)
    MARGINS.append({"case": label or wl.cfg.name, "max_dout": do, "max_dlse": dl, "outputs": int(out.size),
                    "lse_values": int(lse.size)})
    assert do <= TOL_OUT and dl <= TOL_LSE
    return do, dl


def clean(s, plan):
    """Every arrival counter is back at zero and the device raised no data flag."""
    dirty, flags = B.workspace_check(plan, s.workspace)
    assert dirty == 0 and flags == 0
