"""Shared helpers of the GPU parity tests: run a plan through the C ABI and
compare out / lse with the fp64 oracle.

Bars: max|out - oracle| <= 1e-2 and max|lse - oracle| <= 1e-3 (absolute), no
NaN/Inf, for bf16 inputs with fp32 accumulation; a sequence with no cached
tokens must give exactly out = 0 and lse = -inf.
"""
import numpy as np

from cross_cu_load_amd import binding as B
from oracle import attention as A

TOL_OUT, TOL_LSE = 1e-2, 1e-3


def run(wl, cus, xcds, tile=32, policy=B.POLICY_STREAMK_COST, reduce=B.REDUCE_FUSED, tag=""):
    import torch
    print(f"[gpu] {tag} cfg={wl.cfg.name} B={wl.cfg.batch} C={cus} X={xcds} T={tile} policy={policy} "
          f"reduce={reduce}", flush=True)
    plan = B.plan(B.problem_for(wl), wl.seqlens, wl.block_table, num_cus=cus, num_xcds=xcds,
                  tile_tokens=tile, policy=policy)
    s = B.session(wl, plan)
    s.run(reduce)
    torch.cuda.synchronize()
    return s, plan


def compare(s, wl, only=None):
    """Element-wise comparison with the oracle; ``only`` = (b, t, kv_head) units to check."""
    ref_o, ref_l = A.decode_attention_wl(wl, only=only)
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
    print(f"       max|dout|={do:.3e} max|dlse|={dl:.3e}", flush=True)
    assert do <= TOL_OUT and dl <= TOL_LSE
    return do, dl


def clean(s, plan):
    """Every arrival counter is back at zero and the device raised no data flag."""
    dirty, flags = B.workspace_check(plan, s.workspace)
    assert dirty == 0 and flags == 0
