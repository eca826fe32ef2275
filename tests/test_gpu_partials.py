"""The GPU's own split partials, against the oracle and through its merge.

After a call the workspace still holds every split piece's partial (m, l, o),
which the last arriver (fused) or the combine kernel (split + combine) read.
Each piece covers tokens [t0, t1) of its unit's key set (the plan's item), so
the oracle's partial state over exactly those keys pins it:

- the piece's lse must match the oracle's to 1e-3, and its normalised output
  o / l to the bound the arithmetic gives a single piece.  The kernels keep m
  in base 2 (scores scaled by log2 e), so l and o are the same values as with
  natural exponentials and the piece's lse is m ln 2 + ln l.  The sum l adds
  the fp32 weights while the P.V product takes them rounded to bf16
  (relative error <= 2^-9 each), so o / l is a weighted mean of the piece's
  values off by at most 2^-9 max |v|; the MLA kernels store o / r in fp16
  with the row scale r = max |o| beside m and l (o is rebuilt as fp16 x r),
  which adds at most 2^-11 max |v|.  Bar: 1.1 (2^-9 + 2^-11) max |v| over the
  piece's keys.  (A whole output averages many keys and meets the usual
  1e-2; a piece of a few dozen keys need not.)
- Merging the GPU's partials with the oracle's fp64 LSE merge, in split
  order, must reproduce the GPU's own merged out and lse to fp32 rounding
  (the same partials, merged in fp32 on the GPU), and the oracle's unsplit
  result to the usual bars.

This is the split + merge invariant run on the GPU's partials rather than on
the oracle's own (MeldKernel summary, "Core method": partial outputs feed the
just-in-time reduction).
"""
import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W
from oracle import attention as A

from gpu_helpers import TOL_LSE, TOL_OUT, clean, run

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LN2 = float(np.log(2.0))
# fp32 merge of the same partials on the GPU against the fp64 merge: a few
# dozen fp32 roundings of values of magnitude <= max |v| (N(0,1) bf16 values,
# |v| < 8) and of lse values of a few units: well inside 1e-4.
TOL_MERGE_OUT, TOL_MERGE_LSE = 1e-4, 1e-4
PIECE_REL = 1.1 * (2.0 ** -9 + 2.0 ** -11)


def _plan_tables(plan):
    """Items [W][4] (unit, t0, t1, split), unit_nsplit [U], unit_pbase [U] of a plan blob."""
    w = plan.view(np.int32)
    C, U, Wn = int(w[11]), int(w[15]), int(w[17])
    off_items = 32 + ((C + 1 + 3) // 4) * 4
    items = w[off_items:off_items + 4 * Wn].reshape(Wn, 4)
    ns = w[off_items + 4 * Wn:off_items + 4 * Wn + U]
    pb = w[off_items + 4 * Wn + U:off_items + 4 * Wn + 2 * U]
    return items, ns, pb, U, int(w[14])  # H_HPU


def _slot_floats(mode, hpu, dv):
    if mode == W.MODE_GQA:
        return (((2 * hpu + 3) & ~3) + hpu * dv + 63) & ~63
    return (3 * hpu + (hpu * dv + 1) // 2 + 63) & ~63


def _read_slot(ws_bytes, partials_off, slot, slot_floats, mode, hpu, dv):
    """(m in base 2, l, o) of partial slot `slot`, as float64."""
    base = partials_off + 4 * slot * slot_floats
    f = np.frombuffer(ws_bytes, dtype=np.float32, count=slot_floats, offset=base).astype(np.float64)
    m, l = f[:hpu], f[hpu:2 * hpu]
    if mode == W.MODE_GQA:
        o_off = (2 * hpu + 3) & ~3
        o = f[o_off:o_off + hpu * dv].reshape(hpu, dv)
    else:
        r = f[2 * hpu:3 * hpu]
        h = np.frombuffer(ws_bytes, dtype=np.float16, count=hpu * dv, offset=base + 4 * 3 * hpu)
        o = h.astype(np.float64).reshape(hpu, dv) * r[:, None]
    return m, l, o


def _unit_keys(wl, u, hpu):
    """(b, t, query heads, K rows, V rows) of unit u over its whole key set."""
    c = wl.cfg
    Hkv, Tq = c.num_kv_heads, c.q_tokens
    G = c.num_q_heads // Hkv
    bpk = G // hpu
    per_seq = Tq * Hkv * bpk
    b, rem = divmod(u, per_seq)
    t, rem = divmod(rem, Hkv * bpk)
    g, hb = divmod(rem, bpk)
    heads = np.arange(g * G + hb * hpu, g * G + (hb + 1) * hpu)
    k_bits, v_bits = wl.k_cache, wl.v_cache
    if wl.kv_layout == W.KV_HND:
        k_bits = k_bits.transpose(0, 2, 1, 3)
        v_bits = None if v_bits is None else v_bits.transpose(0, 2, 1, 3)
    J = A.key_positions(b, t, wl.seqlens, wl.indices)
    K = A.gather_rows(k_bits, wl.block_table, b, J, c.page_size, head=g)
    V = A.gather_rows(v_bits, wl.block_table, b, J, c.page_size, head=g) if v_bits is not None \
        else K[:, :c.head_dim_v]
    q = A.bf16_to_f64(wl.q[b, t, heads])
    return b, t, heads, q, K, V


def _check_partials(s, wl, plan, label):
    c = wl.cfg
    items, ns, pb, U, hpu = _plan_tables(plan)
    dv = c.head_dim_v
    sf = _slot_floats(c.mode, hpu, dv)
    partials_off = -(-(256 + 128 * U) // 256) * 256
    ws = s.workspace.cpu().numpy().tobytes()
    out = s.out.cpu().numpy().astype(np.float64)
    lse = s.lse.cpu().numpy().astype(np.float64)
    split_units = [u for u in range(U) if ns[u] > 1]
    assert split_units, "the case must split some unit"
    worst = dict(piece_out_over_bound=0.0, piece_out=0.0, piece_lse=0.0, merge_out=0.0, merge_lse=0.0, oracle_out=0.0, oracle_lse=0.0)
    pieces = 0
    for u in split_units:
        b, t, heads, q, K, V = _unit_keys(wl, u, hpu)
        its = items[items[:, 0] == u]
        its = its[np.argsort(its[:, 3])]
        assert list(its[:, 3]) == list(range(ns[u])), f"unit {u}: splits {its[:, 3]}"
        parts = []
        for (_, t0, t1, sp) in its:
            m2, l, o = _read_slot(ws, partials_off, int(pb[u]) + int(sp), sf, c.mode, hpu, dv)
            rm, rl, ro = A.partial_state(q, K[t0:t1], V[t0:t1], c.softmax_scale)
            assert np.all(np.isfinite(m2)) and np.all(l > 0) and np.all(np.isfinite(o))
            err = float(np.max(np.abs(o / l[:, None] - ro / rl[:, None])))
            worst["piece_out"] = max(worst["piece_out"], err)
            worst["piece_out_over_bound"] = max(worst["piece_out_over_bound"],
                                                err / (PIECE_REL * float(np.max(np.abs(V[t0:t1])))))
            worst["piece_lse"] = max(worst["piece_lse"], float(np.max(np.abs(m2 * LN2 + np.log(l)
                                                                                - (rm + np.log(rl))))))
            parts.append((m2 * LN2, l, o))
            pieces += 1
        mo, ml = A.lse_merge(parts)
        go, gl = out[b, t, heads], lse[b, t, heads]
        worst["merge_out"] = max(worst["merge_out"], float(np.max(np.abs(mo - go))))
        worst["merge_lse"] = max(worst["merge_lse"], float(np.max(np.abs(ml - gl))))
        fo, fl = A.attend(q, K, V, c.softmax_scale)
        worst["oracle_out"] = max(worst["oracle_out"], float(np.max(np.abs(mo - fo))))
        worst["oracle_lse"] = max(worst["oracle_lse"], float(np.max(np.abs(ml - fl))))
    print(f"       {label}: {len(split_units)} split units, {pieces} pieces; "
          + " ".join(f"{k}={v:.2e}" for k, v in worst.items()), flush=True)
    assert worst["piece_out_over_bound"] <= 1.0 and worst["piece_lse"] <= TOL_LSE
    assert worst["merge_out"] <= TOL_MERGE_OUT and worst["merge_lse"] <= TOL_MERGE_LSE
    assert worst["oracle_out"] <= TOL_OUT and worst["oracle_lse"] <= TOL_LSE


@pytest.mark.parametrize("reduce", [B.REDUCE_FUSED, B.REDUCE_SPLIT_COMBINE])
@pytest.mark.parametrize("layout", [W.KV_NHD, W.KV_HND])
def test_gqa_partials(dev, reduce, layout):
    import dataclasses
    cfg = dataclasses.replace(W.small_variant(W.CONFIG_BY_NAME["skewed_gqa"], batch=6, seqlen_hi=8000),
                              kv_layout=layout)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, reduce=reduce, tag=f"gqa partials layout={layout}")
    _check_partials(s, wl, plan, f"gqa layout={layout} reduce={reduce}")
    clean(s, plan)


@pytest.mark.parametrize("reduce", [B.REDUCE_FUSED, B.REDUCE_SPLIT_COMBINE])
@pytest.mark.parametrize("name", ["deepseek_mla", "sparse_mla"])
def test_mla_partials(dev, name, reduce):
    base = W.CONFIG_BY_NAME[name]
    cfg = W.small_variant(base, batch=4 if name == "deepseek_mla" else 2, seqlen_hi=3000)
    wl = W.make_workload(cfg)
    s, plan = run(wl, *dev, reduce=reduce, tag=f"{name} partials")
    _check_partials(s, wl, plan, f"{name} reduce={reduce}")
    clean(s, plan)
