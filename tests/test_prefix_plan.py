"""Shared-prefix plans (cc_plan_prefix) on the CPU.

The reference planner in the oracle and the C planner must agree byte for
byte.  What the plan must satisfy, checked from first principles: every
member unit (sequence, KV head) sees each of its tokens exactly once, through
its prefix unit's pieces over [0, prefix_len) and its own pieces over
[prefix_len, L), and its split indices are exactly 0 .. nsplit - 1; a prefix
unit gathers at most 16 query rows; a batch with nothing shared plans exactly
as cc_plan does; the tiles read drop by the prefix re-reads saved.
"""
import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W
from oracle import planner as PL


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 8]))
    P = int(rng.choice([16, 32, 64]))
    Bn = int(rng.integers(1, 13))
    NG = int(rng.integers(0, 4))
    lens_p = [int(rng.integers(0, 6)) * P for _ in range(NG)]
    grp = np.array([int(rng.integers(-1, NG)) if NG else -1 for _ in range(Bn)], np.int32)
    sl = np.array([int(rng.integers(0, 700)) + (lens_p[g] if g >= 0 else 0) for g in grp], np.int32)
    C = int(rng.choice([1, 3, 8, 64, 256]))
    X = int(rng.choice([1, 8]))
    T = int(rng.choice([16, 32, 64]))
    O = int(rng.choice([0, 1, 6]))
    return G, Hkv, P, sl, grp, np.array(lens_p, np.int32), C, X, T, O


def _prefix_plan(G, Hkv, P, sl, grp, lp, C, X, T, O, bt=None):
    maxp = max(1, int(max((int(L) + P - 1) // P for L in sl)))
    npages = max(1, int(sum((int(L) + P - 1) // P for L in sl)))
    prob = B.problem(B.MODE_GQA, len(sl), 1, G * Hkv, Hkv, 64, 64, P, maxp, npages, 0, 0.125)
    ref = PL.plan_prefix(0, len(sl), 1, G * Hkv, Hkv, 64, 64, P, maxp, npages, 0, C, X, T, sl, grp, lp, bt, O)
    return prob, ref


def _coverage(ref, sl, grp, lp, Hkv):
    """Per member unit: its (tok_begin, tok_end, split) list, through prefix units."""
    U = len(sl) * Hkv
    got = {u: [] for u in range(U)}
    for its in ref["chunk_items"]:
        for (u, t0, t1, s) in its:
            if u < U:
                got[u].append((t0, t1, s))
            else:
                h, Lp, members = ref["prefix_units"][u - U]
                assert t1 <= Lp
                for b in members:
                    got[b * Hkv + h].append((t0, t1, s))
    return got


@pytest.mark.parametrize("seed", range(60))
def test_prefix_plan_bytes_and_coverage(lib, seed):
    G, Hkv, P, sl, grp, lp, C, X, T, O = _case(seed)
    prob, ref = _prefix_plan(G, Hkv, P, sl, grp, lp, C, X, T, O)
    blob = B.plan_prefix(prob, sl, grp, lp, num_cus=C, num_xcds=X, tile_tokens=T, unit_cost=O)
    assert blob.tobytes() == ref["blob"]
    B.plan_check(blob, prob, sl)
    assert B.workspace_size(blob) > 0
    h = np.frombuffer(ref["blob"][:128], np.int32)
    assert h[26] == len(ref["prefix_units"])
    # every member unit: tokens [0, L) exactly once, splits 0 .. nsplit-1 in token order
    got = _coverage(ref, sl, grp, lp, Hkv)
    for u, lst in got.items():
        L = int(sl[u // Hkv])
        lst.sort(key=lambda x: x[2])
        assert [s for (_, _, s) in lst] == list(range(len(lst)))
        assert ref["unit_nsplit"][u] == len(lst)
        pos = 0
        for (t0, t1, _) in lst:
            assert t0 == pos and t1 > t0
            pos = t1
        assert pos == L
    # prefix units: one per (group with a prefix, KV head, block of 16 / G members)
    for (h_, Lp, members) in ref["prefix_units"]:
        assert 1 <= len(members) <= 16 // G and Lp > 0
        assert all(grp[b] >= 0 and lp[grp[b]] == Lp for b in members)
    # the tiles read: the prefix once per prefix unit instead of once per member
    own = sum(-(-(int(L) - (int(lp[g]) if g >= 0 else 0)) // T) for L, g in zip(sl, grp)) * Hkv
    shared = sum(-(-Lp // T) for (_, Lp, _) in ref["prefix_units"])
    assert ref["num_tiles"] == own + shared


@pytest.mark.parametrize("seed", range(20))
def test_nothing_shared_is_the_plain_plan(lib, seed):
    """No group, or groups whose prefix is 0 tokens: the same pieces as cc_plan."""
    G, Hkv, P, sl, grp, lp, C, X, T, O = _case(seed)
    prob, _ = _prefix_plan(G, Hkv, P, sl, grp, lp, C, X, T, O)
    plain = B.plan(prob, sl, None, num_cus=C, num_xcds=X, tile_tokens=T, heads_per_unit=G, unit_cost=O)
    for g2, l2 in ((np.full(len(sl), -1, np.int32), lp), (grp, np.zeros_like(lp))):
        b2 = B.plan_prefix(prob, sl, g2, l2, num_cus=C, num_xcds=X, tile_tokens=T, unit_cost=O)
        assert b2.tobytes() == plain.tobytes()


def test_workload_shared_prefix_shape(lib):
    """The shared-prefix workload: one 4096-token prefix for all 64 sequences,
    read by 8 KV heads x 16 prefix units of 4 members."""
    cfg = W.CONFIG_BY_NAME["shared_prefix_gqa"]
    wl = W.make_workload(cfg)
    assert (wl.prefix_group == 0).all() and list(wl.prefix_len) == [cfg.prefix_len]
    prob = B.problem_for(wl)
    blob = B.plan_prefix(prob, wl.seqlens, wl.prefix_group, wl.prefix_len, wl.block_table)
    ref = PL.plan_prefix(cfg.mode, cfg.batch, 1, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim_qk,
                         cfg.head_dim_v, cfg.page_size, wl.max_pages, wl.num_pages, 0, 256, 8, 32, wl.seqlens,
                         wl.prefix_group, wl.prefix_len, wl.block_table, B.UNIT_COST_GQA)
    assert blob.tobytes() == ref["blob"]
    assert len(ref["prefix_units"]) == 8 * 16
    # every member's block-table row names the same prefix pages
    npg = cfg.prefix_len // cfg.page_size
    assert (wl.block_table[:, :npg] == wl.block_table[0, :npg]).all()


@pytest.mark.parametrize("bad", ["not_pages", "short_member", "pages_differ", "group_id", "mla", "g3"])
def test_prefix_inputs_rejected(lib, bad):
    sl = np.array([100, 70, 64], np.int32)
    grp = np.array([0, 0, -1], np.int32)
    lp = np.array([64], np.int32)
    bt = np.array([[0, 1, 2, 3, 4, 5, 6], [0, 1, 2, 3, 7, 8, -1], [9, 10, 11, 12, -1, -1, -1]], np.int32)
    kw = dict(mode=B.MODE_GQA, batch=3, q_tokens=1, num_q_heads=8, num_kv_heads=2, head_dim_qk=64,
              head_dim_v=64, page_size=16, max_pages_per_seq=7, num_pages=13, topk=0, softmax_scale=0.125)
    if bad == "not_pages":
        lp = np.array([40], np.int32)
    elif bad == "short_member":
        lp = np.array([80], np.int32)
    elif bad == "pages_differ":
        bt[1, 2] = 12
    elif bad == "group_id":
        grp = np.array([0, 1, -1], np.int32)
    elif bad == "mla":
        kw.update(mode=B.MODE_MLA, num_q_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512)
    elif bad == "g3":
        kw.update(num_q_heads=6)
    prob = B.problem(**kw)
    with pytest.raises(B.CrossCUError) as ei:
        B.plan_prefix(prob, sl, grp, lp, bt, num_cus=8, num_xcds=1)
    assert ei.value.code == B.CC_ERR_INVALID
    if bad not in ("mla",):
        with pytest.raises(ValueError):
            PL.plan_prefix(kw["mode"], 3, 1, kw["num_q_heads"], kw["num_kv_heads"], 64, 64, 16, 7, 13, 0, 8, 1, 32,
                           sl, grp, lp, bt)
