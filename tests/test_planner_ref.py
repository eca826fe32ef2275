"""Pins of the reference Stream-K planner (CPU only).

The printed facts it is held to: the 732-tasks-over-148-workers split (140 of
5, 8 of 4) and the 4-SM tail-effect timeline.  Everything else is checked by
invariants (every tile exactly once, chunks within one tile of each other,
split counts, partial slots, XCD placement) and by a tile-by-tile brute force
on small inputs, which assigns each tile to a chunk one at a time instead of
cutting ranges.
"""
import json
import os

import numpy as np
import pytest

from cross_cu_load_amd import workloads as W
from oracle import planner as PL

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _plan(lens, C=8, X=1, T=4, G=1, Hkv=1, mode=PL.MODE_GQA, Tq=1, topk=0, hu=None, policy=PL.POLICY_STREAMK):
    lens = np.asarray(lens, np.int32)
    P = 16
    maxp = max(1, int(max((int(L) + P - 1) // P for L in lens)))
    return PL.plan(mode, len(lens), Tq, G * Hkv, Hkv, 64, 64, P, maxp, 1 << 20, topk, C, X, T,
                   hu if hu is not None else G, lens, None, policy)


def test_golden_732_tasks_over_148_workers():
    g = json.load(open(os.path.join(GOLD, "kernelplan_732_tasks_148_workers.json")))
    # 732 one-tile units over 148 chunks
    p = _plan([4] * g["tasks"], C=g["workers"], X=1, T=4)
    sizes = np.diff(p["wg_off"])
    assert int((sizes == 5).sum()) == g["workers_with_5"]
    assert int((sizes == 4).sum()) == g["workers_with_4"]
    assert p["num_tiles"] == g["tasks"]


def test_golden_tail_effect_and_equal_split():
    g = json.load(open(os.path.join(GOLD, "tail_effect_4sm.json")))
    makespan, finish, assign = PL.list_schedule(g["task_ms"], g["num_sms"])
    assert makespan == g["makespan_ms"]
    assert finish == g["finish_ms"]
    assert assign == g["assignment"]
    idle = [makespan - f for f in finish]
    lo, hi = g["idle_window_ms"]
    assert idle[:3] == [hi - lo] * 3 and idle[3] == 0
    # the same work cut into one equal chunk per SM (the Stream-K reading):
    # 620 ms of work in 4 chunks of 155 ms
    total = sum(g["task_ms"])
    per_ms = 5  # cut each task into 5 ms tiles
    tiles = [per_ms] * (total // per_ms)
    p = _plan([1] * len(tiles), C=g["num_sms"], T=1)
    chunk = np.diff(p["wg_off"]) * per_ms
    assert chunk.max() == total / g["num_sms"] == 155


def _check_invariants(p, lens, C, X, T, policy=PL.POLICY_STREAMK, mode=PL.MODE_GQA):
    U = len(lens)
    ntiles = [-(-L // T) for L in lens]
    N = sum(ntiles)
    assert p["num_tiles"] == N and p["num_units"] == U
    # chunk sizes: floor(N/C), +1 on the first N mod C logical chunks
    if policy == PL.POLICY_STREAMK:
        base, rem = divmod(N, C)
        for k, its in enumerate(p["chunk_items"]):
            tiles = sum(-(-(t1 - t0) // T) for (_, t0, t1, _) in its)
            assert tiles == base + (k < rem)
    else:
        # cost of a chunk (16 per tile, the mode's unit cost per unit it
        # starts) is within one tile plus one unit of its share of the total
        K, O = PL.COST_PER_TILE, PL.unit_cost(mode)
        q, r = divmod(K * N + O * sum(n > 0 for n in ntiles), C)
        for k, its in enumerate(p["chunk_items"]):
            cost = sum(K * -(-(t1 - t0) // T) + (O if t0 == 0 else 0) for (_, t0, t1, _) in its)
            assert abs(cost - (q + (k < r))) <= K + O
    # every token of every unit covered exactly once, in order
    cover = [[] for _ in range(U)]
    for its in p["chunk_items"]:
        for (u, t0, t1, s) in its:
            assert t0 % T == 0 and t1 > t0
            assert s == len(cover[u])
            cover[u].append((t0, t1))
    for u in range(U):
        if lens[u] == 0:     # an empty unit: no piece
            assert cover[u] == [] and p["unit_nsplit"][u] == 0
            continue
        assert cover[u][0][0] == 0 and cover[u][-1][1] == lens[u]
        for a, b in zip(cover[u][:-1], cover[u][1:]):
            assert a[1] == b[0]
        assert p["unit_nsplit"][u] == len(cover[u])
    # partial slots: consecutive for split units, -1 for whole units
    nxt = 0
    for u in range(U):
        if p["unit_nsplit"][u] > 1:
            assert p["unit_pbase"][u] == nxt
            nxt += p["unit_nsplit"][u]
        else:
            assert p["unit_pbase"][u] == -1
    assert p["num_partials"] == nxt
    # placement: worker w of logical chunk k sits in domain k div (C/X)
    wok = p["worker_of_chunk"]
    assert sorted(wok) == list(range(C))
    if X > 1 and C % X == 0:
        for k, w in enumerate(wok):
            assert w % X == k // (C // X)
    else:
        assert wok == list(range(C))
    # items of worker w are the pieces of its chunk, in order
    for k, w in enumerate(wok):
        assert p["items"][p["wg_off"][w]:p["wg_off"][w + 1]] == p["chunk_items"][k]


def _brute_force(lens, C, T):
    """Assign tiles one by one: tile i goes to the first chunk that still has quota."""
    ntiles = [-(-L // T) for L in lens]
    N = sum(ntiles)
    quota = [N // C + (1 if k < N % C else 0) for k in range(C)]
    owner = []
    k = 0
    for u, n in enumerate(ntiles):
        for j in range(n):
            while quota[k] == 0:
                k += 1
            quota[k] -= 1
            owner.append((k, u, j))
    chunks = [[] for _ in range(C)]
    for (k, u, j) in owner:
        if chunks[k] and chunks[k][-1][0] == u:
            chunks[k][-1][2] = min((j + 1) * T, lens[u])
        else:
            chunks[k].append([u, j * T, min((j + 1) * T, lens[u])])
    return [[tuple(x) for x in c] for c in chunks]


def _brute_force_cost(lens, C, T):
    """Cost policy, tile by tile: a tile's cost position is the cost of all
    earlier units (16 + 16 per tile each), 16 for its own unit and 16 per
    earlier tile of it; the tile goes to the chunk whose range holds it,
    found by scanning the ranges."""
    K, O = PL.COST_PER_TILE, PL.UNIT_COST
    ntiles = [-(-L // T) for L in lens]
    total = sum(O + K * n for n in ntiles if n > 0)
    ranges = [(k * (total // C) + min(k, total % C), (k + 1) * (total // C) + min(k + 1, total % C))
              for k in range(C)]
    chunks = [[] for _ in range(C)]
    before = 0
    for u, n in enumerate(ntiles):
        for j in range(n):
            pos = before + O + K * j
            k = next(k for k, (a, b) in enumerate(ranges) if a <= pos < b)
            if chunks[k] and chunks[k][-1][0] == u:
                chunks[k][-1][2] = min((j + 1) * T, lens[u])
            else:
                chunks[k].append([u, j * T, min((j + 1) * T, lens[u])])
        if n > 0:
            before += O + K * n
    return [[tuple(x) for x in c] for c in chunks]


@pytest.mark.parametrize("policy", [PL.POLICY_STREAMK, PL.POLICY_STREAMK_COST])
@pytest.mark.parametrize("seed", range(30))
def test_brute_force_and_invariants_small(seed, policy):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(1, 60, size=B)]
    for i in range(B):                  # some sequences with no cached tokens
        if rng.random() < 0.25:
            lens[i] = 0
    C = int(rng.choice([1, 2, 3, 5, 8, 16]))
    X = int(rng.choice([1, 2, 4, 8]))
    T = int(rng.choice([1, 4, 16, 32]))
    p = _plan(lens, C=C, X=X, T=T, policy=policy)
    _check_invariants(p, lens, C, X, T, policy)
    bf = _brute_force(lens, C, T) if policy == PL.POLICY_STREAMK else _brute_force_cost(lens, C, T)
    got = [[(u, t0, t1) for (u, t0, t1, _) in its] for its in p["chunk_items"]]
    assert got == bf


def test_cost_policy_gives_short_units_fewer_tiles():
    # one long unit and many short ones: the chunks made of short units carry
    # a unit cost each, so they get fewer tiles than the equal-tile split gives
    lens = [4096] + [64] * 60
    C, T = 16, 32
    eq = _plan(lens, C=C, T=T)
    co = _plan(lens, C=C, T=T, policy=PL.POLICY_STREAMK_COST)
    tiles = lambda p, k: sum(-(-(t1 - t0) // T) for (_, t0, t1, _) in p["chunk_items"][k])
    assert tiles(co, C - 1) < tiles(eq, C - 1)          # the last chunk holds only short units
    assert tiles(co, 0) >= tiles(eq, 0)                 # the first holds only the long one
    assert co["blob"][80:84] != b"\x00\x00\x00\x00"      # header word 20: policy
    assert np.frombuffer(co["blob"][:96], np.int32)[23] == PL.UNIT_COST


@pytest.mark.parametrize("policy", [PL.POLICY_STREAMK, PL.POLICY_STREAMK_COST])
@pytest.mark.parametrize("C", [1, 3, 8, 148, 256, 304, 1000])
@pytest.mark.parametrize("T", [16, 32, 64])
def test_invariants_on_the_workload_lengths(C, T, policy):
    for cfg in W.CONFIGS:
        lens_b = W.draw_seqlens(cfg)
        hu = cfg.group if cfg.mode == W.MODE_GQA else min(cfg.num_q_heads, 128)
        units_per_b = cfg.q_tokens * cfg.num_kv_heads * (cfg.group // hu)
        per_unit = cfg.topk if cfg.mode == W.MODE_MLA_SPARSE else None
        lens = [per_unit or int(L) for L in lens_b for _ in range(units_per_b)]
        P = cfg.page_size
        maxp = int(max((int(L) + P - 1) // P for L in lens_b))
        p = PL.plan(cfg.mode, cfg.batch, cfg.q_tokens, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim_qk,
                    cfg.head_dim_v, P, maxp, 1 << 20, cfg.topk, C, 8, T, hu, lens_b, None, policy)
        _check_invariants(p, lens, C, 8, T, policy, cfg.mode)


def test_skewed_workload_split_shape():
    cfg = W.CONFIG_BY_NAME["skewed_gqa"]
    lens_b = W.draw_seqlens(cfg)
    p = PL.plan(cfg.mode, cfg.batch, 1, 32, 8, 128, 128, 16, 8192, 1 << 20, 0, 256, 8, 32, 4, lens_b)
    assert p["num_tiles"] == 8 * 4096 + 31 * 8 * 8
    # each long unit spreads over ~30 workers; short units stay whole
    assert max(p["unit_nsplit"][:8]) >= 30
    assert all(n <= 2 for n in p["unit_nsplit"][8:])


@pytest.mark.parametrize("bad", ["seqlen_neg", "topk", "heads", "hu", "page", "tq", "bt_short"])
def test_invalid_inputs_rejected(bad):
    lens = np.array([10, 20], np.int32)
    kw = dict(mode=PL.MODE_GQA, batch=2, q_tokens=1, num_q_heads=8, num_kv_heads=2, head_dim_qk=64,
              head_dim_v=64, page_size=16, max_pages_per_seq=2, num_pages=4, topk=0, num_cus=8,
              num_xcds=1, tile_tokens=16, heads_per_unit=4, seqlens=lens,
              block_table=np.array([[0, -1], [1, 2]], np.int32))
    if bad == "seqlen_neg":
        kw["seqlens"] = np.array([-1, 20], np.int32)
    elif bad == "topk":
        kw.update(mode=PL.MODE_MLA_SPARSE, topk=11, num_q_heads=2, num_kv_heads=1, heads_per_unit=2)
    elif bad == "heads":
        kw["num_q_heads"] = 7
    elif bad == "hu":
        kw["heads_per_unit"] = 3
    elif bad == "page":
        kw["block_table"] = np.array([[0, -1], [1, 4]], np.int32)
    elif bad == "tq":
        kw["q_tokens"] = 2
    elif bad == "bt_short":
        kw["seqlens"] = np.array([10, 40], np.int32)
    with pytest.raises(ValueError):
        PL.plan(**kw)


def test_cost_policy_unit_cost_follows_mode():
    """An MLA unit is charged six tiles, a GQA unit one, and the header says which."""
    lens = [300, 70, 1000]
    for mode, hu, O in ((PL.MODE_GQA, 1, 16), (PL.MODE_MLA, 1, 96)):
        p = _plan(lens, C=4, T=32, mode=mode, hu=hu, policy=PL.POLICY_STREAMK_COST)
        assert np.frombuffer(p["blob"][:96], np.int32)[23] == O == PL.unit_cost(mode)
        _check_invariants(p, lens, 4, 1, 32, PL.POLICY_STREAMK_COST, mode)


@pytest.mark.parametrize("policy", [PL.POLICY_STREAMK, PL.POLICY_STREAMK_COST, PL.POLICY_PER_UNIT])
def test_empty_sequences_get_no_piece(policy):
    """Sequences with no cached tokens: no piece, nsplit 0, no cost; the other
    units are planned exactly as in the batch without them (cost and tile
    positions do not count the empty units)."""
    lens = [0, 37, 0, 0, 120, 5, 0]
    p = _plan(lens, C=8, X=1, T=4, policy=policy)
    if policy != PL.POLICY_PER_UNIT:
        _check_invariants(p, lens, 8, 1, 4, policy)
    assert [p["unit_nsplit"][u] for u in (0, 2, 3, 6)] == [0, 0, 0, 0]
    assert np.frombuffer(p["blob"], np.int32)[24] == 4       # empty units counted in the header
    assert all(u not in (0, 2, 3, 6) for its in p["chunk_items"] for (u, _, _, _) in its)
    if policy != PL.POLICY_PER_UNIT:
        q = _plan([37, 120, 5], C=8, X=1, T=4, policy=policy)
        ren = {0: 1, 1: 4, 2: 5}
        assert [[(ren[u], t0, t1, s) for (u, t0, t1, s) in its] for its in q["chunk_items"]] == p["chunk_items"]
    allempty = _plan([0, 0, 0], C=8, X=1, T=4, policy=policy)
    assert allempty["num_items"] == 0 and allempty["num_tiles"] == 0
    assert allempty["unit_nsplit"] == [0, 0, 0]
