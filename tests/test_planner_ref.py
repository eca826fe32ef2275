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


def _plan(lens, C=8, X=1, T=4, G=1, Hkv=1, mode=PL.MODE_GQA, Tq=1, topk=0, hu=None, policy=PL.POLICY_STREAMK,
          unit_cost=0):
    lens = np.asarray(lens, np.int32)
    P = 16
    maxp = max(1, int(max((int(L) + P - 1) // P for L in lens)))
    return PL.plan(mode, len(lens), Tq, G * Hkv, Hkv, 64, 64, P, maxp, 1 << 20, topk, C, X, T,
                   hu if hu is not None else G, lens, None, policy, unit_cost)


def test_golden_732_tasks_over_148_workers():
    g = json.load(open(os.path.join(GOLD, "kernelplan_732_tasks_148_workers.json")))
    # 732 one-tile units over 148 chunks
    p = _plan([4] * g["tasks"], C=g["workers"], X=1, T=4)
    sizes = np.diff(p["wg_off"])
    assert int((sizes == 5).sum()) == g["workers_with_5"]
    assert int((sizes == 4).sum()) == g["workers_with_4"]
    assert p["num_tiles"] == g["tasks"]
    # the same 732 tasks through the cost split with unit cost 0 (the code
    # path that carries a unit cost): the printed counts again
    pieces = PL._cost_split([1] * g["tasks"], [4] * g["tasks"], g["workers"], 4, 0)
    sizes = np.array([len(c) for c in pieces])
    assert int((sizes == 5).sum()) == g["workers_with_5"] and int((sizes == 4).sum()) == g["workers_with_4"]


def _equal_split_pieces(p):
    return [[(u, t0, t1) for (u, t0, t1, _) in its] for its in p["chunk_items"]]


@pytest.mark.parametrize("seed", range(40))
def test_cost_split_with_unit_cost_zero_is_the_equal_split(seed):
    """The cost split at unit cost 0 and the plain equal tile split give the
    same pieces (chunk by chunk), and the whole plan blob is byte-identical."""
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 9))
    lens = [int(x) for x in rng.integers(0, 400, size=B)]
    C = int(rng.choice([1, 2, 3, 7, 16, 148, 256]))
    T = int(rng.choice([1, 4, 16, 32]))
    eq = _plan(lens, C=C, X=1, T=T)
    ntiles = [-(-L // T) for L in lens]
    assert PL._cost_split(ntiles, lens, C, T, 0) == _equal_split_pieces(eq)


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


def _check_invariants(p, lens, C, X, T, unit_cost=0):
    U = len(lens)
    ntiles = [-(-L // T) for L in lens]
    N = sum(ntiles)
    assert p["num_tiles"] == N and p["num_units"] == U
    # chunk sizes: floor(N/C), +1 on the first N mod C logical chunks
    if unit_cost == 0:
        base, rem = divmod(N, C)
        for k, its in enumerate(p["chunk_items"]):
            tiles = sum(-(-(t1 - t0) // T) for (_, t0, t1, _) in its)
            assert tiles == base + (k < rem)
    else:
        # cost of a chunk (one per tile, the unit cost per unit it starts) is
        # within one tile plus one unit of its share of the total
        O = unit_cost
        q, r = divmod(N + O * sum(n > 0 for n in ntiles), C)
        for k, its in enumerate(p["chunk_items"]):
            cost = sum(-(-(t1 - t0) // T) + (O if t0 == 0 else 0) for (_, t0, t1, _) in its)
            assert abs(cost - (q + (k < r))) <= 1 + O
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


def _brute_force_cost(lens, C, T, O):
    """Cost split, tile by tile: a tile's cost position is the cost of all
    earlier non-empty units (O + one per tile each), O for its own unit and
    one per earlier tile of it; the tile goes to the chunk whose range holds
    it, found by scanning the ranges."""
    K = 1
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


@pytest.mark.parametrize("unit_cost", [0, 1, 3, 6])
@pytest.mark.parametrize("seed", range(30))
def test_brute_force_and_invariants_small(seed, unit_cost):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(1, 60, size=B)]
    for i in range(B):                  # some sequences with no cached tokens
        if rng.random() < 0.25:
            lens[i] = 0
    C = int(rng.choice([1, 2, 3, 5, 8, 16]))
    X = int(rng.choice([1, 2, 4, 8]))
    T = int(rng.choice([1, 4, 16, 32]))
    p = _plan(lens, C=C, X=X, T=T, unit_cost=unit_cost)
    _check_invariants(p, lens, C, X, T, unit_cost)
    got = [[(u, t0, t1) for (u, t0, t1, _) in its] for its in p["chunk_items"]]
    assert got == _brute_force_cost(lens, C, T, unit_cost)
    if unit_cost == 0:      # the two brute forces agree where they should
        assert got == _brute_force(lens, C, T)


def test_cost_policy_gives_short_units_fewer_tiles():
    # one long unit and many short ones: the chunks made of short units carry
    # a unit cost each, so they get fewer tiles than the equal-tile split gives
    lens = [4096] + [64] * 60
    C, T = 16, 32
    eq = _plan(lens, C=C, T=T)
    co = _plan(lens, C=C, T=T, unit_cost=1)
    tiles = lambda p, k: sum(-(-(t1 - t0) // T) for (_, t0, t1, _) in p["chunk_items"][k])
    assert tiles(co, C - 1) < tiles(eq, C - 1)          # the last chunk holds only short units
    assert tiles(co, 0) >= tiles(eq, 0)                 # the first holds only the long one
    assert np.frombuffer(co["blob"][:128], np.int32)[23] == 1      # header word 23: the unit cost
    assert np.frombuffer(eq["blob"][:128], np.int32)[23] == 0


def test_input_hash_is_fnv1a():
    """Header word 25 is FNV-1a over the problem words and the lengths: the
    published FNV-1a test vectors, and a hash that moves with every length."""
    # FNV-1a 32 of the empty input is the offset basis; of b"a" 0xe40c292c
    assert PL.fnv1a32([]) == 2166136261 - (1 << 32)
    h = 2166136261
    for byte in b"a":
        h = ((h ^ byte) * 16777619) & 0xFFFFFFFF
    assert h == 0xE40C292C
    # one int32 word 0x61 hashes its four little-endian bytes 61 00 00 00
    h = 2166136261
    for byte in bytes([0x61, 0, 0, 0]):
        h = ((h ^ byte) * 16777619) & 0xFFFFFFFF
    assert PL.fnv1a32([0x61]) == (h - (1 << 32) if h >= 1 << 31 else h)
    lens = [300, 70, 1000]
    p = _plan(lens, C=4, T=32)
    word = int(np.frombuffer(p["blob"][:128], np.int32)[25])
    for b in range(3):
        other = list(lens)
        other[b] += 1
        assert int(np.frombuffer(_plan(other, C=4, T=32)["blob"][:128], np.int32)[25]) != word
    # knobs of the plan are not inputs: the same inputs under another split hash the same
    assert int(np.frombuffer(_plan(lens, C=7, T=16, unit_cost=6)["blob"][:128], np.int32)[25]) == word


@pytest.mark.parametrize("unit_cost", [0, 1, 6])
@pytest.mark.parametrize("C", [1, 3, 8, 148, 256, 304, 1000])
@pytest.mark.parametrize("T", [16, 32, 64])
def test_invariants_on_the_workload_lengths(C, T, unit_cost):
    for cfg in W.CONFIGS:
        lens_b = W.draw_seqlens(cfg)
        hu = cfg.group if cfg.mode == W.MODE_GQA else min(cfg.num_q_heads, 128)
        units_per_b = cfg.q_tokens * cfg.num_kv_heads * (cfg.group // hu)
        per_unit = cfg.topk if cfg.mode == W.MODE_MLA_SPARSE else None
        lens = [per_unit or int(L) for L in lens_b for _ in range(units_per_b)]
        P = cfg.page_size
        maxp = int(max((int(L) + P - 1) // P for L in lens_b))
        p = PL.plan(cfg.mode, cfg.batch, cfg.q_tokens, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim_qk,
                    cfg.head_dim_v, P, maxp, 1 << 20, cfg.topk, C, 8, T, hu, lens_b, None, PL.POLICY_STREAMK,
                    unit_cost)
        _check_invariants(p, lens, C, 8, T, unit_cost)


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


def test_unit_cost_is_recorded_and_independent_of_mode():
    """The unit cost is an input of the plan, recorded in the header; the
    oracle holds no per-mode tuning (the same lengths and cost give the same
    pieces in every mode)."""
    lens = [300, 70, 1000]
    for O in (0, 1, 6):
        ps = [_plan(lens, C=4, T=32, mode=mode, hu=1, unit_cost=O) for mode in (PL.MODE_GQA, PL.MODE_MLA)]
        for p in ps:
            assert np.frombuffer(p["blob"][:128], np.int32)[23] == O
            _check_invariants(p, lens, 4, 1, 32, O)
        assert ps[0]["chunk_items"] == ps[1]["chunk_items"]
    with pytest.raises(ValueError):
        _plan(lens, unit_cost=-1)


@pytest.mark.parametrize("policy,unit_cost", [(PL.POLICY_STREAMK, 0), (PL.POLICY_STREAMK, 1),
                                              (PL.POLICY_STREAMK, 6), (PL.POLICY_PER_UNIT, 0)])
def test_empty_sequences_get_no_piece(policy, unit_cost):
    """Sequences with no cached tokens: no piece, nsplit 0, no cost; the other
    units are planned exactly as in the batch without them (cost and tile
    positions do not count the empty units)."""
    lens = [0, 37, 0, 0, 120, 5, 0]
    p = _plan(lens, C=8, X=1, T=4, policy=policy, unit_cost=unit_cost)
    if policy != PL.POLICY_PER_UNIT:
        _check_invariants(p, lens, 8, 1, 4, unit_cost)
    assert [p["unit_nsplit"][u] for u in (0, 2, 3, 6)] == [0, 0, 0, 0]
    assert np.frombuffer(p["blob"], np.int32)[24] == 4       # empty units counted in the header
    assert all(u not in (0, 2, 3, 6) for its in p["chunk_items"] for (u, _, _, _) in its)
    if policy != PL.POLICY_PER_UNIT:
        q = _plan([37, 120, 5], C=8, X=1, T=4, policy=policy, unit_cost=unit_cost)
        ren = {0: 1, 1: 4, 2: 5}
        assert [[(ren[u], t0, t1, s) for (u, t0, t1, s) in its] for its in q["chunk_items"]] == p["chunk_items"]
    allempty = _plan([0, 0, 0], C=8, X=1, T=4, policy=policy, unit_cost=unit_cost)
    assert allempty["num_items"] == 0 and allempty["num_tiles"] == 0
    assert allempty["unit_nsplit"] == [0, 0, 0]


@pytest.mark.parametrize("name", ["skewed_gqa", "llama3_8b_gqa", "tiny_gqa", "deepseek_mla", "sparse_mla"])
def test_tail_model_on_the_workloads(name):
    """The tail-effect example's list-scheduling model applied to each decode
    workload's unit tile counts (32-token tiles, 256 CUs): one workgroup per
    unit (the per-unit comparison launch) finishes with its longest unit when
    the units fit one wave, and the Stream-K plan's busiest chunk holds
    exactly ceil(tiles / CUs) tiles.  Their ratio is the model's predicted
    slowdown of the per-unit launch (CSDN Q&A on waves, "Scenario examples":
    the wave tail; "Summary": equal chunks per SM)."""
    c = W.CONFIG_BY_NAME[name]
    sl = W.draw_seqlens(c)
    G = c.num_q_heads // c.num_kv_heads
    hpu = G if c.mode == PL.MODE_GQA else c.num_q_heads
    C, T = 256, 32
    lens = PL.unit_lengths(c.mode, c.batch, c.q_tokens, c.num_q_heads, c.num_kv_heads, hpu, sl, c.topk)
    nt = [-(-L // T) for L in lens]
    N = sum(nt)
    v1, finish, _ = PL.list_schedule(nt, C)
    if len(nt) <= C:
        assert v1 == max(nt)
    assert v1 >= max(nt) and v1 >= N / C
    maxp = max(1, int(max(-(-int(L) // c.page_size) for L in sl)))
    p = PL.plan(c.mode, c.batch, c.q_tokens, c.num_q_heads, c.num_kv_heads, c.head_dim_qk, c.head_dim_v,
                c.page_size, maxp, 1 << 24, c.topk, C, 8, T, hpu, sl, None, PL.POLICY_STREAMK, 0)
    chunk_tiles = [sum(-(-(t1 - t0) // T) for (_, t0, t1, _) in its) for its in p["chunk_items"]]
    assert sum(chunk_tiles) == N and max(chunk_tiles) == -(-N // C)
    print(f"{name}: per-unit makespan {v1:.0f} tiles, Stream-K {max(chunk_tiles)}; predicted ratio "
          f"{v1 / max(chunk_tiles):.1f}")
