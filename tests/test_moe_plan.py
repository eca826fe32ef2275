"""MoE grouped-GEMM plans (cc_moe_plan) on the CPU: byte-identical to the
reference planner, every output tile's k range covered exactly once with
splits 0 .. nsplit - 1, the tiles of each expert's rows and columns, and the
equal split of the (tile, k tile) work at unit cost 0."""
import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from oracle import planner as PL


def _case(seed):
    rng = np.random.default_rng(11000 + seed)
    E = int(rng.integers(1, 20))
    K = 64 * int(rng.integers(1, 9))
    N = PL.MOE_TILE_COLS * int(rng.integers(1, 5))
    et = rng.integers(0, 600, size=E).astype(np.int32)
    et[rng.random(E) < 0.2] = 0
    if et.sum() == 0:
        et[0] = 1
    C = int(rng.choice([1, 3, 8, 64, 256, 1000]))
    X = int(rng.choice([1, 8]))
    O = int(rng.choice([0, 1, 4]))
    policy = int(rng.choice([B.POLICY_STREAMK, B.POLICY_PER_UNIT, B.POLICY_STREAMK_DP]))
    return E, K, N, et, C, X, O, policy


@pytest.mark.parametrize("seed", range(50))
def test_moe_plan_bytes_and_coverage(lib, seed):
    E, K, N, et, C, X, O, policy = _case(seed)
    blob = B.moe_plan(B.moe_problem(E, K, N), et, num_cus=C, num_xcds=X, policy=policy, unit_cost=O)
    ref = PL.plan_moe(E, K, N, et, C, X, policy=policy, unit_cost=O if policy != B.POLICY_PER_UNIT else 0)
    assert blob.tobytes() == ref["blob"]
    assert B.workspace_size(blob) > 0
    # tiles: every (row, column) of every expert exactly once
    off = np.concatenate([[0], np.cumsum(et)])
    cover = np.zeros((int(off[-1]), N), np.int32)
    for (e, r0, rows, c0) in ref["units"]:
        TC = PL.MOE_TILE_COLS
        assert off[e] <= r0 and r0 + rows <= off[e + 1] and 1 <= rows <= PL.MOE_TILE_ROWS and c0 % TC == 0
        cover[r0:r0 + rows, c0:c0 + TC] += 1
    assert np.all(cover == 1)
    # every tile's k range exactly once, splits in order
    got = {u: [] for u in range(ref["num_units"])}
    for its in ref["chunk_items"]:
        for (u, k0, k1, s) in its:
            assert k0 % 64 == 0 and k1 > k0
            got[u].append((s, k0, k1))
    for u, lst in got.items():
        lst.sort()
        assert [s for s, _, _ in lst] == list(range(len(lst))) == list(range(ref["unit_nsplit"][u]))
        assert lst[0][1] == 0 and lst[-1][2] == K
        assert all(a[2] == b[1] for a, b in zip(lst[:-1], lst[1:]))
    if policy == B.POLICY_STREAMK and O == 0:     # the equal split of the k tiles
        n = ref["num_tiles"]
        sizes = sorted(sum((k1 - k0) // 64 for (_, k0, k1, _) in its) for its in ref["chunk_items"])
        assert sizes[0] == n // C and sizes[-1] == -(-n // C)


def test_moe_plan_rejects_bad_inputs(lib):
    prob = B.moe_problem(3, 256, 256)
    for et, kw in (([1, -1, 3], {}), ([0, 0, 0], {})):
        with pytest.raises(B.CrossCUError):
            B.moe_plan(prob, np.array(et, np.int32), **kw)
    with pytest.raises(B.CrossCUError):
        B.moe_plan(B.moe_problem(3, 200, 256), np.array([1, 2, 3], np.int32))      # hidden % 64
    with pytest.raises(B.CrossCUError):
        B.moe_plan(B.moe_problem(3, 256, 200), np.array([1, 2, 3], np.int32))      # out_dim % 256
    with pytest.raises(B.CrossCUError):
        B.moe_plan(B.moe_problem(3, 256, 384), np.array([1, 2, 3], np.int32))      # out_dim % 256


def test_moe_gemm_rejects_before_any_launch(lib):
    import ctypes
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails a host check first
    prob = B.moe_problem(3, 256, 256)
    et = np.array([100, 0, 300], np.int32)
    blob = B.moe_plan(prob, et, num_cus=8, num_xcds=1)
    ws = B.workspace_size(blob)
    call = lambda p, plan=blob, b=ws, tile_ok=True: lib.cc_moe_gemm(ctypes.byref(p), plan.ctypes.data_as(ctypes.c_void_p),
                                                                   fake, fake, fake, fake, fake, b, None)
    assert call(prob, b=ws - 1) == B.CC_ERR_BUFFER
    assert call(B.moe_problem(3, 256, 384)) == B.CC_ERR_PLAN
    odd = B.moe_plan(prob, et, num_cus=8, num_xcds=1, tile_k=32)
    assert call(prob, plan=odd, b=B.workspace_size(odd)) == B.CC_ERR_UNSUPPORTED
    decode_plan = B.plan(B.problem(0, 2, 1, 8, 2, 64, 64, 16, 2, 4, 0, 0.125), np.array([10, 20], np.int32), None,
                         num_cus=8, num_xcds=1)
    assert call(prob, plan=decode_plan, b=1 << 30) == B.CC_ERR_PLAN


@pytest.mark.parametrize("seed", range(12))
def test_streamk_dp_keeps_splits_few(seed):
    """STREAMK_DP deals whole rounds round-robin and splits the rest: nothing
    when the last round is at least three quarters full, the remainder alone
    when it is at least half a round, else the last whole round with it.
    Every tile then has at most three pieces, the whole rounds are tiles
    r C + k in chunk k, and the chunks' work differs by at most one k tile
    (one tile when nothing is split)."""
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(4, 12))
    C = int(rng.integers(2, 12))
    counts = rng.integers(0, 600, E)
    counts[0] = max(counts[0], 1)
    TC = PL.MOE_TILE_COLS
    pl = PL.plan_moe(E, 256, 2 * TC, counts, C, 1, tile_rows=128, policy=PL.POLICY_STREAMK_DP)
    U = pl["num_units"]
    rem = U % C
    whole = rem == 0 or 4 * rem >= 3 * C
    D = -(-U // C) if whole else (U // C if 2 * rem >= C else max(U // C - 1, 0))
    assert max(pl["unit_nsplit"]) <= (1 if whole else 3)
    items = pl["chunk_items"]
    for k in range(C):
        its = items[k]
        dealt = [r * C + k for r in range(D) if r * C + k < U]
        assert [it[0] for it in its[:len(dealt)]] == dealt
        assert all(it[1] == 0 and it[2] == 256 for it in its[:len(dealt)])
    work = [sum((it[2] - it[1]) // 64 for it in items[k]) for k in range(C)]
    assert max(work) - min(work) <= (4 if whole else 1)   # whole: within one tile of 4 k tiles
