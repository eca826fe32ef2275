"""Pins of the indexer oracle (paged indexer score + top-k) against facts that
do not come from its own code: exact integer arithmetic, the error bound of
recursive fp32 summation, a brute-force rank definition of top-k with ties,
and invariance to page placement."""
import numpy as np
import pytest

from cross_cu_load_amd import workloads as W
from oracle import indexer as I


def _bf16(x):
    return W.round_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_scores_exact_on_small_integers():
    # integers |v| <= 16 are exact in bf16; products and partial sums stay far
    # below 2^24, so the fp32 sum is exact and equals the integer dot product
    rng = np.random.default_rng(1)
    q = rng.integers(-16, 17, size=128)
    k = rng.integers(-16, 17, size=(300, 128))
    got = I.scores_fp32(_bf16(q), _bf16(k))
    want = np.array([sum(int(a) * int(b) for a, b in zip(q, row)) for row in k])
    assert np.array_equal(got.astype(np.int64), want)


def test_scores_within_recursive_summation_bound():
    rng = np.random.default_rng(2)
    qb = _bf16(rng.standard_normal(128))
    kb = _bf16(rng.standard_normal((500, 128)))
    got = I.scores_fp32(qb, kb).astype(np.float64)
    q = I.bf16_to_f32(qb).astype(np.float64)
    k = I.bf16_to_f32(kb).astype(np.float64)
    exact = k @ q
    absum = np.abs(k) @ np.abs(q)
    u = 2.0 ** -24
    gamma = 127 * u / (1 - 127 * u)
    assert np.all(np.abs(got - exact) <= gamma * absum)
    # and the bound is not vacuous: a dropped term would break it
    assert np.max(np.abs(k[:, 5] * q[5])) > 10 * np.max(gamma * absum)


def _brute_topk(s, k):
    L = len(s)
    sel = []
    for j in range(L):
        rank = sum(1 for i in range(L) if s[i] > s[j] or (s[i] == s[j] and i < j))
        if rank < k:
            sel.append(j)
    return np.array(sel, dtype=np.int32)


@pytest.mark.parametrize("seed,L,k", [(0, 200, 37), (1, 97, 97), (2, 150, 1), (3, 64, 63)])
def test_topk_matches_rank_definition_with_ties(seed, L, k):
    rng = np.random.default_rng(seed)
    s = rng.integers(-5, 6, size=L).astype(np.float32)   # many equal scores
    assert np.array_equal(I.topk_positions(s, k), _brute_topk(s, k))


def test_topk_all_and_all_equal():
    s = np.random.default_rng(4).standard_normal(50).astype(np.float32)
    assert np.array_equal(I.topk_positions(s, 50), np.arange(50))
    assert np.array_equal(I.topk_positions(np.zeros(40, np.float32), 7), np.arange(7))


def test_gather_rows_follows_block_table():
    P, d = 4, 2
    seqlens = np.array([6, 9], np.int32)
    bt = W.page_table(seqlens, P, True, 5)
    cache = np.zeros((int(bt.max()) + 1, P, d), np.uint16)
    for b in range(2):
        for j in range(int(seqlens[b])):
            cache[bt[b, j // P], j % P] = (b, j)
    for b in range(2):
        rows = I.gather_rows(cache, bt, b, int(seqlens[b]))
        assert np.array_equal(rows[:, 0], np.full(seqlens[b], b)) and np.array_equal(rows[:, 1], np.arange(seqlens[b]))


def test_indexer_topk_invariant_to_page_placement_and_separates_scores():
    cfg = W.small_variant(W.CONFIG_BY_NAME["sparse_mla"], batch=2, seqlen_hi=3000)
    wl = W.make_workload(cfg)
    ix = W.make_indexer_inputs(wl)
    got = I.indexer_topk(ix.q, ix.k_cache, wl.block_table, wl.seqlens, cfg.topk)
    # the same logical cache laid out in sequence order
    ident = W.page_table(wl.seqlens, cfg.page_size, False, 0)
    cache2 = np.empty_like(ix.k_cache)
    for b in range(cfg.batch):
        n = -(-int(wl.seqlens[b]) // cfg.page_size)
        cache2[ident[b, :n]] = ix.k_cache[wl.block_table[b, :n]]
    assert np.array_equal(got, I.indexer_topk(ix.q, cache2, ident, wl.seqlens, cfg.topk))
    # every selected score is >= every unselected one
    for b in range(cfg.batch):
        rows = I.gather_rows(ix.k_cache, wl.block_table, b, int(wl.seqlens[b]))
        for t in range(cfg.q_tokens):
            s = I.scores_fp32(ix.q[b, t], rows)
            m = np.zeros(len(s), bool)
            m[got[b, t]] = True
            assert len(np.unique(got[b, t])) == cfg.topk
            assert s[m].min() >= s[~m].max()
