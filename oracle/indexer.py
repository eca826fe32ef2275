"""Paged indexer score and top-k selection (TEST INFRASTRUCTURE).

Only tests, the package's smoke check and the benchmark's CPU baseline use
this module; the library never does.

What is computed
----------------
Before index-sparse attention a cheap indexer scores every cached token of a
request against each decode query token, and the best-scoring positions
become that token's sparse index set (GLM-5.2 decode article: the layer runs
through "Paged Indexer Score" before TopK and sparse MLA, Summary; the
indexer rank computes the scores and the Top-2048 and publishes the indices,
related-work section on TileRT).  The pages name the steps, not the formula.

Readings of points the pages leave open
---------------------------------------
* One indexer head of dimension d: score(t, j) = sum_i q[t, i] k[j, i], the
  plain dot product of bf16 vectors.
* Precision.  The selection is an integer decision taken on floating-point
  scores, so the score is computed in the kernel's precision and order: fp32,
  each product of two bf16 values (exact in fp32) added to the running sum
  for i = 0 .. d-1 in index order, one rounding per addition.
* Top-k: the k positions of largest score; among equal scores the lower
  position ranks higher.  The result is the set of positions, listed in
  increasing order (the sparse attention that consumes it does not depend on
  the order).
* Paging: token j of request b is row j % P of page block_table[b, j // P].
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def gather_rows(k_cache_bits: np.ndarray, block_table: np.ndarray, b: int, L: int) -> np.ndarray:
    """Rows of tokens 0 .. L-1 of request b, uint16 [L, d]."""
    P = k_cache_bits.shape[1]
    j = np.arange(L)
    return k_cache_bits[block_table[b, j // P], j % P]


def scores_fp32(q_bits: np.ndarray, rows_bits: np.ndarray) -> np.ndarray:
    """score[j] = sum_i q[i] k[j, i] in fp32, products exact, added in index order."""
    q = bf16_to_f32(q_bits)
    k = bf16_to_f32(rows_bits)
    acc = np.zeros(k.shape[0], dtype=np.float32)
    for i in range(q.shape[0]):
        acc = acc + q[i] * k[:, i]   # float32 product (exact) and float32 sum
    return acc


def topk_positions(scores: np.ndarray, k: int) -> np.ndarray:
    """The k positions of largest score (ties: lower position first), ascending."""
    L = scores.shape[0]
    order = np.lexsort((np.arange(L), -scores.astype(np.float64)))
    return np.sort(order[:k]).astype(np.int32)


def indexer_topk(q_bits: np.ndarray, k_cache_bits: np.ndarray, block_table: np.ndarray,
                 seqlens: np.ndarray, topk: int) -> np.ndarray:
    """indices int32 [B, Tq, topk] for indexer queries q [B, Tq, d]."""
    B, Tq, _ = q_bits.shape
    out = np.empty((B, Tq, topk), dtype=np.int32)
    for b in range(B):
        rows = gather_rows(k_cache_bits, block_table, b, int(seqlens[b]))
        for t in range(Tq):
            out[b, t] = topk_positions(scores_fp32(q_bits[b, t], rows), topk)
    return out
