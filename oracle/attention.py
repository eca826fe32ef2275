"""Plain fp64 decode attention over a paged KV cache (TEST INFRASTRUCTURE).

What is computed
----------------
Each decode query token attends over its own sequence's cached keys and
values: out = softmax(scale * q K^T) V and lse = log(sum(exp(scale * q K^T))),
the exact result that the split-KV kernels reach by splitting the key range
and merging partial results (MeldKernel summary, "Key observations": varlen
split-KV attention whose shards finish at different times and are then
reduced; the fusion tutorial, FlashAttention section: softmax attention kept
exact while fused on-chip).

Readings of points the pages leave open
---------------------------------------
* lse is the natural-log log-sum-exp of the scaled scores.
* No mask: a decode token sees all L_b cached tokens of its sequence; in the
  index-sparse mode it sees exactly its own index set.
* GQA head map: query head h reads KV head h // (Hq / Hkv) (contiguous groups).
* MLA: one latent KV row of dk columns serves as K; its first dv columns are V.
* A sequence with no cached tokens (L_b = 0): lse = log of an empty sum =
  -inf, and out = 0.  That pair is the neutral element of the log-sum-exp
  merge (m = -inf, l = 0, o = 0), so an empty key set merged with any other
  leaves it unchanged; the value of out itself (0/0 in the definition) is a
  convention.
* Paged layout: cache[page, slot, kv_head, dim] (token-major, "NHD") or
  cache[page, kv_head, slot, dim] (head-major, "HND"); token j of sequence b
  is page block_table[b, j // P], slot j % P.  Sparse indices are token
  positions within the request's cache.

Everything runs in float64; bf16 inputs are widened exactly.  Every function
here is a direct transcription of the definition, with no blocking or
reordering beyond a library dot product.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: a bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def key_positions(b: int, t: int, seqlens: np.ndarray, indices: np.ndarray | None) -> np.ndarray:
    """The key set J of query token t of sequence b (dense: 0..L_b-1)."""
    if indices is None:
        return np.arange(int(seqlens[b]), dtype=np.int64)
    return np.asarray(indices[b, t], dtype=np.int64)


def gather_rows(cache_bits: np.ndarray, block_table: np.ndarray, b: int, J: np.ndarray,
                page_size: int, head: int | None = None) -> np.ndarray:
    """Rows cache[block_table[b, j // P], j % P] for j in J, as float64 [|J|, H, d]
    (or [|J|, d] of one head when ``head`` is given)."""
    pages = block_table[b, J // page_size]
    if np.any(pages < 0) or np.any(pages >= cache_bits.shape[0]):
        raise ValueError("block_table entry outside the cache")
    if head is None:
        return bf16_to_f64(cache_bits[pages, J % page_size])
    return bf16_to_f64(cache_bits[pages, J % page_size, head])


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> tuple[np.ndarray, np.ndarray]:
    """softmax(scale * q K^T) V and its lse for query rows q [G, dk], K [n, dk], V [n, dv]."""
    if K.shape[0] == 0:                           # empty key set: see the readings above
        return np.zeros((q.shape[0], V.shape[1])), np.full(q.shape[0], -np.inf)
    s = scale * (q @ K.T)                         # [G, n]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    out = (w @ V) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def partial_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Un-normalised partial result of one key subset: (m, l, o).

    m = max score, l = sum exp(s - m), o = sum exp(s - m) v.  These are the
    running max, running sum and un-normalised output that a split piece
    hands to the reduction (MeldKernel summary, "Core method": partial outputs
    feed a just-in-time reduction).  An empty subset has m = -inf, l = 0, o = 0.
    """
    if K.shape[0] == 0:
        return np.full(q.shape[0], -np.inf), np.zeros(q.shape[0]), np.zeros((q.shape[0], V.shape[1]))
    s = scale * (q @ K.T)
    m = s.max(axis=1)
    w = np.exp(s - m[:, None])
    return m, w.sum(axis=1), w @ V


def lse_merge(parts) -> tuple[np.ndarray, np.ndarray]:
    """Exact merge of partial states over disjoint key subsets.

    With M = max_i m_i and c_i = exp(m_i - M):
    L = sum_i c_i l_i, out = sum_i c_i o_i / L, lse = M + log L.
    """
    ms = np.stack([p[0] for p in parts])          # [n, G]
    M = ms.max(axis=0)
    if np.all(M == -np.inf):                      # every part empty: the empty result
        return np.zeros_like(parts[0][2]), M
    c = np.exp(ms - M)                            # 0 for an empty part (m = -inf)
    L = sum(ci * p[1] for ci, p in zip(c, parts))
    O = sum(ci[:, None] * p[2] for ci, p in zip(c, parts))
    return O / L[:, None], M + np.log(L)


def decode_attention(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray | None,
                     block_table: np.ndarray, seqlens: np.ndarray, scale: float,
                     head_dim_v: int | None = None, indices: np.ndarray | None = None,
                     only: list[tuple[int, int, int]] | None = None, head_major: bool = False):
    """Reference decode attention.

    q_bits   uint16 [B, Tq, Hq, dk]
    k_bits   uint16 [pages, P, Hkv, dk]   (MLA: the latent cache, Hkv = 1)
    v_bits   uint16 [pages, P, Hkv, dv], or None: V = first ``head_dim_v``
             columns of the K rows (MLA)
    indices  int32 [B, Tq, topk] for index-sparse decode, else None
    only     optional list of (b, t, kv_head) units to compute; others stay NaN
    head_major  caches are [pages, Hkv, P, d] instead of [pages, P, Hkv, d]

    Returns out float64 [B, Tq, Hq, dv] and lse float64 [B, Tq, Hq].
    """
    if head_major:   # index the same elements through a token-major view
        k_bits = k_bits.transpose(0, 2, 1, 3)
        v_bits = None if v_bits is None else v_bits.transpose(0, 2, 1, 3)
    B, Tq, Hq, dk = q_bits.shape
    P, Hkv = k_bits.shape[1], k_bits.shape[2]
    G = Hq // Hkv
    dv = v_bits.shape[3] if v_bits is not None else int(head_dim_v)
    out = np.full((B, Tq, Hq, dv), np.nan)
    lse = np.full((B, Tq, Hq), np.nan)
    units = only if only is not None else [(b, t, g) for b in range(B) for t in range(Tq) for g in range(Hkv)]
    for b, t, g in units:
        J = key_positions(b, t, seqlens, indices)
        Krows = gather_rows(k_bits, block_table, b, J, P, head=g)
        if v_bits is not None:
            Vrows = gather_rows(v_bits, block_table, b, J, P, head=g)
        else:
            Vrows = Krows[:, :dv]
        qg = bf16_to_f64(q_bits[b, t, g * G:(g + 1) * G])
        o, s = attend(qg, Krows, Vrows, scale)
        out[b, t, g * G:(g + 1) * G] = o
        lse[b, t, g * G:(g + 1) * G] = s
    return out, lse


def decode_attention_wl(wl, only=None):
    """``decode_attention`` on a workload object from the seeded input generator."""
    c = wl.cfg
    return decode_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seqlens,
                            c.softmax_scale, head_dim_v=c.head_dim_v, indices=wl.indices, only=only,
                            head_major=wl.kv_layout == 1)
