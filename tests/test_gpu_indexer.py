"""GPU parity of the paged indexer score + top-k (cc_indexer_topk) against the oracle.

The top-k is an integer decision on fp32 scores; the oracle computes the
scores in the kernel's precision and order, so the index sets must match bit
for bit.  The indices then feed the index-sparse MLA decode, which must match
the fp64 attention oracle run with the oracle's indices.
"""
import dataclasses

import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W
from oracle import attention as A
from oracle import indexer as I

from gpu_helpers import TOL_LSE, TOL_OUT, clean, run

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SPARSE = W.CONFIG_BY_NAME["sparse_mla"]


def _dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def gpu_indexer(wl, ix, topk, block_table=None, err=None):
    c = wl.cfg
    bt = wl.block_table if block_table is None else block_table
    p = B.indexer_problem(c.batch, c.q_tokens, W.INDEXER_DIM, c.page_size, bt.shape[1], ix.k_cache.shape[0], topk)
    scratch = torch.empty(B.indexer_scratch_size(p, wl.seqlens), dtype=torch.uint8, device="cuda")
    out = torch.full((c.batch, c.q_tokens, topk), -7, dtype=torch.int32, device="cuda")
    print(f"[gpu] indexer B={c.batch} Tq={c.q_tokens} L={wl.seqlens.tolist()} P={c.page_size} topk={topk}", flush=True)
    B.indexer_topk(p, wl.seqlens, _dev(ix.q), _dev(ix.k_cache), _dev(bt), scratch, out, err)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("L,topk,page", [(3000, 2048, 64), (2048, 2048, 64), (1, 1, 64), (700, 45, 16),
                                         (5000, 2048, 64), (16384, 2048, 64)])
def test_indexer_topk_bit_exact(dev, L, topk, page):
    cfg = dataclasses.replace(W.small_variant(SPARSE, batch=2, seqlen_hi=L, seed_offset=topk), topk=topk,
                              page_size=page)
    wl = W.make_workload(cfg)
    ix = W.make_indexer_inputs(wl)
    got = gpu_indexer(wl, ix, topk)
    want = I.indexer_topk(ix.q, ix.k_cache, wl.block_table, wl.seqlens, topk)
    assert np.array_equal(got, want)


def test_indexer_ragged_lengths_and_ties(dev):
    # different lengths per request; a key cache of small integers makes many
    # scores equal, so the position tie rule decides
    cfg = dataclasses.replace(W.small_variant(SPARSE, batch=3, seqlen_hi=900), topk=300)
    wl = W.make_workload(cfg, seqlens=np.array([900, 301, 640], np.int32))
    ix = W.make_indexer_inputs(wl)
    rng = np.random.default_rng(3)
    ix = W.IndexerInputs(W.round_to_bf16_bits(rng.integers(-2, 3, ix.q.shape).astype(np.float32)),
                         W.round_to_bf16_bits(rng.integers(-2, 3, ix.k_cache.shape).astype(np.float32)))
    got = gpu_indexer(wl, ix, 300)
    assert np.array_equal(got, I.indexer_topk(ix.q, ix.k_cache, wl.block_table, wl.seqlens, 300))


def test_indexer_full_size_feeds_sparse_decode(dev):
    """Indexer at the sparse workload's full size (2 x 8 tokens, 8192 cached
    tokens, top-2048), then the sparse MLA decode on the GPU's indices."""
    wl = W.make_workload(SPARSE)
    ix = W.make_indexer_inputs(wl)
    got = gpu_indexer(wl, ix, SPARSE.topk)
    want = I.indexer_topk(ix.q, ix.k_cache, wl.block_table, wl.seqlens, SPARSE.topk)
    assert np.array_equal(got, want)
    wl2 = dataclasses.replace(wl, indices=got)
    s, plan = run(wl2, *dev, tag="indexer->sparse")
    ref_o, ref_l = A.decode_attention_wl(dataclasses.replace(wl, indices=want))
    out = s.out.cpu().numpy().astype(np.float64)
    lse = s.lse.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(out - ref_o)) <= TOL_OUT and np.max(np.abs(lse - ref_l)) <= TOL_LSE
    clean(s, plan)


def test_indexer_flags_bad_page(dev):
    cfg = dataclasses.replace(W.small_variant(SPARSE, batch=2, seqlen_hi=500), topk=100)
    wl = W.make_workload(cfg)
    ix = W.make_indexer_inputs(wl)
    bt = wl.block_table.copy()
    bt[1, 2] = ix.k_cache.shape[0] + 5   # outside the cache: clamped on the device and flagged
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_indexer(wl, ix, 100, block_table=bt, err=err)
    assert int(err.item()) & 2
