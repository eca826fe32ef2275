"""GPU parity with non-finite cache contents wherever attention must not look.

A paged cache holds more than the keys a call attends over: the rows of a
sequence's last page past its length, pages no sequence names, and (index-
sparse) every row no index selects.  The kernels read whole 32-token blocks
inside a page, so rows past the end are fetched; their scores are masked and
their probabilities are exactly 0, but 0 times NaN or Inf is NaN, so the
kernels zero those V rows before the products.  Here every cache row outside
the attended set is NaN, +Inf or -Inf (bf16, by row), and the outputs must
still match the fp64 oracle (which reads only the attended rows) to the usual
bar: max|out - oracle| <= 1e-2, max|lse - oracle| <= 1e-3, all finite.
"""
import dataclasses

import numpy as np
import pytest

from cross_cu_load_amd import workloads as W

from gpu_helpers import clean, compare, run

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

_BAD = np.array([0x7FC0, 0x7F80, 0xFF80], np.uint16)  # bf16 NaN, +Inf, -Inf


def _attended(wl):
    """Boolean [num_pages, page_size]: the cache rows the call attends over."""
    P = wl.cfg.page_size
    used = np.zeros((wl.k_cache.shape[0], P), bool)
    for b, L in enumerate(wl.seqlens):
        if wl.indices is not None:
            toks = np.unique(wl.indices[b].reshape(-1))
            toks = toks[(toks >= 0) & (toks < L)]
        else:
            toks = np.arange(int(L))
        pages = wl.block_table[b, toks // P]
        used[pages, toks % P] = True
    return used


def _poison(wl):
    """Every row outside the attended set becomes NaN / +Inf / -Inf (in place)."""
    used = _attended(wl)
    P = wl.cfg.page_size
    rows = np.argwhere(~used)
    assert len(rows) > 0
    bad = _BAD[np.arange(len(rows)) % 3]
    hnd = wl.cfg.kv_layout == W.KV_HND and wl.v_cache is not None
    for cache in (wl.k_cache, wl.v_cache):
        if cache is None:
            continue
        if hnd:    # [num_pages, Hkv, P, d]
            cache[rows[:, 0], :, rows[:, 1], :] = bad[:, None, None]
        else:      # [num_pages, P, Hkv, d]
            cache[rows[:, 0], rows[:, 1], :, :] = bad[:, None, None]
    return int((~used).sum()), used.size // P


# lengths that end inside 32-token blocks and inside pages, and one empty sequence
_SL = np.array([1, 31, 33, 63, 65, 100, 0, 257, 1000], np.int32)


@pytest.mark.parametrize("layout", [W.KV_NHD, W.KV_HND])
def test_gqa_poisoned_rows(dev, layout):
    cfg = dataclasses.replace(W.small_variant(W.CONFIG_BY_NAME["llama3_8b_gqa"], batch=len(_SL), seqlen_hi=1000),
                              kv_layout=layout)
    wl = W.make_workload(cfg, seqlens=_SL)
    n, pages = _poison(wl)
    s, plan = run(wl, *dev, tag=f"gqa poisoned rows layout={layout} ({n} rows of {pages} pages)")
    compare(s, wl, label=f"gqa poisoned rows {'HND' if layout else 'NHD'}")
    clean(s, plan)


@pytest.mark.parametrize("page", [32, 64])
def test_mla_poisoned_rows(dev, page):
    cfg = dataclasses.replace(W.small_variant(W.CONFIG_BY_NAME["deepseek_mla"], batch=len(_SL), seqlen_hi=1000),
                              page_size=page)
    wl = W.make_workload(cfg, seqlens=_SL)
    n, pages = _poison(wl)
    s, plan = run(wl, *dev, tag=f"mla poisoned rows page={page} ({n} rows of {pages} pages)")
    compare(s, wl, label=f"mla poisoned rows page {page}")
    clean(s, plan)


def test_sparse_mla_poisoned_unselected_rows(dev):
    cfg = W.small_variant(W.CONFIG_BY_NAME["sparse_mla"], batch=2, seqlen_hi=1500)
    cfg = dataclasses.replace(cfg, topk=300)
    wl = W.make_workload(cfg)
    n, pages = _poison(wl)
    s, plan = run(wl, *dev, tag=f"sparse poisoned unselected rows ({n} rows of {pages} pages)")
    compare(s, wl, label="sparse mla poisoned unselected rows")
    clean(s, plan)
