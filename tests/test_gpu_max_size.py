"""GPU parity at cache sizes where 32-bit byte offsets would overflow.

One GQA sequence of 1,310,720 cached tokens (5/4 of 2^20) beside a short one,
Llama-3-8B heads (32 q / 8 KV, d 128, page 16): K and V hold 2.7 GB each, so
page offsets pass 2^31 bytes in both page layouts.  One dense MLA sequence of
1,900,000 tokens (page 64) beside a short one: a 2.19 GB latent cache.  The
plans are the benchmark's (one chunk per compute unit, the device's XCDs).

Checked against the fp64 oracle on every output of two KV heads (GQA: the
first and the last) and of every head (MLA), to the usual bar (1e-2 on out,
1e-3 on lse); every other output finite.  The inputs come from the seeded
generator like every other case (N(0,1) bf16, shuffled pages).
"""
import dataclasses

import numpy as np
import pytest

from cross_cu_load_amd import workloads as W

from gpu_helpers import clean, compare, run

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _finite(s):
    assert bool(torch.isfinite(s.out).all()) and bool(torch.isfinite(s.lse).all())


@pytest.mark.parametrize("layout", [W.KV_NHD, W.KV_HND])
def test_gqa_cache_past_2gib(dev, layout):
    cfg = dataclasses.replace(W.CONFIG_BY_NAME["llama3_8b_gqa"], name="llama3_8b_gqa_max", batch=2, seed=1201,
                              kv_layout=layout)
    sl = np.array([1310720, 777], np.int32)
    wl = W.make_workload(cfg, seqlens=sl)
    per_cache = int(wl.k_cache.nbytes)
    assert per_cache > (1 << 31), per_cache
    s, plan = run(wl, *dev, tag=f"max-size gqa {'HND' if layout else 'NHD'}")
    _finite(s)
    compare(s, wl, only=[(0, 0, 0), (0, 0, 7), (1, 0, 0), (1, 0, 7)],
            label=f"gqa 1.31M tokens {'HND' if layout else 'NHD'}")
    clean(s, plan)


def test_mla_cache_past_2gib(dev):
    cfg = dataclasses.replace(W.CONFIG_BY_NAME["deepseek_mla"], name="deepseek_mla_max", batch=2, seed=1202)
    sl = np.array([1900000, 3000], np.int32)
    wl = W.make_workload(cfg, seqlens=sl)
    assert int(wl.k_cache.nbytes) > (1 << 31)
    s, plan = run(wl, *dev, tag="max-size mla")
    _finite(s)
    compare(s, wl, label="mla 1.9M tokens")
    clean(s, plan)
