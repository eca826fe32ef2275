"""The seeded input generator: determinism, shapes, paging and bf16 rounding (CPU only)."""
import numpy as np
import pytest

from cross_cu_load_amd import workloads as W


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 3.0e38],
                 np.float32)
    bits = W.round_to_bf16_bits(f)
    # ties go to even mantissa; above-half rounds up
    assert list(bits[:4]) == [0x3F80, 0x3F80, 0x3F82, 0x3F81]
    assert bits[4] == 0xC020
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(back - f) <= np.abs(f) * 2 ** -8)


def test_seqlen_draws_follow_the_configs():
    c1, c2, c3, c4, c5 = W.CONFIGS
    s1 = W.draw_seqlens(c1)
    assert s1.shape == (4,) and s1.min() >= 1 and s1.max() <= 512
    s2 = W.draw_seqlens(c2)
    assert s2.shape == (64,) and s2.min() >= 128 and s2.max() <= 32768
    # log-uniform: roughly equal mass per octave
    oct_counts = np.histogram(np.log2(s2), bins=8, range=(7, 15))[0]
    assert oct_counts.min() >= 2
    s3 = W.draw_seqlens(c3)
    assert s3[0] == 131072 and np.all(s3[1:] == 256) and s3.shape == (32,)
    s4 = W.draw_seqlens(c4)
    assert s4.min() >= 1024 and s4.max() <= 16384
    assert np.all(W.draw_seqlens(c5) == 8192)
    assert np.array_equal(W.draw_seqlens(c2), s2)


def test_page_table_is_a_permutation_of_used_pages():
    s = np.array([1, 16, 17, 100], np.int32)
    bt = W.page_table(s, 16, True, 5)
    used = []
    for b, L in enumerate(s):
        n = (L + 15) // 16
        used.extend(bt[b, :n])
        assert np.all(bt[b, n:] == -1)
    assert sorted(used) == list(range(len(used)))


@pytest.mark.parametrize("name", ["tiny_gqa", "sparse_mla"])
def test_small_workloads_shapes_and_determinism(name):
    cfg = W.CONFIG_BY_NAME[name]
    a = W.make_workload(cfg)
    b = W.make_workload(cfg)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_cache, b.k_cache)
    assert a.q.shape == (cfg.batch, cfg.q_tokens, cfg.num_q_heads, cfg.head_dim_qk)
    assert a.k_cache.shape[1:] == (cfg.page_size, cfg.num_kv_heads, cfg.head_dim_qk)
    if cfg.mode == W.MODE_MLA_SPARSE:
        assert a.indices.shape == (2, 8, 2048) and a.v_cache is None
        for r in range(2):
            for t in range(8):
                row = a.indices[r, t]
                assert len(np.unique(row)) == 2048 and row.min() >= 0 and row.max() < 8192
    else:
        assert a.v_cache.shape == a.k_cache.shape[:3] + (cfg.head_dim_v,)
    # values look like N(0,1) rounded to bf16
    x = (a.k_cache.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(x.mean())) < 0.05 and abs(float(x.std()) - 1) < 0.05


def test_chunked_fill_is_independent_of_chunk_boundaries():
    a = W.normal_bf16(7, 3, (3, 1 << 21))          # spans two fill chunks
    b = W.normal_bf16(7, 3, (3 << 21,))
    assert np.array_equal(a.reshape(-1), b)
