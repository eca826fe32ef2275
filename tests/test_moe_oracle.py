"""Pins of the fp64 MoE grouped-GEMM oracle (CPU only).

The oracle is held to facts that do not come from itself: a pure-Python
triple loop on tiny inputs, torch float64 matmul (another library), closed
forms (one-hot rows pick a weight column; an identity weight returns X), the
split of K into pieces whose products add up to the whole (the identity the
Stream-K split relies on), invariance to the order of experts, experts with
no rows, and planted mistakes that one of these must catch.
"""
import numpy as np
import pytest
import torch

from cross_cu_load_amd import workloads as W
from oracle import moe as M


def _bits(a):
    """float array -> bf16 bit patterns (exact for values bf16 can hold)."""
    u = np.asarray(a, np.float32).view(np.uint32)
    assert np.all(u & 0xFFFF == 0), "values must be bf16-representable"
    return (u >> 16).astype(np.uint16)


def _rand(rng, shape):
    return _bits(np.round(rng.standard_normal(shape) * 4) / 4)   # quarter steps: exact in bf16


def test_triple_loop_on_tiny_inputs():
    rng = np.random.default_rng(1)
    E, K, N = 3, 5, 4
    counts = [2, 0, 3]
    off = np.concatenate([[0], np.cumsum(counts)])
    x, w = _rand(rng, (5, K)), _rand(rng, (E, N, K))
    y = M.grouped_gemm(x, w, off)
    xf, wf = M.bf16_to_f64(x), M.bf16_to_f64(w)
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            for n in range(N):
                s = 0.0
                for k in range(K):
                    s += xf[r, k] * wf[e, n, k]
                assert y[r, n] == s


def test_matches_torch_float64():
    rng = np.random.default_rng(2)
    E, K, N = 4, 64, 48
    counts = [7, 0, 19, 3]
    off = np.concatenate([[0], np.cumsum(counts)])
    x, w = _rand(rng, (29, K)), _rand(rng, (E, N, K))
    y = M.grouped_gemm(x, w, off)
    xt = torch.from_numpy(M.bf16_to_f64(x))
    wt = torch.from_numpy(M.bf16_to_f64(w))
    for e in range(E):
        a, b = off[e], off[e + 1]
        assert np.allclose(y[a:b], (xt[a:b] @ wt[e].T).numpy(), rtol=0, atol=1e-9)


def test_one_hot_rows_pick_weight_columns_and_identity_weight_returns_x():
    E, K, N = 2, 8, 8
    off = np.array([0, 3, 8])
    x = np.zeros((8, K), np.float32)
    ks = [0, 5, 7, 1, 2, 3, 6, 4]
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    rng = np.random.default_rng(3)
    w = _rand(rng, (E, N, K))
    y = M.grouped_gemm(_bits(x), w, off)
    wf = M.bf16_to_f64(w)
    for r, k in enumerate(ks):
        e = 0 if r < 3 else 1
        assert np.array_equal(y[r], wf[e, :, k])
    eye = np.broadcast_to(np.eye(K, dtype=np.float32), (E, K, K))
    xr = _rand(rng, (8, K))
    assert np.array_equal(M.grouped_gemm(xr, _bits(eye), off), M.bf16_to_f64(xr))


def test_k_split_pieces_add_up_to_the_product():
    """sum over pieces [k_i, k_{i+1}) of X[:, piece] W[:, :, piece]^T equals Y."""
    rng = np.random.default_rng(4)
    E, K, N = 3, 96, 16
    off = np.array([0, 10, 10, 25])
    x, w = _rand(rng, (25, K)), _rand(rng, (E, N, K))
    y = M.grouped_gemm(x, w, off)
    for _ in range(5):
        cuts = np.sort(rng.choice(np.arange(1, K), size=int(rng.integers(1, 6)), replace=False))
        bounds = [0] + list(cuts) + [K]
        s = sum(M.grouped_gemm(np.ascontiguousarray(x[:, a:b]), np.ascontiguousarray(w[:, :, a:b]), off)
                for a, b in zip(bounds[:-1], bounds[1:]))
        assert np.allclose(s, y, rtol=0, atol=1e-9)


def test_expert_order_is_irrelevant_and_empty_experts_add_nothing():
    rng = np.random.default_rng(5)
    E, K, N = 5, 32, 24
    counts = np.array([4, 0, 9, 2, 0])
    off = np.concatenate([[0], np.cumsum(counts)])
    x, w = _rand(rng, (15, K)), _rand(rng, (E, N, K))
    y = M.grouped_gemm(x, w, off)
    perm = np.array([3, 0, 4, 2, 1])
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in perm])
    off2 = np.concatenate([[0], np.cumsum(counts[perm])])
    y2 = M.grouped_gemm(np.ascontiguousarray(x[rows]), np.ascontiguousarray(w[perm]), off2)
    assert np.array_equal(y2, y[rows])
    keep = counts > 0
    off3 = np.concatenate([[0], np.cumsum(counts[keep])])
    assert np.array_equal(M.grouped_gemm(x, np.ascontiguousarray(w[keep]), off3), y)


def test_error_bound_scale():
    rng = np.random.default_rng(6)
    x, w = _rand(rng, (6, 16)), _rand(rng, (2, 8, 16))
    off = np.array([0, 2, 6])
    s = M.abs_product_sums(x, w, off)
    y = M.grouped_gemm(x, w, off)
    assert np.all(s >= np.abs(y)) and M.gamma(4096) == pytest.approx(4096 * 2.0 ** -24 / (1 - 4096 * 2.0 ** -24))


@pytest.mark.parametrize("mutant", ["transposed_weight", "offset_off_by_one", "last_expert_dropped", "no_widen"])
def test_planted_mistakes_are_caught(mutant):
    """A plausible mistake in a copy of the oracle fails the triple-loop pin."""
    rng = np.random.default_rng(7)
    E, K, N = 3, 6, 6
    counts = [2, 3, 2]
    off = np.concatenate([[0], np.cumsum(counts)])
    x, w = _rand(rng, (7, K)), _rand(rng, (E, N, K))

    def bad(xb, wb, o):
        y = np.zeros((xb.shape[0], wb.shape[1]))
        xf, wf = M.bf16_to_f64(xb), M.bf16_to_f64(wb)
        for e in range(E):
            a, b = int(o[e]), int(o[e + 1])
            if mutant == "offset_off_by_one":
                a = max(0, a - 1)
            if mutant == "last_expert_dropped" and e == E - 1:
                continue
            we = wf[e] if mutant != "transposed_weight" else wf[e].T
            if mutant == "no_widen":
                xf = xb.astype(np.float64)
            y[a:b] = xf[a:b] @ we.T
        return y

    xf, wf = M.bf16_to_f64(x), M.bf16_to_f64(w)
    truth = np.zeros((7, N))
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            truth[r] = [sum(xf[r, k] * wf[e, n, k] for k in range(K)) for n in range(N)]
    assert np.array_equal(M.grouped_gemm(x, w, off), truth)
    assert not np.array_equal(bad(x, w, off), truth)


def test_routing_workload_shape():
    cfg = W.MOE_BY_NAME["moe_grouped_gemm"]
    et, tor = W.route(cfg)
    assert et.sum() == cfg.tokens * cfg.top_k and len(tor) == et.sum()
    assert et.max() > 4 * np.median(et)        # skewed
    # each token lands in top_k distinct experts
    off = np.concatenate([[0], np.cumsum(et)])
    seen = {}
    for e in range(cfg.num_experts):
        for t in tor[off[e]:off[e + 1]]:
            seen.setdefault(int(t), set()).add(e)
    assert all(len(s) == cfg.top_k for s in seen.values())
