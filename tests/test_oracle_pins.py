"""Pins of the fp64 attention oracle to facts outside itself (CPU only).

Each check rests on something the oracle's own code does not provide:
IEEE bf16 bit definitions, a loop-level brute force of the definition on tiny
inputs, PyTorch's scaled_dot_product_attention in float64, closed forms
(one key, identical keys, a dominating key) and invariants of the method
(partition + log-sum-exp merge, token permutation, page placement).  The
mutation tests at the end plant plausible mistakes in a copy of the oracle
and check that at least one pin catches each.
"""
import math

import numpy as np
import pytest
import torch

from cross_cu_load_amd import workloads as W
from oracle import attention as A


# ---------------------------------------------------------------- helpers

def _bf16(x):
    return W.round_to_bf16_bits(np.asarray(x, dtype=np.float32))


def paged(rows_bits, seqlens, P, seed=0, shuffle=True):
    """Scatter per-sequence rows [B][L_b, H, d] (uint16) into a paged cache."""
    bt = W.page_table(np.asarray(seqlens, np.int32), P, shuffle, seed)
    npages = int(sum((L + P - 1) // P for L in seqlens))
    H, d = rows_bits[0].shape[1:]
    cache = np.zeros((npages, P, H, d), np.uint16)
    for b, L in enumerate(seqlens):
        for j in range(L):
            cache[bt[b, j // P], j % P] = rows_bits[b][j]
    return cache, bt


def rand_problem(rng, B=3, Hq=4, Hkv=2, dk=8, dv=6, P=4, lens=(1, 5, 9), scale=0.3):
    q = _bf16(rng.standard_normal((B, 1, Hq, dk)))
    K = [_bf16(rng.standard_normal((L, Hkv, dk))) for L in lens]
    V = [_bf16(rng.standard_normal((L, Hkv, dv))) for L in lens]
    kc, bt = paged(K, lens, P, seed=int(rng.integers(1 << 30)))
    # V follows K's block table
    vc = np.zeros((kc.shape[0], P, Hkv, dv), np.uint16)
    for b, L in enumerate(lens):
        for j in range(L):
            vc[bt[b, j // P], j % P] = V[b][j]
    return dict(q=q, K=K, V=V, kc=kc, vc=vc, bt=bt, lens=np.array(lens, np.int32), scale=scale,
                Hq=Hq, Hkv=Hkv, dv=dv)


def run(pr, attend=None):
    return A.decode_attention(pr["q"], pr["kc"], pr["vc"], pr["bt"], pr["lens"], pr["scale"])


# ---------------------------------------------------------------- pins

def test_bf16_widening_matches_ieee_definitions():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x8000, 0x4049], np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, math.inf, -0.0, 3.140625]
    got = A.bf16_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)


def bruteforce(pr):
    """Loop-level transcription of the definition with math.exp; no numpy BLAS."""
    q = A.bf16_to_f64(pr["q"])
    B, _, Hq, dk = q.shape
    G = Hq // pr["Hkv"]
    out = np.zeros((B, 1, Hq, pr["dv"]))
    lse = np.zeros((B, 1, Hq))
    for b in range(B):
        K = A.bf16_to_f64(pr["K"][b])
        V = A.bf16_to_f64(pr["V"][b])
        if len(K) == 0:      # no key: left to the callers (0/0 in the definition)
            continue
        for h in range(Hq):
            g = h // G
            s = [pr["scale"] * sum(float(q[b, 0, h, d]) * float(K[j, g, d]) for d in range(dk))
                 for j in range(len(K))]
            e = [math.exp(x) for x in s]
            Z = sum(e)
            for c in range(pr["dv"]):
                out[b, 0, h, c] = sum(e[j] * float(V[j, g, c]) for j in range(len(K))) / Z
            lse[b, 0, h] = math.log(Z)
    return out, lse


def test_bruteforce_tiny():
    rng = np.random.default_rng(7)
    for lens in [(1, 2, 3), (5, 8, 13), (4,)]:
        pr = rand_problem(rng, B=len(lens), lens=lens)
        o, s = run(pr)
        bo, bs = bruteforce(pr)
        np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(s, bs, rtol=0, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (6, 1)])
def test_matches_torch_sdpa_float64(Hq, Hkv):
    rng = np.random.default_rng(11 + Hq)
    lens = (7, 33, 1, 64)
    pr = rand_problem(rng, B=len(lens), Hq=Hq, Hkv=Hkv, dk=16, dv=16, P=8, lens=lens, scale=1 / 4)
    o, s = run(pr)
    q = torch.from_numpy(A.bf16_to_f64(pr["q"]))
    for b, L in enumerate(lens):
        K = torch.from_numpy(A.bf16_to_f64(pr["K"][b])).permute(1, 0, 2)   # [Hkv, L, d]
        V = torch.from_numpy(A.bf16_to_f64(pr["V"][b])).permute(1, 0, 2)
        qb = q[b, 0][:, None, :]                                          # [Hq, 1, d]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qb[None], K[None], V[None], scale=pr["scale"], enable_gqa=True)[0, :, 0]
        np.testing.assert_allclose(o[b, 0], ref.numpy(), rtol=0, atol=1e-12)
        Kr = K.repeat_interleave(Hq // Hkv, dim=0)
        logits = (qb @ Kr.transpose(1, 2))[:, 0] * pr["scale"]
        np.testing.assert_allclose(s[b, 0], torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_single_key_returns_its_value_row():
    rng = np.random.default_rng(3)
    pr = rand_problem(rng, B=2, lens=(1, 1))
    o, s = run(pr)
    q = A.bf16_to_f64(pr["q"])
    for b in range(2):
        K = A.bf16_to_f64(pr["K"][b])[0]
        V = A.bf16_to_f64(pr["V"][b])[0]
        for h in range(pr["Hq"]):
            g = h // (pr["Hq"] // pr["Hkv"])
            assert np.array_equal(o[b, 0, h], V[g])
            assert s[b, 0, h] == pytest.approx(pr["scale"] * float(q[b, 0, h] @ K[g]), abs=1e-14)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(5)
    L = 37
    pr = rand_problem(rng, B=1, lens=(L,))
    k0 = pr["K"][0][0].copy()
    pr["K"][0][:] = k0
    pr["kc"], pr["bt"] = paged(pr["K"], (L,), 4, seed=9)
    vc = np.zeros((pr["kc"].shape[0], 4, pr["Hkv"], pr["dv"]), np.uint16)
    for j in range(L):
        vc[pr["bt"][0, j // 4], j % 4] = pr["V"][0][j]
    pr["vc"] = vc
    o, s = run(pr)
    V = A.bf16_to_f64(pr["V"][0])
    q = A.bf16_to_f64(pr["q"])
    G = pr["Hq"] // pr["Hkv"]
    for h in range(pr["Hq"]):
        g = h // G
        np.testing.assert_allclose(o[0, 0, h], V[:, g].mean(axis=0), rtol=0, atol=1e-13)
        s0 = pr["scale"] * float(q[0, 0, h] @ A.bf16_to_f64(k0)[g])
        assert s[0, 0, h] == pytest.approx(s0 + math.log(L), abs=1e-12)


def test_dominating_key_limit_and_no_overflow():
    rng = np.random.default_rng(8)
    L, dk, dv = 50, 8, 5
    K = rng.standard_normal((L, dk))
    V = rng.standard_normal((L, dv))
    jstar = 17
    for c in (30.0, 1000.0):
        q = c * K[jstar][None, :]
        o, s = A.attend(q, K, V, 1.0)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
        if c == 1000.0:
            np.testing.assert_allclose(o[0], V[jstar], rtol=0, atol=1e-12)
            assert s[0] == pytest.approx(float(q[0] @ K[jstar]), rel=1e-12)


def test_partition_merge_equals_unsplit():
    rng = np.random.default_rng(12)
    for trial in range(40):
        n = int(rng.integers(1, 300))
        G, dk, dv = 4, 16, 12
        q = rng.standard_normal((G, dk)) * 2
        K = rng.standard_normal((n, dk))
        V = rng.standard_normal((n, dv))
        npieces = int(rng.integers(1, min(n, 64) + 1))
        cuts = np.sort(rng.choice(np.arange(1, n), size=npieces - 1, replace=False)) if npieces > 1 else []
        bounds = [0, *cuts, n]
        parts = [A.partial_state(q, K[a:b], V[a:b], 0.25) for a, b in zip(bounds[:-1], bounds[1:])]
        mo, ms = A.lse_merge(parts)
        o, s = A.attend(q, K, V, 0.25)
        np.testing.assert_allclose(mo, o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ms, s, rtol=1e-12, atol=1e-13)


def test_token_permutation_invariance():
    rng = np.random.default_rng(21)
    lens = (40, 3)
    pr = rand_problem(rng, B=2, lens=lens)
    o, s = run(pr)
    perms = [rng.permutation(L) for L in lens]
    pr2 = dict(pr)
    pr2["K"] = [k[p] for k, p in zip(pr["K"], perms)]
    pr2["V"] = [v[p] for v, p in zip(pr["V"], perms)]
    pr2["kc"], pr2["bt"] = paged(pr2["K"], lens, 4, seed=33)
    vc = np.zeros_like(pr["vc"])
    for b, L in enumerate(lens):
        for j in range(L):
            vc[pr2["bt"][b, j // 4], j % 4] = pr2["V"][b][j]
    pr2["vc"] = vc
    o2, s2 = run(pr2)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(s2, s, rtol=0, atol=1e-13)


def test_page_placement_is_bitwise_irrelevant():
    rng = np.random.default_rng(4)
    lens = (29, 64, 1)
    pr = rand_problem(rng, B=3, lens=lens, P=4)
    o, s = run(pr)
    for P in (1, 16, 64):
        kc, bt = paged(pr["K"], lens, P, seed=P)
        vc = np.zeros((kc.shape[0], P, pr["Hkv"], pr["dv"]), np.uint16)
        for b, L in enumerate(lens):
            for j in range(L):
                vc[bt[b, j // P], j % P] = pr["V"][b][j]
        o2, s2 = A.decode_attention(pr["q"], kc, vc, bt, pr["lens"], pr["scale"])
        assert np.array_equal(o, o2) and np.array_equal(s, s2)


def test_head_major_pages_index_the_same_elements():
    rng = np.random.default_rng(61)
    lens = (29, 3, 64)
    pr = rand_problem(rng, B=3, Hq=8, Hkv=2, lens=lens, P=16)
    o, s = run(pr)
    kh = np.ascontiguousarray(pr["kc"].transpose(0, 2, 1, 3))
    vh = np.ascontiguousarray(pr["vc"].transpose(0, 2, 1, 3))
    o2, s2 = A.decode_attention(pr["q"], kh, vh, pr["bt"], pr["lens"], pr["scale"], head_major=True)
    assert np.array_equal(o, o2) and np.array_equal(s, s2)
    # and a head-major cache read as token-major gives something else
    o3, _ = A.decode_attention(pr["q"], kh.reshape(pr["kc"].shape), vh.reshape(pr["vc"].shape), pr["bt"],
                               pr["lens"], pr["scale"])
    assert not np.allclose(o3, o)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(31)
    lens = (12, 5)
    pr = rand_problem(rng, B=2, Hq=6, Hkv=2, lens=lens)
    o, s = run(pr)
    G = 3
    Krep = [np.repeat(k, G, axis=1) for k in pr["K"]]      # kv head g -> q heads g*G..g*G+G-1
    Vrep = [np.repeat(v, G, axis=1) for v in pr["V"]]
    kc, bt = paged(Krep, lens, 4, seed=2)
    vc = np.zeros((kc.shape[0], 4, 6, pr["dv"]), np.uint16)
    for b, L in enumerate(lens):
        for j in range(L):
            vc[bt[b, j // 4], j % 4] = Vrep[b][j]
    o2, s2 = A.decode_attention(pr["q"], kc, vc, bt, pr["lens"], pr["scale"])
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(s2, s, rtol=0, atol=1e-13)


def test_mla_value_is_leading_latent_columns():
    rng = np.random.default_rng(41)
    lens = (20, 7)
    dk, dv = 24, 16
    q = _bf16(rng.standard_normal((2, 1, 8, dk)))
    K = [_bf16(rng.standard_normal((L, 1, dk))) for L in lens]
    kc, bt = paged(K, lens, 8, seed=1)
    o, s = A.decode_attention(q, kc, None, bt, np.array(lens, np.int32), 0.2, head_dim_v=dv)
    o2, s2 = A.decode_attention(q, kc, np.ascontiguousarray(kc[..., :dv]), bt, np.array(lens, np.int32), 0.2)
    assert np.array_equal(o, o2) and np.array_equal(s, s2)


def test_sparse_equals_dense_attention_over_the_index_set():
    rng = np.random.default_rng(51)
    L, topk, dk, dv, Tq = 300, 40, 24, 16, 3
    q = _bf16(rng.standard_normal((1, Tq, 4, dk)))
    K = [_bf16(rng.standard_normal((L, 1, dk)))]
    kc, bt = paged(K, (L,), 16, seed=5)
    idx = np.stack([rng.choice(L, topk, replace=False) for _ in range(Tq)])[None].astype(np.int32)
    o, s = A.decode_attention(q, kc, None, bt, np.array([L], np.int32), 0.2, head_dim_v=dv, indices=idx)
    for t in range(Tq):
        sub = [K[0][idx[0, t]]]
        kc2, bt2 = paged(sub, (topk,), 16, seed=t)
        o2, s2 = A.decode_attention(q[:, t:t + 1], kc2, None, bt2, np.array([topk], np.int32), 0.2,
                                    head_dim_v=dv)
        np.testing.assert_allclose(o[0, t], o2[0, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(s[0, t], s2[0, 0], rtol=0, atol=1e-13)


# ------------------------------------------------- planted mistakes (mutants)

def _pin_suite(attend_fn, merge_fn, partial_fn, decode_fn):
    """Runs a compact version of the pins above against substituted oracle pieces.

    Returns the list of pins that failed.
    """
    failed = []
    rng = np.random.default_rng(99)
    pr = rand_problem(rng, B=2, Hq=4, Hkv=2, dk=8, dv=6, P=4, lens=(6, 9))
    o, s = decode_fn(pr["q"], pr["kc"], pr["vc"], pr["bt"], pr["lens"], pr["scale"])
    bo, bs = bruteforce(pr)
    if not (np.allclose(o, bo, atol=1e-12, rtol=0) and np.allclose(s, bs, atol=1e-12, rtol=0)):
        failed.append("bruteforce")
    # identical keys -> lse = s + ln L
    q = rng.standard_normal((2, 8))
    K = np.tile(rng.standard_normal((1, 8)), (10, 1))
    V = rng.standard_normal((10, 6))
    o1, s1 = attend_fn(q, K, V, 0.5)
    if not (np.allclose(o1, V.mean(0), atol=1e-12) and np.allclose(s1, 0.5 * q @ K[0] + math.log(10), atol=1e-12)):
        failed.append("identical_keys")
    # overflow guard
    o2, s2 = attend_fn(1000 * K[:1], K, V, 1.0)
    if not (np.all(np.isfinite(o2)) and np.all(np.isfinite(s2))):
        failed.append("overflow")
    # partition + merge
    K2 = rng.standard_normal((40, 8))
    V2 = rng.standard_normal((40, 6))
    parts = [partial_fn(q, K2[a:b], V2[a:b], 0.5) for a, b in ((0, 13), (13, 40))]
    mo, ms = merge_fn(parts)
    ro, rs = attend_fn(q, K2, V2, 0.5)
    if not (np.allclose(mo, ro, atol=1e-12) and np.allclose(ms, rs, atol=1e-12)):
        failed.append("merge")
    return failed


def test_unmodified_oracle_passes_the_compact_pins():
    assert _pin_suite(A.attend, A.lse_merge, A.partial_state, A.decode_attention) == []


_ATTEND = A.attend


def _mut_no_scale(q, K, V, scale):
    return _ATTEND(q, K, V, 1.0)


def _mut_log2_lse(q, K, V, scale):
    o, s = _ATTEND(q, K, V, scale)
    return o, s / math.log(2)


def _mut_no_max_subtract(q, K, V, scale):
    s = scale * (q @ K.T)
    w = np.exp(s)
    l = w.sum(axis=1, keepdims=True)
    return (w @ V) / l, np.log(l)[:, 0]


def _mut_merge_drops_rescale(parts):
    L = sum(p[1] for p in parts)
    O = sum(p[2] for p in parts)
    M = np.stack([p[0] for p in parts]).max(axis=0)
    return O / L[:, None], M + np.log(L)


def _mut_head_map_mod(q_bits, k_bits, v_bits, block_table, seqlens, scale, **kw):
    # query head h reads kv head h % Hkv instead of h // G
    B, Tq, Hq, dk = q_bits.shape
    Hkv = k_bits.shape[2]
    perm = [(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)]
    inv = np.argsort(perm)
    o, s = A.decode_attention(q_bits[:, :, perm], k_bits, v_bits, block_table, seqlens, scale, **kw)
    return o[:, :, inv], s[:, :, inv]


def _mut_kv_gather_mismatch(q_bits, k_bits, v_bits, block_table, seqlens, scale, **kw):
    # V rows gathered with the slot order reversed inside each page, so keys and
    # values no longer pair up (a transposed page/slot index on one side)
    return A.decode_attention(q_bits, k_bits, np.ascontiguousarray(v_bits[:, ::-1]), block_table,
                              seqlens, scale, **kw)


@pytest.mark.parametrize("mutant", ["no_scale", "log2_lse", "no_max_subtract", "merge_drops_rescale",
                                    "head_map_mod", "kv_gather_mismatch"])
def test_planted_mistakes_are_caught(mutant):
    attend, merge, partial, decode = A.attend, A.lse_merge, A.partial_state, A.decode_attention
    if mutant == "no_scale":
        attend = _mut_no_scale

        def decode(*a, **k):
            orig = A.attend
            A.attend = _mut_no_scale
            try:
                return A.decode_attention(*a, **k)
            finally:
                A.attend = orig
    elif mutant == "log2_lse":
        attend = _mut_log2_lse
    elif mutant == "no_max_subtract":
        attend = _mut_no_max_subtract
    elif mutant == "merge_drops_rescale":
        merge = _mut_merge_drops_rescale
    elif mutant == "head_map_mod":
        decode = _mut_head_map_mod
    elif mutant == "kv_gather_mismatch":
        decode = _mut_kv_gather_mismatch
    assert _pin_suite(attend, merge, partial, decode), "a planted mistake went unnoticed"


def test_empty_key_set_is_the_neutral_element_of_the_merge():
    """A sequence with no cached tokens: lse = log of an empty sum = -inf (as
    torch.logsumexp of an empty tensor), out = 0.  That state (m = -inf, l = 0,
    o = 0) merged with any partition of a key set leaves the unsplit result
    unchanged, wherever the empty pieces sit; all-empty merges to (0, -inf)."""
    assert float(torch.logsumexp(torch.empty(0, dtype=torch.float64), 0)) == -math.inf
    rng = np.random.default_rng(31)
    G, dk, dv = 4, 16, 12
    q = rng.standard_normal((G, dk))
    o, s = A.attend(q, np.zeros((0, dk)), np.zeros((0, dv)), 0.25)
    assert np.array_equal(o, np.zeros((G, dv))) and np.all(s == -np.inf)
    for trial in range(20):
        n = int(rng.integers(1, 100))
        K, V = rng.standard_normal((n, dk)), rng.standard_normal((n, dv))
        cut = int(rng.integers(0, n + 1))
        empty = A.partial_state(q, K[:0], V[:0], 0.25)
        parts = [A.partial_state(q, K[:cut], V[:cut], 0.25), empty, A.partial_state(q, K[cut:], V[cut:], 0.25)]
        mo, ms = A.lse_merge(parts)
        ro, rs = A.attend(q, K, V, 0.25)
        np.testing.assert_allclose(mo, ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ms, rs, rtol=1e-12, atol=1e-13)
    mo, ms = A.lse_merge([empty, empty])
    assert np.array_equal(mo, np.zeros((G, dv))) and np.all(ms == -np.inf)


def test_empty_sequences_in_a_paged_batch():
    """Empty sequences in a batch give (0, -inf); the others are unchanged
    from the batch without them (same rows, recomputed by brute force)."""
    rng = np.random.default_rng(32)
    pr = rand_problem(rng, B=5, lens=(0, 5, 0, 9, 1))
    out, lse = run(pr)
    for b in (0, 2):
        assert np.array_equal(out[b], np.zeros_like(out[b])) and np.all(lse[b] == -np.inf)
    bf_o, bf_l = bruteforce(pr)
    keep = [1, 3, 4]
    np.testing.assert_allclose(out[keep], bf_o[keep], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[keep], bf_l[keep], rtol=1e-12, atol=1e-13)


def test_shared_prefix_pages_equal_private_copies():
    """Sequences whose block tables name the same prefix pages (the shared-prefix
    decode) get exactly the results of the same batch with every prefix page
    copied into each sequence's own pages; and each sequence's result is the
    log-sum-exp merge of its prefix part and its own part."""
    import dataclasses
    cfg = dataclasses.replace(W.CONFIG_BY_NAME["shared_prefix_gqa"], prefix_len=0, batch=5, num_q_heads=8,
                              num_kv_heads=2, head_dim_qk=32, head_dim_v=32, softmax_scale=0.2, seed=77)
    sl = np.array([80, 64, 100, 70, 33], np.int32)
    wl = W.make_grouped_workload(cfg, sl, [0, 0, 0, 1, -1], [64, 48])
    o, l = A.decode_attention_wl(wl)
    # private copies: a fresh cache where every (sequence, logical page) has its own page
    P = cfg.page_size
    npg = [(int(L) + P - 1) // P for L in sl]
    bt2 = np.full_like(wl.block_table, -1)
    k2 = np.zeros((sum(npg),) + wl.k_cache.shape[1:], wl.k_cache.dtype)
    v2 = np.zeros_like(k2)
    nxt = 0
    for b, n in enumerate(npg):
        for i in range(n):
            k2[nxt] = wl.k_cache[wl.block_table[b, i]]
            v2[nxt] = wl.v_cache[wl.block_table[b, i]]
            bt2[b, i] = nxt
            nxt += 1
    assert len(set(wl.block_table[:3, :4].ravel())) == 4     # members 0..2 share their 4 prefix pages
    o2, l2 = A.decode_attention(wl.q, k2, v2, bt2, sl, cfg.softmax_scale)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    # prefix part + own part, merged
    G = cfg.group
    for b, Lp in ((0, 64), (2, 64), (3, 48)):
        for g in range(cfg.num_kv_heads):
            q = A.bf16_to_f64(wl.q[b, 0, g * G:(g + 1) * G])
            parts = []
            for J in (np.arange(Lp), np.arange(Lp, int(sl[b]))):
                K = A.gather_rows(wl.k_cache, wl.block_table, b, J, P)[:, g]
                V = A.gather_rows(wl.v_cache, wl.block_table, b, J, P)[:, g]
                parts.append(A.partial_state(q, K, V, cfg.softmax_scale))
            mo, ml = A.lse_merge(parts)
            assert np.allclose(mo, o[b, 0, g * G:(g + 1) * G], rtol=0, atol=1e-12)
            assert np.allclose(ml, l[b, 0, g * G:(g + 1) * G], rtol=0, atol=1e-12)
