"""The C-ABI library on the CPU: exports, plan bytes, validation (no GPU compute).

cc_plan must be byte-identical to the reference planner in the oracle on the
workload lengths and on random inputs; invalid inputs must come back as the
documented error codes before anything touches a device.
"""
import ctypes
import re
import os

import numpy as np
import pytest

from cross_cu_load_amd import binding as B
from cross_cu_load_amd import workloads as W
from oracle import planner as PL

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")


def declared_functions():
    names = set()
    for h in os.listdir(INCLUDE):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(cc_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.cc_version() >= 100
    assert lib.cc_strerror(B.CC_ERR_PLAN)


def _prob(cfg, sl):
    P = cfg.page_size
    maxp = int(max((int(L) + P - 1) // P for L in sl))
    npages = int(sum((int(L) + P - 1) // P for L in sl))
    return B.problem(cfg.mode, cfg.batch, cfg.q_tokens, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim_qk,
                     cfg.head_dim_v, P, maxp, npages, cfg.topk, cfg.softmax_scale), maxp, npages


@pytest.mark.parametrize("name", [c.name for c in W.CONFIGS])
@pytest.mark.parametrize("C,X,T", [(256, 8, 32), (256, 8, 64), (304, 8, 32), (148, 1, 32), (8, 8, 32)])
@pytest.mark.parametrize("policy,unit_cost", [(B.POLICY_STREAMK, 0), (B.POLICY_STREAMK, 1),
                                              (B.POLICY_STREAMK, 6), (B.POLICY_PER_UNIT, 0)])
def test_plan_bytes_match_reference_on_workload_lengths(lib, name, C, X, T, policy, unit_cost):
    cfg = W.CONFIG_BY_NAME[name]
    sl = W.draw_seqlens(cfg)
    prob, maxp, npages = _prob(cfg, sl)
    for hu in ([cfg.group] if cfg.mode == W.MODE_GQA else [32, 64, 128]):
        blob = B.plan(prob, sl, None, num_cus=C, num_xcds=X, tile_tokens=T, heads_per_unit=hu, policy=policy,
                      unit_cost=unit_cost)
        ref = PL.plan(cfg.mode, cfg.batch, cfg.q_tokens, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim_qk,
                      cfg.head_dim_v, cfg.page_size, maxp, npages, cfg.topk, C, X, T, hu, sl, None, policy,
                      unit_cost)
        assert blob.tobytes() == ref["blob"]
        B.plan_check(blob, prob, sl)
        # workspace: 256 B error word area, 128 B of counter words per unit,
        # 256-aligned partial slots of (GQA) fp32 {m[hu], l[hu], pad to 4
        # floats, o[hu][dv]} or (MLA) fp32 {m, l, r}[hu] + fp16 o[hu][dv],
        # rounded up to 64 floats
        if cfg.mode == W.MODE_GQA:
            slot = -(-(-(-2 * hu // 4) * 4 + hu * cfg.head_dim_v) // 64) * 64
        else:
            slot = -(-(3 * hu + hu * cfg.head_dim_v // 2) // 64) * 64
        cnt_end = 256 + 128 * ref["num_units"]
        part = -(-cnt_end // 256) * 256
        want = -(-(part + 4 * slot * ref["num_partials"]) // 256) * 256
        assert B.workspace_size(blob) == want


@pytest.mark.parametrize("seed", range(40))
def test_plan_bytes_match_reference_fuzz(lib, seed):
    rng = np.random.default_rng(1000 + seed)
    mode = int(rng.choice([0, 1, 2]))
    B_ = int(rng.integers(1, 9))
    Tq = 1 if mode != 2 else int(rng.integers(1, 5))
    Hkv = int(rng.choice([1, 2, 8])) if mode == 0 else 1
    G = int(rng.choice([1, 4, 8]))
    Hq = Hkv * G
    hu = int(rng.choice([d for d in (1, 2, 4, 8) if G % d == 0]))
    P = int(rng.choice([1, 16, 64]))
    sl = rng.integers(1, 3000, size=B_).astype(np.int32)
    if mode != 2:                     # dense modes: some sequences with no cached tokens
        sl[rng.random(B_) < 0.25] = 0
    topk = int(rng.integers(1, int(sl.min()) + 1)) if mode == 2 else 0
    maxp = max(1, int(max((int(L) + P - 1) // P for L in sl)))
    npages = max(1, int(sum((int(L) + P - 1) // P for L in sl)))
    bt = W.page_table(sl, P, True, seed)
    C = int(rng.choice([1, 3, 8, 100, 256, 1000]))
    X = int(rng.choice([1, 4, 8]))
    T = int(rng.choice([1, 7, 32, 64]))
    policy = int(rng.integers(0, 2))
    unit_cost = int(rng.choice([0, 1, 2, 6, 40])) if policy == B.POLICY_STREAMK else 0
    prob = B.problem(mode, B_, Tq, Hq, Hkv, 64, 64, P, maxp, npages, topk, 0.125)
    blob = B.plan(prob, sl, bt, num_cus=C, num_xcds=X, tile_tokens=T, heads_per_unit=hu, policy=policy,
                  unit_cost=unit_cost)
    ref = PL.plan(mode, B_, Tq, Hq, Hkv, 64, 64, P, maxp, npages, topk, C, X, T, hu, sl, bt, policy, unit_cost)
    assert blob.tobytes() == ref["blob"]
    B.plan_check(blob, prob, sl)


def _base():
    return dict(mode=0, batch=2, q_tokens=1, num_q_heads=8, num_kv_heads=2, head_dim_qk=64, head_dim_v=64,
                page_size=16, max_pages_per_seq=2, num_pages=4, topk=0, softmax_scale=0.125)


@pytest.mark.parametrize("bad,code", [
    ("seqlen_neg", B.CC_ERR_INVALID), ("heads", B.CC_ERR_INVALID), ("hu", B.CC_ERR_INVALID),
    ("page", B.CC_ERR_PAGE), ("tq", B.CC_ERR_INVALID), ("bt_short", B.CC_ERR_INVALID),
    ("topk", B.CC_ERR_INVALID), ("mode", B.CC_ERR_INVALID), ("cus0", B.CC_ERR_INVALID)])
def test_plan_rejects_invalid_inputs(lib, bad, code):
    kw = _base()
    sl = np.array([10, 20], np.int32)
    bt = np.array([[0, -1], [1, 2]], np.int32)
    hu, cus = 4, 8
    if bad == "seqlen_neg":
        sl = np.array([-1, 20], np.int32)
    elif bad == "heads":
        kw["num_q_heads"] = 7
    elif bad == "hu":
        hu = 3
    elif bad == "page":
        bt = np.array([[0, -1], [1, 4]], np.int32)
    elif bad == "tq":
        kw["q_tokens"] = 2
    elif bad == "bt_short":
        sl = np.array([10, 40], np.int32)
    elif bad == "topk":
        kw.update(mode=2, topk=11, num_q_heads=2, num_kv_heads=1)
        hu = 2
    elif bad == "mode":
        kw["mode"] = 7
    elif bad == "cus0":
        cus = 0
    prob = B.problem(**kw)
    with pytest.raises(B.CrossCUError) as ei:
        B.plan(prob, sl, bt, num_cus=cus, num_xcds=1, tile_tokens=32, heads_per_unit=hu)
    assert ei.value.code == code
    # the Python reference rejects the same inputs
    with pytest.raises(ValueError):
        PL.plan(kw["mode"], kw["batch"], kw["q_tokens"], kw["num_q_heads"], kw["num_kv_heads"], 64, 64, 16, 2,
                4, kw["topk"], cus, 1, 32, hu, sl, bt)


def test_plan_check_binds_the_plan_to_its_lengths(lib):
    """cc_plan_check accepts the inputs a plan was built for and refuses any
    other lengths or shape; cc_plan refuses a negative unit cost."""
    kw = _base()
    prob = B.problem(**kw)
    sl = np.array([10, 20], np.int32)
    blob = B.plan(prob, sl, None, num_cus=8, num_xcds=1, tile_tokens=32, heads_per_unit=4)
    B.plan_check(blob, prob, sl)
    for other in (np.array([10, 19], np.int32), np.array([11, 20], np.int32), np.array([20, 10], np.int32)):
        with pytest.raises(B.CrossCUError) as ei:
            B.plan_check(blob, prob, other)
        assert ei.value.code == B.CC_ERR_PLAN
    with pytest.raises(B.CrossCUError) as ei:
        B.plan_check(blob, B.problem(**{**kw, "num_pages": 5}), sl)
    assert ei.value.code == B.CC_ERR_PLAN
    with pytest.raises(B.CrossCUError) as ei:
        B.plan(prob, sl, None, num_cus=8, num_xcds=1, tile_tokens=32, heads_per_unit=4, unit_cost=-1)
    assert ei.value.code == B.CC_ERR_INVALID


def _corrupt(blob, word, value):
    w = blob.view(np.int32).copy()
    w[word] = value
    return w.view(np.uint8)


def test_plan_structure_is_validated_on_the_host(lib):
    """A blob whose items or unit table are out of range is refused by every
    call that reads a plan (cc_plan_check, cc_workspace_size, cc_decode)
    before anything touches a device."""
    kw = _base()
    prob = B.problem(**kw)
    sl = np.array([10, 20], np.int32)
    blob = B.plan(prob, sl, None, num_cus=3, num_xcds=1, tile_tokens=1, heads_per_unit=4)
    h = blob.view(np.int32)
    C, W_, U = int(h[11]), int(h[17]), int(h[15])
    assert W_ > 3       # several split units
    wg = 32
    it = wg + ((C + 1 + 3) & ~3)
    ns = it + 4 * W_
    bad = {
        "unit": _corrupt(blob, it + 0, U),
        "unit_neg": _corrupt(blob, it + 0, -1),
        "empty_range": _corrupt(blob, it + 2, int(h[it + 1])),
        "past_block_table": _corrupt(blob, it + 4 * (W_ - 1) + 2, 2 * 16 + 1),
        "split": _corrupt(blob, it + 3, int(h[ns + int(h[it])])),
        "wg_descending": _corrupt(blob, wg + 1, W_ + 1),
        "nsplit": _corrupt(blob, ns, int(h[ns]) + 1),
        "pbase": _corrupt(blob, ns + U, 5),
    }
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails a host check first
    n = ctypes.c_size_t()
    for name, b in bad.items():
        with pytest.raises(B.CrossCUError) as ei:
            B.plan_check(b, prob, sl)
        assert ei.value.code == B.CC_ERR_PLAN, name
        assert lib.cc_workspace_size(b.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n)) == B.CC_ERR_PLAN, name
        assert lib.cc_decode(ctypes.byref(prob), b.ctypes.data_as(ctypes.c_void_p), fake, fake, fake, fake, fake,
                             fake, None, fake, fake, fake, 1 << 30, None) == B.CC_ERR_PLAN, name


def test_plan_buffer_too_small_and_bad_blobs(lib):
    prob = B.problem(**_base())
    sl = np.array([10, 20], np.int32)
    opts = B.PlanOpts(8, 1, 32, 4, 0, 0)
    n = ctypes.c_size_t()
    assert lib.cc_plan_size(ctypes.byref(prob), ctypes.byref(opts), sl.ctypes.data_as(B._I32P),
                            ctypes.byref(n)) == 0
    small = np.zeros(n.value - 4, np.uint8)
    rc = lib.cc_plan(ctypes.byref(prob), ctypes.byref(opts), sl.ctypes.data_as(B._I32P), None,
                     small.ctypes.data_as(ctypes.c_void_p), small.nbytes)
    assert rc == B.CC_ERR_BUFFER
    junk = np.zeros(256, np.uint8)
    sz = ctypes.c_size_t()
    assert lib.cc_workspace_size(junk.ctypes.data_as(ctypes.c_void_p), ctypes.byref(sz)) == B.CC_ERR_PLAN


def test_decode_rejects_before_any_launch(lib):
    """Host-side checks of cc_decode return codes without touching a device."""
    kw = _base()
    prob = B.problem(**kw)
    sl = np.array([10, 20], np.int32)
    blob = B.plan(prob, sl, None, num_cus=8, num_xcds=1, tile_tokens=32, heads_per_unit=4)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails a host check first
    hp = blob.ctypes.data_as(ctypes.c_void_p)
    ws_need = B.workspace_size(blob)

    def call(p, plan=hp, ws_bytes=ws_need, v=fake, reduce=0):
        return lib.cc_decode_variant(reduce, ctypes.byref(p), plan, fake, fake, fake, v, fake, fake, None, fake,
                                     fake, fake, ws_bytes, None)

    assert call(prob, ws_bytes=ws_need - 1) == B.CC_ERR_BUFFER
    other = B.problem(**{**kw, "num_pages": 5})
    assert call(other) == B.CC_ERR_PLAN
    assert call(prob, v=None) == B.CC_ERR_INVALID
    assert call(prob, reduce=9) == B.CC_ERR_INVALID
    junk = np.zeros_like(blob)
    assert call(prob, plan=junk.ctypes.data_as(ctypes.c_void_p)) == B.CC_ERR_PLAN
    bad_scale = B.problem(**{**kw, "softmax_scale": 0.0})
    assert call(bad_scale) == B.CC_ERR_INVALID
    # 16-byte accesses: a misaligned out or q is refused
    odd_ptr = ctypes.c_void_p(0x1004)
    assert lib.cc_decode_variant(0, ctypes.byref(prob), hp, fake, fake, fake, fake, fake, fake, None, odd_ptr,
                                 fake, fake, ws_need, None) == B.CC_ERR_INVALID
    assert lib.cc_decode_variant(0, ctypes.byref(prob), hp, fake, odd_ptr, fake, fake, fake, fake, None, fake,
                                 fake, fake, ws_need, None) == B.CC_ERR_INVALID
    # unsupported shapes (head dim 96) are refused before launch
    odd = B.problem(**{**kw, "head_dim_qk": 96, "head_dim_v": 96})
    blob2 = B.plan(odd, sl, None, num_cus=8, num_xcds=1, tile_tokens=32, heads_per_unit=4)
    assert lib.cc_decode(ctypes.byref(odd), blob2.ctypes.data_as(ctypes.c_void_p), fake, fake, fake, fake, fake,
                         fake, None, fake, fake, fake, B.workspace_size(blob2), None) == B.CC_ERR_UNSUPPORTED


def test_mla_decode_rejects_before_any_launch(lib):
    """MLA shape, heads_per_unit, page, tile and indices checks fail on the host."""
    kw = dict(mode=B.MODE_MLA, batch=2, q_tokens=1, num_q_heads=128, num_kv_heads=1, head_dim_qk=576,
              head_dim_v=512, page_size=64, max_pages_per_seq=2, num_pages=4, topk=0, softmax_scale=0.07)
    sl = np.array([100, 20], np.int32)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails a host check first

    def call(p, hu=128, tile=32, indices=None):
        blob = B.plan(p, sl, None, num_cus=8, num_xcds=1, tile_tokens=tile, heads_per_unit=hu)
        return lib.cc_decode(ctypes.byref(p), blob.ctypes.data_as(ctypes.c_void_p), fake, fake, fake, None, fake,
                             fake, indices, fake, fake, fake, B.workspace_size(blob), None)

    prob = B.problem(**kw)
    assert call(prob, hu=64) == B.CC_ERR_UNSUPPORTED
    assert call(prob, tile=48) == B.CC_ERR_UNSUPPORTED
    assert call(B.problem(**{**kw, "page_size": 16, "max_pages_per_seq": 7, "num_pages": 9})) == B.CC_ERR_UNSUPPORTED
    assert call(B.problem(**{**kw, "head_dim_v": 448})) == B.CC_ERR_UNSUPPORTED
    sparse = B.problem(**{**kw, "mode": B.MODE_MLA_SPARSE, "topk": 16})
    assert call(sparse) == B.CC_ERR_INVALID          # no indices
    assert B.kernel_heads_per_unit(prob) == 128 and B.kernel_heads_per_unit(sparse) == 128


def test_debug_kernel_events_needs_both_or_neither(lib):
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the pair is only stored
    assert lib.cc_debug_kernel_events(None, fake) == B.CC_ERR_INVALID
    assert lib.cc_debug_kernel_events(fake, None) == B.CC_ERR_INVALID
    assert lib.cc_debug_kernel_events(None, None) == B.CC_OK


def test_indexer_rejects_before_any_launch(lib):
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails a host check first
    sl = np.array([3000, 100], np.int32)

    def call(p, seqlens=sl, scratch_bytes=1 << 30, q=fake):
        return lib.cc_indexer_topk(ctypes.byref(p), seqlens.ctypes.data_as(B._I32P), q, fake, fake, fake,
                                   scratch_bytes, fake, None, None)

    ok = B.indexer_problem(2, 8, 128, 64, 47, 60, 100)
    n = ctypes.c_size_t()
    assert lib.cc_indexer_scratch_size(ctypes.byref(ok), sl.ctypes.data_as(B._I32P), ctypes.byref(n)) == 0
    assert n.value == 2 * 8 * 3000 * 4
    assert call(B.indexer_problem(2, 8, 128, 64, 47, 60, 101)) == B.CC_ERR_INVALID     # topk > L_1
    assert call(B.indexer_problem(2, 8, 64, 64, 47, 60, 100)) == B.CC_ERR_UNSUPPORTED  # dim
    assert call(B.indexer_problem(2, 17, 128, 64, 47, 60, 100)) == B.CC_ERR_UNSUPPORTED  # q_tokens
    assert call(B.indexer_problem(2, 8, 128, 48, 47, 60, 100)) == B.CC_ERR_INVALID     # page size
    assert call(B.indexer_problem(2, 8, 128, 64, 46, 60, 100)) == B.CC_ERR_INVALID     # block table too narrow
    assert call(ok, seqlens=np.array([20000, 100], np.int32)) == B.CC_ERR_INVALID or \
        call(B.indexer_problem(2, 8, 128, 64, 400, 60, 100), seqlens=np.array([20000, 100], np.int32)) == \
        B.CC_ERR_UNSUPPORTED
    assert call(ok, scratch_bytes=n.value - 4) == B.CC_ERR_BUFFER
    assert call(ok, q=None) == B.CC_ERR_INVALID
