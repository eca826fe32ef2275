"""ctypes binding of libcrosscu.so: argument marshalling only.

Every computation happens in the C library and its HIP kernels.  PyTorch is
used for device memory and streams: tensors are passed as raw pointers
(``data_ptr()``) and the current HIP stream as a handle.  If the library is not
built, every entry point raises; nothing falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcrosscu.so")

CC_OK = 0
CC_ERR_INVALID, CC_ERR_UNSUPPORTED, CC_ERR_BUFFER, CC_ERR_PLAN = -1, -2, -3, -4
CC_ERR_PAGE, CC_ERR_HIP, CC_ERR_DEVICE_DATA = -5, -6, -7
MODE_GQA, MODE_MLA, MODE_MLA_SPARSE = 0, 1, 2
POLICY_STREAMK, POLICY_PER_UNIT, POLICY_STREAMK_DP = 0, 1, 2
UNIT_COST_GQA, UNIT_COST_MLA = 1, 6     # CC_UNIT_COST_GQA / CC_UNIT_COST_MLA
KV_NHD, KV_HND = 0, 1
REDUCE_FUSED, REDUCE_SPLIT_COMBINE = 0, 1

# every symbol include/*.h declares
EXPORTS = ["cc_version", "cc_last_error", "cc_strerror", "cc_device_query", "cc_plan_size", "cc_plan",
           "cc_plan_check", "cc_plan_prefix_size", "cc_plan_prefix",
           "cc_workspace_size", "cc_workspace_init", "cc_workspace_check", "cc_decode",
           "cc_decode_variant", "cc_debug_timeline", "cc_debug_kernel_events", "cc_debug_merge_poll_limit", "cc_probe_read",
           "cc_probe_mfma",
           "cc_indexer_scratch_size", "cc_indexer_topk", "cc_decode_noalloc", "cc_moe_plan_size", "cc_moe_plan",
           "cc_moe_gemm", "cc_moe_gemm_variant"]


class IndexerProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_tokens", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("topk", ctypes.c_int32)]


class Problem(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("batch", ctypes.c_int32), ("q_tokens", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("topk", ctypes.c_int32), ("kv_layout", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class PlanOpts(ctypes.Structure):
    _fields_ = [("num_cus", ctypes.c_int32), ("num_xcds", ctypes.c_int32),
                ("tile_tokens", ctypes.c_int32), ("heads_per_unit", ctypes.c_int32),
                ("policy", ctypes.c_int32), ("unit_cost", ctypes.c_int32)]


class MoEProblem(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("out_dim", ctypes.c_int32)]


class CrossCUError(RuntimeError):
    def __init__(self, code: int, what: str, detail: str):
        super().__init__(f"{what}: {detail} (code {code})")
        self.code = code


_lib = None
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_SZ = ctypes.c_size_t


def load() -> ctypes.CDLL:
    """Loads the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run cross_cu_load_amd.build.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    lib.cc_version.restype = ctypes.c_int
    lib.cc_version.argtypes = []
    lib.cc_last_error.restype = ctypes.c_char_p
    lib.cc_last_error.argtypes = []
    lib.cc_strerror.restype = ctypes.c_char_p
    lib.cc_strerror.argtypes = [ctypes.c_int]
    lib.cc_device_query.argtypes = [ctypes.c_int, _I32P, _I32P]
    lib.cc_plan_size.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(PlanOpts), _I32P,
                                 ctypes.POINTER(_SZ)]
    lib.cc_plan.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(PlanOpts), _I32P, _I32P, _P, _SZ]
    lib.cc_plan_check.argtypes = [_P, ctypes.POINTER(Problem), _I32P]
    lib.cc_plan_prefix_size.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(PlanOpts), _I32P, _I32P,
                                        ctypes.c_int32, _I32P, ctypes.POINTER(_SZ)]
    lib.cc_plan_prefix.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(PlanOpts), _I32P, _I32P, _I32P,
                                   ctypes.c_int32, _I32P, _P, _SZ]
    lib.cc_workspace_size.argtypes = [_P, ctypes.POINTER(_SZ)]
    lib.cc_workspace_init.argtypes = [_P, _SZ, _P]
    lib.cc_workspace_check.argtypes = [_P, _P, _P, _I32P, _I32P]
    dec = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.cc_decode.argtypes = dec
    lib.cc_decode_variant.argtypes = [ctypes.c_int] + dec
    lib.cc_decode_noalloc.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.cc_moe_plan_size.argtypes = [ctypes.POINTER(MoEProblem), ctypes.POINTER(PlanOpts), _I32P, ctypes.POINTER(_SZ)]
    lib.cc_moe_plan.argtypes = [ctypes.POINTER(MoEProblem), ctypes.POINTER(PlanOpts), _I32P, _P, _SZ]
    moe = [ctypes.POINTER(MoEProblem), _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.cc_moe_gemm.argtypes = moe
    lib.cc_moe_gemm_variant.argtypes = [ctypes.c_int] + moe
    lib.cc_debug_timeline.argtypes = [_P, _SZ]
    lib.cc_debug_kernel_events.argtypes = [_P, _P]
    lib.cc_debug_merge_poll_limit.argtypes = [ctypes.c_int]
    lib.cc_indexer_scratch_size.argtypes = [ctypes.POINTER(IndexerProblem), _I32P, ctypes.POINTER(_SZ)]
    lib.cc_indexer_topk.argtypes = [ctypes.POINTER(IndexerProblem), _I32P, _P, _P, _P, _P, _SZ, _P, _P, _P]
    lib.cc_probe_read.argtypes = [_P, ctypes.c_longlong, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, _P, _P]
    lib.cc_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _P]
    for f in EXPORTS:
        if f not in ("cc_last_error", "cc_strerror"):
            getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, what: str) -> None:
    if rc != CC_OK:
        lib = load()
        raise CrossCUError(rc, what, (lib.cc_last_error() or b"").decode() or
                           lib.cc_strerror(rc).decode())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr_i32(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def problem(mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
            max_pages_per_seq, num_pages, topk, softmax_scale, kv_layout=KV_NHD) -> Problem:
    return Problem(mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
                   max_pages_per_seq, num_pages, topk, kv_layout, softmax_scale)


def device_query(device: int = 0) -> tuple[int, int]:
    lib = load()
    cus, xcds = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.cc_device_query(device, ctypes.byref(cus), ctypes.byref(xcds)), "cc_device_query")
    return cus.value, xcds.value


def kernel_heads_per_unit(prob: Problem) -> int:
    """heads_per_unit that cc_decode's kernel for this mode accepts."""
    if prob.mode == MODE_GQA:
        return prob.num_q_heads // prob.num_kv_heads
    return 128


def default_unit_cost(mode: int) -> int:
    """The unit cost (in tiles) measured for the library's kernel of this mode."""
    return UNIT_COST_GQA if mode == MODE_GQA else UNIT_COST_MLA


def plan(prob: Problem, seqlens, block_table=None, num_cus=256, num_xcds=8, tile_tokens=32,
         heads_per_unit=None, policy=POLICY_STREAMK, unit_cost=None) -> np.ndarray:
    """Host plan blob (uint8 array) from cc_plan_size + cc_plan.

    POLICY_STREAMK cuts equal chunks of cost (one per tile plus ``unit_cost``
    per unit; None: the mode's measured default, 0: equal tile counts);
    POLICY_PER_UNIT is one worker per unit."""
    lib = load()
    if heads_per_unit is None:
        heads_per_unit = kernel_heads_per_unit(prob)
    if unit_cost is None:
        unit_cost = default_unit_cost(prob.mode)
    opts = PlanOpts(num_cus, num_xcds, tile_tokens, heads_per_unit, policy, unit_cost)
    sl = _i32(seqlens)
    if sl.shape != (prob.batch,):
        raise ValueError("seqlens must have shape [batch]")
    nbytes = _SZ()
    _check(lib.cc_plan_size(ctypes.byref(prob), ctypes.byref(opts), _ptr_i32(sl), ctypes.byref(nbytes)),
           "cc_plan_size")
    buf = np.zeros(nbytes.value, dtype=np.uint8)
    btp = None
    if block_table is not None:
        bt = _i32(block_table)
        if bt.shape != (prob.batch, prob.max_pages_per_seq):
            raise ValueError("block_table must have shape [batch, max_pages_per_seq]")
        btp = _ptr_i32(bt)
    _check(lib.cc_plan(ctypes.byref(prob), ctypes.byref(opts), _ptr_i32(sl), btp,
                       buf.ctypes.data_as(_P), buf.nbytes), "cc_plan")
    return buf


def plan_prefix(prob: Problem, seqlens, prefix_group, prefix_len, block_table=None, num_cus=256, num_xcds=8,
                tile_tokens=32, unit_cost=None) -> np.ndarray:
    """Shared-prefix plan blob (uint8 array) from cc_plan_prefix_size + cc_plan_prefix."""
    lib = load()
    if unit_cost is None:
        unit_cost = default_unit_cost(prob.mode)
    G = prob.num_q_heads // max(prob.num_kv_heads, 1)
    opts = PlanOpts(num_cus, num_xcds, tile_tokens, G, POLICY_STREAMK, unit_cost)
    sl, grp, ln = _i32(seqlens), _i32(prefix_group), _i32(prefix_len)
    if sl.shape != (prob.batch,) or grp.shape != (prob.batch,):
        raise ValueError("seqlens and prefix_group must have shape [batch]")
    nbytes = _SZ()
    _check(lib.cc_plan_prefix_size(ctypes.byref(prob), ctypes.byref(opts), _ptr_i32(sl), _ptr_i32(grp),
                                   len(ln), _ptr_i32(ln), ctypes.byref(nbytes)), "cc_plan_prefix_size")
    buf = np.zeros(nbytes.value, dtype=np.uint8)
    btp = None
    if block_table is not None:
        bt = _i32(block_table)
        if bt.shape != (prob.batch, prob.max_pages_per_seq):
            raise ValueError("block_table must have shape [batch, max_pages_per_seq]")
        btp = _ptr_i32(bt)
    _check(lib.cc_plan_prefix(ctypes.byref(prob), ctypes.byref(opts), _ptr_i32(sl), btp, _ptr_i32(grp), len(ln),
                              _ptr_i32(ln), buf.ctypes.data_as(_P), buf.nbytes), "cc_plan_prefix")
    return buf


def plan_check(plan_host: np.ndarray, prob: Problem, seqlens) -> None:
    """Raises CrossCUError (CC_ERR_PLAN) unless the plan was built for ``prob`` and these lengths."""
    sl = _i32(seqlens)
    if sl.shape != (prob.batch,):
        raise ValueError("seqlens must have shape [batch]")
    _check(load().cc_plan_check(plan_host.ctypes.data_as(_P), ctypes.byref(prob), _ptr_i32(sl)), "cc_plan_check")


def workspace_size(plan_host: np.ndarray) -> int:
    lib = load()
    n = _SZ()
    _check(lib.cc_workspace_size(plan_host.ctypes.data_as(_P), ctypes.byref(n)), "cc_workspace_size")
    return n.value


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_init(ws, stream=None) -> None:
    lib = load()
    _check(lib.cc_workspace_init(ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                 _stream(stream)), "cc_workspace_init")


def workspace_check(plan_host: np.ndarray, ws, stream=None) -> tuple[int, int]:
    """(non-zero counters, device error flags); synchronises the stream."""
    lib = load()
    dirty, flags = ctypes.c_int32(), ctypes.c_int32()
    rc = lib.cc_workspace_check(plan_host.ctypes.data_as(_P), ctypes.c_void_p(ws.data_ptr()),
                                _stream(stream), ctypes.byref(dirty), ctypes.byref(flags))
    if rc not in (CC_OK, CC_ERR_DEVICE_DATA):
        _check(rc, "cc_workspace_check")
    return dirty.value, flags.value


def debug_timeline(buf) -> None:
    """Sets (a uint64 device tensor of 4 words per worker) or clears (None) the timeline."""
    lib = load()
    if buf is None:
        _check(lib.cc_debug_timeline(None, 0), "cc_debug_timeline")
    else:
        _check(lib.cc_debug_timeline(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size()),
               "cc_debug_timeline")


def debug_merge_poll_limit(polls: int) -> None:
    """MLA in-kernel merge poll limit on the current device (< 0: the default)."""
    _check(load().cc_debug_merge_poll_limit(int(polls)), "cc_debug_merge_poll_limit")


def indexer_problem(batch, q_tokens, dim, page_size, max_pages, num_pages, topk) -> IndexerProblem:
    return IndexerProblem(batch, q_tokens, dim, page_size, max_pages, num_pages, topk)


def indexer_scratch_size(p: IndexerProblem, seqlens: np.ndarray) -> int:
    lib = load()
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    n = _SZ()
    _check(lib.cc_indexer_scratch_size(ctypes.byref(p), sl.ctypes.data_as(_I32P), ctypes.byref(n)),
           "cc_indexer_scratch_size")
    return int(n.value)


def indexer_topk(p: IndexerProblem, seqlens: np.ndarray, q, k_cache, block_table, scratch, indices, err=None,
                 stream=None) -> None:
    """cc_indexer_topk on device tensors; seqlens is a host array."""
    lib = load()
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    _check(lib.cc_indexer_topk(ctypes.byref(p), sl.ctypes.data_as(_I32P), ctypes.c_void_p(q.data_ptr()),
                               ctypes.c_void_p(k_cache.data_ptr()), ctypes.c_void_p(block_table.data_ptr()),
                               ctypes.c_void_p(scratch.data_ptr()), scratch.numel() * scratch.element_size(),
                               ctypes.c_void_p(indices.data_ptr()),
                               None if err is None else ctypes.c_void_p(err.data_ptr()), _stream(stream)),
           "cc_indexer_topk")


def debug_kernel_events(start, stop) -> None:
    """Sets (two torch.cuda.Event objects with timing, already created by a
    record) or clears (None, None) the events later decode calls record at the
    start of their first kernel and the end of their last."""
    lib = load()
    if start is None:
        _check(lib.cc_debug_kernel_events(None, None), "cc_debug_kernel_events")
    else:
        _check(lib.cc_debug_kernel_events(ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)),
               "cc_debug_kernel_events")


def probe_read(buf, method: int, workgroups: int, sink, pages=None, page_bytes: int = 0,
               stream=None) -> None:
    """cc_probe_read on a device tensor (asynchronous)."""
    lib = load()
    npages = 0 if pages is None else pages.numel()
    _check(lib.cc_probe_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(), method,
                             _dp(pages), page_bytes, npages, workgroups, _dp(sink), _stream(stream)),
           "cc_probe_read")


def probe_mfma(workgroups: int, waves_per_workgroup: int, iters: int, sink, stream=None) -> float:
    """cc_probe_mfma (asynchronous); returns the flops of the call."""
    _check(load().cc_probe_mfma(workgroups, waves_per_workgroup, iters, _dp(sink), _stream(stream)), "cc_probe_mfma")
    return float(workgroups) * waves_per_workgroup * iters * 8 * 32768


def _dp(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def decode(prob: Problem, plan_host: np.ndarray, plan_dev, q, k_cache, v_cache, block_table, seqlens,
           indices, out, lse, workspace, reduce: int = REDUCE_FUSED, stream=None) -> None:
    """cc_decode_variant on device tensors (asynchronous on the stream)."""
    lib = load()
    _check(lib.cc_decode_variant(reduce, ctypes.byref(prob), plan_host.ctypes.data_as(_P), _dp(plan_dev),
                                 _dp(q), _dp(k_cache), _dp(v_cache), _dp(block_table), _dp(seqlens),
                                 _dp(indices), _dp(out), _dp(lse), _dp(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "cc_decode")


NOALLOC_WORKSPACE_BYTES = 64 << 20     # CC_NOALLOC_WORKSPACE_BYTES
MODE_MOE = 3
MOE_TILE_ROWS, MOE_TILE_K = 256, 64    # the MoE kernel's output-tile rows and k tile


def moe_problem(num_experts: int, hidden: int, out_dim: int) -> MoEProblem:
    return MoEProblem(num_experts, hidden, out_dim)


MOE_WORKGROUPS_PER_CU = 1  # the MoE kernel's workgroups (128 KiB of LDS each) that fit on one compute unit


def moe_plan(prob: MoEProblem, expert_tokens, num_cus=256 * MOE_WORKGROUPS_PER_CU, num_xcds=8,
             policy=POLICY_STREAMK_DP, unit_cost=None, tile_rows=MOE_TILE_ROWS, tile_k=MOE_TILE_K) -> np.ndarray:
    """MoE grouped-GEMM plan blob (uint8 array).  num_cus: the workers of the
    one wave, MOE_WORKGROUPS_PER_CU per compute unit.  The default policy
    deals whole tiles round-robin and splits only the last round and the
    remainder (POLICY_STREAMK_DP); unit_cost None: one k tile per output tile."""
    lib = load()
    opts = PlanOpts(num_cus, num_xcds, tile_k, tile_rows, policy, 1 if unit_cost is None else unit_cost)
    et = _i32(expert_tokens)
    if et.shape != (prob.num_experts,):
        raise ValueError("expert_tokens must have shape [num_experts]")
    n = _SZ()
    _check(lib.cc_moe_plan_size(ctypes.byref(prob), ctypes.byref(opts), _ptr_i32(et), ctypes.byref(n)),
           "cc_moe_plan_size")
    buf = np.zeros(n.value, dtype=np.uint8)
    _check(lib.cc_moe_plan(ctypes.byref(prob), ctypes.byref(opts), _ptr_i32(et), buf.ctypes.data_as(_P), buf.nbytes),
           "cc_moe_plan")
    return buf


def moe_gemm(prob: MoEProblem, plan_host: np.ndarray, plan_dev, x, w, y, workspace, reduce: int = REDUCE_FUSED,
             stream=None) -> None:
    """cc_moe_gemm_variant on device tensors (asynchronous on the stream)."""
    lib = load()
    _check(lib.cc_moe_gemm_variant(reduce, ctypes.byref(prob), plan_host.ctypes.data_as(_P), _dp(plan_dev), _dp(x),
                                   _dp(w), _dp(y), _dp(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "cc_moe_gemm")


@dataclass
class MoESession:
    """Device-resident MoE inputs, plan and workspace for repeated calls."""

    prob: MoEProblem
    plan_host: np.ndarray
    plan_dev: object
    x: object
    w: object
    y: object
    workspace: object

    def run(self, reduce: int = REDUCE_FUSED, stream=None) -> None:
        moe_gemm(self.prob, self.plan_host, self.plan_dev, self.x, self.w, self.y, self.workspace, reduce, stream)


def moe_session(wl, plan_host: np.ndarray, device="cuda") -> MoESession:
    """Copies a MoE workload (from the seeded generator) and its plan to the device."""
    import torch
    dev = torch.device(device)
    c = wl.cfg
    prob = moe_problem(c.num_experts, c.hidden, c.out_dim)
    ws = torch.empty(workspace_size(plan_host), dtype=torch.uint8, device=dev)
    workspace_init(ws)
    x = torch.from_numpy(np.ascontiguousarray(wl.x).view(np.int16)).to(dev)
    w = torch.from_numpy(np.ascontiguousarray(wl.w).view(np.int16)).to(dev)
    y = torch.empty((wl.x.shape[0], c.out_dim), dtype=torch.float32, device=dev)
    return MoESession(prob, plan_host, torch.from_numpy(plan_host).to(dev), x, w, y, ws)


def decode_noalloc(prob: Problem, plan_host: np.ndarray, plan_dev, q, k_cache, v_cache, block_table, seqlens,
                   indices, out, lse, stream=None) -> None:
    """cc_decode_noalloc on device tensors: the library's own scratch array
    instead of a workspace (asynchronous on the stream)."""
    lib = load()
    _check(lib.cc_decode_noalloc(ctypes.byref(prob), plan_host.ctypes.data_as(_P), _dp(plan_dev), _dp(q),
                                 _dp(k_cache), _dp(v_cache), _dp(block_table), _dp(seqlens), _dp(indices),
                                 _dp(out), _dp(lse), _stream(stream)), "cc_decode_noalloc")


@dataclass
class DeviceSession:
    """Device-resident inputs, plan and workspace for repeated decode calls.

    Holds torch device tensors only; every step of the decode runs in the
    library's kernels.
    """

    prob: Problem
    plan_host: np.ndarray
    plan_dev: object
    q: object
    k: object
    v: object
    block_table: object
    seqlens: object
    indices: object
    out: object
    lse: object
    workspace: object

    def run(self, reduce: int = REDUCE_FUSED, stream=None) -> None:
        decode(self.prob, self.plan_host, self.plan_dev, self.q, self.k, self.v, self.block_table,
               self.seqlens, self.indices, self.out, self.lse, self.workspace, reduce, stream)


def problem_for(wl) -> Problem:
    c = wl.cfg
    return problem(c.mode, c.batch, c.q_tokens, c.num_q_heads, c.num_kv_heads, c.head_dim_qk, c.head_dim_v,
                   c.page_size, wl.max_pages, wl.num_pages, c.topk, c.softmax_scale, wl.kv_layout)


def session(wl, plan_host: np.ndarray, device="cuda") -> DeviceSession:
    """Copies a host workload (from the seeded generator) and its plan to the device."""
    import torch
    dev = torch.device(device)

    def t16(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    def t32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    c = wl.cfg
    prob = problem_for(wl)
    ws = torch.empty(workspace_size(plan_host), dtype=torch.uint8, device=dev)
    workspace_init(ws)
    out = torch.empty((c.batch, c.q_tokens, c.num_q_heads, c.head_dim_v), dtype=torch.float32, device=dev)
    lse = torch.empty((c.batch, c.q_tokens, c.num_q_heads), dtype=torch.float32, device=dev)
    return DeviceSession(prob, plan_host, torch.from_numpy(plan_host).to(dev), t16(wl.q), t16(wl.k_cache),
                         t16(wl.v_cache), t32(wl.block_table), t32(wl.seqlens), t32(wl.indices), out, lse, ws)
