"""Seeded synthetic decode-attention workloads.

This module only draws inputs: sequence lengths, page permutations, bf16 bit
patterns for q / K / V, and sparse index sets.  It holds none of the attention
arithmetic, so both the fp64 oracle and the HIP path can consume the same bits
without sharing any code of the method.

Workload shapes follow the decode settings the source pages discuss: GQA and
MLA decode attention over a paged KV cache (MeldKernel summary, "Experiments
and results"), and index-sparse MLA decode with 2 requests x 8 query tokens,
KV = 8192 and Top-2048 (GLM-5.2 decode article, "Summary").  The pages hold no
dataset, so every tensor is drawn here from N(0, 1) and rounded to bf16.

Random streams are keyed, not sequential: every array is filled in chunks of
2**22 elements, chunk c of array a drawn from
``PCG64(SeedSequence([seed, a, c]))``.  That keeps the draw independent of the
thread count used to fill it.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

MODE_GQA = 0
MODE_MLA = 1
MODE_MLA_SPARSE = 2
KV_NHD = 0   # pages [P][Hkv][d]: token-major
KV_HND = 1   # pages [Hkv][P][d]: head-major

_CHUNK = 1 << 22

# stream ids (the second SeedSequence word)
_S_SEQLENS, _S_PAGES, _S_Q, _S_K, _S_V, _S_IDX, _S_IQ, _S_IK = range(8)


@dataclasses.dataclass(frozen=True)
class Config:
    """One decode workload.  ``seqlen_kind`` picks how lengths are drawn."""

    name: str
    mode: int
    batch: int
    q_tokens: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    page_size: int
    softmax_scale: float
    seqlen_kind: str            # "uniform" | "loguniform" | "skewed" | "fixed"
    seqlen_lo: int = 0
    seqlen_hi: int = 0
    long_len: int = 0           # skewed: the one long sequence
    short_len: int = 0          # skewed: all the others
    topk: int = 0               # sparse: distinct indices per query token
    prefix_len: int = 0         # shared_prefix: tokens every sequence of the batch shares
    shuffle_pages: bool = True
    seed: int = 0
    kv_layout: int = KV_NHD

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


# The five decode workloads.  Seeds are 1000 + position (1-based).
CONFIGS: list[Config] = [
    Config("tiny_gqa", MODE_GQA, batch=4, q_tokens=1, num_q_heads=8, num_kv_heads=2,
           head_dim_qk=64, head_dim_v=64, page_size=512, softmax_scale=1 / math.sqrt(64),
           seqlen_kind="uniform", seqlen_lo=1, seqlen_hi=512, shuffle_pages=False, seed=1001),
    Config("llama3_8b_gqa", MODE_GQA, batch=64, q_tokens=1, num_q_heads=32, num_kv_heads=8,
           head_dim_qk=128, head_dim_v=128, page_size=16, softmax_scale=1 / math.sqrt(128),
           seqlen_kind="loguniform", seqlen_lo=128, seqlen_hi=32768, seed=1002),
    Config("skewed_gqa", MODE_GQA, batch=32, q_tokens=1, num_q_heads=32, num_kv_heads=8,
           head_dim_qk=128, head_dim_v=128, page_size=16, softmax_scale=1 / math.sqrt(128),
           seqlen_kind="skewed", long_len=131072, short_len=256, seed=1003),
    Config("deepseek_mla", MODE_MLA, batch=64, q_tokens=1, num_q_heads=128, num_kv_heads=1,
           head_dim_qk=576, head_dim_v=512, page_size=64, softmax_scale=1 / math.sqrt(192),
           seqlen_kind="uniform", seqlen_lo=1024, seqlen_hi=16384, seed=1004),
    Config("sparse_mla", MODE_MLA_SPARSE, batch=2, q_tokens=8, num_q_heads=128, num_kv_heads=1,
           head_dim_qk=576, head_dim_v=512, page_size=64, softmax_scale=1 / math.sqrt(192),
           seqlen_kind="fixed", seqlen_lo=8192, topk=2048, seed=1005),
]
# Shared-prefix decode (the workload shape of the MeldKernel summary's
# shared-prefix experiment, Fig. 11, whose sizes the page does not give): the
# Llama-3-8B-shaped heads over 64 sequences that all begin with the same
# 4096-token prefix (one set of pages named by every block-table row),
# followed by their own log-uniform [64, 4096]-token suffixes.
SHARED_PREFIX = Config("shared_prefix_gqa", MODE_GQA, batch=64, q_tokens=1, num_q_heads=32, num_kv_heads=8,
                       head_dim_qk=128, head_dim_v=128, page_size=16, softmax_scale=1 / math.sqrt(128),
                       seqlen_kind="shared_prefix", seqlen_lo=64, seqlen_hi=4096, prefix_len=4096, seed=1006)
EXTRA_CONFIGS: list[Config] = [SHARED_PREFIX]
CONFIG_BY_NAME = {c.name: c for c in CONFIGS + EXTRA_CONFIGS}


@dataclasses.dataclass
class Workload:
    """Host arrays of one draw.  bf16 tensors are held as uint16 bit patterns."""

    cfg: Config
    seqlens: np.ndarray        # int32 [B]
    block_table: np.ndarray    # int32 [B, max_pages]; unused entries are -1
    q: np.ndarray              # uint16 [B, Tq, Hq, dk]
    k_cache: np.ndarray        # uint16 [num_pages, P, Hkv, dk] (NHD) or [num_pages, Hkv, P, dk] (HND)
    v_cache: np.ndarray | None  # uint16, as k_cache with dv; None for MLA
    indices: np.ndarray | None  # int32 [B, Tq, topk]; sparse mode only
    prefix_group: np.ndarray | None = None  # int32 [B]: shared-prefix group of each sequence (-1: none)
    prefix_len: np.ndarray | None = None    # int32 [groups]: tokens each group shares

    @property
    def kv_layout(self) -> int:
        return self.cfg.kv_layout

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def unique_kv_bytes(self) -> int:
        """Bytes of the distinct K/V rows the batch attends over: a shared
        prefix counted once per group (equal to kv_bytes without one)."""
        if self.prefix_group is None:
            return self.kv_bytes()
        c = self.cfg
        per_tok = c.num_kv_heads * (c.head_dim_qk + c.head_dim_v) * 2
        toks = int(self.seqlens.astype(np.int64).sum())
        for g, Lp in enumerate(self.prefix_len):
            n = int((self.prefix_group == g).sum())
            if n:
                toks -= (n - 1) * int(Lp)
        return toks * per_tok

    def kv_bytes(self) -> int:
        """Bytes of K/V the attention must read (each used row once)."""
        c = self.cfg
        if c.mode == MODE_GQA:
            per_tok = c.num_kv_heads * (c.head_dim_qk + c.head_dim_v) * 2
            return int(self.seqlens.astype(np.int64).sum()) * per_tok
        per_tok = c.head_dim_qk * 2
        if c.mode == MODE_MLA:
            return int(self.seqlens.astype(np.int64).sum()) * per_tok
        return int(c.batch * c.q_tokens * c.topk) * per_tok


def _gen(seed: int, stream: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, chunk])))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(seed: int, stream: int, shape: tuple[int, ...]) -> np.ndarray:
    """N(0,1) drawn in fp32 and rounded to bf16, filled chunk-parallel."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)

    def fill(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = round_to_bf16_bits(_gen(seed, stream, c).standard_normal(hi - lo, dtype=np.float32))

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def draw_seqlens(cfg: Config) -> np.ndarray:
    g = _gen(cfg.seed, _S_SEQLENS, 0)
    b = cfg.batch
    if cfg.seqlen_kind == "uniform":          # inclusive integer range
        s = g.integers(cfg.seqlen_lo, cfg.seqlen_hi + 1, size=b)
    elif cfg.seqlen_kind == "loguniform":     # L = round(exp(u)), u ~ U[ln lo, ln hi]
        u = g.uniform(math.log(cfg.seqlen_lo), math.log(cfg.seqlen_hi), size=b)
        s = np.clip(np.rint(np.exp(u)), cfg.seqlen_lo, cfg.seqlen_hi)
    elif cfg.seqlen_kind == "skewed":         # the long sequence first, then the short ones
        s = np.full(b, cfg.short_len)
        s[0] = cfg.long_len
    elif cfg.seqlen_kind == "fixed":
        s = np.full(b, cfg.seqlen_lo)
    elif cfg.seqlen_kind == "shared_prefix":  # the prefix, then a log-uniform suffix
        u = g.uniform(math.log(cfg.seqlen_lo), math.log(cfg.seqlen_hi), size=b)
        s = cfg.prefix_len + np.clip(np.rint(np.exp(u)), cfg.seqlen_lo, cfg.seqlen_hi)
    else:
        raise ValueError(cfg.seqlen_kind)
    return s.astype(np.int32)


def page_table(seqlens: np.ndarray, page_size: int, shuffle: bool, seed: int) -> np.ndarray:
    """Block table over exactly the pages the sequences need.

    Logical page i of sequence b gets a physical page id; with ``shuffle`` the
    ids are a seeded random permutation of 0..num_pages-1, else they are laid
    out in sequence order.  Unused entries are -1.
    """
    npg = (seqlens.astype(np.int64) + page_size - 1) // page_size
    total = int(npg.sum())
    maxp = int(npg.max()) if len(npg) else 0
    phys = np.arange(total, dtype=np.int32)
    if shuffle:
        phys = _gen(seed, _S_PAGES, 0).permutation(total).astype(np.int32)
    bt = np.full((len(seqlens), max(maxp, 1)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(npg):
        bt[b, :n] = phys[off:off + n]
        off += int(n)
    return bt


def shared_page_table(seqlens: np.ndarray, page_size: int, prefix_pages: int, shuffle: bool,
                      seed: int) -> np.ndarray:
    """Block table in which every sequence's first ``prefix_pages`` entries name
    the same pages (a shared prefix) and the rest its own pages; physical ids
    are a seeded permutation of all the pages with ``shuffle``."""
    return grouped_page_table(seqlens, np.zeros(len(seqlens), np.int32), np.array([prefix_pages * page_size]),
                              page_size, shuffle, seed)


def grouped_page_table(seqlens: np.ndarray, prefix_group: np.ndarray, prefix_len: np.ndarray, page_size: int,
                       shuffle: bool, seed: int) -> np.ndarray:
    """Block table for prefix groups: the members of group g (prefix_group[b]
    == g) name the same first prefix_len[g] / page_size pages, every other
    page belongs to one sequence; physical ids are a seeded permutation of all
    the pages with ``shuffle``."""
    npg_prefix = [int(L) // page_size for L in prefix_len]
    own = np.array([(int(L) - (int(prefix_len[g]) if g >= 0 else 0) + page_size - 1) // page_size
                    for L, g in zip(seqlens, prefix_group)], np.int64)
    total = sum(npg_prefix) + int(own.sum())
    phys = np.arange(total, dtype=np.int32)
    if shuffle:
        phys = _gen(seed, _S_PAGES, 0).permutation(total).astype(np.int32)
    first = np.cumsum([0] + npg_prefix)          # group g's pages: phys[first[g]:first[g + 1]]
    maxp = max([(npg_prefix[g] if g >= 0 else 0) + int(n) for g, n in zip(prefix_group, own)] + [1])
    bt = np.full((len(seqlens), maxp), -1, dtype=np.int32)
    off = int(first[-1])
    for b, (g, n) in enumerate(zip(prefix_group, own)):
        k = 0
        if g >= 0:
            k = npg_prefix[g]
            bt[b, :k] = phys[first[g]:first[g + 1]]
        bt[b, k:k + n] = phys[off:off + n]
        off += int(n)
    return bt


def make_grouped_workload(cfg: Config, seqlens, prefix_group, prefix_len) -> Workload:
    """A GQA workload whose sequences share prefixes by group (-1: none); the
    values are drawn as in make_workload."""
    seqlens = np.asarray(seqlens, np.int32)
    prefix_group = np.asarray(prefix_group, np.int32)
    prefix_len = np.asarray(prefix_len, np.int32)
    bt = grouped_page_table(seqlens, prefix_group, prefix_len, cfg.page_size, cfg.shuffle_pages, cfg.seed)
    num_pages = max(int(bt.max()) + 1, 1)
    P = cfg.page_size
    q = normal_bf16(cfg.seed, _S_Q, (cfg.batch, cfg.q_tokens, cfg.num_q_heads, cfg.head_dim_qk))
    k = normal_bf16(cfg.seed, _S_K, (num_pages, P, cfg.num_kv_heads, cfg.head_dim_qk))
    v = normal_bf16(cfg.seed, _S_V, (num_pages, P, cfg.num_kv_heads, cfg.head_dim_v))
    if cfg.kv_layout == KV_HND:
        k = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
        v = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    return Workload(cfg, seqlens, bt, q, k, v, None, prefix_group, prefix_len)


def make_workload(cfg: Config, seqlens: np.ndarray | None = None) -> Workload:
    """Draw one workload.  ``seqlens`` overrides the configured length draw."""
    if seqlens is None:
        seqlens = draw_seqlens(cfg)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    prefix_group = prefix_len = None
    if cfg.prefix_len > 0:   # one group: every sequence shares the prefix pages
        if cfg.prefix_len % cfg.page_size or int(seqlens.min()) < cfg.prefix_len:
            raise ValueError("the prefix must be whole pages and no longer than any sequence")
        bt = shared_page_table(seqlens, cfg.page_size, cfg.prefix_len // cfg.page_size, cfg.shuffle_pages,
                               cfg.seed)
        num_pages = int(bt.max()) + 1
        prefix_group = np.zeros(len(seqlens), np.int32)
        prefix_len = np.array([cfg.prefix_len], np.int32)
    else:
        bt = page_table(seqlens, cfg.page_size, cfg.shuffle_pages, cfg.seed)
        num_pages = int(((seqlens.astype(np.int64) + cfg.page_size - 1) // cfg.page_size).sum())
    P = cfg.page_size
    q = normal_bf16(cfg.seed, _S_Q, (cfg.batch, cfg.q_tokens, cfg.num_q_heads, cfg.head_dim_qk))
    k = normal_bf16(cfg.seed, _S_K, (num_pages, P, cfg.num_kv_heads, cfg.head_dim_qk))
    v = None
    if cfg.mode == MODE_GQA:
        v = normal_bf16(cfg.seed, _S_V, (num_pages, P, cfg.num_kv_heads, cfg.head_dim_v))
    if cfg.kv_layout == KV_HND:   # same logical content, head-major pages
        k = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
        v = None if v is None else np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    idx = None
    if cfg.mode == MODE_MLA_SPARSE:
        idx = np.empty((cfg.batch, cfg.q_tokens, cfg.topk), dtype=np.int32)
        for b in range(cfg.batch):
            for t in range(cfg.q_tokens):
                g = _gen(cfg.seed, _S_IDX, b * cfg.q_tokens + t)
                idx[b, t] = g.choice(int(seqlens[b]), size=cfg.topk, replace=False)
    return Workload(cfg, seqlens, bt, q, k, v, idx, prefix_group, prefix_len)


def small_variant(cfg: Config, batch: int, seqlen_hi: int, seed_offset: int = 0) -> Config:
    """A reduced copy of ``cfg`` for oracle-sized parity runs (same heads/dims/paging)."""
    kw = dataclasses.asdict(cfg)
    kw.update(name=cfg.name + "_small", batch=batch, seed=cfg.seed + 100 + seed_offset)
    if cfg.mode == MODE_MLA_SPARSE:
        kw.update(seqlen_kind="fixed", seqlen_lo=seqlen_hi, topk=min(cfg.topk, seqlen_hi))
    elif cfg.prefix_len > 0:   # keep the prefix shape: a shorter prefix and suffixes
        plen = max(cfg.page_size, (seqlen_hi // 2) // cfg.page_size * cfg.page_size)
        kw.update(prefix_len=plen, seqlen_lo=1, seqlen_hi=max(1, seqlen_hi - plen))
    else:
        kw.update(seqlen_kind="uniform", seqlen_lo=1, seqlen_hi=seqlen_hi)
    return Config(**kw)


# ---------------------------------------------------------------- indexer inputs
# The step before index-sparse attention: a cheap indexer scores every cached
# token of a request against each decode query token, and the top-k positions
# become the sparse index sets (GLM-5.2 decode article: "Paged Indexer Score"
# ahead of TopK and sparse MLA; Top-2048).  One indexer query per decode token
# and one indexer key per cached token, on the same pages as the latent cache.
INDEXER_DIM = 128


@dataclasses.dataclass
class IndexerInputs:
    q: np.ndarray        # uint16 [B, Tq, dim]: indexer query of each decode token
    k_cache: np.ndarray  # uint16 [num_pages, P, dim]: indexer key of each cached token


def make_indexer_inputs(wl: Workload, dim: int = INDEXER_DIM) -> IndexerInputs:
    """Indexer query and key bits for a workload's requests (same block table and pages)."""
    c = wl.cfg
    q = normal_bf16(c.seed, _S_IQ, (c.batch, c.q_tokens, dim))
    k = normal_bf16(c.seed, _S_IK, (wl.num_pages, c.page_size, dim))
    return IndexerInputs(q, k)


# ---------------------------------------------------------------- MoE grouped GEMM
# Routing sends each token to top_k of E experts, so the experts receive very
# different row counts (MeldKernel summary, "Problem and motivation": expert
# token counts differ from SM to SM).  The pages give no MoE shapes; these are
# a DeepSeek/Qwen-like layer: 64 experts, hidden 4096, expert output 2048,
# 4096 tokens routed top-8 with Zipf-skewed expert popularity (a seeded
# permutation of p_e proportional to 1 / (rank + 1)).
_S_MOE_ROUTE, _S_MOE_X, _S_MOE_W = 20, 21, 22


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    num_experts: int
    hidden: int          # K
    out_dim: int         # N
    tokens: int
    top_k: int
    zipf: float = 1.0    # popularity of the expert of rank i proportional to (i + 1) ** -zipf
    seed: int = 0


MOE_CONFIGS = [
    MoEConfig("moe_grouped_gemm", num_experts=64, hidden=4096, out_dim=2048, tokens=4096, top_k=8, seed=1007),
]
MOE_BY_NAME = {c.name: c for c in MOE_CONFIGS}


@dataclasses.dataclass
class MoEWorkload:
    cfg: MoEConfig
    expert_tokens: np.ndarray   # int32 [E]: rows routed to each expert
    offsets: np.ndarray         # int32 [E + 1]: expert e owns rows offsets[e] .. offsets[e + 1] - 1
    token_of_row: np.ndarray    # int32 [R]: the token each routed row copies
    x: np.ndarray               # uint16 [R, K]: routed rows, sorted by expert
    w: np.ndarray               # uint16 [E, N, K]: expert weights ([out, in])

    def flops(self) -> float:
        c = self.cfg
        return 2.0 * float(self.expert_tokens.sum()) * c.hidden * c.out_dim

    def bytes_min(self) -> int:
        """Each input read once and the output written once: X, the weights of
        experts with rows, Y (fp32)."""
        c = self.cfg
        used = int((self.expert_tokens > 0).sum())
        R = int(self.expert_tokens.sum())
        return R * c.hidden * 2 + used * c.out_dim * c.hidden * 2 + R * c.out_dim * 4


def route(cfg: MoEConfig) -> tuple[np.ndarray, np.ndarray]:
    """(expert_tokens [E], token_of_row [R]): each token picks top_k distinct
    experts with probability proportional to the Zipf popularity."""
    g = _gen(cfg.seed, _S_MOE_ROUTE, 0)
    rank = g.permutation(cfg.num_experts)
    p = (rank + 1.0) ** -cfg.zipf
    p /= p.sum()
    picks = [g.choice(cfg.num_experts, size=cfg.top_k, replace=False, p=p) for _ in range(cfg.tokens)]
    pairs = sorted((int(e), t) for t, es in enumerate(picks) for e in es)
    expert_tokens = np.bincount([e for e, _ in pairs], minlength=cfg.num_experts).astype(np.int32)
    token_of_row = np.array([t for _, t in pairs], np.int32)
    return expert_tokens, token_of_row


def make_moe_workload(cfg: MoEConfig, expert_tokens=None) -> MoEWorkload:
    """Draw a MoE workload; ``expert_tokens`` overrides the routing (rows then
    copy tokens 0, 1, ... in order)."""
    if expert_tokens is None:
        expert_tokens, token_of_row = route(cfg)
    else:
        expert_tokens = np.asarray(expert_tokens, np.int32)
        token_of_row = np.arange(int(expert_tokens.sum()), dtype=np.int32) % max(cfg.tokens, 1)
    offsets = np.concatenate([[0], np.cumsum(expert_tokens)]).astype(np.int32)
    xt = normal_bf16(cfg.seed, _S_MOE_X, (max(cfg.tokens, 1), cfg.hidden))
    x = np.ascontiguousarray(xt[token_of_row]) if len(token_of_row) else np.zeros((0, cfg.hidden), np.uint16)
    w = normal_bf16(cfg.seed, _S_MOE_W, (cfg.num_experts, cfg.out_dim, cfg.hidden))
    return MoEWorkload(cfg, expert_tokens, offsets, token_of_row, x, w)


def small_moe(cfg: MoEConfig, num_experts: int, hidden: int, out_dim: int, tokens: int, top_k: int,
              seed_offset: int = 0) -> MoEConfig:
    return dataclasses.replace(cfg, name=cfg.name + "_small", num_experts=num_experts, hidden=hidden,
                               out_dim=out_dim, tokens=tokens, top_k=top_k, seed=cfg.seed + 100 + seed_offset)
