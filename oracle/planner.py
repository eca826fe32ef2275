"""Reference Stream-K work plan for split-KV decode (TEST INFRASTRUCTURE).

The method (CSDN Q&A on waves and FlashMLA's Stream-K, "Summary"): cut the
total work into exactly as many equal chunks as there are compute units and
launch a single wave, so no unit idles behind a slow tail.  The mapping is
decided at run time from the real sequence lengths and the hardware shape
(MeldKernel summary, "Core method"), and only this host plan is rebuilt when
the lengths change (GLM-5.2 decode article, MegaRTP design, point 1).  The
host emits fixed-size work descriptors per worker (same article: 732 tile
tasks over 148 worker queues give 140 queues of 5 and 8 of 4).

Readings (the pages fix only "equal, one chunk per compute unit"):
* cost model: KV tiles of T tokens; a unit of length L has ceil(L / T) tiles.
* unit: the query heads sharing one K/V stream for one query token,
  u = ((b * Tq + t) * Hkv + g) * (G / Hu) + hb; units are ordered by u.
* tiles are laid out unit-major; chunk k takes floor(N / C) tiles, plus one
  for the first N mod C chunks, contiguously.
* an empty unit (a sequence with no cached tokens) has no tiles, gets no
  piece and carries no cost; its unit_nsplit is 0.
* unit_cost (a plan input, in tiles, default 0): with unit_cost = 0 the
  split is exactly the equal tile split above.  With unit_cost = c > 0 what
  is split evenly is the cost of the work, one per tile plus c per non-empty
  unit for the fixed work of starting and finishing it; a unit occupies a
  contiguous cost range with its overhead first, and a tile belongs to the
  chunk whose cost range holds the tile's starting position.  Chunk k's
  range is [k * q + min(k, r), (k+1) * q + min(k+1, r)) for total cost =
  q C + r.  The value of c is a caller's choice (a measured property of a
  kernel), not part of the method; the pages' split is c = 0.
* a piece is a chunk's intersection with one unit; its split index counts the
  unit's pieces in chunk order; split units get consecutive partial slots.
* placement: with X locality domains (XCDs) and C divisible by X, logical
  chunk k runs on worker w = (k mod C/X) * X + k div (C/X), so consecutive
  chunks (the pieces of one unit) share a domain when the hardware places
  worker w in domain w mod X.  Otherwise w = k.
* binding to the inputs: header word 25 is the 32-bit FNV-1a hash of the
  little-endian bytes of the int32 words (mode, batch, q_tokens, num_q_heads,
  num_kv_heads, head_dim_qk, head_dim_v, page_size, max_pages_per_seq,
  num_pages, topk, seqlens[0 .. batch)), so a plan can be checked against the
  lengths it is used with (GLM-5.2 decode article, MegaRTP design: the plan is
  rebuilt, not reused, when the lengths change).

The byte layout below is the contract with the C planner; it is written out
here independently and compared byte for byte.
"""
from __future__ import annotations

import struct

import numpy as np

PLAN_MAGIC = 0x4C504343          # "CCPL" little-endian
PLAN_VERSION = 3
HEADER_WORDS = 32               # words 0..26 below, the rest zero
ITEM_WORDS = 4                   # unit, tok_begin, tok_end, split
PREFIX_WORDS = 20                # a prefix-table row: kv_head, members, prefix_len, pieces, member ids[16]
PREFIX_ROWS = 16                 # query rows one prefix unit gathers (members x group size)

MODE_GQA, MODE_MLA, MODE_MLA_SPARSE, MODE_MOE = 0, 1, 2, 3
MOE_DESC_WORDS = 4               # a MoE unit: expert, first row, rows, first column
MOE_TILE_COLS = 256              # output columns of a MoE unit (the C planner's fixed tile width)
MOE_TILE_ROWS = 256              # output rows of a MoE unit (the kernel's tile height)
POLICY_STREAMK, POLICY_PER_UNIT, POLICY_STREAMK_DP = 0, 1, 2


def fnv1a32(words) -> int:
    """32-bit FNV-1a (offset basis 2166136261, prime 16777619) of the
    little-endian bytes of int32 ``words``, returned as a signed int32."""
    h = 2166136261
    for byte in struct.pack("<%di" % len(words), *[int(w) for w in words]):
        h ^= byte
        h = (h * 16777619) & 0xFFFFFFFF
    return h - (1 << 32) if h >= 1 << 31 else h


def input_hash(mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
               max_pages_per_seq, num_pages, topk, seqlens) -> int:
    """Header word 25: the hash that ties a plan to its problem and lengths."""
    return fnv1a32([mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
                    max_pages_per_seq, num_pages, topk] + [int(L) for L in seqlens])


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def unit_lengths(mode: int, batch: int, q_tokens: int, num_q_heads: int, num_kv_heads: int,
                 heads_per_unit: int, seqlens, topk: int) -> list[int]:
    G = num_q_heads // num_kv_heads
    hb = G // heads_per_unit
    lens = []
    for b in range(batch):
        L = topk if mode == MODE_MLA_SPARSE else int(seqlens[b])
        lens.extend([L] * (q_tokens * num_kv_heads * hb))
    return lens


def validate(mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
             max_pages_per_seq, num_pages, topk, num_cus, num_xcds, tile_tokens, heads_per_unit,
             seqlens, block_table=None, policy=POLICY_STREAMK, unit_cost=0) -> None:
    if mode not in (MODE_GQA, MODE_MLA, MODE_MLA_SPARSE):
        raise ValueError("mode")
    if policy not in (POLICY_STREAMK, POLICY_PER_UNIT):
        raise ValueError("policy")
    if unit_cost < 0:
        raise ValueError("unit_cost")
    if batch < 1 or q_tokens < 1 or num_q_heads < 1 or num_kv_heads < 1:
        raise ValueError("shape")
    if mode != MODE_MLA_SPARSE and q_tokens != 1:
        raise ValueError("dense decode has one query token per sequence")
    if num_q_heads % num_kv_heads:
        raise ValueError("heads")
    G = num_q_heads // num_kv_heads
    if heads_per_unit < 1 or G % heads_per_unit:
        raise ValueError("heads_per_unit")
    if head_dim_qk < 1 or head_dim_v < 1 or page_size < 1 or max_pages_per_seq < 1 or num_pages < 1:
        raise ValueError("dims")
    if num_cus < 1 or num_xcds < 1 or tile_tokens < 1:
        raise ValueError("opts")
    for b in range(batch):
        L = int(seqlens[b])
        if L < 0:
            raise ValueError("seqlen")
        if _ceil_div(L, page_size) > max_pages_per_seq:
            raise ValueError("seqlen beyond block table")
        if mode == MODE_MLA_SPARSE and (topk < 1 or topk > L):
            raise ValueError("topk")
        if block_table is not None:
            row = np.asarray(block_table)[b, :_ceil_div(L, page_size)]
            if np.any(row < 0) or np.any(row >= num_pages):
                raise ValueError("page")


def plan(mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
         max_pages_per_seq, num_pages, topk, num_cus, num_xcds, tile_tokens, heads_per_unit,
         seqlens, block_table=None, policy=POLICY_STREAMK, unit_cost=0) -> dict:
    """Build the plan; returns its fields and the serialised ``blob``.

    ``policy`` POLICY_PER_UNIT is the comparison launch with one worker per
    unit and no split (num_cus is then ignored and the worker count is U).
    ``unit_cost`` (POLICY_STREAMK, in tiles): 0 is the equal tile split.
    """
    validate(mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
             max_pages_per_seq, num_pages, topk, num_cus, num_xcds, tile_tokens, heads_per_unit,
             seqlens, block_table, policy, unit_cost)
    C, X, T = num_cus, num_xcds, tile_tokens
    lens = unit_lengths(mode, batch, q_tokens, num_q_heads, num_kv_heads, heads_per_unit, seqlens, topk)
    U = len(lens)
    if policy == POLICY_PER_UNIT:
        C = U
    ntiles = [_ceil_div(L, T) for L in lens]
    N = sum(ntiles)

    if policy == POLICY_PER_UNIT:
        chunk_pieces = [[(k, 0, lens[k])] if lens[k] > 0 else [] for k in range(C)]
    else:
        chunk_pieces = _chunks(ntiles, lens, C, T, unit_cost)

    nsplit = [0] * U
    items_by_chunk = []
    for pieces in chunk_pieces:
        its = []
        for (v, t0, t1) in pieces:
            its.append((v, t0, t1, nsplit[v]))
            nsplit[v] += 1
        items_by_chunk.append(its)
    pbase = []
    S = 0
    for n in nsplit:
        if n > 1:
            pbase.append(S)
            S += n
        else:
            pbase.append(-1)

    header = [0] * HEADER_WORDS
    header[:23] = [PLAN_MAGIC, PLAN_VERSION, mode, batch, q_tokens, num_q_heads, num_kv_heads,
                   head_dim_qk, head_dim_v, page_size, topk, C, X, T, heads_per_unit, U, N, 0, S,
                   max(nsplit) if nsplit else 0, policy, max_pages_per_seq, num_pages]
    header[23] = unit_cost if policy == POLICY_STREAMK else 0
    header[24] = sum(1 for n in nsplit if n == 0)      # units with no piece (empty sequences)
    header[25] = input_hash(mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v,
                            page_size, max_pages_per_seq, num_pages, topk, seqlens)
    return _serialise(header, items_by_chunk, nsplit, pbase, [], policy != POLICY_PER_UNIT, C, X,
                      dict(num_units=U, num_tiles=N, num_partials=S, unit_len=lens))


def _serialise(header, items_by_chunk, nsplit, pbase, prefix_rows, spread, C, X, fields) -> dict:
    """Worker placement, then the blob: header, wg_off (padded to 4 words),
    items, unit_nsplit, unit_pbase and the prefix table rows."""
    if spread and X > 1 and C % X == 0:
        CX = C // X
        worker_of_chunk = [(k % CX) * X + k // CX for k in range(C)]
    else:
        worker_of_chunk = list(range(C))
    chunk_of_worker = [0] * C
    for k, w in enumerate(worker_of_chunk):
        chunk_of_worker[w] = k

    wg_off = [0]
    items = []
    for w in range(C):
        its = items_by_chunk[chunk_of_worker[w]]
        items.extend(its)
        wg_off.append(len(items))
    W = len(items)
    header = list(header)
    header[17] = W
    pad = (-(C + 1)) % 4                 # keeps the item array 16-byte aligned
    words = (header + wg_off + [0] * pad + [x for it in items for x in it] + nsplit + pbase +
             [x for row in prefix_rows for x in row])
    for x in words:
        if not (-2**31 <= x < 2**31):
            raise ValueError("plan does not fit int32")
    blob = struct.pack("<%di" % len(words), *words)
    return dict(blob=blob, num_items=W, wg_off=wg_off, items=items, unit_nsplit=nsplit, unit_pbase=pbase,
                worker_of_chunk=worker_of_chunk, chunk_items=items_by_chunk, **fields)


def _equal_split(ntiles, lens, C: int, T: int):
    """The equal tile split: chunk k takes floor(N / C) tiles, one more for
    k < N mod C, contiguously in the unit-major tile order; pieces
    (unit, tok_begin, tok_end) per chunk, an empty unit getting none."""
    first_tile = []
    acc = 0
    for n in ntiles:
        first_tile.append(acc)
        acc += n
    N, U = acc, len(ntiles)
    base, rem = divmod(N, C)
    u = 0
    chunk_pieces = []
    for k in range(C):
        start = k * base + min(k, rem)
        end = start + base + (1 if k < rem else 0)
        pieces = []
        while u < U and first_tile[u] + ntiles[u] <= start:
            u += 1
        v = u
        while end > start and v < U and first_tile[v] < end:
            if ntiles[v] == 0:     # an empty unit gets no piece
                v += 1
                continue
            tb = max(start, first_tile[v]) - first_tile[v]
            te = min(end, first_tile[v] + ntiles[v]) - first_tile[v]
            pieces.append((v, tb * T, min(te * T, lens[v])))
            if first_tile[v] + ntiles[v] > end:
                break
            v += 1
        chunk_pieces.append(pieces)
    return chunk_pieces


def _chunks(ntiles, lens, C: int, T: int, unit_cost: int):
    """Pieces per chunk of the Stream-K split: the equal tile split at unit
    cost 0, the cost split otherwise."""
    return _cost_split(ntiles, lens, C, T, unit_cost) if unit_cost > 0 else _equal_split(ntiles, lens, C, T)


def _cost_split(ntiles, lens, C: int, T: int, O: int):
    """Chunks of the cost split: pieces (unit, tok_begin, tok_end) per chunk.

    Unit u's cost range starts at cs[u] = sum over earlier non-empty units of
    (O + n), O the unit cost in tiles; its tile i starts at cs[u] + O + i and
    belongs to the chunk whose range holds that position.  With O = 0 a tile's
    position is its index in the unit-major tile order, so this is the equal
    tile split.
    """
    total = sum(O + n for n in ntiles if n > 0)
    q, r = divmod(total, C)
    bound = [k * q + min(k, r) for k in range(C + 1)]   # chunk k: [bound[k], bound[k+1])
    pieces: list[list[tuple[int, int, int]]] = [[] for _ in range(C)]
    cs, k = 0, 0
    for u, n in enumerate(ntiles):
        if n == 0:      # an empty unit: no piece, no cost
            continue
        i = 0
        while i < n:
            start = cs + O + i
            while bound[k + 1] <= start:
                k += 1
            # tiles of u whose start lies before the end of chunk k
            last = min(n, bound[k + 1] - cs - O)
            pieces[k].append((u, i * T, min(last * T, lens[u])))
            i = last
        cs += O + n
    return pieces


def validate_prefix(batch, num_q_heads, num_kv_heads, page_size, seqlens, prefix_group, prefix_len,
                    block_table=None) -> None:
    """Shared-prefix inputs: prefix_group[b] is -1 or a group id in
    [0, len(prefix_len)); prefix_len[g] is a whole number of pages; every
    member of a group holds at least its prefix; with a block table, every
    member's first prefix_len / page_size pages are the same pages."""
    G = num_q_heads // num_kv_heads
    if PREFIX_ROWS % G:
        raise ValueError("group size must divide 16")
    NG = len(prefix_len)
    if len(prefix_group) != batch:
        raise ValueError("prefix_group")
    for g in range(NG):
        if prefix_len[g] < 0 or prefix_len[g] % page_size:
            raise ValueError("prefix_len must be a whole number of pages")
    first = {}
    for b in range(batch):
        g = int(prefix_group[b])
        if g == -1:
            continue
        if not (0 <= g < NG):
            raise ValueError("prefix group id")
        Lp = int(prefix_len[g])
        if int(seqlens[b]) < Lp:
            raise ValueError("a member is shorter than its group's prefix")
        if block_table is not None and Lp > 0:
            row = list(np.asarray(block_table)[b, :Lp // page_size])
            if g in first and first[g] != row:
                raise ValueError("members of a group do not share the prefix pages")
            first.setdefault(g, row)


def plan_prefix(mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
                max_pages_per_seq, num_pages, topk, num_cus, num_xcds, tile_tokens, seqlens,
                prefix_group, prefix_len, block_table=None, unit_cost=0) -> dict:
    """A Stream-K plan in which sequences sharing a prefix read it once.

    The shared-prefix decode the MeldKernel summary measures ("Experiments and
    results", Fig. 11): sequences b with prefix_group[b] = g hold the same
    first prefix_len[g] tokens (the same pages).  Readings:
    * prefix units: for each group in id order, each KV head, and each block
      of 16 / G members (in sequence order), one unit over tokens
      [0, prefix_len) whose 16 query rows are the members' G heads; its work
      is read once for all of them.
    * the sequences' own units (b, h) then cover [prefix_len_b, L_b) only
      (prefix_len_b = 0 outside a group or for a group with no prefix).
    * unit order for the split: every prefix unit (ids U .. U + P - 1, U =
      batch * Hkv), then the sequences' units in the usual order; the chunks
      are cut as in ``plan`` (equal tiles at unit cost 0).
    * splits of a member unit: the pieces of its prefix unit first (split
      index = the piece's index within the prefix unit, in chunk order), then
      its own pieces; unit_nsplit counts both, and partial slots are laid out
      as in ``plan``.  A prefix piece's partial for a member holds that
      member's rows, so each member's result is the log-sum-exp merge of all
      its splits, the same identity as for any split.
    * the blob appends one PREFIX_WORDS row per prefix unit: KV head, number
      of members, prefix length, number of pieces, member sequence ids (-1
      padded to 16); header word 26 counts the rows.
    GQA with one query token, heads_per_unit = G, only.
    """
    if mode != MODE_GQA or q_tokens != 1:
        raise ValueError("shared prefixes: GQA decode with one query token")
    G = num_q_heads // num_kv_heads if num_kv_heads and num_q_heads % num_kv_heads == 0 else 0
    validate(mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
             max_pages_per_seq, num_pages, topk, num_cus, num_xcds, tile_tokens, max(G, 1), seqlens,
             block_table, POLICY_STREAMK, unit_cost)
    validate_prefix(batch, num_q_heads, num_kv_heads, page_size, seqlens, prefix_group, prefix_len,
                    block_table)
    C, X, T, Hkv = num_cus, num_xcds, tile_tokens, num_kv_heads
    Mp = PREFIX_ROWS // G
    U = batch * Hkv

    lp_of = [0] * batch
    prefix_units = []           # (kv_head, prefix_len, member sequences)
    for g in range(len(prefix_len)):
        members = [b for b in range(batch) if int(prefix_group[b]) == g]
        Lp = int(prefix_len[g])
        if Lp == 0 or not members:
            continue
        for b in members:
            lp_of[b] = Lp
        for h in range(Hkv):
            for i in range(0, len(members), Mp):
                prefix_units.append((h, Lp, members[i:i + Mp]))
    P = len(prefix_units)
    prefix_of = {}              # member unit -> its prefix unit
    for p, (h, Lp, members) in enumerate(prefix_units):
        for b in members:
            prefix_of[b * Hkv + h] = p

    # the work list in split order: (unit id, first token, end token)
    work = [(U + p, 0, Lp) for p, (h, Lp, members) in enumerate(prefix_units)]
    work += [(b * Hkv + h, lp_of[b], int(seqlens[b])) for b in range(batch) for h in range(Hkv)]
    lens = [te - t0 for (_, t0, te) in work]
    ntiles = [_ceil_div(L, T) for L in lens]
    N = sum(ntiles)
    chunk_pieces = _chunks(ntiles, lens, C, T, unit_cost)

    pieces_of_prefix = [0] * P
    for pieces in chunk_pieces:
        for (v, _, _) in pieces:
            if work[v][0] >= U:
                pieces_of_prefix[work[v][0] - U] += 1
    own = [0] * U               # own pieces numbered so far
    seen_prefix = [0] * P
    items_by_chunk = []
    for pieces in chunk_pieces:
        its = []
        for (v, a, e) in pieces:
            unit, t0, _ = work[v]
            if unit >= U:
                split = seen_prefix[unit - U]
                seen_prefix[unit - U] += 1
            else:
                before = pieces_of_prefix[prefix_of[unit]] if unit in prefix_of else 0
                split = before + own[unit]
                own[unit] += 1
            its.append((unit, t0 + a, t0 + e, split))
        items_by_chunk.append(its)
    nsplit = [own[u] + (pieces_of_prefix[prefix_of[u]] if u in prefix_of else 0) for u in range(U)]
    pbase = []
    S = 0
    for n in nsplit:
        if n > 1:
            pbase.append(S)
            S += n
        else:
            pbase.append(-1)
    rows = [[h, len(members), Lp, pieces_of_prefix[p]] + members + [-1] * (PREFIX_ROWS - len(members))
            for p, (h, Lp, members) in enumerate(prefix_units)]

    header = [0] * HEADER_WORDS
    header[:23] = [PLAN_MAGIC, PLAN_VERSION, mode, batch, q_tokens, num_q_heads, num_kv_heads,
                   head_dim_qk, head_dim_v, page_size, topk, C, X, T, G, U, N, 0, S,
                   max(nsplit) if nsplit else 0, POLICY_STREAMK, max_pages_per_seq, num_pages]
    header[23] = unit_cost
    header[24] = sum(1 for n in nsplit if n == 0)
    header[25] = input_hash(mode, batch, q_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v,
                            page_size, max_pages_per_seq, num_pages, topk, seqlens)
    header[26] = P
    return _serialise(header, items_by_chunk, nsplit, pbase, rows, True, C, X,
                      dict(num_units=U, num_tiles=N, num_partials=S, unit_len=lens, prefix_units=prefix_units,
                           prefix_pieces=pieces_of_prefix))


def plan_moe(num_experts, hidden, out_dim, expert_tokens, num_cus, num_xcds, tile_rows=MOE_TILE_ROWS, tile_cols=MOE_TILE_COLS,
             tile_k=64, policy=POLICY_STREAMK, unit_cost=0) -> dict:
    """A Stream-K plan for the MoE grouped GEMM Y_e = X_e W_e^T.

    The same split as ``plan`` applied to another imbalanced workload (the
    MeldKernel summary instantiates the method on MoE: "Problem and
    motivation", "Core method").  Readings:
    * unit: one tile_rows x tile_cols output tile of one expert, (expert e,
      column block, row block) in that order, so the row blocks of one
      column block (which read the same weight tile) are adjacent; an expert
      with no rows has no unit.
    * a unit's length is the hidden size K, cut into tiles of tile_k: the
      split is over the (unit, k tile) work exactly as ``plan`` splits
      (unit, KV tile) work; a piece is a unit's k range within one chunk and
      its split index counts the unit's pieces in chunk order.
    * POLICY_STREAMK_DP (the data-parallel + Stream-K form of the same equal
      split): the first D C tiles go whole, tile r C + k to chunk k in round
      r, so the tiles computed at the same time are neighbours that share
      weight and row tiles in cache; the remaining U - D C tiles have their k
      tiles split over the chunks as above.  With R = U mod C: R = 0 or
      4 R >= 3 C (a last round at least three quarters full) splits nothing,
      the last round's tiles going whole to chunks 0 .. R - 1; 2 R >= C
      splits the remainder alone (at least half a tile per chunk); a smaller
      remainder takes the last whole round with it (at least one tile per
      chunk).  Every chunk gets the same work to within one tile (within one
      k tile when something is split), and a split tile has at most three
      pieces (unit cost 0): the sum of a split tile reads one or two other
      partials, not a share of a small remainder cut C ways.  The three
      quarters are this library's reading of when a split costs more than
      the idle quarter round it saves (a split tile's partials are written
      and read back whole).
    * the blob has ``plan``'s layout with mode 3, batch = E, head_dim_qk = K,
      head_dim_v = N, page_size = tile_cols, heads_per_unit = tile_rows,
      tile_tokens = tile_k, one page, and then MOE_DESC_WORDS per unit
      (expert, first row, rows, first column); word 25 is ``input_hash`` of
      those header values with expert_tokens in place of seqlens.
    """
    E, K, N = num_experts, hidden, out_dim
    if E < 1 or K < 1 or N < 1 or K % tile_k or N % tile_cols:
        raise ValueError("MoE shape: K a multiple of tile_k, N of tile_cols")
    if (policy not in (POLICY_STREAMK, POLICY_PER_UNIT, POLICY_STREAMK_DP) or unit_cost < 0 or num_cus < 1
            or num_xcds < 1):
        raise ValueError("opts")
    counts = [int(n) for n in expert_tokens]
    if len(counts) != E or min(counts) < 0:
        raise ValueError("expert_tokens")
    units = []
    row0 = 0
    for e in range(E):
        for nt in range(N // tile_cols):
            for mt in range(_ceil_div(counts[e], tile_rows)):
                units.append((e, row0 + mt * tile_rows, min(tile_rows, counts[e] - mt * tile_rows),
                              nt * tile_cols))
        row0 += counts[e]
    U = len(units)
    if U == 0:
        raise ValueError("no rows")
    lens = [K] * U
    ntiles = [K // tile_k] * U
    C = U if policy == POLICY_PER_UNIT else num_cus
    if policy == POLICY_PER_UNIT:
        chunk_pieces = [[(k, 0, K)] for k in range(C)]
    elif policy == POLICY_STREAMK_DP:
        # whole tiles dealt round-robin (tile r C + k to chunk k, round by
        # round), then the remaining tiles' k tiles split as in ``plan``; a
        # remainder of less than half a round takes the last round with it
        rem = U % C
        whole = rem == 0 or 4 * rem >= 3 * C
        full = -(-U // C) if whole else (U // C if 2 * rem >= C else max(U // C - 1, 0))
        chunk_pieces = [[(r * C + k, 0, K) for r in range(full) if r * C + k < U] for k in range(C)]
        rest = _chunks(ntiles[full * C:], lens[full * C:], C, tile_k, unit_cost) if U > full * C else [[]] * C
        for k in range(C):
            chunk_pieces[k] += [(full * C + v, a, b) for (v, a, b) in rest[k]]
    else:
        chunk_pieces = _chunks(ntiles, lens, C, tile_k, unit_cost)
    nsplit = [0] * U
    items_by_chunk = []
    for pieces in chunk_pieces:
        its = []
        for (v, t0, t1) in pieces:
            its.append((v, t0, t1, nsplit[v]))
            nsplit[v] += 1
        items_by_chunk.append(its)
    pbase, S = [], 0
    for n in nsplit:
        if n > 1:
            pbase.append(S)
            S += n
        else:
            pbase.append(-1)
    header = [0] * HEADER_WORDS
    header[:23] = [PLAN_MAGIC, PLAN_VERSION, MODE_MOE, E, 1, 1, 1, K, N, tile_cols, 0, C, num_xcds, tile_k,
                   tile_rows, U, sum(ntiles), 0, S, max(nsplit), policy, 1, 1]
    header[23] = unit_cost if policy != POLICY_PER_UNIT else 0
    header[24] = 0
    header[25] = input_hash(MODE_MOE, E, 1, 1, 1, K, N, tile_cols, 1, 1, 0, counts)
    return _serialise(header, items_by_chunk, nsplit, pbase, [list(u) for u in units], policy != POLICY_PER_UNIT,
                      C, num_xcds, dict(num_units=U, num_tiles=sum(ntiles), num_partials=S, units=units))


def plan_for(wl, num_cus=256, num_xcds=8, tile_tokens=32, heads_per_unit=None,
             policy=POLICY_STREAMK, unit_cost=0) -> dict:
    """``plan`` for a workload object from the seeded input generator."""
    c = wl.cfg
    hu = heads_per_unit if heads_per_unit is not None else c.num_q_heads // c.num_kv_heads
    return plan(c.mode, c.batch, c.q_tokens, c.num_q_heads, c.num_kv_heads, c.head_dim_qk, c.head_dim_v,
                c.page_size, wl.max_pages, wl.num_pages, c.topk, num_cus, num_xcds, tile_tokens, hu,
                wl.seqlens, wl.block_table, policy, unit_cost)


def list_schedule(task_times, num_workers: int):
    """Greedy list scheduling: each task, in order, starts on the earliest-free worker.

    The hardware block scheduler of the tail-effect example (CSDN Q&A on
    waves, "Scenario examples") behaves this way.  Returns (makespan,
    per-worker finish times, per-worker assignment).
    """
    free = [0.0] * num_workers
    assign = [[] for _ in range(num_workers)]
    for i, t in enumerate(task_times):
        w = min(range(num_workers), key=lambda j: (free[j], j))
        assign[w].append(i)
        free[w] += t
    return max(free), free, assign
