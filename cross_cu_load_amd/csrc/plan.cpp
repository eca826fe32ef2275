// Host planner: the Stream-K split of a decode batch into one equal chunk of
// KV tiles per compute unit, run as a single wave (CSDN Q&A on waves and
// FlashMLA's Stream-K, "Summary").  The split is computed from the real
// sequence lengths and the hardware shape at run time (MeldKernel summary,
// "Core method") and serialised as fixed-size work descriptors per worker
// (GLM-5.2 decode article, MegaRTP design: host-built per-worker queues).
//
// Plain C++17 with no HIP dependency.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "plan.h"

namespace cc {

namespace {
thread_local std::string g_err;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tiles of T tokens covering a length: a shift when T is a power of two (the
// usual case), since 64-bit division dominates the planner's time otherwise.
struct TileCount {
  int64_t T;
  int shift = -1;
  explicit TileCount(int64_t t) : T(t) {
    if ((t & (t - 1)) == 0)
      for (shift = 0; (int64_t{1} << shift) < t; ++shift) {}
  }
  int64_t operator()(int64_t len) const { return shift >= 0 ? (len + T - 1) >> shift : ceil_div(len, T); }
};

struct Inputs {
  const cc_problem* p;
  const cc_plan_opts* o;
  const int32_t* seqlens;
  const int32_t* block_table;
};

int validate(const Inputs& in) {
  const cc_problem& p = *in.p;
  const cc_plan_opts& o = *in.o;
  if (p.mode < CC_MODE_GQA || p.mode > CC_MODE_MLA_SPARSE) {
    set_error("unknown mode %d", p.mode);
    return CC_ERR_INVALID;
  }
  if (o.policy != CC_POLICY_STREAMK && o.policy != CC_POLICY_PER_UNIT) {
    set_error("unknown policy %d", o.policy);
    return CC_ERR_INVALID;
  }
  if (o.unit_cost < 0) {
    set_error("unit_cost %d must be >= 0", o.unit_cost);
    return CC_ERR_INVALID;
  }
  if (p.batch < 1 || p.q_tokens < 1 || p.num_q_heads < 1 || p.num_kv_heads < 1) {
    set_error("batch, q_tokens and head counts must be >= 1");
    return CC_ERR_INVALID;
  }
  if (p.mode != CC_MODE_MLA_SPARSE && p.q_tokens != 1) {
    set_error("dense decode takes one query token per sequence (q_tokens=%d)", p.q_tokens);
    return CC_ERR_INVALID;
  }
  if (p.num_q_heads % p.num_kv_heads) {
    set_error("num_q_heads %d not a multiple of num_kv_heads %d", p.num_q_heads, p.num_kv_heads);
    return CC_ERR_INVALID;
  }
  const int32_t G = p.num_q_heads / p.num_kv_heads;
  if (o.heads_per_unit < 1 || G % o.heads_per_unit) {
    set_error("heads_per_unit %d must divide the group size %d", o.heads_per_unit, G);
    return CC_ERR_INVALID;
  }
  if (p.head_dim_qk < 1 || p.head_dim_v < 1 || p.page_size < 1 || p.max_pages_per_seq < 1 ||
      p.num_pages < 1) {
    set_error("head dims, page_size, max_pages_per_seq and num_pages must be >= 1");
    return CC_ERR_INVALID;
  }
  if (o.num_cus < 1 || o.num_xcds < 1 || o.tile_tokens < 1) {
    set_error("num_cus, num_xcds and tile_tokens must be >= 1");
    return CC_ERR_INVALID;
  }
  for (int32_t b = 0; b < p.batch; ++b) {
    const int32_t L = in.seqlens[b];
    if (L < 0) {
      set_error("seqlens[%d] = %d is negative", b, L);
      return CC_ERR_INVALID;
    }
    const int64_t pages = ceil_div(L, p.page_size);
    if (pages > p.max_pages_per_seq) {
      set_error("seqlens[%d] = %d needs %lld pages > max_pages_per_seq %d", b, L, (long long)pages,
                p.max_pages_per_seq);
      return CC_ERR_INVALID;
    }
    if (p.mode == CC_MODE_MLA_SPARSE && (p.topk < 1 || p.topk > L)) {
      set_error("topk %d outside [1, seqlens[%d] = %d]", p.topk, b, L);
      return CC_ERR_INVALID;
    }
    if (in.block_table) {
      const int32_t* row = in.block_table + (int64_t)b * p.max_pages_per_seq;
      for (int64_t i = 0; i < pages; ++i) {
        if (row[i] < 0 || row[i] >= p.num_pages) {
          set_error("block_table[%d][%lld] = %d outside [0, %d)", b, (long long)i, row[i],
                    p.num_pages);
          return CC_ERR_PAGE;
        }
      }
    }
  }
  return CC_OK;
}

struct Built {
  bool size_only = false;   // stop once the word count is known
  int64_t total = 0;        // words in the blob
  std::vector<int32_t> words;
};

// Shared-prefix inputs of cc_plan_prefix (absent for cc_plan).
struct PrefixInputs {
  const int32_t* group;  // [batch]: -1 or a group id in [0, num_groups)
  int32_t num_groups;
  const int32_t* len;    // [num_groups]: prefix tokens, whole pages
};

// The split cuts a list of work entries in order: a unit id and the token
// range [t0, t0 + len) of it that the entry covers.
struct Work { int64_t unit, t0, len; };
// A piece: work entry w, tokens [a, e) relative to the entry's t0.
struct Piece { int64_t w, a, e; };
struct Item { int64_t u, t0, t1, s; };

// Elements are appended field by field.  A braced temporary is built on the
// stack with 8-byte stores and copied out with 16-byte loads, which defeats
// store-to-load forwarding and cost ~20 cycles per element, most of the
// planner's time.
void add_work(std::vector<Work>& v, int64_t unit, int64_t t0, int64_t len) {
  Work& x = v.emplace_back();
  x.unit = unit; x.t0 = t0; x.len = len;
}
void add_piece(std::vector<Piece>& v, int64_t w, int64_t a, int64_t e) {
  Piece& x = v.emplace_back();
  x.w = w; x.a = a; x.e = e;
}
void add_item(std::vector<Item>& v, int64_t u, int64_t t0, int64_t t1, int64_t s) {
  Item& x = v.emplace_back();
  x.u = u; x.t0 = t0; x.t1 = t1; x.s = s;
}

// Pieces grouped by chunk: chunk k's pieces are pieces[off[k] .. off[k + 1]).
// One flat list, not a list per chunk: a plan of a few hundred chunks would
// otherwise spend most of its time allocating.
struct Chunks {
  std::vector<int64_t> off;
  std::vector<Piece> pieces;
  int64_t count() const { return (int64_t)off.size() - 1; }
};

// Pieces per chunk of the equal split of cost: one per tile plus O per
// non-empty entry, each entry's cost first; a tile goes to the chunk whose
// cost range holds its starting position (with O = 0, the equal tile split).
Chunks split_chunks(const std::vector<Work>& work, int64_t C, int64_t T, int64_t O) {
  const TileCount tiles(T);
  int64_t busy = 0, N = 0;
  for (const Work& x : work) {
    const int64_t n = tiles(x.len);
    N += n;
    busy += n > 0;
  }
  // Each of the C - 1 chunk boundaries cuts at most one entry in two, so
  // busy + C - 1 pieces at most; written through a pointer, not appended.
  Chunks ch;
  ch.off.assign(C + 1, 0);
  ch.pieces.resize(busy + C);
  Piece* out = ch.pieces.data();
  int64_t np = 0;
  const int64_t total = O * busy + N;
  const int64_t q = total / C, r = total % C;
  auto bound = [&](int64_t k) { return k * q + (k < r ? k : r); };  // chunk k: [bound(k), bound(k+1))
  int64_t cs = 0, k = 0;
  for (int64_t w = 0; w < (int64_t)work.size(); ++w) {
    const int64_t L = work[w].len, n = tiles(L);
    if (n == 0) continue;  // an empty entry gets no piece and costs nothing
    for (int64_t i = 0; i < n;) {
      while (bound(k + 1) <= cs + O + i) ++k;
      int64_t last = bound(k + 1) - cs - O;  // tiles of w starting before chunk k ends
      if (last > n) last = n;
      if (np == (int64_t)ch.pieces.size()) {  // not reached (the bound above); kept as a guard
        ch.pieces.resize(2 * np + 1);
        out = ch.pieces.data();
      }
      out[np].w = w;
      out[np].a = i * T;
      out[np].e = last * T < L ? last * T : L;
      ++np;
      ++ch.off[k + 1];
      i = last;
    }
    cs += O + n;
  }
  ch.pieces.resize(np);
  for (int64_t j = 0; j < C; ++j) ch.off[j + 1] += ch.off[j];
  return ch;
}

// One piece per non-empty entry, chunk u holding entry u (the per-unit policy).
Chunks whole_chunks(const std::vector<Work>& work) {
  Chunks ch;
  const int64_t C = (int64_t)work.size();
  ch.off.assign(C + 1, 0);
  ch.pieces.reserve(C);
  for (int64_t u = 0; u < C; ++u) {
    if (work[u].len > 0) add_piece(ch.pieces, u, 0, work[u].len);
    ch.off[u + 1] = (int64_t)ch.pieces.size();
  }
  return ch;
}

// Items of pieces whose entry is the unit itself: split indices in chunk order.
std::vector<Item> unit_items(const Chunks& ch, std::vector<int64_t>& nsplit) {
  std::vector<Item> items(ch.pieces.size());
  for (size_t i = 0; i < items.size(); ++i) {
    const Piece& pc = ch.pieces[i];
    items[i].u = pc.w;
    items[i].t0 = pc.a;
    items[i].t1 = pc.e;
    items[i].s = nsplit[pc.w]++;
  }
  return items;
}

// The blob: header, wg_off (padded), items in worker order, unit_nsplit,
// unit_pbase, prefix table rows.  Logical chunk k's items are
// items[off[k] .. off[k + 1]).  With out->size_only, only the word count.
int serialise(const cc_problem& p, const cc_plan_opts& o, const int32_t* seqlens, int64_t C, int64_t U,
              int64_t N, int64_t hpu, const std::vector<int64_t>& off, const std::vector<Item>& items,
              const std::vector<int64_t>& nsplit, const std::vector<int32_t>& prefix_rows, Built* out) {
  const int64_t W = (int64_t)items.size();
  const int64_t total = kHeaderWords + wg_words(C) + kItemWords * W + 2 * U + (int64_t)prefix_rows.size();
  if (N > INT32_MAX || C > INT32_MAX || W > INT32_MAX || U > INT32_MAX || total > INT32_MAX) {
    set_error("plan too large for int32 fields");
    return CC_ERR_INVALID;
  }
  out->total = total;
  if (out->size_only) return CC_OK;
  std::vector<int64_t> pbase(U, -1);
  int64_t S = 0, maxsplit = 0, empty = 0;
  for (int64_t u = 0; u < U; ++u) {
    if (nsplit[u] > 1) { pbase[u] = S; S += nsplit[u]; }
    if (nsplit[u] > maxsplit) maxsplit = nsplit[u];
    empty += nsplit[u] == 0;
  }
  // worker of each logical chunk: consecutive chunks share an XCD
  std::vector<int64_t> chunk_of_worker(C);
  const int64_t X = o.num_xcds;
  const bool spread = o.policy != CC_POLICY_PER_UNIT && X > 1 && C % X == 0;
  for (int64_t k = 0; k < C; ++k) {
    const int64_t w = spread ? (k % (C / X)) * X + k / (C / X) : k;
    chunk_of_worker[w] = k;
  }
  const int64_t P = (int64_t)prefix_rows.size() / kPrefixWords;  // S <= W: every slot is an item
  std::vector<int32_t>& w = out->words;
  w.assign(total, 0);
  int32_t* h = w.data();
  h[H_MAGIC] = kPlanMagic;
  h[H_VERSION] = kPlanVersion;
  h[H_MODE] = p.mode;
  h[H_BATCH] = p.batch;
  h[H_QTOKENS] = p.q_tokens;
  h[H_HQ] = p.num_q_heads;
  h[H_HKV] = p.num_kv_heads;
  h[H_DQK] = p.head_dim_qk;
  h[H_DV] = p.head_dim_v;
  h[H_PAGE] = p.page_size;
  h[H_TOPK] = p.topk;
  h[H_WORKERS] = (int32_t)C;
  h[H_XCDS] = o.num_xcds;
  h[H_TILE] = o.tile_tokens;
  h[H_HPU] = (int32_t)hpu;
  h[H_UNITS] = (int32_t)U;
  h[H_TILES] = (int32_t)N;
  h[H_ITEMS] = (int32_t)W;
  h[H_PARTIALS] = (int32_t)S;
  h[H_MAXSPLIT] = (int32_t)maxsplit;
  h[H_POLICY] = o.policy;
  h[H_MAXPAGES] = p.max_pages_per_seq;
  h[H_NUMPAGES] = p.num_pages;
  h[H_UNIT_COST] = o.policy != CC_POLICY_PER_UNIT ? o.unit_cost : 0;
  h[H_EMPTY] = (int32_t)empty;
  h[H_HASH] = input_hash(p, seqlens);
  h[H_PREFIX] = (int32_t)P;
  int32_t* wg = h + kHeaderWords;
  int32_t* it = wg + wg_words(C);
  int64_t n = 0;
  for (int64_t wk = 0; wk < C; ++wk) {
    wg[wk] = (int32_t)n;
    const int64_t k = chunk_of_worker[wk];
    for (int64_t i = off[k]; i < off[k + 1]; ++i) {
      const Item& x = items[i];
      it[4 * n + 0] = (int32_t)x.u;
      it[4 * n + 1] = (int32_t)x.t0;
      it[4 * n + 2] = (int32_t)x.t1;
      it[4 * n + 3] = (int32_t)x.s;
      ++n;
    }
  }
  wg[C] = (int32_t)n;
  int32_t* ns = it + 4 * W;
  int32_t* pb = ns + U;
  for (int64_t u = 0; u < U; ++u) {
    ns[u] = (int32_t)nsplit[u];
    pb[u] = (int32_t)pbase[u];
  }
  std::copy(prefix_rows.begin(), prefix_rows.end(), pb + U);
  return CC_OK;
}

// The whole plan as int32 words.  Returns CC_OK or an error code.
int build(const Inputs& in, Built* out) {
  int rc = validate(in);
  if (rc) return rc;
  const cc_problem& p = *in.p;
  const cc_plan_opts& o = *in.o;
  const int64_t G = p.num_q_heads / p.num_kv_heads;
  const int64_t blocks_per_kv = G / o.heads_per_unit;
  const int64_t units_per_seq = (int64_t)p.q_tokens * p.num_kv_heads * blocks_per_kv;
  const int64_t U = units_per_seq * p.batch;
  const int64_t T = o.tile_tokens;

  // units units_per_seq * b .. units_per_seq * (b + 1) - 1 belong to sequence b
  std::vector<Work> work;
  work.reserve(U);
  const TileCount tiles(T);
  int64_t N = 0;
  for (int64_t b = 0, u = 0; b < p.batch; ++b) {
    const int64_t L = p.mode == CC_MODE_MLA_SPARSE ? p.topk : in.seqlens[b];
    N += tiles(L) * units_per_seq;
    for (int64_t j = 0; j < units_per_seq; ++j, ++u) add_work(work, u, 0, L);
  }
  const int64_t C = o.policy == CC_POLICY_PER_UNIT ? U : o.num_cus;
  const Chunks ch = o.policy == CC_POLICY_PER_UNIT ? whole_chunks(work) : split_chunks(work, C, T, o.unit_cost);
  std::vector<int64_t> nsplit(U, 0);
  const std::vector<Item> items = unit_items(ch, nsplit);
  return serialise(p, o, in.seqlens, C, U, N, o.heads_per_unit, ch.off, items, nsplit, {}, out);
}

// Shared-prefix inputs: group ids in range, prefixes of whole pages, members
// at least as long as their prefix and (with a block table) holding the same
// prefix pages.
int validate_prefix(const Inputs& in, const PrefixInputs& pre) {
  const cc_problem& p = *in.p;
  const cc_plan_opts& o = *in.o;
  if (p.mode != CC_MODE_GQA || p.q_tokens != 1) {
    set_error("shared prefixes: GQA decode with one query token");
    return CC_ERR_INVALID;
  }
  if (o.policy != CC_POLICY_STREAMK) {
    set_error("shared prefixes: policy must be CC_POLICY_STREAMK");
    return CC_ERR_INVALID;
  }
  const int32_t G = p.num_q_heads / p.num_kv_heads;
  if (kPrefixRows % G || o.heads_per_unit != G) {
    set_error("shared prefixes: the group size %d must divide 16 and heads_per_unit equal it", G);
    return CC_ERR_INVALID;
  }
  if (pre.num_groups < 0 || !pre.group || (pre.num_groups > 0 && !pre.len)) {
    set_error("shared prefixes: null group ids or lengths");
    return CC_ERR_INVALID;
  }
  for (int32_t g = 0; g < pre.num_groups; ++g) {
    if (pre.len[g] < 0 || pre.len[g] % p.page_size) {
      set_error("prefix_len[%d] = %d is not a whole number of %d-token pages", g, pre.len[g], p.page_size);
      return CC_ERR_INVALID;
    }
  }
  std::vector<int32_t> first(pre.num_groups, -1);  // first member of each group
  for (int32_t b = 0; b < p.batch; ++b) {
    const int32_t g = pre.group[b];
    if (g == -1) continue;
    if (g < 0 || g >= pre.num_groups) {
      set_error("prefix_group[%d] = %d outside [-1, %d)", b, g, pre.num_groups);
      return CC_ERR_INVALID;
    }
    const int32_t Lp = pre.len[g];
    if (in.seqlens[b] < Lp) {
      set_error("sequence %d (length %d) is shorter than its group's prefix of %d", b, in.seqlens[b], Lp);
      return CC_ERR_INVALID;
    }
    if (in.block_table && Lp > 0) {
      if (first[g] < 0) {
        first[g] = b;
      } else {
        const int32_t* r0 = in.block_table + (int64_t)first[g] * p.max_pages_per_seq;
        const int32_t* r1 = in.block_table + (int64_t)b * p.max_pages_per_seq;
        for (int32_t i = 0; i < Lp / p.page_size; ++i) {
          if (r0[i] != r1[i]) {
            set_error("sequences %d and %d share prefix group %d but not its page %d", first[g], b, g, i);
            return CC_ERR_INVALID;
          }
        }
      }
    }
  }
  return CC_OK;
}

// A shared-prefix plan: prefix units (group, KV head, block of 16 / G
// members) over [0, prefix_len), then every sequence's own units over
// [prefix_len_b, L_b); a member's splits are its prefix unit's pieces, then
// its own.
int build_prefix(const Inputs& in, const PrefixInputs& pre, Built* out) {
  int rc = validate(in);
  if (rc) return rc;
  rc = validate_prefix(in, pre);
  if (rc) return rc;
  const cc_problem& p = *in.p;
  const cc_plan_opts& o = *in.o;
  const int64_t G = p.num_q_heads / p.num_kv_heads, Hkv = p.num_kv_heads, Mp = kPrefixRows / G;
  const int64_t U = (int64_t)p.batch * Hkv, T = o.tile_tokens, C = o.num_cus;

  std::vector<int64_t> lp_of(p.batch, 0);
  std::vector<int32_t> rows;                  // prefix table
  std::vector<int64_t> prefix_of(U, -1);      // member unit -> prefix unit
  std::vector<int64_t> members;
  for (int32_t g = 0; g < pre.num_groups; ++g) {
    members.clear();
    for (int32_t b = 0; b < p.batch; ++b)
      if (pre.group[b] == g) members.push_back(b);
    const int32_t Lp = pre.len[g];
    if (Lp == 0 || members.empty()) continue;
    for (int64_t b : members) lp_of[b] = Lp;
    for (int64_t h = 0; h < Hkv; ++h) {
      for (size_t i = 0; i < members.size(); i += Mp) {
        const int64_t pu = (int64_t)rows.size() / kPrefixWords;
        const size_t n = std::min<size_t>(Mp, members.size() - i);
        rows.push_back((int32_t)h);
        rows.push_back((int32_t)n);
        rows.push_back(Lp);
        rows.push_back(0);  // pieces, filled below
        for (size_t j = 0; j < (size_t)kPrefixRows; ++j) {
          const int32_t b = j < n ? (int32_t)members[i + j] : -1;
          rows.push_back(b);
          if (b >= 0) prefix_of[b * Hkv + h] = pu;
        }
      }
    }
  }
  const int64_t P = (int64_t)rows.size() / kPrefixWords;
  // work list in split order: every prefix unit, then the sequences' own units
  std::vector<Work> work;
  work.reserve(P + U);
  int64_t N = 0;
  for (int64_t pu = 0; pu < P; ++pu) add_work(work, U + pu, 0, rows[pu * kPrefixWords + 2]);
  for (int64_t b = 0; b < p.batch; ++b)
    for (int64_t h = 0; h < Hkv; ++h) add_work(work, b * Hkv + h, lp_of[b], in.seqlens[b] - lp_of[b]);
  const TileCount tiles(T);
  for (const Work& x : work) N += tiles(x.len);
  const Chunks ch = split_chunks(work, C, T, o.unit_cost);

  std::vector<int64_t> pieces(P, 0);
  for (const Piece& pc : ch.pieces)
    if (work[pc.w].unit >= U) ++pieces[work[pc.w].unit - U];
  std::vector<int64_t> own(U, 0), seen(P, 0);
  std::vector<Item> items;
  items.reserve(ch.pieces.size());
  for (const Piece& pc : ch.pieces) {   // chunk order
    const Work& x = work[pc.w];
    int64_t s;
    if (x.unit >= U) {
      s = seen[x.unit - U]++;
    } else {
      s = (prefix_of[x.unit] >= 0 ? pieces[prefix_of[x.unit]] : 0) + own[x.unit]++;
    }
    add_item(items, x.unit, x.t0 + pc.a, x.t0 + pc.e, s);
  }
  std::vector<int64_t> nsplit(U);
  for (int64_t u = 0; u < U; ++u) nsplit[u] = own[u] + (prefix_of[u] >= 0 ? pieces[prefix_of[u]] : 0);
  for (int64_t pu = 0; pu < P; ++pu) rows[pu * kPrefixWords + 3] = (int32_t)pieces[pu];
  return serialise(p, o, in.seqlens, C, U, N, G, ch.off, items, nsplit, rows, out);
}

// MoE grouped GEMM plan: output tiles (expert, column block, row block) of
// heads_per_unit rows and 128 columns, each of length K cut into tile_tokens-
// wide k tiles, split as any plan.
int build_moe(const cc_moe_problem& mp, const cc_plan_opts& o, const int32_t* expert_tokens, Built* out) {
  const int64_t E = mp.num_experts, K = mp.hidden, N = mp.out_dim;
  const int64_t BM = o.heads_per_unit, BN = kMoeTileCols, BK = o.tile_tokens;
  if (E < 1 || K < 1 || N < 1 || BM < 1 || BK < 1 || K % BK || N % BN) {
    set_error("MoE plan: experts, hidden and out_dim >= 1, hidden a multiple of tile_tokens %lld and out_dim of %lld",
              (long long)BK, (long long)BN);
    return CC_ERR_INVALID;
  }
  if (o.policy != CC_POLICY_STREAMK && o.policy != CC_POLICY_PER_UNIT && o.policy != CC_POLICY_STREAMK_DP) {
    set_error("unknown policy %d", o.policy);
    return CC_ERR_INVALID;
  }
  if (o.unit_cost < 0 || o.num_cus < 1 || o.num_xcds < 1) {
    set_error("num_cus, num_xcds >= 1 and unit_cost >= 0");
    return CC_ERR_INVALID;
  }
  std::vector<int32_t> desc;
  int64_t row0 = 0;
  for (int64_t e = 0; e < E; ++e) {
    const int64_t n = expert_tokens[e];
    if (n < 0) {
      set_error("expert_tokens[%lld] = %lld is negative", (long long)e, (long long)n);
      return CC_ERR_INVALID;
    }
    for (int64_t nt = 0; nt < N / BN; ++nt) {
      for (int64_t mt = 0; mt < ceil_div(n, BM); ++mt) {
        desc.push_back((int32_t)e);
        desc.push_back((int32_t)(row0 + mt * BM));
        desc.push_back((int32_t)std::min<int64_t>(BM, n - mt * BM));
        desc.push_back((int32_t)(nt * BN));
      }
    }
    row0 += n;
  }
  const int64_t U = (int64_t)desc.size() / kMoeDescWords;
  if (U == 0) {
    set_error("MoE plan: no expert has rows");
    return CC_ERR_INVALID;
  }
  std::vector<Work> work;
  work.reserve(U);
  for (int64_t u = 0; u < U; ++u) add_work(work, u, 0, K);
  const int64_t C = o.policy == CC_POLICY_PER_UNIT ? U : o.num_cus;
  Chunks ch;
  if (o.policy == CC_POLICY_PER_UNIT) {
    ch = whole_chunks(work);
  } else if (o.policy == CC_POLICY_STREAMK_DP) {
    // whole tiles round-robin, round by round; the remaining tiles are split
    // (a last round at least three quarters full runs whole, a remainder of
    // less than half a round takes the last whole round with it)
    const int64_t rem = U % C;
    const bool whole = rem == 0 || 4 * rem >= 3 * C;
    const int64_t full = whole ? (U + C - 1) / C : (2 * rem >= C ? U / C : std::max<int64_t>(U / C - 1, 0));
    Chunks sk;
    if (U > full * C) {
      const std::vector<Work> rest(work.begin() + full * C, work.end());
      sk = split_chunks(rest, C, BK, o.unit_cost);
    }
    ch.off.assign(C + 1, 0);
    ch.pieces.reserve(std::min(full * C, U) + sk.pieces.size());
    for (int64_t k = 0; k < C; ++k) {
      for (int64_t r = 0; r < full; ++r)
        if (r * C + k < U) add_piece(ch.pieces, r * C + k, 0, K);
      if (!sk.off.empty())
        for (int64_t i = sk.off[k]; i < sk.off[k + 1]; ++i) {
          const Piece& pc = sk.pieces[i];
          add_piece(ch.pieces, full * C + pc.w, pc.a, pc.e);
        }
      ch.off[k + 1] = (int64_t)ch.pieces.size();
    }
  } else {
    ch = split_chunks(work, C, BK, o.unit_cost);
  }
  std::vector<int64_t> nsplit(U, 0);
  const std::vector<Item> items = unit_items(ch, nsplit);
  // the header words of a plan, with the MoE meanings
  cc_problem p{};
  p.mode = CC_MODE_MOE;
  p.batch = (int32_t)E;
  p.q_tokens = 1;
  p.num_q_heads = 1;
  p.num_kv_heads = 1;
  p.head_dim_qk = (int32_t)K;
  p.head_dim_v = (int32_t)N;
  p.page_size = (int32_t)BN;
  p.max_pages_per_seq = 1;
  p.num_pages = 1;
  const int64_t N_tiles = U * (K / BK);
  int rc = serialise(p, o, expert_tokens, C, U, N_tiles, BM, ch.off, items, nsplit, desc, out);
  if (rc) return rc;
  if (!out->size_only) out->words[H_PREFIX] = 0;  // the trailing table holds tile descriptors, not prefix units
  return CC_OK;
}

int check_args(const cc_problem* prob, const cc_plan_opts* opts, const int32_t* seqlens) {
  if (!prob || !opts || !seqlens) {
    set_error("null argument");
    return CC_ERR_INVALID;
  }
  return CC_OK;
}

}  // namespace

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
}

const char* last_error() { return g_err.c_str(); }

int parse_plan(const void* blob, PlanView* v) {
  if (!blob || !v) {
    set_error("null plan");
    return CC_ERR_PLAN;
  }
  const int32_t* h = static_cast<const int32_t*>(blob);
  if (h[H_MAGIC] != kPlanMagic || h[H_VERSION] != kPlanVersion) {
    set_error("not a plan blob (magic %08x, version %d)", (unsigned)h[H_MAGIC], h[H_VERSION]);
    return CC_ERR_PLAN;
  }
  const int64_t C = h[H_WORKERS], W = h[H_ITEMS], U = h[H_UNITS], S = h[H_PARTIALS];
  const int64_t T = h[H_TILE], hpu = h[H_HPU];
  if (C < 1 || W < 0 || U < 1 || S < 0 || T < 1 || hpu < 1 || h[H_BATCH] < 1 || h[H_QTOKENS] < 1 ||
      h[H_PAGE] < 1 || h[H_MAXPAGES] < 1) {
    set_error("corrupt plan header");
    return CC_ERR_PLAN;
  }
  v->header = h;
  v->off_wg = kHeaderWords;
  v->off_items = v->off_wg + wg_words(C);
  v->off_nsplit = v->off_items + kItemWords * W;
  v->off_pbase = v->off_nsplit + U;
  v->wg_off = h + v->off_wg;
  v->items = h + v->off_items;
  v->unit_nsplit = h + v->off_nsplit;
  v->unit_pbase = h + v->off_pbase;
  const int64_t P = h[H_PREFIX];
  const bool moe = h[H_MODE] == CC_MODE_MOE;
  if (P < 0 || (P > 0 && (h[H_MODE] != CC_MODE_GQA || hpu < 1 || kPrefixRows % hpu))) {
    set_error("corrupt plan header (prefix units)");
    return CC_ERR_PLAN;
  }
  v->off_prefix = v->off_pbase + U;
  v->prefix = h + v->off_prefix;
  v->off_moe = v->off_prefix;
  v->moe_desc = moe ? h + v->off_moe : nullptr;
  v->bytes = (v->off_prefix + kPrefixWords * P + (moe ? kMoeDescWords * U : 0)) * sizeof(int32_t);
  if (v->wg_off[0] != 0 || v->wg_off[C] != W) {
    set_error("corrupt plan offsets");
    return CC_ERR_PLAN;
  }
  for (int64_t w = 0; w < C; ++w) {
    if (v->wg_off[w + 1] < v->wg_off[w]) {
      set_error("plan worker offsets descend at worker %lld", (long long)w);
      return CC_ERR_PLAN;
    }
  }
  // partial slots: consecutive blocks for split units, -1 for the others
  int64_t slots = 0, maxsplit = 0, empty = 0;
  for (int64_t u = 0; u < U; ++u) {
    const int64_t ns = v->unit_nsplit[u], pb = v->unit_pbase[u];
    if (ns < 0 || (ns > 1 ? pb != slots : pb != -1)) {
      set_error("plan unit %lld: %lld pieces, partial base %lld", (long long)u, (long long)ns, (long long)pb);
      return CC_ERR_PLAN;
    }
    if (ns > 1) slots += ns;
    if (ns > maxsplit) maxsplit = ns;
    empty += ns == 0;
  }
  if (slots != S || maxsplit != h[H_MAXSPLIT] || empty != h[H_EMPTY]) {
    set_error("plan unit table disagrees with its header");
    return CC_ERR_PLAN;
  }
  // prefix table: KV head, 1 .. 16 / hpu members (sequences), a prefix of
  // whole pages, at least one piece; every member's unit counts the pieces
  const int64_t B = h[H_BATCH], Hkv = h[H_HKV];
  for (int64_t pu = 0; pu < P; ++pu) {
    const int32_t* r = v->prefix + kPrefixWords * pu;
    bool ok = r[0] >= 0 && r[0] < Hkv && r[1] >= 1 && r[1] <= kPrefixRows / hpu && r[2] > 0 &&
              r[2] % h[H_PAGE] == 0 && r[3] >= 1;
    for (int32_t j = 0; ok && j < kPrefixRows; ++j) {
      const int64_t b = r[4 + j];
      ok = j < r[1] ? (b >= 0 && b < B && v->unit_nsplit[b * Hkv + r[0]] >= r[3]) : b == -1;
    }
    if (!ok) {
      set_error("plan prefix unit %lld is malformed", (long long)pu);
      return CC_ERR_PLAN;
    }
  }
  // items: unit in range, a non-empty tile-aligned token range inside the
  // unit's key set, a split index below the unit's piece count
  // MoE output tiles: expert in range, rows 1 .. rows per tile, whole column blocks
  for (int64_t u = 0; moe && u < U; ++u) {
    const int32_t* d = v->moe_desc + kMoeDescWords * u;
    if (d[0] < 0 || d[0] >= h[H_BATCH] || d[1] < 0 || d[2] < 1 || d[2] > hpu || d[3] < 0 ||
        d[3] % h[H_PAGE] || d[3] + h[H_PAGE] > h[H_DV]) {
      set_error("plan MoE tile %lld is malformed", (long long)u);
      return CC_ERR_PLAN;
    }
  }
  const bool sparse = h[H_MODE] == CC_MODE_MLA_SPARSE;
  const int64_t tmax = moe ? (int64_t)h[H_DQK] : sparse ? (int64_t)h[H_TOPK] : (int64_t)h[H_MAXPAGES] * h[H_PAGE];
  for (int64_t i = 0; i < W; ++i) {
    const int32_t* it = v->items + kItemWords * i;
    const int64_t u = it[0], tb = it[1], te = it[2], s = it[3];
    const bool pre = u >= U && u < U + P;
    const int64_t end = pre ? v->prefix[kPrefixWords * (u - U) + 2] : tmax;
    const int64_t ns = pre ? v->prefix[kPrefixWords * (u - U) + 3] : (u >= 0 && u < U ? v->unit_nsplit[u] : 0);
    if (u < 0 || u >= U + P || tb < 0 || (pre ? tb % T : (tb % T && tb % h[H_PAGE])) || te <= tb || te > end ||
        s < 0 || s >= ns) {
      set_error("plan item %lld (unit %lld, tokens [%lld, %lld), split %lld) out of range", (long long)i,
                (long long)u, (long long)tb, (long long)te, (long long)s);
      return CC_ERR_PLAN;
    }
  }
  return CC_OK;
}

int32_t input_hash(const cc_problem& p, const int32_t* seqlens) {
  uint32_t h = 2166136261u;
  auto word = [&](int32_t x) {
    const uint32_t u = (uint32_t)x;
    for (int i = 0; i < 4; ++i) {
      h ^= (u >> (8 * i)) & 0xffu;
      h *= 16777619u;
    }
  };
  for (int32_t x : {p.mode, p.batch, p.q_tokens, p.num_q_heads, p.num_kv_heads, p.head_dim_qk, p.head_dim_v,
                    p.page_size, p.max_pages_per_seq, p.num_pages, p.topk})
    word(x);
  for (int32_t b = 0; b < p.batch; ++b) word(seqlens[b]);
  return (int32_t)h;
}

int plan_matches(const PlanView& v, const cc_problem& p) {
  const int32_t* h = v.header;
  if (h[H_MODE] != p.mode || h[H_BATCH] != p.batch || h[H_QTOKENS] != p.q_tokens ||
      h[H_HQ] != p.num_q_heads || h[H_HKV] != p.num_kv_heads || h[H_DQK] != p.head_dim_qk ||
      h[H_DV] != p.head_dim_v || h[H_PAGE] != p.page_size || h[H_TOPK] != p.topk ||
      h[H_MAXPAGES] != p.max_pages_per_seq || h[H_NUMPAGES] != p.num_pages) {
    set_error("plan was built for another problem shape");
    return CC_ERR_PLAN;
  }
  return CC_OK;
}

WorkspaceLayout workspace_layout(const PlanView& v, int64_t counter_units) {
  WorkspaceLayout L;
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  L.counters_off = 256;  // the error word lives at offset 0
  if (counter_units < v.units()) counter_units = v.units();
  L.partials_off = align(L.counters_off + sizeof(int32_t) * L.counter_words(counter_units));
  const size_t hpu = (size_t)v.header[H_HPU], dv = (size_t)v.header[H_DV];
  if (v.header[H_MODE] == CC_MODE_MOE) {
    // an fp32 output tile: rows per tile x columns per tile
    L.slot_floats = (hpu * (size_t)v.header[H_PAGE] + 63) & ~size_t(63);
  } else if (v.header[H_MODE] == CC_MODE_GQA) {
    // fp32 {m[hpu], l[hpu], pad to 4 floats, o[hpu][dv]}: o starts 16-byte aligned
    const size_t o_off = (2 * hpu + 3) & ~size_t(3);
    L.slot_floats = (o_off + hpu * dv + 63) & ~size_t(63);
  } else {
    // fp32 {m[hpu], l[hpu], r[hpu]}, then o[hpu][dv] as fp16 row / r (the MLA kernels)
    L.slot_floats = (3 * hpu + (hpu * dv + 1) / 2 + 63) & ~size_t(63);
  }
  L.total = align(L.partials_off + sizeof(float) * L.slot_floats * (size_t)v.partials());
  return L;
}

}  // namespace cc

extern "C" {

int cc_plan_size(const cc_problem* prob, const cc_plan_opts* opts, const int32_t* seqlens,
                 size_t* bytes) {
  int rc = cc::check_args(prob, opts, seqlens);
  if (rc) return rc;
  if (!bytes) {
    cc::set_error("null bytes");
    return CC_ERR_INVALID;
  }
  cc::Built b;
  b.size_only = true;
  rc = cc::build({prob, opts, seqlens, nullptr}, &b);
  if (rc) return rc;
  *bytes = b.total * sizeof(int32_t);
  return CC_OK;
}

int cc_plan(const cc_problem* prob, const cc_plan_opts* opts, const int32_t* seqlens,
            const int32_t* block_table, void* plan, size_t bytes) {
  int rc = cc::check_args(prob, opts, seqlens);
  if (rc) return rc;
  if (!plan) {
    cc::set_error("null plan buffer");
    return CC_ERR_INVALID;
  }
  cc::Built b;
  rc = cc::build({prob, opts, seqlens, block_table}, &b);
  if (rc) return rc;
  const size_t need = b.words.size() * sizeof(int32_t);
  if (bytes < need) {
    cc::set_error("plan buffer holds %zu bytes, needs %zu", bytes, need);
    return CC_ERR_BUFFER;
  }
  std::memcpy(plan, b.words.data(), need);
  return CC_OK;
}

int cc_plan_prefix_size(const cc_problem* prob, const cc_plan_opts* opts, const int32_t* seqlens,
                        const int32_t* prefix_group, int32_t num_groups, const int32_t* prefix_len,
                        size_t* bytes) {
  int rc = cc::check_args(prob, opts, seqlens);
  if (rc) return rc;
  if (!bytes) {
    cc::set_error("null bytes");
    return CC_ERR_INVALID;
  }
  cc::Built b;
  b.size_only = true;
  rc = cc::build_prefix({prob, opts, seqlens, nullptr}, {prefix_group, num_groups, prefix_len}, &b);
  if (rc) return rc;
  *bytes = b.total * sizeof(int32_t);
  return CC_OK;
}

int cc_plan_prefix(const cc_problem* prob, const cc_plan_opts* opts, const int32_t* seqlens,
                   const int32_t* block_table, const int32_t* prefix_group, int32_t num_groups,
                   const int32_t* prefix_len, void* plan, size_t bytes) {
  int rc = cc::check_args(prob, opts, seqlens);
  if (rc) return rc;
  if (!plan) {
    cc::set_error("null plan buffer");
    return CC_ERR_INVALID;
  }
  cc::Built b;
  rc = cc::build_prefix({prob, opts, seqlens, block_table}, {prefix_group, num_groups, prefix_len}, &b);
  if (rc) return rc;
  const size_t need = b.words.size() * sizeof(int32_t);
  if (bytes < need) {
    cc::set_error("plan buffer holds %zu bytes, needs %zu", bytes, need);
    return CC_ERR_BUFFER;
  }
  std::memcpy(plan, b.words.data(), need);
  return CC_OK;
}

int cc_moe_plan_size(const cc_moe_problem* prob, const cc_plan_opts* opts, const int32_t* expert_tokens,
                     size_t* bytes) {
  if (!prob || !opts || !expert_tokens || !bytes) {
    cc::set_error("null argument");
    return CC_ERR_INVALID;
  }
  cc::Built b;
  b.size_only = true;
  const int rc = cc::build_moe(*prob, *opts, expert_tokens, &b);
  if (rc) return rc;
  *bytes = b.total * sizeof(int32_t);
  return CC_OK;
}

int cc_moe_plan(const cc_moe_problem* prob, const cc_plan_opts* opts, const int32_t* expert_tokens, void* plan,
                size_t bytes) {
  if (!prob || !opts || !expert_tokens || !plan) {
    cc::set_error("null argument");
    return CC_ERR_INVALID;
  }
  cc::Built b;
  const int rc = cc::build_moe(*prob, *opts, expert_tokens, &b);
  if (rc) return rc;
  const size_t need = b.words.size() * sizeof(int32_t);
  if (bytes < need) {
    cc::set_error("plan buffer holds %zu bytes, needs %zu", bytes, need);
    return CC_ERR_BUFFER;
  }
  std::memcpy(plan, b.words.data(), need);
  return CC_OK;
}

int cc_plan_check(const void* plan, const cc_problem* prob, const int32_t* seqlens) {
  if (!plan || !prob || !seqlens) {
    cc::set_error("null argument");
    return CC_ERR_INVALID;
  }
  cc::PlanView v;
  int rc = cc::parse_plan(plan, &v);
  if (rc) return rc;
  rc = cc::plan_matches(v, *prob);
  if (rc) return rc;
  const int32_t want = cc::input_hash(*prob, seqlens);
  if (v.header[cc::H_HASH] != want) {
    cc::set_error("plan was built for other sequence lengths (hash %08x, these inputs %08x)",
                  (unsigned)v.header[cc::H_HASH], (unsigned)want);
    return CC_ERR_PLAN;
  }
  return CC_OK;
}

int cc_workspace_size(const void* plan_host, size_t* bytes) {
  cc::PlanView v;
  int rc = cc::parse_plan(plan_host, &v);
  if (rc) return rc;
  if (!bytes) {
    cc::set_error("null bytes");
    return CC_ERR_INVALID;
  }
  *bytes = cc::workspace_layout(v).total;
  return CC_OK;
}

}  // extern "C"
