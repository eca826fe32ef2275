// Host-side view of a work-plan blob (shared by the planner and the launcher).
//
// Blob layout, int32 little-endian words:
//   header[32]           fields below (H_*); words past H_HASH are zero
//   wg_off[C + 1]        items of worker w are items[wg_off[w] .. wg_off[w+1]),
//                        zero-padded to a multiple of 4 words so items[] is
//                        16-byte aligned
//   items[W][4]          unit, tok_begin, tok_end, split (index of the piece
//                        within its unit, in token order)
//   unit_nsplit[U]       pieces of each unit
//   unit_pbase[U]        first partial slot of a split unit, -1 if unsplit
//   prefix[P][20]        shared-prefix units (cc_plan_prefix): KV head, number
//                        of members, prefix length, number of pieces, member
//                        sequence ids (-1 padded to 16); items name prefix
//                        unit p as unit U + p
//   moe_desc[U][4]       MoE plans (mode CC_MODE_MOE, cc_moe_plan): expert,
//                        first row, rows, first column of each output tile.
//                        Their header reuses words: batch = experts, dqk =
//                        hidden K, dv = output N, tile = k per tile, hpu = rows
//                        per tile, page = columns per tile; items' token
//                        ranges are k ranges
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/crosscu.h"

namespace cc {

constexpr int32_t kPlanMagic = 0x4C504343;  // "CCPL"
constexpr int32_t kPlanVersion = 3;
constexpr int kHeaderWords = 32;
constexpr int kItemWords = 4;
constexpr int kPrefixWords = 20;
constexpr int kMoeDescWords = 4;  // a MoE unit: expert, first row, rows, first column
constexpr int kMoeTileCols = 256; // output columns of a MoE tile
constexpr int kMoeTileRows = 256; // output rows of a MoE tile (the plan's heads_per_unit)
constexpr int kPrefixRows = 16;  // query rows a prefix unit gathers (members x group size)

enum HeaderField {
  H_MAGIC = 0, H_VERSION, H_MODE, H_BATCH, H_QTOKENS, H_HQ, H_HKV, H_DQK, H_DV, H_PAGE, H_TOPK,
  H_WORKERS, H_XCDS, H_TILE, H_HPU, H_UNITS, H_TILES, H_ITEMS, H_PARTIALS, H_MAXSPLIT, H_POLICY,
  H_MAXPAGES, H_NUMPAGES,
  H_UNIT_COST,  // per-unit cost (tiles) of CC_POLICY_STREAMK, else 0
  H_EMPTY,      // units with no piece (sequences with no cached tokens)
  H_HASH,       // FNV-1a of the problem's int32 fields and seqlens (input_hash)
  H_PREFIX      // shared-prefix units (rows of the prefix table)
};

struct PlanView {
  const int32_t* header = nullptr;
  const int32_t* wg_off = nullptr;
  const int32_t* items = nullptr;
  const int32_t* unit_nsplit = nullptr;
  const int32_t* unit_pbase = nullptr;
  const int32_t* prefix = nullptr;
  const int32_t* moe_desc = nullptr;
  size_t bytes = 0;
  // word offsets of the arrays inside the blob (valid for a device copy too)
  size_t off_wg = 0, off_items = 0, off_nsplit = 0, off_pbase = 0, off_prefix = 0, off_moe = 0;

  int32_t workers() const { return header[H_WORKERS]; }
  int32_t units() const { return header[H_UNITS]; }
  int32_t num_items() const { return header[H_ITEMS]; }
  int32_t partials() const { return header[H_PARTIALS]; }
  int32_t prefix_units() const { return header[H_PREFIX]; }
};

// Parses and checks a host blob: header, worker offsets ascending, every
// item's unit, token range and split index in range, partial slots laid out
// consecutively.  Returns CC_OK or CC_ERR_PLAN (message set).
int parse_plan(const void* blob, PlanView* v);

// 32-bit FNV-1a of the little-endian bytes of (mode, batch, q_tokens,
// num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
// max_pages_per_seq, num_pages, topk, seqlens[0 .. batch)) as int32 words.
int32_t input_hash(const cc_problem& p, const int32_t* seqlens);

// Checks that a parsed plan was built for `prob`.
int plan_matches(const PlanView& v, const cc_problem& prob);

// Thread-local error text.
void set_error(const char* fmt, ...);
const char* last_error();

// Words of wg_off[] including the alignment padding.
inline int64_t wg_words(int64_t workers) { return (workers + 1 + 3) & ~int64_t(3); }

// int32 words per unit in the workspace counter area: the arrival counter,
// the merge-claim mask, then padding, so that every unit's words sit in a
// 128-byte line of their own (workgroups poll them while others stream).
constexpr int kCounterStride = 32;

// Workspace layout of a plan: error word and counters first, then partials.
struct WorkspaceLayout {
  size_t counters_off = 0;   // bytes; int32[U][kCounterStride]
  static size_t counter_words(int64_t units) { return kCounterStride * (size_t)units; }
  size_t partials_off = 0;   // bytes; S slots: GQA fp32 {m[hpu], l[hpu], pad to 4, o[hpu][dv]},
                             // MLA fp32 {m[hpu], l[hpu], r[hpu]} + fp16 o[hpu][dv]
  size_t slot_floats = 0;    // floats per partial slot
  size_t total = 0;
};
// counter_units: units the counter area is sized for (>= the plan's units; -1:
// exactly the plan's), so that a workspace shared by plans of different sizes
// can keep its counters and its partials apart.
WorkspaceLayout workspace_layout(const PlanView& v, int64_t counter_units = -1);

}  // namespace cc
