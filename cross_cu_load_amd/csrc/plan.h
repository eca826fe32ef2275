// Host-side view of a work-plan blob (shared by the planner and the launcher).
//
// Blob layout, int32 little-endian words:
//   header[32]           fields below (H_*); words past H_EMPTY are zero
//   wg_off[C + 1]        items of worker w are items[wg_off[w] .. wg_off[w+1]),
//                        zero-padded to a multiple of 4 words so items[] is
//                        16-byte aligned
//   items[W][4]          unit, tok_begin, tok_end, split (index of the piece
//                        within its unit, in token order)
//   unit_nsplit[U]       pieces of each unit
//   unit_pbase[U]        first partial slot of a split unit, -1 if unsplit
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/crosscu.h"

namespace cc {

constexpr int32_t kPlanMagic = 0x4C504343;  // "CCPL"
constexpr int32_t kPlanVersion = 2;
constexpr int kHeaderWords = 32;
constexpr int kItemWords = 4;

enum HeaderField {
  H_MAGIC = 0, H_VERSION, H_MODE, H_BATCH, H_QTOKENS, H_HQ, H_HKV, H_DQK, H_DV, H_PAGE, H_TOPK,
  H_WORKERS, H_XCDS, H_TILE, H_HPU, H_UNITS, H_TILES, H_ITEMS, H_PARTIALS, H_MAXSPLIT, H_POLICY,
  H_MAXPAGES, H_NUMPAGES,
  H_UNIT_COST,  // per-unit cost of CC_POLICY_STREAMK_COST, else 0
  H_EMPTY       // units with no piece (sequences with no cached tokens)
};

struct PlanView {
  const int32_t* header = nullptr;
  const int32_t* wg_off = nullptr;
  const int32_t* items = nullptr;
  const int32_t* unit_nsplit = nullptr;
  const int32_t* unit_pbase = nullptr;
  size_t bytes = 0;
  // word offsets of the arrays inside the blob (valid for a device copy too)
  size_t off_wg = 0, off_items = 0, off_nsplit = 0, off_pbase = 0;

  int32_t workers() const { return header[H_WORKERS]; }
  int32_t units() const { return header[H_UNITS]; }
  int32_t num_items() const { return header[H_ITEMS]; }
  int32_t partials() const { return header[H_PARTIALS]; }
};

// Parses and checks a host blob; returns CC_OK or CC_ERR_PLAN (message set).
int parse_plan(const void* blob, PlanView* v);

// Checks that a parsed plan was built for `prob`.
int plan_matches(const PlanView& v, const cc_problem& prob);

// Thread-local error text.
void set_error(const char* fmt, ...);
const char* last_error();

// Words of wg_off[] including the alignment padding.
inline int64_t wg_words(int64_t workers) { return (workers + 1 + 3) & ~int64_t(3); }

// Cost model of CC_POLICY_STREAMK_COST: one tile costs kCostPerTile, and each
// unit adds unit_cost(mode) (the plan header's last word records it).  A GQA
// unit's start and finish cost about one tile; an MLA unit's (the 128-head
// partial written and published, the next query token's q loaded) about six.
constexpr int64_t kCostPerTile = 16;
constexpr int64_t kUnitCostGqa = 16;
constexpr int64_t kUnitCostMla = 96;
inline int64_t unit_cost(int mode) { return mode == CC_MODE_GQA ? kUnitCostGqa : kUnitCostMla; }

// int32 words per unit in the workspace counter area: the arrival counter,
// the merge-claim mask, then padding, so that every unit's words sit in a
// 128-byte line of their own (workgroups poll them while others stream).
constexpr int kCounterStride = 32;

// Workspace layout of a plan: error word and counters first, then partials.
struct WorkspaceLayout {
  size_t counters_off = 0;   // bytes; int32[U][kCounterStride]
  static size_t counter_words(const PlanView& v) { return kCounterStride * (size_t)v.units(); }
  size_t partials_off = 0;   // bytes; S slots {m[hpu], l[hpu], pad to 4, o[hpu][dv]}
  size_t slot_floats = 0;    // floats per partial slot
  size_t total = 0;
};
WorkspaceLayout workspace_layout(const PlanView& v);

}  // namespace cc
