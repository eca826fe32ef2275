// Kernel launch interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/crosscu.h"

namespace cc {

// Everything a decode launch needs, resolved on the host from the problem,
// the plan header and the workspace layout.
struct DecodeArgs {
  // problem
  int mode, batch, q_tokens, hq, hkv, dqk, dv, page_size, max_pages, num_pages, topk, kv_layout;
  float scale_log2;  // softmax_scale * log2(e): scores are kept in base 2
  // plan (device pointers into the plan copy)
  int workers, units, hpu, tile;
  const int32_t* wg_off;
  const int4* items;  // unit, tok_begin, tok_end, split
  const int32_t* unit_nsplit;
  const int32_t* unit_pbase;
  const int32_t* prefix;  // shared-prefix table rows (prefix_units of them)
  int prefix_units;
  // tensors (device)
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* indices;
  float* out;
  float* lse;
  // workspace (device)
  int32_t* err;
  int32_t* counters;
  float* partials;
  int slot_floats;
  int reduce;  // CC_REDUCE_*
  // optional in-kernel timeline (kTimelineWords x uint64 per workgroup), null when off
  unsigned long long* timeline;
  // optional events recorded at the start of the call's first kernel and the
  // end of its last (hipExtLaunchKernel), null when off
  hipEvent_t ev_start;
  hipEvent_t ev_stop;
};

// Everything a MoE grouped GEMM launch needs.
struct MoeArgs {
  int K, N, workers, units, slot_floats, reduce, partials_count;
  const int32_t* wg_off;
  const int4* items;  // unit, k_begin, k_end, split
  const int32_t* unit_nsplit;
  const int32_t* unit_pbase;
  const int32_t* desc;  // per unit: expert, first row, rows, first column
  const uint16_t* x;
  const uint16_t* w;
  float* y;
  int32_t* counters;
  float* partials;
  unsigned long long* timeline;
  hipEvent_t ev_start;
  hipEvent_t ev_stop;
};
hipError_t launch_moe(const MoeArgs& a, hipStream_t s);

// The debug kernel events set by cc_debug_kernel_events (null when off).
void kernel_events(hipEvent_t* start, hipEvent_t* stop);

// cc_decode_variant's checks and launches on a given workspace whose counter
// area is sized for counter_units units (-1: the plan's own count).  The
// no-allocation entry point passes its scratch array and a fixed capacity.
int decode_checked(int reduce, const cc_problem* prob, const void* plan_host, const void* plan_dev, const void* q,
                   const void* k_cache, const void* v_cache, const int32_t* block_table, const int32_t* seqlens,
                   const int32_t* indices, float* out, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream, int64_t counter_units);

// uint64 words per workgroup in the debug timeline
constexpr int kTimelineWords = 8;

// Device error-word bits.
constexpr int kErrSeqlen = 1;
constexpr int kErrPage = 2;
constexpr int kErrIndex = 4;

hipError_t launch_gqa(const DecodeArgs& a, hipStream_t s);
hipError_t launch_mla(const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine(const DecodeArgs& a, hipStream_t s);
hipError_t launch_mla_combine(const DecodeArgs& a, hipStream_t s);
// Sets the MLA kernel's merge poll limit on the current device (< 0: the default).
hipError_t set_mla_merge_poll_limit(int polls);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace cc
