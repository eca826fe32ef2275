// C ABI of the decode library: argument checks, plan/problem consistency,
// workspace carving and kernel launches.  Everything here runs on the host
// and touches device memory only through enqueued kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/crosscu.h"
#include "../../include/crosscu_debug.h"
#include "fill.h"
#include "launch.h"
#include "plan.h"

namespace {

// debug timeline buffer (process-wide; set by cc_debug_timeline)
void* g_timeline = nullptr;
size_t g_timeline_bytes = 0;
// debug kernel events (process-wide; set by cc_debug_kernel_events)
hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int hip_fail(hipError_t e, const char* what) {
  cc::set_error("%s: %s", what, hipGetErrorString(e));
  return CC_ERR_HIP;
}

// Shapes the GQA kernel implements.
int check_gqa(const cc_problem& p, const cc::PlanView& v) {
  const int G = p.num_q_heads / p.num_kv_heads;
  if (p.head_dim_qk != p.head_dim_v || (p.head_dim_qk != 64 && p.head_dim_qk != 128)) {
    cc::set_error("GQA kernel: head_dim_qk == head_dim_v in {64, 128} (got %d, %d)",
                  p.head_dim_qk, p.head_dim_v);
    return CC_ERR_UNSUPPORTED;
  }
  if (G > 16) {
    cc::set_error("GQA kernel: group size %d > 16", G);
    return CC_ERR_UNSUPPORTED;
  }
  if (v.header[cc::H_HPU] != G) {
    cc::set_error("GQA kernel: heads_per_unit must equal the group size %d", G);
    return CC_ERR_UNSUPPORTED;
  }
  if (!is_pow2(p.page_size) || p.page_size < 16) {
    cc::set_error("GQA kernel: page_size must be a power of two >= 16 (got %d)", p.page_size);
    return CC_ERR_UNSUPPORTED;
  }
  if (v.header[cc::H_TILE] % 32) {
    cc::set_error("GQA kernel: tile_tokens must be a multiple of 32 (got %d)", v.header[cc::H_TILE]);
    return CC_ERR_UNSUPPORTED;
  }
  return CC_OK;
}

// Shapes the MLA kernels implement (dense and index-sparse).
int check_mla(const cc_problem& p, const cc::PlanView& v) {
  if (p.num_kv_heads != 1 || p.num_q_heads != 128 || p.head_dim_qk != 576 || p.head_dim_v != 512) {
    cc::set_error("MLA kernel: 128 query heads over one 576-wide latent head with dv 512 "
                  "(got Hq %d, Hkv %d, dk %d, dv %d)", p.num_q_heads, p.num_kv_heads, p.head_dim_qk,
                  p.head_dim_v);
    return CC_ERR_UNSUPPORTED;
  }
  if (v.header[cc::H_HPU] != 128) {
    cc::set_error("MLA kernel: heads_per_unit must be 128 (one unit per query token)");
    return CC_ERR_UNSUPPORTED;
  }
  if (!is_pow2(p.page_size) || (p.mode == CC_MODE_MLA && p.page_size < 32)) {
    cc::set_error("MLA kernel: page_size must be a power of two (>= 32 for dense MLA), got %d", p.page_size);
    return CC_ERR_UNSUPPORTED;
  }
  if (v.header[cc::H_TILE] % 32) {
    cc::set_error("MLA kernel: tile_tokens must be a multiple of 32 (got %d)", v.header[cc::H_TILE]);
    return CC_ERR_UNSUPPORTED;
  }
  // a workgroup packs each split piece it publishes (unit, split index) into one word
  if (v.units() >= (1 << 20) || v.header[cc::H_MAXSPLIT] > 512) {
    cc::set_error("MLA kernel: at most 2^20 - 1 units and 512 splits per unit (got %d units, %d splits)",
                  v.units(), v.header[cc::H_MAXSPLIT]);
    return CC_ERR_UNSUPPORTED;
  }
  return CC_OK;
}

int decode_impl(int reduce, const cc_problem* prob, const void* plan_host, const void* plan_dev,
                const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                const int32_t* seqlens, const int32_t* indices, float* out, float* lse,
                void* workspace, size_t workspace_bytes, void* stream, int64_t counter_units = -1) {
  if (!prob || !plan_host || !plan_dev || !q || !k_cache || !block_table || !seqlens || !out ||
      !lse || !workspace) {
    cc::set_error("null argument");
    return CC_ERR_INVALID;
  }
  // the kernels move q, K, V, out and partials in 16-byte accesses
  auto misaligned = [](const void* ptr) { return ptr && (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; };
  if (misaligned(q) || misaligned(k_cache) || misaligned(v_cache) || misaligned(out) || misaligned(workspace)) {
    cc::set_error("q, k_cache, v_cache, out and workspace must be 16-byte aligned");
    return CC_ERR_INVALID;
  }
  if (reduce != CC_REDUCE_FUSED && reduce != CC_REDUCE_SPLIT_COMBINE) {
    cc::set_error("unknown reduction %d", reduce);
    return CC_ERR_INVALID;
  }
  cc::PlanView v;
  int rc = cc::parse_plan(plan_host, &v);
  if (rc) return rc;
  rc = cc::plan_matches(v, *prob);
  if (rc) return rc;
  const cc::WorkspaceLayout wl = cc::workspace_layout(v, counter_units);
  if (workspace_bytes < wl.total) {
    cc::set_error("workspace holds %zu bytes, the plan needs %zu", workspace_bytes, wl.total);
    return CC_ERR_BUFFER;
  }
  if (prob->kv_layout != CC_KV_NHD && prob->kv_layout != CC_KV_HND) {
    cc::set_error("unknown kv_layout %d", prob->kv_layout);
    return CC_ERR_INVALID;
  }
  if (!(prob->softmax_scale > 0.f) || !std::isfinite(prob->softmax_scale)) {
    cc::set_error("softmax_scale must be finite and > 0");
    return CC_ERR_INVALID;
  }
  const cc_problem& p = *prob;
  if (p.mode == CC_MODE_GQA) {
    if (!v_cache) {
      cc::set_error("GQA needs a V cache");
      return CC_ERR_INVALID;
    }
    rc = check_gqa(p, v);
    if (rc) return rc;
  } else {
    if (p.mode == CC_MODE_MLA_SPARSE && !indices) {
      cc::set_error("index-sparse MLA needs indices");
      return CC_ERR_INVALID;
    }
    rc = check_mla(p, v);
    if (rc) return rc;
  }

  const int32_t* pd = static_cast<const int32_t*>(plan_dev);
  char* ws = static_cast<char*>(workspace);
  cc::DecodeArgs a{};
  a.mode = p.mode;
  a.batch = p.batch;
  a.q_tokens = p.q_tokens;
  a.hq = p.num_q_heads;
  a.hkv = p.num_kv_heads;
  a.dqk = p.head_dim_qk;
  a.dv = p.head_dim_v;
  a.page_size = p.page_size;
  a.max_pages = p.max_pages_per_seq;
  a.num_pages = p.num_pages;
  a.topk = p.topk;
  a.kv_layout = p.kv_layout;
  a.scale_log2 = (float)((double)p.softmax_scale * 1.4426950408889634);
  a.workers = v.workers();
  a.units = v.units();
  a.hpu = v.header[cc::H_HPU];
  a.tile = v.header[cc::H_TILE];
  a.wg_off = pd + v.off_wg;
  a.items = reinterpret_cast<const int4*>(pd + v.off_items);
  a.unit_nsplit = pd + v.off_nsplit;
  a.unit_pbase = pd + v.off_pbase;
  a.prefix = pd + v.off_prefix;
  a.prefix_units = v.prefix_units();
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.block_table = block_table;
  a.seqlens = seqlens;
  a.indices = indices;
  a.out = out;
  a.lse = lse;
  a.err = reinterpret_cast<int32_t*>(ws);
  a.counters = reinterpret_cast<int32_t*>(ws + wl.counters_off);
  a.partials = reinterpret_cast<float*>(ws + wl.partials_off);
  a.slot_floats = (int)wl.slot_floats;
  a.reduce = reduce;
  a.timeline = (g_timeline && g_timeline_bytes >= (size_t)v.workers() * 8 * cc::kTimelineWords)
                   ? static_cast<unsigned long long*>(g_timeline)
                   : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool combine = reduce == CC_REDUCE_SPLIT_COMBINE && v.partials() > 0;
  const bool has_empty = v.header[cc::H_EMPTY] > 0;  // sequences with no cached tokens
  a.ev_start = g_ev_start;
  hipError_t e;
  if (has_empty) {
    a.ev_stop = nullptr;
    e = cc::launch_empty_units(a, s);
    if (e != hipSuccess) return hip_fail(e, "empty-unit launch");
    a.ev_start = nullptr;
  }
  a.ev_stop = combine ? nullptr : g_ev_stop;
  e = p.mode == CC_MODE_GQA ? cc::launch_gqa(a, s) : cc::launch_mla(a, s);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (combine) {
    a.ev_start = nullptr;
    a.ev_stop = g_ev_stop;
    e = cc::launch_combine(a, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return CC_OK;
}

}  // namespace

namespace cc {
int decode_checked(int reduce, const cc_problem* prob, const void* plan_host, const void* plan_dev, const void* q,
                   const void* k_cache, const void* v_cache, const int32_t* block_table, const int32_t* seqlens,
                   const int32_t* indices, float* out, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream, int64_t counter_units) {
  return decode_impl(reduce, prob, plan_host, plan_dev, q, k_cache, v_cache, block_table, seqlens, indices, out,
                     lse, workspace, workspace_bytes, stream, counter_units);
}

void kernel_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = g_ev_start;
  *stop = g_ev_stop;
}
}  // namespace cc

extern "C" {

int cc_version(void) { return 100; }

int cc_debug_timeline(void* buf, size_t bytes) {
  g_timeline = buf;
  g_timeline_bytes = buf ? bytes : 0;
  return CC_OK;
}

int cc_debug_kernel_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) {
    cc::set_error("cc_debug_kernel_events: give both events or neither");
    return CC_ERR_INVALID;
  }
  g_ev_start = static_cast<hipEvent_t>(start_event);
  g_ev_stop = static_cast<hipEvent_t>(stop_event);
  return CC_OK;
}

int cc_debug_merge_poll_limit(int polls) {
  const hipError_t e = cc::set_mla_merge_poll_limit(polls);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyToSymbol(merge poll limit)");
  return CC_OK;
}

const char* cc_last_error(void) { return cc::last_error(); }

const char* cc_strerror(int code) {
  switch (code) {
    case CC_OK: return "ok";
    case CC_ERR_INVALID: return "invalid argument";
    case CC_ERR_UNSUPPORTED: return "unsupported problem";
    case CC_ERR_BUFFER: return "buffer too small";
    case CC_ERR_PLAN: return "plan malformed or built for another problem";
    case CC_ERR_PAGE: return "page id outside the cache";
    case CC_ERR_HIP: return "HIP runtime error";
    case CC_ERR_DEVICE_DATA: return "device reported bad data";
    default: return "unknown error code";
  }
}

int cc_device_query(int device, int32_t* num_cus, int32_t* num_xcds) {
  if (!num_cus || !num_xcds) {
    cc::set_error("null argument");
    return CC_ERR_INVALID;
  }
  int v = 0;
  hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiProcessorCount)");
  *num_cus = v;
  int x = 1;
  e = hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, device);
  if (e != hipSuccess || x < 1) x = 1;
  *num_xcds = x;
  return CC_OK;
}

int cc_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace || bytes % 4) {
    cc::set_error("workspace must be non-null and a multiple of 4 bytes");
    return CC_ERR_INVALID;
  }
  hipError_t e = cc::launch_fill_zero(workspace, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "workspace fill");
  return CC_OK;
}

int cc_workspace_check(const void* plan_host, const void* workspace, void* stream,
                       int32_t* dirty_counters, int32_t* device_flags) {
  if (!workspace || !dirty_counters || !device_flags) {
    cc::set_error("null argument");
    return CC_ERR_INVALID;
  }
  cc::PlanView v;
  int rc = cc::parse_plan(plan_host, &v);
  if (rc) return rc;
  const cc::WorkspaceLayout wl = cc::workspace_layout(v);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  std::vector<int32_t> cnt(cc::WorkspaceLayout::counter_words(v.units()));
  int32_t flags = 0;
  const char* ws = static_cast<const char*>(workspace);
  e = hipMemcpy(&flags, ws, sizeof flags, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(error word)");
  e = hipMemcpy(cnt.data(), ws + wl.counters_off, cnt.size() * sizeof(int32_t),
                hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(counters)");
  int32_t dirty = 0;
  for (int32_t c : cnt) dirty += c != 0;
  *dirty_counters = dirty;
  *device_flags = flags;
  if (dirty || flags) {
    cc::set_error("workspace: %d non-zero counters, device flags 0x%x", dirty, flags);
    return CC_ERR_DEVICE_DATA;
  }
  return CC_OK;
}

int cc_decode(const cc_problem* prob, const void* plan_host, const void* plan_dev, const void* q,
              const void* k_cache, const void* v_cache, const int32_t* block_table,
              const int32_t* seqlens, const int32_t* indices, float* out, float* lse,
              void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(CC_REDUCE_FUSED, prob, plan_host, plan_dev, q, k_cache, v_cache, block_table,
                     seqlens, indices, out, lse, workspace, workspace_bytes, stream);
}

int cc_moe_gemm_variant(int reduce, const cc_moe_problem* prob, const void* plan_host, const void* plan_dev,
                        const void* x, const void* w, float* y, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!prob || !plan_host || !plan_dev || !x || !w || !y || !workspace) {
    cc::set_error("null argument");
    return CC_ERR_INVALID;
  }
  if (reduce != CC_REDUCE_FUSED && reduce != CC_REDUCE_SPLIT_COMBINE) {
    cc::set_error("unknown reduction %d", reduce);
    return CC_ERR_INVALID;
  }
  cc::PlanView v;
  int rc = cc::parse_plan(plan_host, &v);
  if (rc) return rc;
  const int32_t* h = v.header;
  if (h[cc::H_MODE] != CC_MODE_MOE || h[cc::H_BATCH] != prob->num_experts || h[cc::H_DQK] != prob->hidden ||
      h[cc::H_DV] != prob->out_dim) {
    cc::set_error("plan was not built for this MoE problem");
    return CC_ERR_PLAN;
  }
  if (h[cc::H_HPU] != cc::kMoeTileRows || h[cc::H_TILE] != 64 || prob->hidden % 64 || prob->out_dim % cc::kMoeTileCols) {
    cc::set_error("MoE kernel: %d-row tiles (heads_per_unit), 64-wide k tiles (tile_tokens), hidden %% 64 == 0, "
                  "out_dim %% %d == 0", cc::kMoeTileRows, cc::kMoeTileCols);
    return CC_ERR_UNSUPPORTED;
  }
  if ((int64_t)prob->hidden * (std::max(cc::kMoeTileRows, cc::kMoeTileCols) - 1) * 2 + 1024 > INT32_MAX || (int64_t)v.units() >= (1 << 21)) {
    cc::set_error("MoE kernel: hidden too large for 32-bit row offsets or too many tiles");
    return CC_ERR_UNSUPPORTED;
  }
  const cc::WorkspaceLayout wl = cc::workspace_layout(v);
  if (workspace_bytes < wl.total) {
    cc::set_error("workspace holds %zu bytes, the plan needs %zu", workspace_bytes, wl.total);
    return CC_ERR_BUFFER;
  }
  const int32_t* pd = static_cast<const int32_t*>(plan_dev);
  char* ws = static_cast<char*>(workspace);
  cc::MoeArgs a{};
  a.K = prob->hidden;
  a.N = prob->out_dim;
  a.workers = v.workers();
  a.units = v.units();
  a.slot_floats = (int)wl.slot_floats;
  a.reduce = reduce;
  a.partials_count = v.partials();
  a.wg_off = pd + v.off_wg;
  a.items = reinterpret_cast<const int4*>(pd + v.off_items);
  a.unit_nsplit = pd + v.off_nsplit;
  a.unit_pbase = pd + v.off_pbase;
  a.desc = pd + v.off_moe;
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = y;
  a.counters = reinterpret_cast<int32_t*>(ws + wl.counters_off);
  a.partials = reinterpret_cast<float*>(ws + wl.partials_off);
  a.timeline = (g_timeline && g_timeline_bytes >= (size_t)v.workers() * 8 * cc::kTimelineWords)
                   ? static_cast<unsigned long long*>(g_timeline)
                   : nullptr;
  a.ev_start = g_ev_start;
  a.ev_stop = g_ev_stop;
  const hipError_t e = cc::launch_moe(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "MoE launch");
  return CC_OK;
}

int cc_moe_gemm(const cc_moe_problem* prob, const void* plan_host, const void* plan_dev, const void* x,
                const void* w, float* y, void* workspace, size_t workspace_bytes, void* stream) {
  return cc_moe_gemm_variant(CC_REDUCE_FUSED, prob, plan_host, plan_dev, x, w, y, workspace, workspace_bytes,
                             stream);
}

int cc_decode_variant(int reduce, const cc_problem* prob, const void* plan_host,
                      const void* plan_dev, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table, const int32_t* seqlens,
                      const int32_t* indices, float* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return decode_impl(reduce, prob, plan_host, plan_dev, q, k_cache, v_cache, block_table, seqlens,
                     indices, out, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"
