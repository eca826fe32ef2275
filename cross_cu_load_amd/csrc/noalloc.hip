// cc_decode for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The split pieces' partials, the per-unit arrival counters and the error
// word live in `scratch`, a file-scope device array of
// CC_NOALLOC_WORKSPACE_BYTES that every GPU the library runs on holds until
// the process ends, instead of a caller-provided workspace.  In host code the
// array's name is only a stand-in for the symbol: its device address (one per
// device) comes from hipGetSymbolAddress on the first call on that device and
// is the only thing passed to kernels.  That first call also enqueues one
// clear of the whole array on its stream.  The array's layout does not depend
// on the plan: the error word, then arrival counters for up to
// CC_NOALLOC_MAX_UNITS units, then the partial slots.  The decode kernels
// leave every counter they use at zero, and no plan's partials ever land on
// a counter, so a call finds all counters zero whatever plans ran before it.
// All calls on one device share the array: calls that may overlap (different
// streams without ordering) race.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "../../include/crosscu.h"
#include "launch.h"
#include "plan.h"

static __device__ __align__(256) char scratch[CC_NOALLOC_WORKSPACE_BYTES];

namespace cc {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once set up

// The scratch array's address on the current device (set up on first use).
int scratch_of_current_device(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("hipGetDevice: %s", hipGetErrorString(e));
    return CC_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device %d outside the %d devices cc_decode_noalloc keeps a scratch address for", dev,
              kMaxDevices);
    return CC_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return CC_ERR_HIP;
    }
    e = launch_fill_zero(p, CC_NOALLOC_WORKSPACE_BYTES, s);
    if (e != hipSuccess) {
      set_error("scratch clear on device %d: %s", dev, hipGetErrorString(e));
      return CC_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CC_OK;
}

}  // namespace
}  // namespace cc

extern "C" int cc_decode_noalloc(const cc_problem* prob, const void* plan_host, const void* plan_dev,
                                 const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seqlens, const int32_t* indices,
                                 float* out, float* lse, void* stream) {
  // the size check needs only the host plan: refuse before touching a device
  cc::PlanView v;
  int rc = cc::parse_plan(plan_host, &v);
  if (rc) return rc;
  if (v.units() > CC_NOALLOC_MAX_UNITS) {
    cc::set_error("the plan has %d units; cc_decode_noalloc's scratch array counts arrivals for %d "
                  "(use cc_decode with a workspace)", v.units(), CC_NOALLOC_MAX_UNITS);
    return CC_ERR_BUFFER;
  }
  const size_t need = cc::workspace_layout(v, CC_NOALLOC_MAX_UNITS).total;
  if (need > (size_t)CC_NOALLOC_WORKSPACE_BYTES) {
    cc::set_error("the plan needs %zu bytes of workspace; cc_decode_noalloc's scratch array holds %zu "
                  "(use cc_decode with a workspace)", need, (size_t)CC_NOALLOC_WORKSPACE_BYTES);
    return CC_ERR_BUFFER;
  }
  void* ws = nullptr;
  rc = cc::scratch_of_current_device(static_cast<hipStream_t>(stream), &ws);
  if (rc) return rc;
  return cc::decode_checked(CC_REDUCE_FUSED, prob, plan_host, plan_dev, q, k_cache, v_cache, block_table, seqlens,
                            indices, out, lse, ws, CC_NOALLOC_WORKSPACE_BYTES, stream, CC_NOALLOC_MAX_UNITS);
}
