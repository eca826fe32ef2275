// Output of the units a plan gives no piece: sequences with no cached tokens.
//
// Softmax attention over an empty key set has lse = log of an empty sum =
// -inf; out is set to 0, which with lse = -inf is the neutral element of the
// log-sum-exp merge of partial results (MeldKernel summary, "Core method":
// partial outputs feed a just-in-time reduction), so such a sequence merged
// with any other key range leaves that range's result unchanged.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cmath>
#include <cstdint>

#include "fill.h"

namespace cc {
namespace fill {

// One workgroup per unit; units with pieces return at once.  Unit u's query
// rows are u * rows .. u * rows + rows - 1 of the flattened [B][Tq][Hq]; it
// belongs to sequence u / units_per_seq.  A unit the plan left empty whose
// sequence does have cached tokens (a plan built for other lengths) is
// flagged in the error word and gets NaN.
__global__ void empty_units_kernel(const int32_t* __restrict__ unit_nsplit, const int32_t* __restrict__ seqlens,
                                   int units_per_seq, int rows, int dv, float* out, float* lse, int32_t* err) {
  const int u = blockIdx.x;
  if (unit_nsplit[u] != 0) return;
  const bool stale = seqlens[u / units_per_seq] != 0;
  if (stale && threadIdx.x == 0) atomicOr(err, kErrSeqlen);
  const float o = stale ? __builtin_nanf("") : 0.f, l = stale ? __builtin_nanf("") : -INFINITY;
  const size_t r0 = (size_t)u * rows;
  for (int i = threadIdx.x; i < rows * dv; i += blockDim.x) out[r0 * dv + i] = o;
  for (int i = threadIdx.x; i < rows; i += blockDim.x) lse[r0 + i] = l;
}

}  // namespace fill

hipError_t launch_empty_units(const DecodeArgs& a, hipStream_t s) {
  const int units_per_seq = a.q_tokens * (a.hq / a.hpu);
  hipExtLaunchKernelGGL(fill::empty_units_kernel, dim3(a.units), dim3(256), 0u, s, a.ev_start, a.ev_stop, 0u,
                        a.unit_nsplit, a.seqlens, units_per_seq, a.hpu, a.dv, a.out, a.lse, a.err);
  return hipGetLastError();
}

}  // namespace cc
