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
// rows are u * rows .. u * rows + rows - 1 of the flattened [B][Tq][Hq].
__global__ void empty_units_kernel(const int32_t* __restrict__ unit_nsplit, int rows, int dv, float* out,
                                   float* lse) {
  const int u = blockIdx.x;
  if (unit_nsplit[u] != 0) return;
  const size_t r0 = (size_t)u * rows;
  for (int i = threadIdx.x; i < rows * dv; i += blockDim.x) out[r0 * dv + i] = 0.f;
  for (int i = threadIdx.x; i < rows; i += blockDim.x) lse[r0 + i] = -INFINITY;
}

}  // namespace fill

hipError_t launch_empty_units(const DecodeArgs& a, hipStream_t s) {
  hipExtLaunchKernelGGL(fill::empty_units_kernel, dim3(a.units), dim3(256), 0u, s, a.ev_start, a.ev_stop, 0u,
                        a.unit_nsplit, a.hpu, a.dv, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace cc
