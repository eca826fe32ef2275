// Streaming-read probe: the HBM read bandwidth a persistent grid reaches on
// this device with each of the load paths the decode kernels can use.  It is
// the practical ceiling the decode's KV GB/s is quoted against.
//
// Every workgroup reads one contiguous share of the buffer (or, with a page
// list, whole pages in the listed order, as a paged KV cache is read) and
// folds the data into one word per thread so no load is dead.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>

#include "../../include/crosscu.h"
#include "../../include/crosscu_debug.h"
#include "launch.h"

namespace cc {
namespace probe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kThreads = 512;
constexpr int kUnroll = 8;  // 16-byte loads in flight per lane (register path)

template <bool NT>
__device__ __forceinline__ void lds_dma16(const char* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr)lds, 16, 0, NT ? 2 : 0);  // policy 2: nt
}
template <bool NT>
__device__ __forceinline__ u32x4 load16(const char* p) {
  return NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)) : *reinterpret_cast<const u32x4*>(p);
}

// method 0: global_load_dwordx4 into registers, kUnroll per lane in flight.
// method 1: global_load_lds_dwordx4 into one 16 KiB LDS slot per wave.
// method 2: global_load_lds_dwordx4 into two 8 KiB LDS slots per wave (ping-pong).
// methods 3 and 4: methods 0 and 2 with the non-temporal cache policy (nt).
template <bool NT>
__global__ void __launch_bounds__(kThreads, 1)
read_probe(const char* __restrict__ buf, long long bytes, int method, const int* __restrict__ pages,
           int page_bytes, int num_pages, uint32_t* __restrict__ sink) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // unit of work: 16 KiB per wave-step; a workgroup covers its share in steps
  const long long step_bytes = 16384;
  const long long nsteps = bytes / step_bytes;
  const long long per_wg = (nsteps + gridDim.x - 1) / gridDim.x;
  const long long s0 = blockIdx.x * per_wg;
  const long long s1 = s0 + per_wg < nsteps ? s0 + per_wg : nsteps;
  auto src_of = [&](long long st) -> const char* {
    long long off = st * step_bytes;
    if (pages) {  // step -> (page in list, offset inside the page)
      const long long per_page = page_bytes / step_bytes;
      const long long pi = st / per_page;
      off = (long long)pages[pi % num_pages] * page_bytes + (st - pi * per_page) * step_bytes;
    }
    return buf + off;
  };
  uint32_t acc = 0;
  const int nw = kThreads / 64;
  if (method == 0) {
    for (long long st = s0 + wave; st < s1; st += nw) {
      const char* p = src_of(st) + lane * 16;
      u32x4 v[kUnroll * 2];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = load16<NT>(p + u * 1024);
#pragma unroll
      for (int u = 0; u < 16; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  } else {
    const int slot_bytes = method == 1 ? 16384 : 8192;
    const int nslots = method == 1 ? 1 : 2;
    char* region = smem + wave * 16384;
    const int chunks = slot_bytes / 1024;  // DMA instructions per slot fill
    long long st = s0 + wave;
    // sub-steps of slot_bytes
    const long long sub = step_bytes / slot_bytes;
    long long k = 0, kend = 0;
    for (long long t = s0 + wave; t < s1; t += nw) kend += sub;
    auto issue = [&](long long kk) {
      const long long t = s0 + wave + (kk / sub) * nw;
      const char* p = src_of(t) + (kk % sub) * slot_bytes + lane * 16;
      char* dst = region + (kk % nslots) * slot_bytes;
      for (int c = 0; c < chunks; ++c) lds_dma16<NT>(p + c * 1024, dst + c * 1024);
    };
    (void)st;
    if (kend > 0) issue(0);
    for (k = 0; k < kend; ++k) {
      if (nslots == 2 && k + 1 < kend) {
        issue(k + 1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(8) : "memory");  // the older slot's 8 transfers done
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      const char* src = region + (k % nslots) * slot_bytes;
      for (int c = 0; c < chunks; ++c) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + c * 1024 + lane * 16);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (nslots == 1 && k + 1 < kend) issue(k + 1);
    }
  }
  sink[blockIdx.x * kThreads + tid] = acc;
}

// MFMA ceiling probe: each wave runs `iters` rounds of kChains independent
// v_mfma_f32_32x32x16_bf16 accumulations on register operands (no memory
// traffic), so the rate it reaches is the practical dense bf16 MFMA rate of
// the device for that many waves per SIMD.  The accumulators are folded
// into sink so no product is dead.
constexpr int kChains = 8;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kProbeMaxWaves = 8;
__global__ void __launch_bounds__(64 * kProbeMaxWaves) mfma_probe(int iters, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  u32x4 a = {0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  u32x4 b = {0x3f803f80u, 0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u};
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = __builtin_bit_cast(uint32_t, s);
}

}  // namespace probe
}  // namespace cc

extern "C" int cc_probe_read(const void* buf, long long bytes, int method, const int32_t* pages,
                             int page_bytes, int num_pages, int workgroups, void* sink, void* stream) {
  using namespace cc::probe;
  if (!buf || !sink || bytes < 16384 || method < 0 || method > 4 || workgroups < 1) return CC_ERR_INVALID;
  if (pages && (page_bytes < 16384 || page_bytes % 16384 || num_pages < 1)) return CC_ERR_INVALID;
  const bool nt = method >= 3;
  const int m = method == 3 ? 0 : (method == 4 ? 2 : method);
  const size_t lds = m == 0 ? 0 : (size_t)(kThreads / 64) * 16384;
  const void* fn = nt ? reinterpret_cast<const void*>(&read_probe<true>) : reinterpret_cast<const void*>(&read_probe<false>);
  if (lds > 65536 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return CC_ERR_HIP;
  hipEvent_t ev0, ev1;
  cc::kernel_events(&ev0, &ev1);
  if (nt)
    hipExtLaunchKernelGGL(read_probe<true>, dim3(workgroups), dim3(kThreads), (uint32_t)lds,
                          static_cast<hipStream_t>(stream), ev0, ev1, 0u, static_cast<const char*>(buf), bytes, m,
                          pages, page_bytes, num_pages, static_cast<uint32_t*>(sink));
  else
    hipExtLaunchKernelGGL(read_probe<false>, dim3(workgroups), dim3(kThreads), (uint32_t)lds,
                          static_cast<hipStream_t>(stream), ev0, ev1, 0u, static_cast<const char*>(buf), bytes, m,
                          pages, page_bytes, num_pages, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? CC_OK : CC_ERR_HIP;
}

extern "C" int cc_probe_mfma(int workgroups, int waves_per_workgroup, int iters, void* sink, void* stream) {
  using namespace cc::probe;
  if (!sink || workgroups < 1 || waves_per_workgroup < 1 || waves_per_workgroup > kProbeMaxWaves || iters < 1)
    return CC_ERR_INVALID;
  hipEvent_t ev0, ev1;
  cc::kernel_events(&ev0, &ev1);
  hipExtLaunchKernelGGL(mfma_probe, dim3(workgroups), dim3(64 * waves_per_workgroup), 0u,
                        static_cast<hipStream_t>(stream), ev0, ev1, 0u, iters, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? CC_OK : CC_ERR_HIP;
}
