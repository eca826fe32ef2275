// Persistent Stream-K grouped GEMM for the experts of a MoE layer on gfx950.
//
// Routed rows sorted by expert: Y[r, :] = X[r, :] . W[e]^T for the rows r of
// expert e.  The experts' row counts differ widely (MeldKernel summary,
// "Problem and motivation"), so a launch of one workgroup per output tile
// leaves most compute units idle behind the big experts' tiles.  Here the
// host plan cuts the (output tile, k tile) work into one equal chunk per
// compute unit and the grid is one wave of workgroups (CSDN Q&A on waves and
// FlashMLA's Stream-K, "Summary"); a tile whose k range spans two chunks is
// summed just in time by the piece that finishes last (MeldKernel summary,
// "Core method"), in split order, so the result does not depend on timing.
//
// A workgroup is 8 waves, two per SIMD; wave (wm, wn) = (w / 4, w % 4) owns
// the 128 x 64 block (wm, wn) of the 256 x 256 output tile as 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per lane).  Both operands
// are K-contiguous (X rows; W rows = output columns), so a lane's 8-element
// MFMA operand is one 16-byte LDS read.  Each 64-wide k step of the operand
// tiles (32 KiB of X, 32 KiB of W) goes HBM -> LDS with
// global_load_lds_dwordx4 into one of two stages while the other computes;
// one workgroup per compute unit (128 KiB of LDS).  A k step gives each SIMD
// 2048 clocks of MFMA work against one barrier, one wait and 64 KiB moved per
// CU: the fixed cost of a step (the barrier, the operand reads' first round
// trip, the transfers' issue) is what a grouped GEMM with experts this small
// loses most to, and the larger tile halves it per flop, outweighing the rows
// it pads (an expert's last tile is cut to its rows).  In LDS, row r's 16-byte
// chunk c sits at chunk position c ^ ((r / 2) % 8) of the row's 128 bytes: a
// 16-byte read by 16 lanes of 16 consecutive rows' chunk c then covers the
// 64 banks (256 bytes) once, as two rows share one 256-byte bank line.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>

#include "../../include/crosscu.h"
#include "launch.h"
#include "merge.h"
#include "plan.h"

namespace cc {
namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kBM = kMoeTileRows, kBN = kMoeTileCols, kBK = 64;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kStages = 2;
constexpr int kTileA = kBM * kBK * 2;            // X tile of one stage: 32 KiB
constexpr int kTileB = kBN * kBK * 2;            // W tile of one stage: 32 KiB
constexpr int kDmaA = kTileA / 1024 / kWaves;    // 1 KiB transfers per wave and stage: 4 of X
constexpr int kDmaB = kTileB / 1024 / kWaves;    // and 4 of W
constexpr int kAcc = 128;                         // accumulators per lane: 4 x 2 blocks x 16
static_assert(kBN == kBM && kWaves == 8, "waves form a 2 x 4 grid of 128 x 64 blocks");

__shared__ __attribute__((aligned(16))) char lds_a[kStages][kTileA];
__shared__ __attribute__((aligned(16))) char lds_b[kStages][kTileB];

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const char* uni_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  return reinterpret_cast<const char*>((uintptr_t)((uint64_t)(uint32_t)uni((int)(uint32_t)v) |
                                                   ((uint64_t)(uint32_t)uni((int)(uint32_t)(v >> 32)) << 32)));
}

// HBM -> LDS copy of 16 bytes per lane: lane i's bytes from sbase + voff land
// at lds + 16 i (sbase and lds wave-uniform).  Inline asm: the kernel orders
// its stages with explicit waits and barriers, which the compiler's own wait
// insertion cannot see through.  M0 carries the LDS address; one wait state
// separates its write from the transfer.
__device__ __forceinline__ void lds_dma16(const char* sbase, uint32_t voff, char* lds) {
  const uint32_t m0 = uni((int)(uint32_t)(uintptr_t)(lds_ptr)lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}

struct Params {
  int K, N, slot_floats, reduce;
};

// Where accumulator idx = 16 (2 i + j) + r of thread (wave, lane) sits in the
// 256 x 256 tile: block (i, j) of the wave's 128 x 64 block, MFMA output
// register r.
__device__ __forceinline__ int acc_row(int wave, int lane, int idx) {
  const int i = idx >> 5, r = idx & 15;
  return (wave >> 2) * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wave, int lane, int idx) {
  const int j = (idx >> 4) & 1;
  return (wave & 3) * 64 + 32 * j + (lane & 31);
}

// Sum of a split tile's partials in split order, written to Y.  A partial
// slot holds accumulator idx of thread t at idx * kThreads + t.  Run by all
// kThreads threads of a workgroup (one per accumulator column of the slot):
// rounds of kIn accumulators, the loads of up to kSp splits of a round issued
// before any is used, so a tile of a few splits takes kAcc / kIn load round
// trips.
__device__ __forceinline__ void merge_tile(const float* pb, int ns, int slot_floats, const int32_t* d, int N,
                                           float* __restrict__ y, int t) {
  const int wave = t >> 6, lane = t & 63;
  const int row0 = d[1], rows = d[2], col0 = d[3];
  constexpr int kIn = 16;  // accumulators per round
  constexpr int kSp = 4;   // splits per round
  for (int i0 = 0; i0 < kAcc; i0 += kIn) {
    float s[kIn];
#pragma unroll
    for (int q = 0; q < kIn; ++q) s[q] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += kSp) {
      float v[kSp][kIn];
#pragma unroll
      for (int sp = 0; sp < kSp; ++sp) {
        const bool ok = s0 + sp < ns;
        const float* ps = pb + (size_t)(ok ? s0 + sp : 0) * slot_floats + (size_t)i0 * kThreads + t;
#pragma unroll
        for (int q = 0; q < kIn; ++q) v[sp][q] = ok ? partial_load(ps + (size_t)q * kThreads) : 0.f;
      }
#pragma unroll
      for (int sp = 0; sp < kSp; ++sp) {
        if (s0 + sp < ns) {  // in split order; absent splits add nothing (not even +0)
#pragma unroll
          for (int q = 0; q < kIn; ++q) s[q] += v[sp][q];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kIn; ++q) {
      const int m = acc_row(wave, lane, i0 + q);
      if (m < rows) y[(size_t)(row0 + m) * N + col0 + acc_col(wave, lane, i0 + q)] = s[q];
    }
  }
}

__global__ void __launch_bounds__(kThreads, 1)
moe_gemm_kernel(const Params p, const int32_t* __restrict__ wg_off, const int4* __restrict__ items,
                const int32_t* __restrict__ unit_nsplit, const int32_t* __restrict__ unit_pbase,
                const int32_t* __restrict__ desc, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                float* __restrict__ y, int32_t* counters, float* partials, unsigned long long* timeline) {
  __shared__ int sh_done[2];
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63;
  const int K = p.K, N = p.N;

  unsigned long long* tl = timeline ? timeline + kTimelineWords * blockIdx.x : nullptr;
  if (tl && tid == 0) {
    tl[0] = __builtin_amdgcn_s_memrealtime();
    tl[5] = xcc_id();
  }
  const int i0 = uni(wg_off[blockIdx.x]), i1 = uni(wg_off[blockIdx.x + 1]);
  if (i0 >= i1) {
    if (tl && tid == 0) tl[1] = tl[2] = tl[3] = tl[4] = tl[0];
    return;
  }

  // cursor over the chunk: item, its tile, and the k position
  struct Cur {
    int it, u, e, row0, rows, col0, kb, k1, split;
  };
  auto load = [&](Cur& c, int it) {
    const int4 t = items[it];
    c.it = it;
    c.u = uni(t.x);
    c.kb = uni(t.y);
    c.k1 = uni(t.z);
    c.split = uni(t.w);
    const int32_t* d = desc + kMoeDescWords * c.u;
    c.e = uni(d[0]);
    c.row0 = uni(d[1]);
    c.rows = uni(d[2]);
    c.col0 = uni(d[3]);
  };

  // X transfer i of this wave moves rows 8 q .. 8 q + 7 (q = kDmaA wave + i)
  // of the X tile, W transfer i rows 8 q .. (q = kDmaB wave + i) of the W
  // tile: lane L takes row 8 q + L / 8, k chunk (L % 8) ^ ((row / 2) % 8);
  // rows of X past the tile's last row repeat it (their outputs are dropped)
  uint32_t voff_b[kDmaB];
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int n = 8 * (kDmaB * wave + i) + (lane >> 3);
    voff_b[i] = (uint32_t)((n * K + 8 * ((lane & 7) ^ ((n >> 1) & 7))) * 2);
  }
  auto issue = [&](const Cur& c, int stage) {
    const char* sa = uni_ptr(reinterpret_cast<const char*>(x) + ((size_t)c.row0 * K + c.kb) * 2);
    const char* sb = uni_ptr(reinterpret_cast<const char*>(w) + (((size_t)c.e * N + c.col0) * K + c.kb) * 2);
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) {
      const int q = kDmaA * wave + i;
      const int r = 8 * q + (lane >> 3);
      const uint32_t voff_a = (uint32_t)((min(r, c.rows - 1) * K + 8 * ((lane & 7) ^ ((r >> 1) & 7))) * 2);
      lds_dma16(sa, voff_a, lds_a[stage] + 1024 * q);
    }
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) lds_dma16(sb, voff_b[i], lds_b[stage] + 1024 * (kDmaB * wave + i));
  };

  // operand reads: block i (j) of the wave's rows (columns) is row
  // base + lane % 32 of its tile (base a multiple of 32, so (row / 2) % 8 is
  // (lane / 2) % 8); k step ks reads chunk 2 ks + lane / 32
  const int arow = (wave >> 2) * 128 + (lane & 31), bcol = (wave & 3) * 64 + (lane & 31);
  auto chunk_pos = [&](int row, int ks) { return row * 128 + (((2 * ks + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4); };

  f32x16 acc[4][2];
  auto zero = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  };
  zero();

  Cur c;
  load(c, i0);
  Cur f = c;
  bool fvalid = true;
  auto advance = [&](Cur& a) -> bool {  // false past the chunk's last k step
    a.kb += kBK;
    if (a.kb < a.k1) return true;
    if (a.it + 1 >= i1) return false;
    load(a, a.it + 1);
    return true;
  };
  issue(f, 0);
  fvalid = advance(f);

  // split pieces this workgroup holds (a chunk's first and last items):
  // unit << 10 | split, -1 for none; they arrive after the stream
  int pend[2] = {-1, -1};
  int stage = 0;
  for (;;) {
    wait_vmem();  // this wave's transfers of the current stage (and any stores) are complete
    barrier();    // every wave's are, and every wave is done with the other stage
    if (fvalid) {
      issue(f, stage ^ 1);
      fvalid = advance(f);
    }
    const char* ta = lds_a[stage];
    const char* tb = lds_b[stage];
    u32x4 av[4][4], bv[2][4];
    auto rd = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i][ks] = *reinterpret_cast<const u32x4*>(ta + chunk_pos(arow + 32 * i, ks));
#pragma unroll
      for (int i = 0; i < 2; ++i) bv[i][ks] = *reinterpret_cast<const u32x4*>(tb + chunk_pos(bcol + 32 * i, ks));
    };
    // operand reads one k step ahead of the products, in a fixed order
    // (sched barriers): left to itself the scheduler waits out an LDS round
    // trip before every few MFMAs, and with more than 15 reads in flight the
    // wait count saturates and the first product waits for all of them.
    // The next item's scalar loads (if any) are done first: with a scalar
    // load outstanding the compiler can only wait for LDS reads with
    // lgkmcnt(0).
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
    rd(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) rd(ks + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i][ks]),
                                                            __builtin_bit_cast(bf16x8, bv[j][ks]), acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c.kb + kBK >= c.k1) {
      // -------- the item ends: the tile, or this piece's partial of it
      const int ns = uni(unit_nsplit[c.u]);
      if (ns == 1) {
#pragma unroll
        for (int idx = 0; idx < kAcc; ++idx) {
          const int m = acc_row(wave, lane, idx);
          if (m < c.rows)
            y[(size_t)(c.row0 + m) * N + c.col0 + acc_col(wave, lane, idx)] = acc[idx >> 5][(idx >> 4) & 1][idx & 15];
        }
      } else {
        float* ps = partials + (size_t)(uni(unit_pbase[c.u]) + c.split) * p.slot_floats;
#pragma unroll
        for (int idx = 0; idx < kAcc; ++idx)
          partial_store(ps + (size_t)idx * kThreads + tid, acc[idx >> 5][(idx >> 4) & 1][idx & 15]);
        if (p.reduce == CC_REDUCE_FUSED) {
          if (pend[0] < 0)
            pend[0] = (c.u << 10) | c.split;
          else
            pend[1] = (c.u << 10) | c.split;
        }
      }
      zero();
    }
    if (!advance(c)) break;
    stage ^= 1;
  }
  if (tl && tid == 0) tl[1] = tl[2] = __builtin_amdgcn_s_memrealtime();

  if (pend[0] >= 0) {
    // every partial store of the workgroup is complete (device-coherent,
    // see partial_store), then one arrival per piece; the piece that
    // completes a tile sums it (every other piece has arrived) and resets
    // its counter
    wait_vmem();
    __syncthreads();
    if (tid == 0) {
      for (int q = 0; q < 2; ++q) {
        sh_done[q] = 0;
        if (pend[q] < 0) continue;
        const int u = pend[q] >> 10;
        const int old = atomicAdd(&counters[kCounterStride * u], 1);
        if (old == unit_nsplit[u] - 1) {
          __hip_atomic_store(&counters[kCounterStride * u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          sh_done[q] = 1;
        }
      }
    }
    __syncthreads();
    if (tl && tid == 0) tl[3] = __builtin_amdgcn_s_memrealtime();
    for (int q = 0; q < 2; ++q) {
      if (pend[q] < 0 || !sh_done[q]) continue;
      const int u = pend[q] >> 10;
      merge_tile(partials + (size_t)uni(unit_pbase[u]) * p.slot_floats, uni(unit_nsplit[u]), p.slot_floats,
                 desc + kMoeDescWords * u, N, y, tid);
    }
  } else if (tl && tid == 0) {
    tl[3] = tl[1];
  }
  if (tl && tid == 0) tl[4] = __builtin_amdgcn_s_memrealtime();
}

// Split-then-combine comparison: one workgroup per split tile sums it.
__global__ void __launch_bounds__(kThreads)
moe_combine_kernel(int N, int slot_floats, const int32_t* __restrict__ unit_nsplit,
                   const int32_t* __restrict__ unit_pbase, const int32_t* __restrict__ desc,
                   const float* __restrict__ partials, float* __restrict__ y) {
  const int u = blockIdx.x;
  const int ns = unit_nsplit[u];
  if (ns <= 1) return;
  merge_tile(partials + (size_t)unit_pbase[u] * slot_floats, ns, slot_floats, desc + kMoeDescWords * u, N, y,
             threadIdx.x);
}

}  // namespace moe

hipError_t launch_moe(const MoeArgs& a, hipStream_t s) {
  moe::Params p;
  p.K = a.K;
  p.N = a.N;
  p.slot_floats = a.slot_floats;
  p.reduce = a.reduce;
  hipExtLaunchKernelGGL(moe::moe_gemm_kernel, dim3(a.workers), dim3(moe::kThreads), 0u, s, a.ev_start,
                        a.reduce == CC_REDUCE_SPLIT_COMBINE && a.partials_count > 0 ? nullptr : a.ev_stop, 0u, p,
                        a.wg_off, a.items, a.unit_nsplit, a.unit_pbase, a.desc, a.x, a.w, a.y, a.counters,
                        a.partials, a.timeline);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.reduce != CC_REDUCE_SPLIT_COMBINE || a.partials_count == 0) return e;
  hipExtLaunchKernelGGL(moe::moe_combine_kernel, dim3(a.units), dim3(moe::kThreads), 0u, s, nullptr, a.ev_stop,
                        0u, a.N, a.slot_floats, a.unit_nsplit, a.unit_pbase, a.desc, a.partials, a.y);
  return hipGetLastError();
}

}  // namespace cc
