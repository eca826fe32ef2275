// Persistent split-KV MLA decode attention for gfx950 (MI355X), dense and
// index-sparse.
//
// MLA shape: 128 query heads share one latent KV row of 576 bf16 per token;
// the whole row is K, its first 512 columns are V.  One workgroup of 4 waves
// per compute unit runs the equal chunk of KV tiles the host plan gave it
// (CSDN Q&A on waves and FlashMLA's Stream-K, "Summary"); sequences split
// across compute units are merged inside this kernel by the piece that
// arrives last (MeldKernel summary, "Core method").
//
// A unit is one query token's block of 64 heads (the two head blocks of a
// token are adjacent units, so their chunks stream the same tokens at the
// same time and the second read is served by the memory-side cache).  The 64
// heads are split over the 4 waves (16 each) and every wave sees every KV
// token: two dense contractions on v_mfma_f32_16x16x32_bf16 tiles,
//   S^T[16 tokens][16 heads] = K[16][576] . Q^T[576][16]   (2 halves x 18 k-steps)
//   O[16 heads][512]        += P[16][32 tokens] . V[32][512]  (32 tiles)
// Q^T stays in registers (72), O in accumulation registers (128).  S^T leaves
// each head's scores in the layout P needs as an A operand.
//
// A 32-token tile (36 KiB) streams HBM -> LDS with global_load_lds_dwordx4
// through a 3-stage ring shared by the 4 waves, so two tiles are in flight
// while one computes.  Each token's first 512 columns are one transfer into an
// LDS row padded to 1040 bytes (rows 260 dwords apart fall in different banks,
// so the MFMA operand reads are conflict free and every lane's address is one
// base register plus an immediate); the 64 rope columns are stored
// column-major, [chunk][token], which is conflict free for the same reads.
//
// The running max is only moved when a head's block max exceeds it by more
// than 2^8 (in base 2): probabilities stay below 256, and the costly rescale
// of 256 accumulators happens on a handful of blocks per sequence.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/crosscu.h"
#include "launch.h"
#include "merge.h"

namespace cc {
namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeads = 64;             // heads per unit (= per workgroup)
constexpr int kHW = kHeads / kWaves;   // heads per wave (16)
constexpr int kDqk = 576, kDv = 512;
constexpr int kRowBytes = kDqk * 2;    // 1152
constexpr int kBlk = 32;               // tokens per tile
constexpr int kKSteps = kDqk / 32;     // 18
constexpr int kRowPad = 1040;          // LDS bytes per token row (1024 + 16 pad)
constexpr int kRopeOff = kBlk * kRowPad;
constexpr int kStageBytes = kRopeOff + kBlk * 128;   // 37376
constexpr int kStages = 3;
constexpr int kDmaPerWave = (kBlk + 4) / kWaves;  // 32 row transfers + 4 rope transfers
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLazy = 8.f;           // log2 headroom before the max is moved

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ void lds_dma16(const char* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr)lds, 16, 0, 0);
}
__device__ __forceinline__ unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct Params {
  int hq, q_tokens, max_pages, num_pages, log2_page, topk;
  float scale_log2;
  int slot_floats;
  int reduce;
};

struct Item {
  int unit, tb, te, split, nsplit, pbase;
};

template <bool SPARSE>
__global__ void __launch_bounds__(kThreads, 1)
mla_decode_kernel(const Params p, const int32_t* __restrict__ wg_off, const int4* __restrict__ items,
                  const int32_t* __restrict__ unit_nsplit, const int32_t* __restrict__ unit_pbase,
                  const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kc,
                  const int32_t* __restrict__ bt, const int32_t* __restrict__ seqlens,
                  const int32_t* __restrict__ indices, float* __restrict__ out, float* __restrict__ lse,
                  int32_t* err, int32_t* counters, float* partials, unsigned long long* timeline) {
  extern __shared__ __attribute__((aligned(16))) char ring[];  // kStages x kStageBytes
  __shared__ __attribute__((aligned(16))) float merge_lds[merge_lds_floats(kThreads, kHeads)];
  __shared__ int sh_last;

  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;  // MFMA row/column, lane group

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
  auto load_item = [&](int it) {
    const int4 t = items[it];
    Item I;
    I.unit = uni(t.x);
    I.tb = uni(t.y);
    I.te = uni(t.z);
    I.split = uni(t.w);
    I.nsplit = uni(unit_nsplit[I.unit]);
    I.pbase = uni(unit_pbase[I.unit]);
    return I;
  };
  int nblk = 0;
  for (int i = i0; i < i1; ++i) {
    const int4 t = items[i];
    nblk += (uni(t.z) - uni(t.y) + kBlk - 1) / kBlk;
  }

  // unit = (b * Tq + t) * 2 + head block; q token row (b * Tq + t)
  const int hblocks = p.hq / kHeads;
  const int page_mask = (1 << p.log2_page) - 1;
  auto row_of = [&](int b, int tok) -> long long {  // cache row of token `tok` of sequence b
    int lp = min(tok >> p.log2_page, p.max_pages - 1);
    int pg = uni(bt[(size_t)b * p.max_pages + lp]);
    if ((unsigned)pg >= (unsigned)p.num_pages) {
      atomicOr(err, kErrPage);
      pg = pg < 0 ? 0 : p.num_pages - 1;
    }
    return (long long)pg * (1 << p.log2_page) + (tok & page_mask);
  };

  // ---- issue the tile of block (item I, block j) into ring stage st
  // row transfer j2 < 32: token j2, its first 1024 bytes -> LDS row j2 (1040 apart)
  // rope transfer r < 4: lane i takes rope chunk 2r + i/32 of token i%32 -> [chunk][token]
  auto fetch = [&](const Item& I, int j, int st) {
    char* dst = ring + st * kStageBytes;
    const int b = I.unit / hblocks / p.q_tokens;
    const int tok0 = I.tb + j * kBlk;
    const int tl_last = min(tok0 + kBlk, I.te) - 1;  // rows past the item end re-read the last valid row
    if constexpr (!SPARSE) {
      // a 32-token block lies inside one page (pages hold >= 32 tokens): rows are contiguous
      const char* base = reinterpret_cast<const char*>(kc) + row_of(b, tok0) * kRowBytes;
      const int nvalid = tl_last - tok0 + 1;
#pragma unroll
      for (int q = 0; q < kDmaPerWave; ++q) {
        const int j2 = wave + kWaves * q;  // transfer index 0..35 (uniform)
        if (j2 < kBlk) {
          const int t = min(j2, nvalid - 1);
          lds_dma16(base + (size_t)t * kRowBytes + 16 * lane, dst + j2 * kRowPad);
        } else {
          const int r = j2 - kBlk;
          const int t = min(lane & 31, nvalid - 1);
          lds_dma16(base + (size_t)t * kRowBytes + 1024 + 16 * (2 * r + (lane >> 5)), dst + kRopeOff + r * 1024);
        }
      }
    } else {
      const int32_t* idx = indices + (size_t)(I.unit / hblocks) * p.topk;
      const int L = seqlens[b];
#pragma unroll
      for (int q = 0; q < kDmaPerWave; ++q) {
        const int j2 = wave + kWaves * q;
        if (j2 < kBlk) {
          int tok = uni(idx[min(tok0 + j2, tl_last)]);
          if ((unsigned)tok >= (unsigned)L) {
            atomicOr(err, kErrIndex);
            tok = 0;
          }
          const char* row = reinterpret_cast<const char*>(kc) + row_of(b, tok) * kRowBytes;
          lds_dma16(row + 16 * lane, dst + j2 * kRowPad);
        } else {
          const int r = j2 - kBlk;
          int tok = idx[min(tok0 + (lane & 31), tl_last)];
          tok = ((unsigned)tok < (unsigned)L) ? tok : 0;
          const int lp = min(tok >> p.log2_page, p.max_pages - 1);
          int pg = bt[(size_t)b * p.max_pages + lp];
          pg = ((unsigned)pg < (unsigned)p.num_pages) ? pg : 0;
          const long long rw = (long long)pg * (1 << p.log2_page) + (tok & page_mask);
          lds_dma16(reinterpret_cast<const char*>(kc) + rw * kRowBytes + 1024 + 16 * (2 * r + (lane >> 5)),
                    dst + kRopeOff + r * 1024);
        }
      }
    }
  };

  // LDS read addresses of the MFMA operands: one base per operand, the rest immediate
  //   K, half hh, k-step ks < 16: token 16hh + lr, dims 32ks + 8lg -> lr*1040 + 16lg + hh*16*1040 + 64ks
  //   rope, half hh, k-step 16 + r: token 16hh + lr, chunk 4r + lg -> rope + lg*512 + 16lr + hh*256 + r*2048
  //   V, dv group g4, slot i: token tau(lg, i) = 4lg + i (i < 4), 16 + 4lg + i-4 (i >= 4),
  //     chunk 16 g4 + lr -> (4lg*1040 + 16lr) + (i<4 ? i : 12 + i)*1040 + 256 g4
  const uint32_t kbase = lr * kRowPad + 16 * lg;
  const uint32_t rbase = kRopeOff + 512 * lg + 16 * lr;
  const uint32_t vbase = 4 * lg * kRowPad + 16 * lr;

  // Q^T operand of the wave's 16 heads: lane holds head lr, dims 32 ks + 8 lg .. +8
  u32x4 qv[kKSteps];
  auto load_q = [&](int unit) {
    const size_t row = (size_t)(unit / hblocks) * p.hq + (size_t)(unit % hblocks) * kHeads + wave * kHW + lr;
    const uint16_t* qp = qg + row * kDqk + 8 * lg;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qv[s] = *reinterpret_cast<const u32x4*>(qp + 32 * s);
  };

  // ------------------------------------------------ the block stream
  Item cur = load_item(i0);
  int cur_it = i0, cur_j = 0, cur_nb = (cur.te - cur.tb + kBlk - 1) / kBlk;
  // producer cursor (two tiles ahead)
  Item pI = cur;
  int p_it = i0, p_j = 0, p_nb = cur_nb;
  auto advance = [&](Item& I, int& it, int& j, int& nb) {
    if (++j == nb) {
      ++it;
      if (it < i1) {
        I = load_item(it);
        j = 0;
        nb = (I.te - I.tb + kBlk - 1) / kBlk;
      }
    }
  };
  fetch(pI, p_j, 0);
  advance(pI, p_it, p_j, p_nb);
  if (nblk > 1) {
    fetch(pI, p_j, 1);
    advance(pI, p_it, p_j, p_nb);
  }
  load_q(cur.unit);

  float m_run = -INFINITY, l_run = 0.f;  // per lane: head lr (four lanes per head)
  f32x4 o[4][8];                          // dv group g4, column c: dv = 128 g4 + 8 lr + c; rows heads 4lg+r
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[g4][c] = f32x4{};
  bool fresh = true;  // no block of the current item seen yet

  for (int k = 0; k < nblk; ++k) {
    const int st = k % kStages;
    // tile k has landed in LDS for every wave; tile k-1's stage is free
    if (k + 1 < nblk) wait_vmcnt<kDmaPerWave>(); else wait_vmcnt<0>();
    wait_lds();
    barrier();
    if (k + 2 < nblk) {
      fetch(pI, p_j, (k + 2) % kStages);
      advance(pI, p_it, p_j, p_nb);
    }
    const char* tile = ring + st * kStageBytes;
    const int tok0 = cur.tb + cur_j * kBlk;
    const int nv = min(kBlk, cur.te - tok0);

    // S^T = K Q^T, two 16-token halves
    f32x4 s0 = {}, s1 = {};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      s0 = mfma16(*reinterpret_cast<const u32x4*>(tile + kbase + 64 * ks), qv[ks], s0);
      s1 = mfma16(*reinterpret_cast<const u32x4*>(tile + kbase + 16 * kRowPad + 64 * ks), qv[ks], s1);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      s0 = mfma16(*reinterpret_cast<const u32x4*>(tile + rbase + 2048 * r), qv[16 + r], s0);
      s1 = mfma16(*reinterpret_cast<const u32x4*>(tile + rbase + 256 + 2048 * r), qv[16 + r], s1);
    }
    const bool item_ends = cur_j == cur_nb - 1;
    if (item_ends && k + 1 < nblk) {
      // q of the next item replaces this one as soon as the scores no longer need it
      load_q(uni(items[cur_it + 1].x));
    }
    // scores (base 2), masked past the item end; x[i] is token tau(lg, i)
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (4 * lg + i < nv) ? s0[i] * p.scale_log2 : -INFINITY;
      x[4 + i] = (16 + 4 * lg + i < nv) ? s1[i] * p.scale_log2 : -INFINITY;
    }
    float bmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    // move the reference max only when some head needs it
    const bool need = bmax > m_run + kLazy;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float mnew = fmaxf(m_run, bmax);
      const float alpha = fast_exp2(m_run - mnew);
      l_run *= alpha;
      m_run = mnew;
      if (!fresh) {  // O rows of register r are heads 4 lg + r
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float a = __shfl(alpha, 4 * lg + rr);
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
            for (int c = 0; c < 8; ++c) o[g4][c][rr] *= a;
        }
      }
    }
    fresh = false;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = fast_exp2(x[i] - m_run);
      psum += x[i];
    }
    l_run += psum;
    const u32x4 pa = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};

    // O += P V; rows past the item end read zeros
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x4 vr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        vr[i] = *reinterpret_cast<const u32x4*>(tile + vbase + (i < 4 ? i : 12 + i) * kRowPad + 256 * g4);
        const int tau = (i < 4) ? 4 * lg + i : 16 + 4 * lg + (i - 4);
        if (tau >= nv) vr[i] = u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4 vb;
#pragma unroll
        for (int pi = 0; pi < 4; ++pi) {
          const uint32_t a0 = vr[2 * pi][c >> 1];
          const uint32_t a1 = vr[2 * pi + 1][c >> 1];
          vb[pi] = (c & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
        }
        o[g4][c] = mfma16(pa, vb, o[g4][c]);
      }
    }

    if (item_ends) {
      // -------- finish the item: this workgroup holds the whole piece
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      const int hb = cur.unit % hblocks;
      const size_t qrow = (size_t)(cur.unit / hblocks) * p.hq + (size_t)hb * kHeads;  // first head of the unit
      const int hw0 = wave * kHW;                                                       // wave's first head in the unit
      if (cur.nsplit == 1) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int hh = 4 * lg + rr;
          const float inv = 1.f / __shfl(l_tot, hh);
          float* orow = out + (qrow + hw0 + hh) * kDv + 8 * lr;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            *reinterpret_cast<f32x4*>(orow + 128 * g4) =
                f32x4{o[g4][0][rr] * inv, o[g4][1][rr] * inv, o[g4][2][rr] * inv, o[g4][3][rr] * inv};
            *reinterpret_cast<f32x4*>(orow + 128 * g4 + 4) =
                f32x4{o[g4][4][rr] * inv, o[g4][5][rr] * inv, o[g4][6][rr] * inv, o[g4][7][rr] * inv};
          }
        }
        if (lane < 16) lse[qrow + hw0 + lane] = (m_run + __log2f(l_tot)) * kLn2;
      } else {
        float* ps = partials + (size_t)(cur.pbase + cur.split) * p.slot_floats;
        if (lane < 16) {
          ps[hw0 + lane] = m_run;
          ps[kHeads + hw0 + lane] = l_tot;
        }
        float* po = ps + partial_o_offset(kHeads) + (size_t)hw0 * kDv;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int hh = 4 * lg + rr;
          float* orow = po + (size_t)hh * kDv + 8 * lr;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            *reinterpret_cast<f32x4*>(orow + 128 * g4) = f32x4{o[g4][0][rr], o[g4][1][rr], o[g4][2][rr], o[g4][3][rr]};
            *reinterpret_cast<f32x4*>(orow + 128 * g4 + 4) = f32x4{o[g4][4][rr], o[g4][5][rr], o[g4][6][rr], o[g4][7][rr]};
          }
        }
        if (p.reduce == CC_REDUCE_FUSED) {
          __syncthreads();  // every wave's share of the partial is written
          if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const int old = atomicAdd(&counters[cur.unit], 1);
            const bool last = old == cur.nsplit - 1;
            if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            sh_last = last;
          }
          __syncthreads();
          if (uni(sh_last)) {
            merge_splits<kThreads>(partials + (size_t)cur.pbase * p.slot_floats, cur.nsplit, p.slot_floats,
                                   kHeads, kDv, out + qrow * kDv, lse + qrow, merge_lds);
            if (tid == 0) __hip_atomic_store(&counters[cur.unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      if (k + 1 < nblk) {
        ++cur_it;
        cur = load_item(cur_it);
        cur_j = 0;
        cur_nb = (cur.te - cur.tb + kBlk - 1) / kBlk;
        m_run = -INFINITY;
        l_run = 0.f;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
          for (int c = 0; c < 8; ++c) o[g4][c] = f32x4{};
        fresh = true;
      }
    } else {
      ++cur_j;
    }
  }
  if (tl && tid == 0) tl[1] = tl[2] = tl[3] = tl[4] = __builtin_amdgcn_s_memrealtime();
}

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

}  // namespace mla

hipError_t launch_mla(const DecodeArgs& a, hipStream_t s) {
  mla::Params p;
  p.hq = a.hq;
  p.q_tokens = a.q_tokens;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.log2_page = mla::ilog2(a.page_size);
  p.topk = a.topk;
  p.scale_log2 = a.scale_log2;
  p.slot_floats = a.slot_floats;
  p.reduce = a.reduce;
  const size_t lds = (size_t)mla::kStages * mla::kStageBytes;
  hipError_t e;
  if (a.mode == CC_MODE_MLA_SPARSE) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mla::mla_decode_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    mla::mla_decode_kernel<true><<<a.workers, mla::kThreads, lds, s>>>(
        p, a.wg_off, a.items, a.unit_nsplit, a.unit_pbase, a.q, a.k, a.block_table, a.seqlens, a.indices,
        a.out, a.lse, a.err, a.counters, a.partials, a.timeline);
  } else {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mla::mla_decode_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    mla::mla_decode_kernel<false><<<a.workers, mla::kThreads, lds, s>>>(
        p, a.wg_off, a.items, a.unit_nsplit, a.unit_pbase, a.q, a.k, a.block_table, a.seqlens, a.indices,
        a.out, a.lse, a.err, a.counters, a.partials, a.timeline);
  }
  return hipGetLastError();
}

}  // namespace cc
