// Paged indexer score and top-k selection (the step that produces the index
// sets of index-sparse decode attention: GLM-5.2 decode article, "Paged
// Indexer Score" ahead of TopK and sparse MLA, Summary; the Top-2048 the
// indexer rank publishes, related-work section on TileRT).
//
// Two kernels.  The score kernel gives each lane one cached token and two
// decode tokens: the lane reads the token's 256-byte key row into registers
// (the request's query rows sit in LDS) and runs an fp32 FMA chain over the
// 128 dimensions in index order for each decode token (a bf16 x bf16 product
// is exact in fp32, so each FMA rounds once, exactly as an add of the exact
// product).  It is a streaming read of the key cache, a few MB.
//
// The top-k kernel gives each decode token one 1024-thread workgroup: the
// scores become order-preserving unsigned keys in LDS, a radix select over
// digits of 12, 12 and 8 bits finds the k-th largest key T and how many keys
// equal to T belong to the result, and a stable compaction in position order writes
// every key above T plus the first such keys equal to T.  Integer work on
// the score bits, so the result is exact and deterministic.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>

#include "../../include/crosscu.h"
#include "../../include/crosscu_indexer.h"
#include "launch.h"
#include "plan.h"

namespace cc {
namespace indexer {

constexpr int kDim = 128;
constexpr int kMaxTq = 16;
constexpr int kMaxB = 64;
constexpr int kMaxL = 16384;
constexpr int kScoreThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kErrPage = 2;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Lens {
  int32_t L[kMaxB];
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// grid (ceil(max L * lpt / 256), B): lane = (cached token j, pair of decode
// tokens p), p fastest (lpt = ceil(tq / 2) rounded up to a power of two, the
// lanes of one token).  The request's query rows are staged in LDS once per
// workgroup; each lane loads its token's key row into registers and runs two
// independent FMA chains over the 128 dimensions in index order, one per
// decode token (2p and 2p + 1).
__global__ void __launch_bounds__(kScoreThreads)
indexer_score_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                     const int32_t* __restrict__ bt, Lens lens, int tq, int log2lpt, int log2p, int max_pages,
                     int num_pages, int ld, float* __restrict__ scores, int32_t* __restrict__ err) {
  __shared__ u32x4 qs[kMaxTq][kDim / 8];
  const int b = blockIdx.y;
  const int L = lens.L[b];
  {
    const u32x4* qb = reinterpret_cast<const u32x4*>(q + (size_t)b * tq * kDim);
    for (int i = threadIdx.x; i < tq * (kDim / 8); i += kScoreThreads) qs[i / (kDim / 8)][i % (kDim / 8)] = qb[i];
  }
  __syncthreads();
  const int t = blockIdx.x * kScoreThreads + threadIdx.x;
  const int j = t >> log2lpt, m0 = 2 * (t & ((1 << log2lpt) - 1));
  if (j >= L || m0 >= tq) return;
  const int m1 = m0 + 1 < tq ? m0 + 1 : m0;  // an odd last token: the second chain repeats the first
  int pg = bt[(size_t)b * max_pages + (j >> log2p)];
  if ((unsigned)pg >= (unsigned)num_pages) {
    if (err) atomicOr(err, kErrPage);
    pg = pg < 0 ? 0 : num_pages - 1;
  }
  const u32x4* row = reinterpret_cast<const u32x4*>(
      kc + (((size_t)pg << log2p) + (size_t)(j & ((1 << log2p) - 1))) * kDim);
  u32x4 r[kDim / 8];
#pragma unroll
  for (int c = 0; c < kDim / 8; ++c) r[c] = row[c];
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int c = 0; c < kDim / 8; ++c) {
    const u32x4 q0 = qs[m0][c], q1 = qs[m1][c];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      a0 = __builtin_fmaf(bf16_lo(q0[w]), bf16_lo(r[c][w]), a0);
      a1 = __builtin_fmaf(bf16_lo(q1[w]), bf16_lo(r[c][w]), a1);
      a0 = __builtin_fmaf(bf16_hi(q0[w]), bf16_hi(r[c][w]), a0);
      a1 = __builtin_fmaf(bf16_hi(q1[w]), bf16_hi(r[c][w]), a1);
    }
  }
  scores[(size_t)(b * tq + m0) * ld + j] = a0;
  if (m1 != m0) scores[(size_t)(b * tq + m1) * ld + j] = a1;
}

constexpr int kWavesT = kTopkThreads / 64;

// Sum over the first kWavesT lanes of v, for every lane of the wave: lane l
// holds wave l's contribution (zero where it does not count), and a butterfly
// over groups of 16 lanes adds them in four steps instead of a chain of LDS
// reads.  Integer sums: the order does not matter.
__device__ __forceinline__ uint32_t sum_wave_lanes(uint32_t v) {
  static_assert(kWavesT == 16, "one butterfly group per workgroup's waves");
#pragma unroll
  for (int o = 1; o < kWavesT; o <<= 1) v += __shfl_xor(v, o);
  return __builtin_amdgcn_readfirstlane(v);
}

// Inclusive suffix sum over the workgroup in thread order: thread t gets the
// sum of x over threads >= t.
__device__ __forceinline__ uint32_t block_suffix_sum(uint32_t x, uint32_t* wtot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_down(incl, o);
    if (lane + o < 64) incl += t;
  }
  __syncthreads();  // wtot free from a previous use
  if (lane == 0) wtot[wave] = incl;
  __syncthreads();
  const uint32_t after = sum_wave_lanes(lane < kWavesT && lane > wave ? wtot[lane] : 0u);
  return incl + after;
}

// Radix-select passes, most significant first: key bits [20, 32), [8, 20),
// [0, 8).  A float key's top 12 bits are its sign, exponent and 3 mantissa
// bits, so the first pass already spreads the scores over many bins (8-bit
// digits would put nearly all of them in a few bins, and their LDS atomics
// would serialize).
constexpr int kPasses = 3;
__device__ constexpr int kPassShift[kPasses] = {20, 8, 0};
__device__ constexpr int kPassBits[kPasses] = {12, 12, 8};
constexpr int kBins = 1 << 12;

// grid B * Tq; one workgroup per decode token
__global__ void __launch_bounds__(kTopkThreads)
indexer_topk_kernel(const float* __restrict__ scores, int ld, Lens lens, int tq, int topk,
                    int32_t* __restrict__ out) {
  __shared__ uint32_t keys[kMaxL];
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wtot[kWavesT];
  __shared__ uint32_t wcount[2][kWavesT];  // per wave: keys above T, keys equal to T
  __shared__ uint32_t sh_digit, sh_above;
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const int L = lens.L[r / tq];
  const float* s = scores + (size_t)r * ld;
  {
    // every score load of a thread issued before any is used (one round trip)
    constexpr int kPer = kMaxL / kTopkThreads;
    uint32_t v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = tid + u * kTopkThreads;
      v[u] = j < L ? __float_as_uint(s[j]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = tid + u * kTopkThreads;
      uint32_t x = v[u];
      if (x == 0x80000000u) x = 0u;  // -0 ranks with +0
      if (j < L) keys[j] = (x & 0x80000000u) ? ~x : (x | 0x80000000u);
    }
  }
  // radix select of the topk-th largest key
  uint32_t prefix = 0, mask = 0;
  uint32_t kk = (uint32_t)topk;  // rank still to place among keys matching prefix
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int shift = kPassShift[pass], nb = 1 << kPassBits[pass];
    for (int i = tid; i < nb; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < L; j += kTopkThreads) {
      const uint32_t k = keys[j];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    // thread t owns bins [per t, per t + per); the digit is the bin where the
    // count of larger keys first reaches kk, scanning from the top bin down
    const int per = nb >= kTopkThreads ? nb / kTopkThreads : 1;
    const int b0 = tid * per;
    uint32_t own = 0;
    for (int i = 0; i < per; ++i)
      if (b0 + i < nb) own += hist[b0 + i];
    const uint32_t incl = block_suffix_sum(own, wtot);  // keys in bins >= b0
    const uint32_t above = incl - own;                  // keys in bins >= b0 + per
    if (above < kk && kk <= incl) {
      uint32_t c = above;
      int d = b0 + per - 1;
      while (c + hist[d] < kk) c += hist[d--];
      sh_digit = (uint32_t)d;
      sh_above = c;
    }
    __syncthreads();
    kk -= sh_above;
    prefix |= sh_digit << shift;
    mask |= (uint32_t)(nb - 1) << shift;
  }
  const uint32_t T = prefix;  // the topk-th largest key; kk keys equal to it are kept
  // Stable compaction in position order.  Wave w owns positions [w P, (w + 1) P)
  // and walks them 64 at a time (lane = position), so key reads hit distinct
  // LDS banks and index writes are contiguous; ballots give each lane its rank
  // among the keys above T, and among those equal to T, before it.  The first
  // kk keys equal to T in position order are kept.
  const int lane = tid & 63, wave = tid >> 6;
  const int P = (L + kWavesT * 64 - 1) / (kWavesT * 64) * 64;
  const int jw = wave * P;
  const unsigned long long below = (1ull << lane) - 1;
  int gt = 0, eq = 0;  // this wave's counts (wave-uniform)
  for (int i = 0; i < P; i += 64) {
    const int j = jw + i + lane;
    const bool in = j < L;
    const uint32_t k = in ? keys[j] : 0u;
    gt += __popcll(__ballot(in && k > T));
    eq += __popcll(__ballot(in && k == T));
  }
  if (lane == 0) {
    wcount[0][wave] = gt;
    wcount[1][wave] = eq;
  }
  __syncthreads();
  const bool earlier = lane < wave;  // lane l < kWavesT stands for wave l
  const int gt_before = (int)sum_wave_lanes(earlier ? wcount[0][lane] : 0u);
  const int eq_before = (int)sum_wave_lanes(earlier ? wcount[1][lane] : 0u);
  int pos = gt_before + min((int)kk, eq_before);  // results before this wave's positions
  int eqr = eq_before;                            // keys equal to T before the current 64
  int32_t* o = out + (size_t)r * topk;
  for (int i = 0; i < P; i += 64) {
    const int j = jw + i + lane;
    const bool in = j < L;
    const uint32_t k = in ? keys[j] : 0u;
    const bool g = in && k > T, q = in && k == T;
    const unsigned long long qb = __ballot(q);
    const bool take = g || (q && eqr + __popcll(qb & below) < (int)kk);
    const unsigned long long tb = __ballot(take);
    const int p = pos + __popcll(tb & below);
    if (take && p < topk) o[p] = j;
    pos += __popcll(tb);
    eqr += __popcll(qb);
  }
}

}  // namespace indexer
}  // namespace cc

namespace {
bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}
// Host checks shared by both calls; max L into *maxl.
int check(const cc_indexer_problem* p, const int32_t* seqlens, int* maxl) {
  using namespace cc::indexer;
  if (!p || !seqlens) {
    cc::set_error("cc_indexer: null problem or seqlens");
    return CC_ERR_INVALID;
  }
  if (p->batch < 1 || p->q_tokens < 1 || p->dim < 1 || !pow2(p->page_size) || p->max_pages_per_seq < 1 ||
      p->num_pages < 1 || p->topk < 1) {
    cc::set_error("cc_indexer: bad problem sizes");
    return CC_ERR_INVALID;
  }
  if (p->dim != kDim || p->q_tokens > kMaxTq || p->batch > kMaxB) {
    cc::set_error("cc_indexer: implemented for dim 128, q_tokens <= 16, batch <= 64");
    return CC_ERR_UNSUPPORTED;
  }
  int m = 0;
  for (int b = 0; b < p->batch; ++b) {
    const int L = seqlens[b];
    if (L < 1 || p->topk > L || (L + p->page_size - 1) / p->page_size > p->max_pages_per_seq) {
      cc::set_error("cc_indexer: request %d: length %d, topk %d, pages %d", b, L, p->topk, p->max_pages_per_seq);
      return CC_ERR_INVALID;
    }
    if (L > kMaxL) {
      cc::set_error("cc_indexer: request %d: length %d above 16384", b, L);
      return CC_ERR_UNSUPPORTED;
    }
    m = L > m ? L : m;
  }
  *maxl = m;
  return CC_OK;
}
}  // namespace

extern "C" int cc_indexer_scratch_size(const cc_indexer_problem* p, const int32_t* seqlens, size_t* bytes) {
  if (!bytes) return CC_ERR_INVALID;
  int maxl = 0;
  const int rc = check(p, seqlens, &maxl);
  if (rc != CC_OK) return rc;
  *bytes = (size_t)p->batch * p->q_tokens * maxl * sizeof(float);
  return CC_OK;
}

extern "C" int cc_indexer_topk(const cc_indexer_problem* p, const int32_t* seqlens, const void* q,
                               const void* k_cache, const int32_t* block_table, void* scratch, size_t scratch_bytes,
                               int32_t* indices, int32_t* err, void* stream) {
  using namespace cc::indexer;
  int maxl = 0;
  const int rc = check(p, seqlens, &maxl);
  if (rc != CC_OK) return rc;
  if (!q || !k_cache || !block_table || !scratch || !indices) {
    cc::set_error("cc_indexer_topk: null device pointer");
    return CC_ERR_INVALID;
  }
  const size_t need = (size_t)p->batch * p->q_tokens * maxl * sizeof(float);
  if (scratch_bytes < need) {
    cc::set_error("cc_indexer_topk: scratch %zu bytes, need %zu", scratch_bytes, need);
    return CC_ERR_BUFFER;
  }
  Lens lens = {};
  for (int b = 0; b < p->batch; ++b) lens.L[b] = seqlens[b];
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* sc = static_cast<float*>(scratch);
  hipEvent_t ev0, ev1;  // debug kernel events (cc_debug_kernel_events): start of the first, end of the last
  cc::kernel_events(&ev0, &ev1);
  const int log2lpt = ilog2((p->q_tokens + 1) / 2);
  const long long lanes = (long long)maxl << log2lpt;
  hipExtLaunchKernelGGL(indexer_score_kernel, dim3((unsigned)((lanes + kScoreThreads - 1) / kScoreThreads), p->batch),
                        dim3(kScoreThreads), 0u, s, ev0, nullptr, 0u, static_cast<const uint16_t*>(q),
                        static_cast<const uint16_t*>(k_cache), block_table, lens, p->q_tokens, log2lpt,
                        ilog2(p->page_size), p->max_pages_per_seq, p->num_pages, maxl, sc, err);
  hipExtLaunchKernelGGL(indexer_topk_kernel, dim3(p->batch * p->q_tokens), dim3(kTopkThreads), 0u, s, nullptr, ev1,
                        0u, static_cast<const float*>(sc), maxl, lens, p->q_tokens, p->topk, indices);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    cc::set_error("cc_indexer_topk: %s", hipGetErrorString(e));
    return CC_ERR_HIP;
  }
  return CC_OK;
}
