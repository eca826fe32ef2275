// Persistent split-KV MLA decode attention for gfx950 (MI355X), dense and
// index-sparse.
//
// MLA shape: 128 query heads share one latent KV row of 576 bf16 per token;
// the whole row is K, its first 512 columns are V.  One workgroup of 8 waves
// per compute unit runs the equal chunk of KV tiles the host plan gave it
// (CSDN Q&A on waves and FlashMLA's Stream-K, "Summary"); sequences split
// across compute units are merged inside this kernel by the piece that
// arrives last (MeldKernel summary, "Core method").
//
// A unit is one query token's block of 64 heads (the two head blocks of a
// token are adjacent units, so their chunks stream the same tokens at the
// same time and the second read is served by the memory-side cache).  Each
// pair of waves owns 16 heads and every wave sees every KV token of the tile.
// The two waves of a pair split the work of the two dense contractions
// (v_mfma_f32_16x16x32_bf16 tiles):
//   S^T[32 tokens][16 heads] = K[32][576] . Q^T[576][16]: wave h of the pair
//     sums k-steps 9h .. 9h+8 (dims 288h .. 288h+287) and the pair adds the
//     two partials through LDS, in the same order in both waves, so both hold
//     bitwise the same scores and run the same softmax;
//   O[16 heads][512] += P[16][32] . V[32][512]: wave h accumulates dv columns
//     256h .. 256h+255.
// Per wave that is 9 k-steps of Q^T (36 registers) and 64 accumulators, which
// leaves the register file room for the operand pipeline.  S^T leaves each
// head's scores in the layout P needs as an A operand; V is transposed in
// registers with one byte permute per word.
//
// A 32-token tile (36 KiB) streams HBM -> LDS with global_load_lds_dwordx4
// through a 3-stage ring, so two tiles are in flight while one computes.  Wave
// w moves tokens w, w+8, w+16, w+24: each token's first 512 columns are one
// transfer into an LDS row padded to 1040 bytes (rows 260 dwords apart fall in
// different banks, so the MFMA operand reads are conflict free and every
// lane's address is one base register plus an immediate), and the 64 rope
// columns of its 4 tokens are one half-wave transfer into the wave's own
// 512-byte region, 16-byte chunks in [token][chunk] order with the chunk index
// XOR-ed by bit 0 of the token slot; regions 544 bytes apart keep the rope
// operand reads conflict free too.  The fetch needs no per-lane loads, so it
// never waits behind the transfers in flight.
//
// The running max is only moved when a head's block max exceeds it by more
// than 2^8 (in base 2): probabilities stay below 256, and the rescale of the
// accumulators happens on a handful of blocks per sequence.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

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

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeads = 64;                  // heads per unit (= per workgroup)
constexpr int kHG = 16;                     // heads per wave pair
constexpr int kDqk = 576, kDv = 512;
constexpr int kRowBytes = kDqk * 2;         // 1152
constexpr int kBlk = 32;                    // tokens per tile
constexpr int kKHalf = 9;                   // 32-dim k-steps of q.k per wave of a pair
constexpr int kRowPad = 1040;               // LDS bytes per token row (1024 + 16 pad)
constexpr int kRopeOff = kBlk * kRowPad;
constexpr int kRopeWave = 544;              // LDS bytes between the waves' rope regions (512 + 32)
constexpr int kStageBytes = kRopeOff + (kWaves - 1) * kRopeWave + 512;   // 37600
constexpr int kRowsPerWave = kBlk / kWaves;                              // 4
constexpr int kDmaPerWave = kRowsPerWave + 1;                            // + 1 rope transfer
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLazy = 8.f;                // log2 headroom before the max is moved

// The three ring stages and the exchange buffer of the score partials.
__shared__ __attribute__((aligned(16))) char ring0[kStageBytes];
__shared__ __attribute__((aligned(16))) char ring1[kStageBytes];
__shared__ __attribute__((aligned(16))) char ring2[kStageBytes];
__shared__ __attribute__((aligned(16))) f32x4 xch[kWaves][2][64];

template <int S>
__device__ __forceinline__ char* stage() {
  return S == 0 ? ring0 : (S == 1 ? ring1 : ring2);
}
template <int S>
using IC = std::integral_constant<int, S>;

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
// HBM -> LDS transfer of 16 bytes per active lane: lane i's bytes land at
// lds + 16 i (lds wave-uniform).  Written as inline asm on purpose: the
// compiler's own wait insertion cannot tell which stage a transfer targets and
// would wait for every transfer in flight before any LDS read; the kernel
// orders the ring itself with explicit vmcnt waits and barriers.  M0 carries
// the LDS address (the compiler uses M0 nowhere else in these kernels); one
// wait state separates its write from the transfer.  The transfers carry the
// non-temporal cache policy (nt): a streaming read reaches ~6.7 TB/s with it
// and ~5.7 TB/s without on MI355X.
__device__ __forceinline__ void lds_dma16(const char* src, char* lds) {
  const uint32_t m0 = uni((int)(uint32_t)(uintptr_t)(lds_ptr)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(src), "s"(m0) : "memory", "m0");
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

// K^T operand reads of wave half H for both 16-token halves of the tile:
// k-step ks < 16 is latent dims 32 ks .. from the padded rows, ks >= 16 rope.
template <int H>
__device__ __forceinline__ void scores_half(const char* tile, uint32_t kbase, uint32_t rbase,
                                            const u32x4 (&qv)[kKHalf], f32x4& s0, f32x4& s1) {
#pragma unroll
  for (int jb = 0; jb < kKHalf; jb += 3) {
    u32x4 ka[3], kb[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int ks = H * kKHalf + jb + u;
      const uint32_t off0 = ks < 16 ? kbase + 64 * ks : rbase + 64 * (ks - 16);
      const uint32_t off1 = ks < 16 ? kbase + 16 * kRowPad + 64 * ks : rbase + 256 + 64 * (ks - 16);
      ka[u] = *reinterpret_cast<const u32x4*>(tile + off0);
      kb[u] = *reinterpret_cast<const u32x4*>(tile + off1);
    }
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      s0 = mfma16(ka[u], qv[jb + u], s0);
      s1 = mfma16(kb[u], qv[jb + u], s1);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool SPARSE>
__global__ void __launch_bounds__(kThreads, 1)
mla_decode_kernel(const Params p, const int32_t* __restrict__ wg_off, const int4* __restrict__ items,
                  const int32_t* __restrict__ unit_nsplit, const int32_t* __restrict__ unit_pbase,
                  const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kc,
                  const int32_t* __restrict__ bt, const int32_t* __restrict__ seqlens,
                  const int32_t* __restrict__ indices, float* __restrict__ out, float* __restrict__ lse,
                  int32_t* err, int32_t* counters, float* partials, unsigned long long* timeline) {
  __shared__ __attribute__((aligned(16))) float merge_lds[merge_lds_floats(kThreads, kHeads)];
  __shared__ int sh_last;

  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63;
  const int hg = wave >> 1, half = wave & 1;  // head group of the pair, half of the pair
  const int lr = lane & 15, lg = lane >> 4;   // MFMA row/column, lane group

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

  // ---- issue the tile of block (item I, block j) into the stage at dst
  // row transfer q < 4: token j2 = wave + 8q, its first 1024 bytes -> LDS row j2 (1040 apart)
  // rope transfer (lanes 0..31): lane l takes token wave + 8(l/8), chunk (l%8) ^ ((l/8)%2)
  const int rq = (lane >> 3) & 3;  // token slot of this lane's rope chunk
  const int rchunk = (lane & 7) ^ (rq & 1);
  auto fetch = [&](const Item& I, int j, char* dst) {
    const int b = I.unit / hblocks / p.q_tokens;
    const int tok0 = I.tb + j * kBlk;
    const int tl_last = min(tok0 + kBlk, I.te) - 1;  // rows past the item end re-read the last valid row
    char* rope_dst = dst + kRopeOff + wave * kRopeWave;
    if constexpr (!SPARSE) {
      // a 32-token block lies inside one page (pages hold >= 32 tokens): rows are contiguous
      const char* base = reinterpret_cast<const char*>(kc) + row_of(b, tok0) * kRowBytes;
      const int nvalid = tl_last - tok0 + 1;
#pragma unroll
      for (int q = 0; q < kRowsPerWave; ++q) {
        const int j2 = wave + kWaves * q;
        lds_dma16(base + (size_t)min(j2, nvalid - 1) * kRowBytes + 16 * lane, dst + j2 * kRowPad);
      }
      const int t = min(wave + kWaves * rq, nvalid - 1);
      if (lane < 32) lds_dma16(base + (size_t)t * kRowBytes + 1024 + 16 * rchunk, rope_dst);
    } else {
      const int32_t* idx = indices + (size_t)(I.unit / hblocks) * p.topk;
      const int L = uni(seqlens[b]);
      const char* rope_src = nullptr;
#pragma unroll
      for (int q = 0; q < kRowsPerWave; ++q) {
        const int j2 = wave + kWaves * q;
        int tok = uni(idx[min(tok0 + j2, tl_last)]);
        if ((unsigned)tok >= (unsigned)L) {
          atomicOr(err, kErrIndex);
          tok = 0;
        }
        const char* row = reinterpret_cast<const char*>(kc) + row_of(b, tok) * kRowBytes;
        lds_dma16(row + 16 * lane, dst + j2 * kRowPad);
        if (rq == q) rope_src = row;
      }
      if (lane < 32) lds_dma16(rope_src + 1024 + 16 * rchunk, rope_dst);
    }
  };

  // LDS read addresses of the MFMA operands: one base per operand, the rest immediate
  //   K, half hh, k-step ks < 16: token 16hh + lr, dims 32ks + 8lg -> lr*1040 + 16lg + hh*16*1040 + 64ks
  //   rope, half hh, k-step 16 + r: token t = 16hh + lr, chunk 4r + lg, stored by wave t%8 at slot t/8
  //     -> rope + (lr%8)*544 + (lr/8)*128 + 16 (lg ^ lr/8) + hh*256 + r*64
  //   V, dv group g4, slot i: token tau(lg, i) = 4lg + i (i < 4), 16 + 4lg + i-4 (i >= 4),
  //     chunk 16 g4 + lr -> (4lg*1040 + 16lr) + (i<4 ? i : 12 + i)*1040 + 256 g4
  const uint32_t kbase = lr * kRowPad + 16 * lg;
  const uint32_t rbase = kRopeOff + (lr & 7) * kRopeWave + 128 * (lr >> 3) + 16 * (lg ^ (lr >> 3));
  const uint32_t vbase = 4 * lg * kRowPad + 16 * lr + 512 * half;  // this wave's dv half

  // Q^T operand: lane holds head 16 hg + lr, dims 288 half + 32 j + 8 lg .. +8.
  // The q loads are followed by kDmaPerWave stores of zero into the unused
  // words 4, 8, .., 20 of the workspace header: the compiler counts those (it
  // does not see the asm transfers), so it waits for q with vmcnt(kDmaPerWave),
  // which leaves exactly the next tile's transfers in flight, instead of vmcnt(0).
  u32x4 qv[kKHalf];
  auto load_q = [&](int unit) {
    const size_t row = (size_t)(unit / hblocks) * p.hq + (size_t)(unit % hblocks) * kHeads + hg * kHG + lr;
    const uint16_t* qp = qg + row * kDqk + 8 * lg + 32 * kKHalf * half;
#pragma unroll
    for (int j = 0; j < kKHalf; ++j) qv[j] = *reinterpret_cast<const u32x4*>(qp + 32 * j);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) err[4 * (i + 1)] = 0;  // every lane, same word: no branch
    asm volatile("" ::: "memory");
  };

  // ------------------------------------------------ the block stream
  // Every iteration issues exactly one tile fetch (kDmaPerWave transfers per
  // wave), after the score products and after the next item's q loads, so the
  // loads outstanding at the top of iteration k are, oldest first: tile k,
  // [the q loads of iteration k-1], tile k+1.  Past the last block the fetch
  // re-reads the current block into the free stage (never read again).
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
  load_q(cur.unit);
  fetch(pI, p_j, stage<0>());
  advance(pI, p_it, p_j, p_nb);
  if (nblk > 1) {
    fetch(pI, p_j, stage<1>());
    advance(pI, p_it, p_j, p_nb);
  } else {
    fetch(cur, 0, stage<1>());
  }

  float m_run = -INFINITY, l_run = 0.f;  // per lane: head lr of the pair (four lanes per head)
  f32x4 o[2][8];                          // dv group 2 half + gg, column c: dv = 128 g4 + 8 lr + c; rows heads 4lg+r
#pragma unroll
  for (int gg = 0; gg < 2; ++gg)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[gg][c] = f32x4{};
  bool fresh = true;  // no block of the current item seen yet

  // one block: tile k in stage ST; the fetch two blocks ahead goes to stage (ST + 2) % 3
  auto step = [&](auto stage_c, int k) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_c)::value;
    // tile k (and any q loads, issued before tile k+1's transfers) has landed
    // for every wave; tile k-1's stage and the exchange buffer are free
    wait_vmcnt<kDmaPerWave>();
    wait_lds();
    barrier();
    const char* tile = stage<ST>();
    const int tok0 = cur.tb + cur_j * kBlk;
    const int nv = min(kBlk, cur.te - tok0);

    // partial S^T of this wave's dims half, then the pair's sum
    f32x4 s0 = {}, s1 = {};
    if (half == 0)
      scores_half<0>(tile, kbase, rbase, qv, s0, s1);
    else
      scores_half<1>(tile, kbase, rbase, qv, s0, s1);
    xch[wave][0][lane] = s0;
    xch[wave][1][lane] = s1;
    const bool item_ends = cur_j == cur_nb - 1;
    if (item_ends && k + 1 < nblk) {
      // q of the next item replaces this one as soon as the scores no longer need it
      load_q(uni(items[cur_it + 1].x));
    }
    if (k + 2 < nblk) {
      fetch(pI, p_j, stage<(ST + 2) % 3>());
      advance(pI, p_it, p_j, p_nb);
    } else {
      fetch(cur, cur_j, stage<(ST + 2) % 3>());
    }
    wait_lds();
    barrier();
    s0 += xch[wave ^ 1][0][lane];  // IEEE addition commutes: both waves of the pair get the same sum
    s1 += xch[wave ^ 1][1][lane];

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
          for (int gg = 0; gg < 2; ++gg)
#pragma unroll
            for (int c = 0; c < 8; ++c) o[gg][c][rr] *= a;
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

    // O += P V over this wave's dv half.  Rows past the item end hold a copy of
    // the last valid row (finite) and their probabilities are exactly 0, so
    // they add nothing.
    u32x4 vr[2][8];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        vr[gg][i] = *reinterpret_cast<const u32x4*>(tile + vbase + (i < 4 ? i : 12 + i) * kRowPad + 256 * gg);
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        // B operand of column 8 lr + c: element i = V[tau(lg, i)][col], two per word
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        u32x4 vb;
#pragma unroll
        for (int pi = 0; pi < 4; ++pi)
          vb[pi] = __builtin_amdgcn_perm(vr[gg][2 * pi + 1][c >> 1], vr[gg][2 * pi][c >> 1], sel);
        o[gg][c] = mfma16(pa, vb, o[gg][c]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    if (item_ends) {
      // -------- finish the item: this workgroup holds the whole piece
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      const size_t qrow = (size_t)cur.unit * kHeads;  // first head of the unit: (b Tq + t) Hq + 64 hb
      const int h0 = hg * kHG;                        // pair's first head in the unit
      if (cur.nsplit == 1) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int hh = 4 * lg + rr;
          const float inv = 1.f / __shfl(l_tot, hh);
          float* orow = out + (qrow + h0 + hh) * kDv + 256 * half + 8 * lr;
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            *reinterpret_cast<f32x4*>(orow + 128 * gg) =
                f32x4{o[gg][0][rr] * inv, o[gg][1][rr] * inv, o[gg][2][rr] * inv, o[gg][3][rr] * inv};
            *reinterpret_cast<f32x4*>(orow + 128 * gg + 4) =
                f32x4{o[gg][4][rr] * inv, o[gg][5][rr] * inv, o[gg][6][rr] * inv, o[gg][7][rr] * inv};
          }
        }
        if (half == 0 && lane < 16) lse[qrow + h0 + lane] = (m_run + __log2f(l_tot)) * kLn2;
      } else {
        float* ps = partials + (size_t)(cur.pbase + cur.split) * p.slot_floats;
        if (half == 0 && lane < 16) {
          ps[h0 + lane] = m_run;
          ps[kHeads + h0 + lane] = l_tot;
        }
        float* po = ps + partial_o_offset(kHeads) + (size_t)h0 * kDv + 256 * half;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int hh = 4 * lg + rr;
          float* orow = po + (size_t)hh * kDv + 8 * lr;
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            *reinterpret_cast<f32x4*>(orow + 128 * gg) = f32x4{o[gg][0][rr], o[gg][1][rr], o[gg][2][rr], o[gg][3][rr]};
            *reinterpret_cast<f32x4*>(orow + 128 * gg + 4) = f32x4{o[gg][4][rr], o[gg][5][rr], o[gg][6][rr], o[gg][7][rr]};
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
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
          for (int c = 0; c < 8; ++c) o[gg][c] = f32x4{};
        fresh = true;
      }
    } else {
      ++cur_j;
    }
  };
  for (int k = 0; k < nblk; k += 3) {
    step(IC<0>{}, k);
    if (k + 1 < nblk) step(IC<1>{}, k + 1);
    if (k + 2 < nblk) step(IC<2>{}, k + 2);
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
  if (a.mode == CC_MODE_MLA_SPARSE) {
    mla::mla_decode_kernel<true><<<a.workers, mla::kThreads, 0, s>>>(
        p, a.wg_off, a.items, a.unit_nsplit, a.unit_pbase, a.q, a.k, a.block_table, a.seqlens, a.indices,
        a.out, a.lse, a.err, a.counters, a.partials, a.timeline);
  } else {
    mla::mla_decode_kernel<false><<<a.workers, mla::kThreads, 0, s>>>(
        p, a.wg_off, a.items, a.unit_nsplit, a.unit_pbase, a.q, a.k, a.block_table, a.seqlens, a.indices,
        a.out, a.lse, a.err, a.counters, a.partials, a.timeline);
  }
  return hipGetLastError();
}

}  // namespace cc
