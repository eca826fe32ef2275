// Persistent split-KV GQA decode attention for gfx950 (MI355X).
//
// One workgroup of 8 wavefronts per compute unit runs the equal chunk of KV
// tiles the host plan gave it, so the whole batch is one wave with no tail
// (CSDN Q&A on waves and FlashMLA's Stream-K, "Summary").  Pieces of a
// sequence that other compute units also work on are merged inside this
// kernel by whichever piece arrives last (MeldKernel summary, "Core method":
// just-in-time reduction, no separate reduction kernel).  The softmax is the
// streaming form that keeps the result exact while fused (fusion tutorial,
// FlashAttention section).
//
// Inside a workgroup the chunk is cut again into 8 equal contiguous runs of
// 32-token blocks, one per wave.  A wave streams its run through a private
// LDS slot: the next block's K and V rows go HBM -> LDS with
// global_load_lds_dwordx4 (no registers held while in flight) while the
// current block, read back with ds_read_b128, computes:
//   S^T[token][head] = K[token][:] . Q[head][:]   v_mfma_f32_16x16x32_bf16
//   O[head][dv]     += P[head][token] . V[token][dv]
// Each lane fetches exactly the 16 bytes it later needs as an MFMA operand, so
// LDS reads are conflict-free and need no barrier.  Computing S^T puts each
// head's 8 scores of a block in one lane in exactly the A-operand layout P
// needs, so the softmax needs no data movement beyond two cross-lane max
// steps; V is transposed in registers with bit operations.
// Items a wave cannot finish alone (shared with another wave, or split across
// compute units) leave their (m, l, o) in LDS; after one barrier the whole
// workgroup merges them and runs the arrival-counter protocol.
//
// Scores are kept in base 2: s2 = scale * log2(e) * q.k, lse = ln2 * (m2 + log2 l).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>

#include "../../include/crosscu.h"
#include "launch.h"
#include "merge.h"
#include "plan.h"

namespace cc {
namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlk = 32;  // tokens per wave step
constexpr int kPrefixMergeChunk = 4;  // splits per merge round in the shared-prefix kernel
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// two fp32 -> packed bf16 (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Marks a value the whole wave agrees on, so it lives in a scalar register and
// addresses built from it use the scalar-base load forms.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ size_t uni64(size_t x) {
  return (size_t)(uint32_t)uni((int)(uint32_t)x) | ((size_t)(uint32_t)uni((int)(uint32_t)(x >> 32)) << 32);
}

// Asynchronous copy global -> LDS: lane i's bytes from sbase + voff land at
// lds + i * bytes (sbase and lds wave-uniform, voff per lane).  Inline asm on
// purpose: the compiler's own wait insertion cannot tell the stream slots from
// the merge slots that reuse them and would put a full vmcnt wait (which also
// waits for every output store in flight) before each LDS read; the kernel
// waits for its transfers explicitly.  M0 carries the LDS address (the
// compiler uses M0 nowhere else in this kernel); one wait state separates its
// write from the transfer.  The KV cache is read once per decode, so the
// transfers carry the non-temporal cache policy (nt): on MI355X a streaming
// read of this kind reaches ~6.7 TB/s with it and ~5.7 TB/s without.
__device__ __forceinline__ void lds_dma16(const char* sbase, uint32_t voff, char* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_ptr)lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(voff), "s"(sbase), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const char* sbase, uint32_t voff, char* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_ptr)lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1 nt"
               :: "v"(voff), "s"(sbase), "s"(m0) : "memory", "m0");
}

// Id of the XCD this wave runs on (hardware register XCC_ID, low 4 bits).
__device__ __forceinline__ unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Per-head-dim geometry of one 32-token block in a wave's LDS slot.
template <int D>
struct Geo;
template <>
struct Geo<128> {
  using vvec = u32x4;                        // 8 bf16 of one V row per lane
  static constexpr int KS = 4;               // k-steps of 32 dims
  static constexpr int W = 8;                // dv columns per lane
  static constexpr int kBytes = 2 * KS * 1024;
  static constexpr int vDmaBytes = 16;       // bytes per lane per V transfer
  static constexpr int vDmas = 8;
  static constexpr int ring = kBytes + vDmas * 64 * vDmaBytes;  // 16 KiB
};
template <>
struct Geo<64> {
  using vvec = u32x2;                        // 4 bf16
  static constexpr int KS = 2;
  static constexpr int W = 4;
  static constexpr int kBytes = 2 * KS * 1024;
  static constexpr int vDmaBytes = 4;        // 8-byte LDS transfers do not exist: two of 4
  static constexpr int vDmas = 16;
  static constexpr int ring = kBytes + vDmas * 64 * vDmaBytes;  // 8 KiB
};

template <int D>
struct BlockRegs {
  u32x4 k[2][Geo<D>::KS];        // K rows (A operand), two 16-token halves
  typename Geo<D>::vvec v[8];    // V rows of tokens tau(lane/16, i)
};

struct Params {
  int hq, hkv, group, max_pages, num_pages, log2_page;
  // byte strides of the paged cache: a page, a KV head inside a page, and one
  // token of one head inside a page (token-major or head-major page layout)
  long long page_bytes;
  int head_bytes, token_bytes;
  float scale_log2;
  int slot_floats;   // floats per partial slot in the workspace
  int region_bytes;  // LDS bytes per wave (stream slot, later its merge slots)
  int reduce;
  int units;         // sequence units (b, g); items name shared-prefix unit p as units + p
};

// wave-uniform position in the chunk
struct Cursor {
  int it;     // item index
  int j;      // 32-token block inside the item
  int nb;     // blocks in the item (from the plan)
  int unit, tb, te, split;
  int lim;    // min(te, seqlens[b]): tokens at or past it are masked
  int bad;    // the plan does not match seqlens[b] for this item (an int: no padding)
  int nsplit; // pieces of the unit across the grid
  int pbase;  // first partial slot of the unit (split units)
  // shared-prefix plans: the KV head, the sequence whose block-table row is
  // read, the prefix unit (-1: a sequence's own unit) and its query rows
  int g, b0, pu, rows;
};

__device__ __forceinline__ int blocks_of(int tb, int te) { return (te - tb + kBlk - 1) / kBlk; }

// PREFIX: the plan has shared-prefix units (items with unit >= p.units): a
// prefix unit gathers the G query heads of up to 16 / G member sequences as
// its query rows over the prefix they share, and each member counts the
// prefix unit's pieces as splits of its own (the prefix table row: KV head,
// members, prefix length, pieces, member ids).  A member's own pieces are
// then splits too, wherever they sit in a chunk, so a wave that holds a whole
// piece of a split unit (prefix or own) finishes it itself: each member's
// output or partial, its arrival, and the merge of a member it completes.  A
// piece shared by waves goes through the LDS slots like any shared item.
template <int D, bool PREFIX>
__global__ void __launch_bounds__(kThreads, 1)
gqa_decode_kernel(const Params p, const int32_t* __restrict__ wg_off, const int4* __restrict__ items,
                  const int32_t* __restrict__ unit_nsplit, const int32_t* __restrict__ unit_pbase,
                  const int32_t* __restrict__ prefix_tab,
                  const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kc,
                  const uint16_t* __restrict__ vc, const int32_t* __restrict__ bt,
                  const int32_t* __restrict__ seqlens, float* __restrict__ out,
                  float* __restrict__ lse, int32_t* err, int32_t* counters, float* partials,
                  unsigned long long* timeline) {
  using GE = Geo<D>;
  constexpr int KS = GE::KS;
  constexpr int W = GE::W;
  using vvec = typename GE::vvec;
  extern __shared__ __attribute__((aligned(16))) char smem[];  // kWaves regions
  // arrivals one workgroup makes after its stream: one per split item, and
  // with shared prefixes one per member of each prefix item in the slots
  // (at most 8 such items of at most 16 members), plus those the waves put off
  // for the whole split pieces they finished (kWaveArrivals each)
  constexpr int kWaveArrivals = PREFIX ? 32 : 1;
  constexpr int kArrivals = PREFIX ? 2 * kWaves + 8 * kPrefixRows + kWaves * kWaveArrivals : 2 * kWaves;
  __shared__ int wave_arr[kWaves][kWaveArrivals][3];  // a wave's put-off arrivals: unit, nsplit, first slot
  __shared__ int wave_narr[kWaves];
  // a prefix item in a merge slot: per member, its unit, its first output
  // row, its splits and its first partial slot (filled when the slot is)
  constexpr int kMemSlots = PREFIX ? 2 * kWaves : 1;
  __shared__ int slot_mem[kMemSlots][kPrefixRows][4];
  __shared__ int slot_item[2 * kWaves];
  __shared__ int slot_meta[2 * kWaves][4];  // unit, split, nsplit, pbase (a prefix item: rows) of the slot's item
  __shared__ int done_units[kArrivals][3];  // units this workgroup completes: {pbase, nsplit, out row}
  __shared__ float slot_w[2 * kWaves][16];    // phase-1 weight of each merge slot, per head
  __shared__ float item_L[2 * kWaves][16];    // phase-1 sum L of each item, per head
  __shared__ float item_M[2 * kWaves][16];    // phase-1 max M of each item, per head
  __shared__ int it_slot[2 * kWaves];         // phase-1 items: first slot,
  __shared__ unsigned it_mask[2 * kWaves];    // the slots holding it,
  __shared__ int num_items;                   // and how many
  __shared__ int split_list[kArrivals][3];    // arrivals: unit, nsplit, first partial slot
  __shared__ int num_split;
  __shared__ int num_done;
  __shared__ int slots_ready;  // waves whose slot entries are written (no shared prefixes)
  __shared__ int waves_done;   // waves past their stream (no shared prefixes)

  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int G = p.group;
  // rows of a merge slot: a unit's G heads, or with shared prefixes the up
  // to 16 query rows of a prefix unit
  const int SR = PREFIX ? kPrefixRows : G;
  const int slot_stride = SR * (D + 2);  // floats of one (m, l, o) merge slot
  const int page_mask = (1 << p.log2_page) - 1;
  char* const region = smem + wave * p.region_bytes;
  auto merge_slot = [&](int sl) -> float* {
    return reinterpret_cast<float*>(smem + (sl >> 1) * p.region_bytes) + (sl & 1) * slot_stride;
  };

  unsigned long long* tl = timeline ? timeline + kTimelineWords * blockIdx.x : nullptr;
  if (tl && tid == 0) {
    tl[0] = __builtin_amdgcn_s_memrealtime();
    tl[5] = xcc_id();
  }
  const int i0 = uni(wg_off[blockIdx.x]), i1 = uni(wg_off[blockIdx.x + 1]);
  if (i0 >= i1) {
    if (tl && tid == 0) tl[1] = tl[2] = tl[3] = tl[4] = tl[6] = tl[7] = tl[0];
    return;
  }

  int nblk = 0;
  for (int i = i0; i < i1; ++i) {
    const int4 t = items[i];
    nblk += blocks_of(uni(t.y), uni(t.z));
  }
  const int s = (int)(((long long)nblk * wave) / kWaves);
  const int e = (int)(((long long)nblk * (wave + 1)) / kWaves);

  if (tid < 2 * kWaves) slot_item[tid] = -1;
  if (PREFIX && tid < kWaves) wave_narr[tid] = 0;
  if (tid == 0) {
    slots_ready = 0;
    waves_done = 0;
  }
  __syncthreads();

  auto load_item = [&](Cursor& c, int it) {
    const int4 t = items[it];
    c.it = it;
    c.unit = uni(t.x);
    c.tb = uni(t.y);
    c.te = uni(t.z);
    c.split = uni(t.w);
    c.nb = blocks_of(c.tb, c.te);
    if constexpr (PREFIX) {
      if (c.unit >= p.units) {
        // a shared-prefix piece: its unit's row of the prefix table.  The
        // plan must still match the lengths: the prefix's last piece ends at
        // the prefix, every member holds the prefix, and a member whose last
        // split this piece is has no tokens past it.
        c.pu = c.unit - p.units;
        const int32_t* r = prefix_tab + kPrefixWords * c.pu;
        c.g = uni(r[0]);
        const int nmem = uni(r[1]), Lp = uni(r[2]);
        c.nsplit = uni(r[3]);
        c.pbase = -1;
        c.b0 = uni(r[4]);
        c.rows = nmem * G;
        c.bad = c.te > Lp || (c.split == c.nsplit - 1 && c.te != Lp);
        for (int j = 0; j < nmem; ++j) {
          const int b = uni(r[4 + j]);
          const int L = uni(seqlens[b]), ns = uni(unit_nsplit[b * p.hkv + c.g]);
          c.bad = c.bad || L < Lp || (c.split == ns - 1 && L != Lp);
        }
        c.lim = min(c.te, Lp);
        if (c.bad && lane == 0) atomicOr(err, kErrSeqlen);
        return;
      }
      c.pu = -1;
      c.b0 = c.unit / p.hkv;
      c.g = c.unit - c.b0 * p.hkv;
      c.rows = G;
    }
    c.nsplit = uni(unit_nsplit[c.unit]);
    c.pbase = uni(unit_pbase[c.unit]);
    // a plan built for other lengths: a piece past the sequence end, or the
    // unit's last piece ending before it.  Such an item is flagged and its
    // running sum starts at NaN, so the unit's out and lse come out NaN
    // through every merge; tokens past the sequence end are masked.
    const int L = uni(seqlens[c.unit / p.hkv]);
    c.bad = c.te > L || (c.split == c.nsplit - 1 && c.te != L);
    c.lim = min(c.te, L);
    if (c.bad && lane == 0) atomicOr(err, kErrSeqlen);
  };

  auto page_of = [&](const int32_t* row, int tok) {
    int lp = min(tok >> p.log2_page, p.max_pages - 1);
    int pg = uni(row[lp]);
    if ((unsigned)pg >= (unsigned)p.num_pages) {
      atomicOr(err, kErrPage);
      pg = pg < 0 ? 0 : p.num_pages - 1;
    }
    return pg;
  };

  // Every 16-token half of a block lies inside one page (blocks start at
  // multiples of 16 — an item starts at a multiple of 32, or of the page size
  // past a shared prefix — and pages hold a power of two >= 16 tokens), so a lane's
  // offset from the half's first row never changes: only the two half bases,
  // wave-uniform, move from block to block.  A half with no valid token
  // reads half 0 again; rows past the valid length stay inside their page and
  // are masked (scores) or zeroed (values) in compute.
  const uint32_t tstride = (uint32_t)p.token_bytes;
  const uint32_t koff = lr * tstride + lg * 16;
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (4 * lg + i) * tstride + W * lr * (uint32_t)sizeof(uint16_t);

  // Global sources of one block: the K and V rows of its two 16-token halves.
  struct Src {
    const char* k0;
    const char* k1;
    const char* v0;
    const char* v1;
  };
  auto sources = [&](const Cursor& c) {
    // a prefix unit reads its first member's block-table row (every member
    // names the same prefix pages)
    const int b = uni(PREFIX ? c.b0 : c.unit / p.hkv);
    const int g = uni(PREFIX ? c.g : c.unit - b * p.hkv);
    const int32_t* row = bt + (size_t)b * p.max_pages;
    const int tok0 = c.tb + c.j * kBlk;
    const int h1 = (tok0 + 16 < c.lim) ? tok0 + 16 : tok0;
    const size_t go = (size_t)g * p.head_bytes;
    // wave-uniform by construction; through readfirstlane so that the
    // transfers' scalar base operands stay scalar whatever the compiler infers
    const size_t o0 = uni64((size_t)page_of(row, tok0) * p.page_bytes + go + (size_t)(tok0 & page_mask) * tstride);
    const size_t o1 = uni64((size_t)page_of(row, h1) * p.page_bytes + go + (size_t)(h1 & page_mask) * tstride);
    Src S;
    S.k0 = reinterpret_cast<const char*>(kc) + o0;
    S.k1 = reinterpret_cast<const char*>(kc) + o1;
    S.v0 = reinterpret_cast<const char*>(vc) + o0;
    S.v1 = reinterpret_cast<const char*>(vc) + o1;
    return S;
  };

  // Stream one block into this wave's LDS slot.
  auto fetch = [&](const Src& S) {
    // K: lane takes token lr of each half, dims 32*ks + 8*lg .. +8
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      lds_dma16(S.k0 + ks * 64, koff, region + ks * 1024);
      lds_dma16(S.k1 + ks * 64, koff, region + (KS + ks) * 1024);
    }
    // V: lane takes tokens tau(lg, i) = 4lg+i (i<4), 16+4lg+(i-4) (i>=4), dims W*lr .. +W
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const char* base = i < 4 ? S.v0 : S.v1;
      if constexpr (GE::vDmaBytes == 16) {
        lds_dma16(base, voff[i & 3], region + GE::kBytes + i * 1024);
      } else {
        lds_dma4(base, voff[i & 3], region + GE::kBytes + (2 * i) * 256);
        lds_dma4(base + 4, voff[i & 3], region + GE::kBytes + (2 * i + 1) * 256);
      }
    }
  };

  // The streamed block, back from LDS into operand registers.
  auto unpack = [&](BlockRegs<D>& r) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        r.k[h][ks] = *reinterpret_cast<const u32x4*>(region + (h * KS + ks) * 1024 + lane * 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (GE::vDmaBytes == 16) {
        r.v[i] = *reinterpret_cast<const u32x4*>(region + GE::kBytes + i * 1024 + lane * 16);
      } else {
        r.v[i] = u32x2{*reinterpret_cast<const uint32_t*>(region + GE::kBytes + (2 * i) * 256 + lane * 4),
                       *reinterpret_cast<const uint32_t*>(region + GE::kBytes + (2 * i + 1) * 256 +
                                                          lane * 4)};
      }
    }
  };

  // (m, l, o) of this wave for item `it` into merge slot sl (real heads only).
  // slot layout: m[SR], l[SR], o[SR][D] (rows past the item's own are not written)
  auto put_slot = [&](int sl, const Cursor& cu, float m, float l, const f32x4* o) {
    float* sb = merge_slot(sl);
    const int rows = PREFIX ? cu.rows : G;
    if (lane < rows) {
      sb[lane] = m;
      sb[SR + lane] = l;
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int hh = 4 * lg + rr;
      if (hh < rows) {
#pragma unroll
        for (int cc = 0; cc < W; ++cc) sb[2 * SR + hh * D + W * lr + cc] = o[cc][rr];
      }
    }
    if constexpr (PREFIX) {
      if (cu.pu >= 0) {
        const int32_t* r = prefix_tab + kPrefixWords * cu.pu;
        if (lane < uni(r[1])) {
          const int b = r[4 + lane], mu = b * p.hkv + cu.g;
          slot_mem[sl][lane][0] = mu;
          slot_mem[sl][lane][1] = b * p.hq + cu.g * G;
          slot_mem[sl][lane][2] = unit_nsplit[mu];
          slot_mem[sl][lane][3] = unit_pbase[mu];
        }
      }
    }
    if (PREFIX && lane == 0) {  // (without shared prefixes written before the stream)
      slot_item[sl] = cu.it;
      slot_meta[sl][0] = cu.unit;
      slot_meta[sl][1] = cu.split;
      slot_meta[sl][2] = cu.nsplit;
      slot_meta[sl][3] = cu.pu >= 0 ? cu.rows : cu.pbase;  // a prefix item's query rows
    }
  };

  // A whole piece of a split unit in one wave (with shared prefixes any
  // piece can be one: a prefix piece, and a sequence's own piece, which the
  // prefix makes a split, anywhere in a chunk).  Its rows belong to members
  // j = row / G: the prefix unit's members, or the sequence itself.  Each
  // member's rows go out as its output when it has no other split, else as
  // its partial of split cu.split.  The arrivals for those partials are put
  // off to the end of the workgroup's stream (the wave's list in LDS), so
  // the stream does not stop for them; only when the wave's list is full
  // does the wave arrive itself, once its stores are complete, and merge any
  // member it completes.
  int narr = 0;  // this wave's put-off arrivals
  auto wave_finish = [&](const Cursor& cu, float m, float l, const f32x4* o) {
    if constexpr (PREFIX) {
      const bool pre = cu.pu >= 0;
      const int32_t* r = prefix_tab + kPrefixWords * (pre ? cu.pu : 0);
      const int nmem = pre ? uni(r[1]) : 1;
      const int o_off = partial_o_offset(G);
      unsigned arrive = 0;  // members with a partial (bit j)
      for (int j = 0; j < nmem; ++j) {
        const int b = pre ? uni(r[4 + j]) : cu.b0;
        const int mu = b * p.hkv + cu.g;
        const int ns = uni(unit_nsplit[mu]);
        const size_t row0 = (size_t)b * p.hq + (size_t)cu.g * G;  // the member's first output row
        if (ns == 1) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int hh = 4 * lg + rr;
            const float inv = 1.f / __shfl(l, hh);
            if (hh / G == j) {
              float* op = out + (row0 + hh - j * G) * D + W * lr;
#pragma unroll
              for (int c4 = 0; c4 < W; c4 += 4)
                *reinterpret_cast<f32x4*>(op + c4) = f32x4{o[c4][rr] * inv, o[c4 + 1][rr] * inv,
                                                           o[c4 + 2][rr] * inv, o[c4 + 3][rr] * inv};
            }
          }
          if (lane < kPrefixRows && lane / G == j) lse[row0 + lane - j * G] = (m + __log2f(l)) * kLn2;
        } else {
          float* ps = partials + (size_t)(uni(unit_pbase[mu]) + cu.split) * p.slot_floats;
          if (lane < kPrefixRows && lane / G == j) {
            partial_store(ps + lane - j * G, m);
            partial_store(ps + G + lane - j * G, l);
          }
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int hh = 4 * lg + rr;
            if (hh / G == j) {
#pragma unroll
              for (int cc = 0; cc < W; ++cc) partial_store(ps + o_off + (hh - j * G) * D + W * lr + cc, o[cc][rr]);
            }
          }
          if (p.reduce == CC_REDUCE_FUSED && narr < kWaveArrivals) {
            if (lane == 0) {
              wave_arr[wave][narr][0] = mu;
              wave_arr[wave][narr][1] = ns;
              wave_arr[wave][narr][2] = uni(unit_pbase[mu]);
            }
            ++narr;
          } else {
            arrive |= 1u << j;
          }
        }
      }
      if (arrive && p.reduce == CC_REDUCE_FUSED) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are complete
        const bool on = lane < nmem && ((arrive >> lane) & 1);
        int b = 0, mu = 0, ns = 0, old = -1;
        if (on) {
          b = pre ? r[4 + lane] : cu.b0;
          mu = b * p.hkv + cu.g;
          ns = unit_nsplit[mu];
          old = atomicAdd(&counters[kCounterStride * mu], 1);
        }
        const bool done = on && old == ns - 1;
        if (done) __hip_atomic_store(&counters[kCounterStride * mu], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (unsigned long long db = __ballot(done); db; db &= db - 1) {
          const int j = __builtin_ctzll(db);
          const int bj = __builtin_amdgcn_readlane(b, j), muj = __builtin_amdgcn_readlane(mu, j);
          const int nsj = __builtin_amdgcn_readlane(ns, j);
          const float* pb = partials + (size_t)uni(unit_pbase[muj]) * p.slot_floats;
          merge_unit_direct<64, kPrefixMergeChunk>(pb, nsj, (size_t)bj * p.hq + (size_t)cu.g * G, p.slot_floats, G,
                                                   D, out, lse, lane);
        }
      }
    }
  };

  // Wave 0's list of the items left in merge slots, in slot order: each
  // distinct item's first slot and the slots holding it, and the split ones
  // among them (unit, nsplit, first partial slot).
  auto scan_slots = [&]() {
    // one lane per merge slot, compacted with ballots so the list stays in
    // slot order
    const int me = lane < 2 * kWaves ? slot_item[lane] : -1;
    unsigned mask = 0;
    bool before = false;
#pragma unroll
    for (int t = 0; t < 2 * kWaves; ++t) {
      const bool same = __builtin_amdgcn_readlane(me, t) == me;
      mask |= (unsigned)same << t;
      before |= same && t < lane;
    }
    const bool first = lane < 2 * kWaves && me >= 0 && !before;
    const int ns = first ? slot_meta[lane][2] : 0;
    // (a prefix item's arrivals are its members', listed below)
    const bool split = ns > 1 && (!PREFIX || slot_meta[lane][0] < p.units);
    const unsigned long long fb = __ballot(first), sb = __ballot(split);
    const unsigned long long below = (1ull << lane) - 1;
    if (first) {
      const int n = __popcll(fb & below);
      it_slot[n] = lane;
      it_mask[n] = mask;
    }
    if (split) {
      const int k = __popcll(sb & below);
      split_list[k][0] = slot_meta[lane][0];
      split_list[k][1] = ns;
      split_list[k][2] = slot_meta[lane][3];
    }
    int nsp = __popcll(sb);
    if constexpr (PREFIX) {
      // each member with other splits arrives once for a prefix item
      for (unsigned long long pm = __ballot(first && slot_meta[lane][0] >= p.units); pm; pm &= pm - 1) {
        const int sl = __builtin_ctzll(pm);
        const int nmem = uni(slot_meta[sl][3]) / G;
        for (int j0 = 0; j0 < nmem; j0 += 64) {
          const int j = j0 + lane;
          int mu = 0, ns2 = 0, pb = 0;
          if (j < nmem) {
            mu = slot_mem[sl][j][0];
            ns2 = slot_mem[sl][j][2];
            pb = slot_mem[sl][j][3];
          }
          const bool add = j < nmem && ns2 > 1;
          const unsigned long long ab = __ballot(add);
          if (add) {
            const int k = nsp + __popcll(ab & below);
            split_list[k][0] = mu;
            split_list[k][1] = ns2;
            split_list[k][2] = pb;
          }
          nsp += __popcll(ab);
        }
      }
    }
    if constexpr (PREFIX) {
      // the waves' put-off arrivals
      for (int w = 0; w < kWaves; ++w) {
        const int n = wave_narr[w];
        for (int i = lane; i < n; i += 64) {
          split_list[nsp + i][0] = wave_arr[w][i][0];
          split_list[nsp + i][1] = wave_arr[w][i][1];
          split_list[nsp + i][2] = wave_arr[w][i][2];
        }
        nsp += n;
      }
    }
    if (lane == 0) {
      num_items = __popcll(fb);
      num_split = nsp;
    }
  };

  if (s < e) {
    // ------------------------------------------------ the wave's run [s, e)
    Cursor c;
    {
      int it = i0, cum = 0;
      load_item(c, it);
      while (cum + c.nb <= s) {
        cum += c.nb;
        load_item(c, ++it);
      }
      c.j = s - cum;
    }
    const int first_it = c.it;

    // Q^T operand of a unit: lane holds head lr, dims 32*ks + 8*lg .. +8 (zero rows past G)
    // (a prefix unit's row lr is head lr % G of member lr / G)
    auto load_q = [&](const Cursor& cu, u32x4* qd) {
      int b, g, hh, rows;
      if constexpr (PREFIX) {
        g = cu.g;
        rows = cu.rows;
        hh = min(lr, rows - 1);
        b = cu.b0;
        if (cu.pu >= 0) {
          // member ids as scalars, the lane's one picked out by selects
          const int32_t* r = prefix_tab + kPrefixWords * cu.pu + 4;
          const int jm = hh / G;
#pragma unroll
          for (int j = 1; j < kPrefixRows; ++j) {
            const int v = uni(r[j]);
            b = jm == j ? v : b;
          }
          hh -= jm * G;
        }
      } else {
        b = cu.unit / p.hkv;
        g = cu.unit - b * p.hkv;
        rows = G;
        hh = min(lr, G - 1);
      }
      const uint16_t* qp = qg + ((size_t)b * p.hq + (size_t)g * G + hh) * D + lg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 t = *reinterpret_cast<const u32x4*>(qp + ks * 32);
        qd[ks] = lr < rows ? t : u32x4{0, 0, 0, 0};
      }
    };

    u32x4 qv[KS], qn[KS];
    load_q(c, qv);
    fetch(sources(c));
    if constexpr (!PREFIX) {
      // A wave's merge slots hold its first and last items unless it finishes
      // an item alone (the whole item, unsplit, written out directly); its
      // middle items are whole units.  Without shared prefixes that is known
      // from the plan: the slot entries are written here, under the first
      // transfers' latency, and the first wave to end its stream builds the
      // merge list from them while the others still stream (not after the
      // workgroup's last wave, on the critical path).
      Cursor z = c;
      int itz = c.it, cz = s - c.j;  // cz: the chunk block where item itz starts
      while (cz + z.nb < e) {        // block e - 1 lies in item itz
        cz += z.nb;
        load_item(z, ++itz);
      }
      auto claim = [&](int sl, const Cursor& cu, bool whole) {
        if (!(whole && cu.nsplit == 1) && lane == 0) {
          slot_item[sl] = cu.it;
          slot_meta[sl][0] = cu.unit;
          slot_meta[sl][1] = cu.split;
          slot_meta[sl][2] = cu.nsplit;
          slot_meta[sl][3] = cu.pbase;
        }
      };
      claim(2 * wave, c, c.j == 0 && s - c.j + c.nb <= e);
      if (itz != c.it) claim(2 * wave + 1, z, cz + z.nb <= e);
      if (lane == 0) __hip_atomic_fetch_add(&slots_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }

    // the first item's state when it is neither written out nor the last item
    bool stashed = false;
    Cursor c_first = c;
    float m_first = 0.f, l_first = 0.f;
    f32x4 o_first[W];

    int k = s;
    for (;;) {
      // -------- item c.it, blocks c.j .. jend-1 of it
      const int j0 = c.j;
      const int jend = min(c.nb, c.j + (e - k));
      float m_run = -INFINITY, l_run = c.bad ? __builtin_nanf("") : 0.f;
      f32x4 o[W];
#pragma unroll
      for (int cc = 0; cc < W; ++cc) o[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
      Cursor n = c;
      for (; c.j < jend; ++c.j, ++k) {
        const bool more = k + 1 < e;
        Src S{};
        if (more) {  // next block's sources (scalar loads, hidden under the DMA in flight)
          if (c.j + 1 < c.nb) {
            n.j = c.j + 1;
          } else {  // the next block opens the next item: fetch its q as well
            load_item(n, c.it + 1);
            n.j = 0;
            load_q(n, qn);
          }
          S = sources(n);
        }
        BlockRegs<D> cur;
        wait_vmem();  // block k is in the slot (and any q loads landed)
        unpack(cur);
        wait_lds();   // slot read: it may be refilled
        if (more) fetch(S);

        // S^T = K Q^T for the block's two 16-token halves
        const int tok0 = c.tb + c.j * kBlk;
        const int nv = min(kBlk, c.lim - tok0);  // valid tokens in the block
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s0 = mfma_bf16(cur.k[0][ks], qv[ks], s0);
          s1 = mfma_bf16(cur.k[1][ks], qv[ks], s1);
        }
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = (4 * lg + i < nv) ? s0[i] * p.scale_log2 : -INFINITY;
          x[4 + i] = (16 + 4 * lg + i < nv) ? s1[i] * p.scale_log2 : -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - mnew);
        float pr[8];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pr[i] = fast_exp2(x[i] - mnew);
          psum += pr[i];
        }
        l_run = l_run * alpha + psum;
        m_run = mnew;
        const u32x4 pa = {pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]), pack_bf16(pr[4], pr[5]),
                          pack_bf16(pr[6], pr[7])};

        // O = alpha * O + P V   (rows of O are heads 4*lg + rr)
        if (nv < kBlk) {  // rows past the end may hold anything: zero them
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int rel = (i < 4) ? 4 * lg + i : 16 + 4 * lg + (i - 4);
            if (rel >= nv) cur.v[i] = vvec{};
          }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float a = __shfl(alpha, 4 * lg + rr);
#pragma unroll
          for (int cc = 0; cc < W; ++cc) o[cc][rr] *= a;
        }
#pragma unroll
        for (int cc = 0; cc < W; ++cc) {
          u32x4 vb;
#pragma unroll
          for (int pi = 0; pi < 4; ++pi) {
            const uint32_t a0 = cur.v[2 * pi][cc >> 1];
            const uint32_t a1 = cur.v[2 * pi + 1][cc >> 1];
            vb[pi] = (cc & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
          }
          o[cc] = mfma_bf16(pa, vb, o[cc]);
        }
      }
      --c.j;  // last block of this item run by the wave

      // -------- end of this wave's part of the item
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      const bool whole = j0 == 0 && c.j == c.nb - 1;
      if (PREFIX && whole && (c.pu >= 0 || c.nsplit > 1)) {
        wave_finish(c, m_run, l_tot, o);
      } else if (whole && c.nsplit == 1) {
        const int b = c.unit / p.hkv, g = c.unit - (c.unit / p.hkv) * p.hkv;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int hh = 4 * lg + rr;
          const float inv = 1.f / __shfl(l_tot, hh);
          if (hh < G) {
            float* op = out + ((size_t)b * p.hq + (size_t)g * G + hh) * D + W * lr;
#pragma unroll
            for (int c4 = 0; c4 < W; c4 += 4) {
              *reinterpret_cast<f32x4*>(op + c4) = f32x4{o[c4][rr] * inv, o[c4 + 1][rr] * inv,
                                                         o[c4 + 2][rr] * inv, o[c4 + 3][rr] * inv};
            }
          }
        }
        if (lane < G) lse[(size_t)b * p.hq + (size_t)g * G + lane] = (m_run + __log2f(l_tot)) * kLn2;
      } else if (k < e) {
        // only a wave's first and last items can be shared or split; this is
        // the first and more follow: keep it until the slot stops streaming
        stashed = true;
        c_first = c;
        m_first = m_run;
        l_first = l_tot;
#pragma unroll
        for (int cc = 0; cc < W; ++cc) o_first[cc] = o[cc];
      } else {
        put_slot(2 * wave + (c.it == first_it ? 0 : 1), c, m_run, l_tot, o);
      }
      if (k >= e) break;
      c = n;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qv[ks] = qn[ks];
    }
    if (stashed) put_slot(2 * wave, c_first, m_first, l_first, o_first);
    if (PREFIX && lane == 0) wave_narr[wave] = narr;
  }
  if constexpr (!PREFIX) {
    // a wave with no blocks holds no slot; the first wave past its stream
    // builds the merge list once every wave's entries are in (each wave
    // writes them before it streams, so the wait ends)
    if (s >= e && lane == 0)
      __hip_atomic_fetch_add(&slots_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    int first = 0;
    if (lane == 0)
      first = __hip_atomic_fetch_add(&waves_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
    if (uni(first)) {
      while (__hip_atomic_load(&slots_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kWaves)
        __builtin_amdgcn_s_sleep(1);
      scan_slots();
    }
  }

  __syncthreads();
  if (tl && tid == 0) tl[1] = __builtin_amdgcn_s_memrealtime();

  // ------------------------------------------------ workgroup-level merges
  // Phase 1: every item the waves left in LDS is merged over its waves and
  // written out (whole unit) or handed on as this piece's partial.  All items
  // at once: (a) one thread per (item, head) takes the max over the item's
  // slots, the sum L and each slot's weight exp2(m - M); (b) after a barrier a
  // flat loop over (item, element) adds the weighted outputs in slot (token)
  // order.  Only the slots that hold an item are read.
  if (PREFIX && tid < 64) scan_slots();
  __syncthreads();
  if (tl && tid == 0) tl[6] = __builtin_amdgcn_s_memrealtime();
  const int nit = uni(num_items);
  const int GD = G * D;
  const int SD = SR * D;  // elements of a slot's output (rows past an item's own are skipped)
  // One lane per (item, row, merge slot), the 16 slots of a row in 16
  // consecutive lanes: a slot's (m, l), then the row's max M and sum
  // L = sum l exp2(m - M) by butterflies inside the 16 lanes (every lane of a
  // group takes part: groups are all valid or all past the end).
  static_assert(2 * kWaves == 16, "one lane per merge slot in groups of 16");
  for (int base = 0; base < nit * SR * 16; base += kThreads) {
    const int idx = base + tid;
    const bool valid = idx < nit * SR * 16;
    const int t = idx & 15, r = idx >> 4;
    const int ii = valid ? r / SR : 0, hh = valid ? r - ii * SR : 0;
    const bool on = valid && ((it_mask[ii] >> t) & 1);
    const float* sb = merge_slot(t);
    const float m = on ? sb[hh] : -INFINITY;
    const float l = on ? sb[SR + hh] : 0.f;
    float M = m;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 16));
    const float f = fast_exp2(m - M);  // 0 for slots of other items
    float L = l * f;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) L += __shfl_xor(L, o, 16);
    if (on) slot_w[t][hh] = f;
    if (valid && t == 0) {
      item_M[ii][hh] = M;
      item_L[ii][hh] = L;
    }
  }
  __syncthreads();
  if (tl && tid == 0) tl[7] = __builtin_amdgcn_s_memrealtime();
  for (int idx = tid; idx < nit * SD; idx += kThreads) {
    const int ii = uni(idx / SD);  // SR * D is a multiple of 64: one item per wave and pass
    const int e = idx - ii * SD, hh = e / D;
    const unsigned mask = uni(it_mask[ii]);
    const int sl0 = uni(it_slot[ii]);
    const int unit = uni(slot_meta[sl0][0]), split = uni(slot_meta[sl0][1]), ns = uni(slot_meta[sl0][2]);
    if (PREFIX && hh >= (unit >= p.units ? uni(slot_meta[sl0][3]) : G)) continue;  // rows of the item
    float O = 0.f;
    for (unsigned mm = mask; mm; mm &= mm - 1) {
      const int t = __builtin_ctz(mm);
      O += merge_slot(t)[2 * SR + e] * slot_w[t][hh];
    }
    const bool head_lane = e - hh * D == 0;
    if (PREFIX && unit >= p.units) {
      // a prefix item: row hh is head hh % G of member hh / G
      const int j = hh / G, hr = hh - j * G, col = e - hh * D;
      const size_t row = (size_t)slot_mem[sl0][j][1] + hr;
      if (slot_mem[sl0][j][2] == 1) {
        out[row * D + col] = O / item_L[ii][hh];
        if (head_lane) lse[row] = (item_M[ii][hh] + __log2f(item_L[ii][hh])) * kLn2;
      } else {
        float* pslot = partials + (size_t)(slot_mem[sl0][j][3] + split) * p.slot_floats;
        partial_store(pslot + partial_o_offset(G) + hr * D + col, O);
        if (head_lane) {
          partial_store(pslot + hr, item_M[ii][hh]);
          partial_store(pslot + G + hr, item_L[ii][hh]);
        }
      }
    } else if (ns == 1) {
      out[(size_t)unit * GD + e] = O / item_L[ii][hh];  // row of unit (b, g): b Hq + g G = unit G
      if (head_lane) lse[(size_t)unit * G + hh] = (item_M[ii][hh] + __log2f(item_L[ii][hh])) * kLn2;
    } else {
      float* pslot = partials + (size_t)(uni(slot_meta[sl0][3]) + split) * p.slot_floats;
      partial_store(pslot + partial_o_offset(G) + e, O);
      if (head_lane) {
        partial_store(pslot + hh, item_M[ii][hh]);
        partial_store(pslot + G + hh, item_L[ii][hh]);
      }
    }
  }
  if (tl && tid == 0) tl[2] = __builtin_amdgcn_s_memrealtime();
  if (p.reduce == CC_REDUCE_FUSED) {
    // Phase 2: every wave's partial stores are complete (device-coherent, see
    // partial_store), then one arrival per split item; the piece that
    // completes a unit merges it and resets its counter (every other piece has
    // arrived).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid < 64) {
      // one lane per arrival (64 at a time): the arrivals in one atomic
      // instruction; the lanes that completed their unit are compacted in
      // list order
      const int nsp = uni(num_split);
      int nd = 0;
      for (int i0a = 0; i0a < nsp; i0a += 64) {
        const int i = i0a + lane;
        const bool on = i < nsp;
        int unit = 0, ns = 0, old = -1;
        if (on) {
          unit = split_list[i][0];
          ns = split_list[i][1];
          old = atomicAdd(&counters[kCounterStride * unit], 1);
        }
        const bool done = on && old == ns - 1;
        const unsigned long long db = __ballot(done);
        if (done) {
          __hip_atomic_store(&counters[kCounterStride * unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int d = nd + __popcll(db & ((1ull << lane) - 1));
          done_units[d][0] = split_list[i][2];
          done_units[d][1] = ns;
          done_units[d][2] = unit * G;  // output row of unit (b, g): b Hq + g G
        }
        nd += __popcll(db);
      }
      if (lane == 0) num_done = nd;
    }
    __syncthreads();
    if (tl && tid == 0) tl[3] = __builtin_amdgcn_s_memrealtime();
    // Phase 3: the units this workgroup completed, merged together
    const int nd = uni(num_done);
    if (nd > 0) {
      // with shared prefixes a workgroup may complete many small units
      // (members): all at once.  Every merge of this kernel then takes its
      // splits 4 at a time (kPrefixMergeChunk, also in wave_finish), so the
      // bits of a unit do not depend on which workgroup completes it.
      if (PREFIX)
        merge_units_batched<kThreads, 2, kPrefixMergeChunk>(partials, done_units, nd, p.slot_floats, G, D, out, lse);
      else
        merge_units_grouped<kThreads>(partials, done_units, nd, p.slot_floats, G, D, out, lse,
                                      reinterpret_cast<float*>(smem));
    }
  }
  if (tl && tid == 0) {
    if (p.reduce != CC_REDUCE_FUSED) tl[3] = tl[2];
    tl[4] = __builtin_amdgcn_s_memrealtime();
  }
}

// Merge kernel of the split-then-combine comparison: one workgroup per unit.
constexpr int kCombineThreads = 256;
__global__ void __launch_bounds__(kCombineThreads)
combine_kernel(int hq, int hkv, int group, int hpu, int dv, int slot_floats,
               const int32_t* __restrict__ unit_nsplit, const int32_t* __restrict__ unit_pbase,
               const float* __restrict__ partials, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) float lds[merge_lds_floats(kCombineThreads, 128)];
  const int u = blockIdx.x;
  const int ns = unit_nsplit[u];
  if (ns <= 1) return;
  const int hb_per_kv = group / hpu;
  const int hb = u % hb_per_kv;
  const int g = (u / hb_per_kv) % hkv;
  const int bt = u / (hb_per_kv * hkv);  // b * q_tokens + t
  const size_t orow = (size_t)bt * hq + (size_t)g * group + (size_t)hb * hpu;
  merge_splits<kCombineThreads>(partials + (size_t)unit_pbase[u] * slot_floats, ns, slot_floats, hpu, dv,
                                out + orow * dv, lse + orow, lds);
}

__global__ void fill_zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

}  // namespace gqa

using namespace gqa;

template <int D, bool PREFIX>
hipError_t launch_gqa_kernel(const Params& p, const DecodeArgs& a, size_t lds, hipStream_t s) {
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gqa::gqa_decode_kernel<D, PREFIX>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipExtLaunchKernelGGL(gqa::gqa_decode_kernel<D, PREFIX>, dim3(a.workers), dim3(kThreads), (uint32_t)lds, s,
                        a.ev_start, a.ev_stop, 0u, p, a.wg_off, a.items, a.unit_nsplit, a.unit_pbase, a.prefix, a.q,
                        a.k, a.v, a.block_table, a.seqlens, a.out, a.lse, a.err, a.counters, a.partials, a.timeline);
  return hipGetLastError();
}

hipError_t launch_gqa(const DecodeArgs& a, hipStream_t s) {
  Params p;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.group = a.hq / a.hkv;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.log2_page = ilog2(a.page_size);
  const long long head_row = (long long)a.dqk * sizeof(uint16_t);
  p.page_bytes = (long long)a.page_size * a.hkv * head_row;
  if (a.kv_layout == CC_KV_HND) {  // [page][head][token][dim]
    p.head_bytes = (int)(a.page_size * head_row);
    p.token_bytes = (int)head_row;
  } else {                         // [page][token][head][dim]
    p.head_bytes = (int)head_row;
    p.token_bytes = (int)(a.hkv * head_row);
  }
  p.scale_log2 = a.scale_log2;
  p.slot_floats = a.slot_floats;
  p.reduce = a.reduce;
  p.units = a.units;
  const bool prefix = a.prefix_units > 0;
  const int ring = a.dqk == 128 ? Geo<128>::ring : Geo<64>::ring;
  const int slot_rows = prefix ? kPrefixRows : p.group;
  const int slots = 2 * slot_rows * (a.dqk + 2) * (int)sizeof(float);
  p.region_bytes = ((ring > slots ? ring : slots) + 15) & ~15;
  const size_t lds = (size_t)kWaves * p.region_bytes;
  if (a.dqk == 128)
    return prefix ? launch_gqa_kernel<128, true>(p, a, lds, s) : launch_gqa_kernel<128, false>(p, a, lds, s);
  return prefix ? launch_gqa_kernel<64, true>(p, a, lds, s) : launch_gqa_kernel<64, false>(p, a, lds, s);
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t s) {
  if (a.mode != CC_MODE_GQA) return launch_mla_combine(a, s);  // MLA partials hold fp16 rows
  hipExtLaunchKernelGGL(combine_kernel, dim3(a.units), dim3(kCombineThreads), 0u, s, a.ev_start, a.ev_stop, 0u,
                        a.hq, a.hkv, a.hq / a.hkv, a.hpu, a.dv, a.slot_floats, a.unit_nsplit, a.unit_pbase,
                        a.partials, a.out, a.lse);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  fill_zero_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<uint32_t*>(ptr), words);
  return hipGetLastError();
}

}  // namespace cc
