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
// A unit is one query token with all 128 heads, so every KV row is read from
// HBM once per query token.  Wave w owns heads 32w .. 32w+31 and runs both
// dense contractions on v_mfma_f32_32x32x16_bf16 tiles, one wave per SIMD with
// the whole register file:
//   S^T[32 tokens][32 heads] = K[32][576] . Q^T[576][32]   (36 k-steps; Q^T in
//     108 VGPRs and 9 KiB of LDS per wave for the whole item),
//   O^T[512][32 heads]      += V^T[512][32] . P^T[32][32]  (16 column blocks of
//     32 dv x 32 heads: 256 accumulators, held in AGPRs).
// S^T leaves lane (n, g) with head n's scores of tokens 8j + 4g + i, which is
// exactly the P^T operand of the two 16-token k-blocks of O^T once the tokens
// of a k-block are ordered {16b + 4g + i, 16b + 8 + 4g + i}.  Each lane of O^T
// belongs to one head, so softmax rescales are lane-local.  V^T operands come
// straight from gfx950's transposing LDS read (ds_read_b64_tr_b16): two reads
// give a lane 8 tokens of one dv column.
//
// A 32-token tile (36.5 KiB) streams HBM -> LDS with global_load_lds_dwordx4
// through a 3-stage ring, so two tiles are in flight while one computes.  Wave
// w moves tokens 8w .. 8w+7: each token's first 512 columns are one transfer
// into an LDS row placed so that both the K operand reads and the transposed
// V reads are bank-conflict free (every lane's address is one base register
// plus an immediate), and the 64 rope columns of
// its 8 tokens are one transfer into a [token][chunk] area whose 16-byte chunk
// c of token t sits at slot c ^ ((t >> 1) & 7), which keeps the rope operand
// reads conflict free.  The fetch needs no per-lane loads, so it never waits
// behind the transfers in flight.
//
// The running max is only moved when a head's block max exceeds it by more
// than 2^8 (in base 2): probabilities stay below 256, and the rescale of the
// accumulators happens on a handful of blocks per sequence.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>
#include <type_traits>

#include "../../include/crosscu.h"
#include "launch.h"
#include "merge.h"
#include "plan.h"

namespace cc {
namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeads = 128;                 // heads per unit (= per workgroup)
constexpr int kHW = 32;                     // heads per wave
constexpr int kDqk = 576, kDv = 512;
constexpr int kRowBytes = kDqk * 2;         // 1152
constexpr int kBlk = 32;                    // tokens per tile
constexpr int kKSteps = kDqk / 16;          // 36 k-steps of q.k
constexpr int kLatentSteps = 32;            // k-steps inside the first 512 columns
constexpr int kQReg = 27;                   // k-steps of Q^T held in registers (the rest in LDS)
// LDS row of token t (its first 512 columns): 1088 t + 16 ((t / 4) % 4).  Row
// starts fall on 16-byte bank slot 4 (t % 4) + (t / 4) % 4 modulo 256 bytes, so
// 16 consecutive tokens hit 16 different slots (K operand reads) and 4
// consecutive tokens start 64 bytes apart (transposed V reads): both conflict free.
__host__ __device__ constexpr int row_lds(int t) { return 1088 * t + 16 * ((t >> 2) & 3); }
constexpr int kRopeOff = 34816;             // >= row_lds(31) + 1024, 256-aligned
constexpr int kStageBytes = kRopeOff + kBlk * 128;   // 38912
static_assert(row_lds(kBlk - 1) + 1024 <= kRopeOff, "rows overlap the rope area");
constexpr int kRowsPerWave = kBlk / kWaves;          // 8
constexpr int kDmaPerWave = kRowsPerWave + 1;        // + 1 rope transfer
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLazy = 8.f;                // log2 headroom before the max is moved
constexpr int kPreS = 4;                    // K operand reads in flight ahead of the score MFMAs
constexpr int kPreV = 4;                    // V^T operands in flight ahead of the output MFMAs

__shared__ __attribute__((aligned(16))) char ring[3][kStageBytes];
__shared__ __attribute__((aligned(16))) char qlds[kWaves][(kKSteps - kQReg) * 1024];



// ---- The output accumulators: a0 .. a255, owned by inline asm.
// O^T block d (32 dv rows x 32 heads, 16 registers per lane) lives in
// a[16 d .. 16 d + 15] for the whole kernel.  Every instruction that touches
// them is inline asm below: the compiler itself never allocates an AGPR in this
// kernel (its values fit the 256 VGPRs; a test checks the generated code), and
// its register allocator cannot keep 256 accumulators in place once VALU code
// (the rescale, the reset) touches them.  Because the compiler does not see
// these registers, the asm carries the wait states CDNA3/4 require around an
// XDL (MFMA) result: 18 independent cycles before a VALU, memory or
// v_accvgpr_read access to it, 2 after a VALU write (v_accvgpr_write) before
// an MFMA reads it.  Back-to-back accumulation into the same block needs none.
template <class F, int... I>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}
// Declares a0 .. a255 used, so the launch reserves them (the asm statements
// below name them only in their text).
__device__ __forceinline__ void acc_reserve() {
  asm volatile("" :::
    "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15",
    "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31",
    "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47",
    "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63",
    "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79",
    "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95",
    "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111",
    "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127",
    "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143",
    "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159",
    "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175",
    "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191",
    "a192", "a193", "a194", "a195", "a196", "a197", "a198", "a199", "a200", "a201", "a202", "a203", "a204", "a205", "a206", "a207",
    "a208", "a209", "a210", "a211", "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", "a223",
    "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", "a234", "a235", "a236", "a237", "a238", "a239",
    "a240", "a241", "a242", "a243", "a244", "a245", "a246", "a247", "a248", "a249", "a250", "a251", "a252", "a253", "a254", "a255");
}
__device__ __forceinline__ void wait_xdl_result() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory"); }
__device__ __forceinline__ void wait_valu_to_xdl() { asm volatile("s_nop 1" ::: "memory"); }
template <int D>
__device__ __forceinline__ void acc_zero1(const u32x4& z) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 a[%c1:%c2], %0, %0, 0" ::"v"(z), "n"(16 * D), "n"(16 * D + 15));
}
template <int... D>
__device__ __forceinline__ void acc_zero_all(const u32x4& z, std::integer_sequence<int, D...>) {
  (acc_zero1<D>(z), ...);
}
// 16 MFMAs with zero operands and a zero accumulator write zeros to a0 .. a255.
__device__ __forceinline__ void acc_zero() {
  const u32x4 z = {0u, 0u, 0u, 0u};
  wait_xdl_result();
  acc_zero_all(z, std::make_integer_sequence<int, 16>{});
}
template <int R>
__device__ __forceinline__ void acc_scale1(float s) {
  float t;
  asm volatile("v_accvgpr_read_b32 %0, a%c2\n\tv_mul_f32 %0, %0, %1\n\tv_accvgpr_write_b32 a%c2, %0"
               : "=&v"(t)
               : "v"(s), "n"(R));
}
template <int... R>
__device__ __forceinline__ void acc_scale_all(float s, std::integer_sequence<int, R...>) {
  (acc_scale1<R>(s), ...);
}
__device__ __forceinline__ void acc_scale(float s) {
  wait_xdl_result();
  acc_scale_all(s, std::make_integer_sequence<int, 256>{});
  wait_valu_to_xdl();
}
// max |a_i| over a0 .. a255 (one register read at a time).
template <int R>
__device__ __forceinline__ void acc_absmax1(float& m) {
  float t;
  asm volatile("v_accvgpr_read_b32 %1, a%c2\n\tv_max_f32 %0, %0, |%1|" : "+v"(m), "=&v"(t) : "n"(R));
}
template <int... R>
__device__ __forceinline__ float acc_absmax_all(std::integer_sequence<int, R...>) {
  float m = 0.f;
  (acc_absmax1<R>(m), ...);
  return m;
}
__device__ __forceinline__ float acc_absmax() { return acc_absmax_all(std::make_integer_sequence<int, 256>{}); }
template <int R>
__device__ __forceinline__ float acc_read() {
  float x;
  asm volatile("v_accvgpr_read_b32 %0, a%c1" : "=v"(x) : "n"(R));
  return x;
}
// O^T block d (dv 32 d .. 32 d + 31) += V^T P^T.  P^T is written by VALU code
// the compiler may place right before this statement, so the statement starts
// with the 2 wait states an MFMA operand needs after a VALU write.
template <int D>
__device__ __forceinline__ void pv1(const u32x4& v, const u32x4& p) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 a[%c2:%c3], %0, %1, a[%c2:%c3]" ::"v"(v), "v"(p),
               "n"(16 * D), "n"(16 * D + 15));
}
// Transposed 8-byte LDS read (ds_read_b64_tr_b16): within each 16-lane group,
// lane i receives element i % 4 of the chunks supplied by lanes i / 4 + 4 e.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16* lp;
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(lds_ptr)p);
  return __builtin_bit_cast(u32x2, r);
}
// The score chain keeps its accumulator in VGPRs (the AGPRs hold the output
// accumulators): written as inline asm with VGPR operands.  Back-to-back
// accumulation into the same registers needs no wait states; before VALU reads
// the result, mfma32_v_drain provides the 18 independent cycles a 32x32 XDL
// result needs on CDNA3/4.
__device__ __forceinline__ void mfma32_v_first(f32x16& d, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_v(f32x16& d, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_v_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory"); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
// The value through a VGPR move the compiler cannot see into, so the code
// that uses it treats it as per-lane.  The post-stream merge takes its split
// count and slot size this way: as scalars, the loop counts and addresses
// derived from them raise the kernel's scalar register pressure, and the
// allocator then spills scalars inside the tile loop.
__device__ __forceinline__ int in_vgpr(int x) {
  int r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
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
// The same transfer with a scalar base and a per-lane offset, the LDS address
// given as a number (no pointer conversion).  (An immediate offset on this
// instruction would move the LDS destination as well as the source.)
__device__ __forceinline__ void lds_dma16n(const char* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
// The same transfer with a scalar base and a per-lane offset.
__device__ __forceinline__ void lds_dma16s(const char* sbase, uint32_t voff, char* lds) {
  const uint32_t m0 = uni((int)(uint32_t)(uintptr_t)(lds_ptr)lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(voff), "s"(sbase), "s"(m0) : "memory", "m0");
}
// 16 bytes per lane at p + OFF into v, a load the compiler does not track:
// the kernel's own vmcnt waits make it complete before v is read.  v is an
// in-out operand, so the load lands in the registers that hold the value it
// replaces and the compiler has no reason to copy it while it is in flight
// (a test checks the generated code for that).
template <int OFF>
__device__ __forceinline__ void load16_async(u32x4& v, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "+v"(v) : "v"(p), "n"(OFF) : "memory");
}
// A dword load the compiler does not track: the kernel's own vmcnt waits make
// it complete before the value is read with take_dword (both are ordered asm).
__device__ __forceinline__ uint32_t load_dword_async(const int32_t* ptr) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(ptr) : "memory");
  return v;
}
__device__ __forceinline__ int take_dword(uint32_t v) {
  int s;
  asm volatile("v_readfirstlane_b32 %0, %1" : "=s"(s) : "v"(v) : "memory");
  return s;
}
// 16-byte store with the device-coherent policy (sc1): it writes through this
// XCD's L2, so once vmcnt clears the bytes are visible to every XCD.  Asm, so
// the compiler does not count it: the kernel waits for it explicitly.  A store
// of more than 8 bytes needs one wait state before a VALU instruction may
// overwrite its data registers; the compiler inserts that only for stores it
// can see, so the statement ends with it.
__device__ __forceinline__ void store16_coherent(char* p, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}
// A VGPR written by load_dword_async, read only after the wait that covers
// the load (ordered asm, so nothing that uses the value moves above it).
__device__ __forceinline__ uint32_t take_vgpr(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v) : "memory");
  return r;
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
  int L;  // index-sparse: length of the unit's sequence (valid row ids are < L)
};

// A split piece's partial (one workspace slot): m[128] at float 0, l[128] at
// 128, r[128] at 256, then o[128][512] in fp16 at float 384, each head row o
// divided by its own r = max |o| (fp32), so the halves hold values in [-1, 1]
// and the rounding error of the merged output stays below max |v| 2^-12.
// Half the bytes of an fp32 partial: the piece writes 128 KiB, the merger
// reads 128 KiB per piece.
constexpr int kPartL = kHeads, kPartR = 2 * kHeads, kPartO = 3 * kHeads;
constexpr int kPartRowLds = 272;  // LDS bytes per head row of a transposed partial quarter (256 + pad)
static_assert(kPartRowLds * kHW * kWaves <= kStageBytes, "partial transpose fits one stage");
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// Merge of heads h0 .. h0 + nh - 1 (nh <= 128) of a unit's split partials by
// one workgroup.  Threads 0 .. nh - 1, one per head, load every split's (m, l)
// of their head (16 splits in flight), form (M, L) and the lse, and stage the
// split weights c_s = exp2(m_s - M) r_s / L for up to kMergeChunk splits in
// LDS.  Then all threads stream the output in 16-byte columns (8 halves),
// consecutive threads on consecutive columns, kMergeCols columns x
// kMergeSplits splits = 32 loads in flight per thread; columns past the head
// range repeat the thread's first column and are not stored.  Splits are
// combined in index order, so the result does not depend on which piece
// arrived last or which workgroup merges the range.  The partials were
// published with device-coherent stores before their pieces' arrivals (or a
// kernel boundary); the caller has performed the matching acquire.
constexpr int kMergeChunk = 64;  // split weights staged per pass
constexpr int kMergeCols = 4;    // 16-byte columns per thread per round
constexpr int kMergeSplits = 8;  // splits per round

// Arrival counter of a split unit: pieces that have published (low half) and
// pieces done with the unit's merge (upper half).
constexpr int kArriveMask = 0xffff;
constexpr int kLeaveShift = 16;
constexpr int kLeave = 1 << kLeaveShift;
// A unit's merge is cut into at most kSlices head ranges of whole 8-head
// blocks; slice k of nsl starts at head slice_head(k, nsl).
constexpr int kSlices = 16;
__device__ __forceinline__ int slice_head(int k, int nsl) { return 8 * ((16 * k) / nsl); }
// Polls of a unit's counter a finished piece makes (each after a sleep of
// kPollSleep x 64 clocks) before it leaves the unit's slices to the others.
constexpr int kSpinLimit = 512;
constexpr int kPollSleep = 8;
// The poll limit in use on this device (cc_debug_merge_poll_limit lowers it to
// exercise the path where pieces stop waiting).
__device__ int g_merge_poll_limit = kSpinLimit;
__host__ __device__ constexpr int merge_lds_floats_mla(int nh) { return 2 * nh + kMergeChunk * nh; }
__device__ __forceinline__ void merge_unit(const float* pb, int ns, int slot_floats, float* out, float* lse,
                                           float* lds, int h0, int nh) {
  float* ml = lds;            // M[nh], 1/L[nh]
  float* coef = lds + 2 * nh;  // [split in pass][head]
  const int tid = threadIdx.x;
  __syncthreads();  // the LDS is free: every wave is past its last tile (or the previous merge)
  if (tid < nh) {
    const int h = h0 + tid;
    float M = -INFINITY, L = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 16) {
      float mt[16], lt[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = s0 + i < ns;
        const float* ps = pb + (size_t)(ok ? s0 + i : 0) * slot_floats;
        mt[i] = ok ? ps[h] : -INFINITY;
        lt[i] = ok ? ps[kPartL + h] : 0.f;
      }
      float Mc = M;
#pragma unroll
      for (int i = 0; i < 16; ++i) Mc = fmaxf(Mc, mt[i]);
      L *= fast_exp2(M - Mc);  // 0 on the first chunk
#pragma unroll
      for (int i = 0; i < 16; ++i) L += lt[i] * fast_exp2(mt[i] - Mc);
      M = Mc;
    }
    ml[tid] = M;
    ml[nh + tid] = 1.f / L;
    lse[h] = (M + __log2f(L)) * kLn2;
  }
  typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
  const int slot16 = slot_floats / 4;                    // 16-byte words per slot
  const u32x4_* o16 = reinterpret_cast<const u32x4_*>(pb + kPartO) + (size_t)h0 * (kDv / 8);
  f32x4* out4 = reinterpret_cast<f32x4*>(out) + (size_t)h0 * (kDv / 4);
  const int ncols = nh * (kDv / 8);                      // 16-byte columns of the head range
  for (int c0 = 0; c0 < ns; c0 += kMergeChunk) {
    const int nc = min(kMergeChunk, ns - c0);
    __syncthreads();  // (M, 1/L) visible; the previous pass's weights consumed
    for (int i = tid; i < nc * nh; i += kThreads) {
      const int sp = i / nh, hl = i - (i / nh) * nh;
      const float* ps = pb + (size_t)(c0 + sp) * slot_floats;
      coef[i] = fast_exp2(ps[h0 + hl] - ml[hl]) * ps[kPartR + h0 + hl] * ml[nh + hl];
    }
    __syncthreads();
    // a round past the last split re-reads the last one with weight 0; a
    // column past the range (e >= ncols) re-reads column e0 (< ncols)
    for (int e0 = tid; e0 < ncols; e0 += kThreads * kMergeCols) {
      f32x8 acc[kMergeCols];
      int col[kMergeCols];
#pragma unroll
      for (int u = 0; u < kMergeCols; ++u) {
        const int e = e0 + kThreads * u;
        col[u] = e < ncols ? e : e0;
        if (c0 == 0) {
          acc[u] = f32x8{};
        } else {
          const f32x4 a = out4[2 * col[u]], b = out4[2 * col[u] + 1];
          acc[u] = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        }
      }
      for (int s0 = 0; s0 < nc; s0 += kMergeSplits) {
        u32x4_ v[kMergeCols][kMergeSplits];
#pragma unroll
        for (int t = 0; t < kMergeSplits; ++t) {
          const u32x4_* src = o16 + (size_t)(c0 + min(s0 + t, nc - 1)) * slot16;  // wave-uniform base
#pragma unroll
          for (int u = 0; u < kMergeCols; ++u) v[u][t] = src[col[u]];
        }
        __builtin_amdgcn_sched_barrier(0);  // one round of loads live at a time
#pragma unroll
        for (int u = 0; u < kMergeCols; ++u) {
          const int hl = col[u] / (kDv / 8);
#pragma unroll
          for (int t = 0; t < kMergeSplits; ++t) {
            const float c = s0 + t < nc ? coef[(s0 + t) * nh + hl] : 0.f;
            acc[u] += c * __builtin_convertvector(__builtin_bit_cast(f16x8, v[u][t]), f32x8);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < kMergeCols; ++u) {
        if (e0 + kThreads * u < ncols) {
          const int e = col[u];
          out4[2 * e] = f32x4{acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
          out4[2 * e + 1] = f32x4{acc[u][4], acc[u][5], acc[u][6], acc[u][7]};
        }
      }
    }
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
  __shared__ int sh_pend[2];
  __shared__ uint32_t sh_claim;

  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;  // MFMA row/column, lane group

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
    I.L = SPARSE ? uni(seqlens[I.unit / p.q_tokens]) : 0;
    return I;
  };
  // The workgroup's items, one lane each (64 at a time, every load in
  // flight together): their block count, and whether the plan matches the
  // lengths — no piece may end past its unit's key count (seqlens[b] dense,
  // topk index-sparse) and a unit's last piece must end exactly there.  A
  // plan built for other lengths turns this workgroup's softmax scale into
  // NaN, which carries through every merge into the out and lse of each unit
  // it works on, and sets the error word's seqlen bit.
  int nblk = 0;
  bool stale = false;
  for (int i = i0; i < i1; i += 64) {
    const int ii = i + lane;
    int nb = 0;
    bool bad = false;
    if (ii < i1) {
      const int4 t = items[ii];
      nb = (t.z - t.y + kBlk - 1) / kBlk;
      const int len = SPARSE ? p.topk : seqlens[t.x / p.q_tokens];
      bad = t.z > len || (t.w == unit_nsplit[t.x] - 1 && t.z != len);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) nb += __shfl_xor(nb, o);
    nblk += uni(nb);
    stale |= __builtin_amdgcn_ballot_w64(bad) != 0;
  }
  if (stale && tid == 0) atomicOr(err, kErrSeqlen);
  // wave-uniform, kept in a scalar register (a per-lane copy would cost the
  // tile loop a VGPR)
  const float scale_log2 =
      __builtin_bit_cast(float, uni(__builtin_bit_cast(int, stale ? __builtin_nanf("") : p.scale_log2)));

  // unit = b * Tq + t (one unit per query token)
  const int page_mask = (1 << p.log2_page) - 1;

  // block-table entry of block j of item I (dense)
  auto bt_entry = [&](const Item& I, int j) -> const int32_t* {
    const int lp = min((I.tb + j * kBlk) >> p.log2_page, p.max_pages - 1);
    return bt + (size_t)(I.unit / p.q_tokens) * p.max_pages + lp;
  };

  // ---- issue the tile of block (item I, block j) into the stage at dst
  // row transfer q < 8: token 8 wave + q, its first 1024 bytes -> LDS row row_lds(t)
  // rope transfer: lane l takes token rt = 8 wave + l / 8, LDS slot l % 8 holds chunk (l % 8) ^ ((rt / 2) % 8)
  const int rslot = lane >> 3;
  const int rt = kRowsPerWave * wave + rslot;
  const int rchunk = (lane & 7) ^ ((rt >> 1) & 7);
  // dense: a 32-token block lies inside one page (pages hold >= 32 tokens), so
  // its rows are contiguous and all 32 of them lie inside the page.  The
  // transfers read all 32 rows; past the item end those are whatever the page
  // holds, so the step that uses such a tile zeroes their V columns (their
  // scores are masked).  The address arithmetic is per step: wave w moves
  // rows 8w .. 8w+3 from base + 9216 w (LDS row_lds(8w + q) = wb0 + 1088 q)
  // and rows 8w+4 .. 8w+7 from 4608 bytes further (wb1 + 1088 q), row q at
  // per-lane offset 16 lane + 1152 (q % 4), and the rope columns of its 8
  // rows with a per-lane offset of their own.
  struct DenseFetch {
    const char* r0;    // row 8 wave of the block
    const char* r4;    // row 8 wave + 4
    const char* base;  // row 0
  };
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_ptr)&ring[0][0];
  const uint32_t wb0 = uni(row_lds(kRowsPerWave * wave));
  const uint32_t wb1 = uni(row_lds(kRowsPerWave * wave + 4) - 4 * 1088);
  const uint32_t wbr = uni(kRopeOff + 1024 * wave);
  const uint32_t rope_voff = rt * kRowBytes + 1024 + 16 * rchunk;
  auto dense_prep = [&](const Item& I, int j, int pg) -> DenseFetch {
    const int tok0 = I.tb + j * kBlk;
    if ((unsigned)pg >= (unsigned)p.num_pages) {
      atomicOr(err, kErrPage);
      pg = pg < 0 ? 0 : p.num_pages - 1;
    }
    DenseFetch F;
    F.base = reinterpret_cast<const char*>(kc) + ((long long)pg * (1 << p.log2_page) + (tok0 & page_mask)) * kRowBytes;
    F.r0 = F.base + kRowsPerWave * kRowBytes * wave;
    F.r4 = F.r0 + 4 * kRowBytes;
    return F;
  };
  // transfer Q of a dense block into the stage at LDS address st_lds
  auto dense_piece = [&](const DenseFetch& F, auto qc, uint32_t st_lds) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    if constexpr (q < 4)
      lds_dma16n(F.r0, 16 * lane + kRowBytes * q, st_lds + wb0 + 1088 * q);
    else if constexpr (q < kRowsPerWave)
      lds_dma16n(F.r4, 16 * lane + kRowBytes * (q - 4), st_lds + wb1 + 1088 * q);
    else
      lds_dma16n(F.base, rope_voff, st_lds + wbr);
  };
  // index-sparse: lane l of wave w stands for row rt = 8 w + l / 8 of a tile
  // (the row its rope transfer takes).  The row ids of a tile are loaded two
  // steps before its transfers and the block-table entries of those rows one
  // step before, as untracked dword loads issued ahead of that step's
  // transfers: the wait at the top of the next step covers them, so no step
  // waits on the index or block-table round trips.  Rows past the item end
  // repeat its last row (a cursor past the last item repeats the last row of
  // the chunk: its transfers fill a stage that is never read).
  auto sid_ptr = [&](const Item& I, int j) -> const int32_t* {
    const int tok0 = I.tb + j * kBlk;
    const int tl_last = min(tok0 + kBlk, I.te) - 1;
    return indices + (size_t)I.unit * p.topk + min(tok0 + rt, tl_last);
  };
  auto sid_check = [&](const Item& I, uint32_t sid) -> uint32_t {
    const bool bad = sid >= (uint32_t)I.L;  // an invalid id reads token 0 instead
    if (bad) atomicOr(err, kErrIndex);
    return bad ? 0u : sid;
  };
  auto spg_ptr = [&](const Item& I, uint32_t sid) -> const int32_t* {
    return bt + (size_t)(I.unit / p.q_tokens) * p.max_pages + min((int)(sid >> p.log2_page), p.max_pages - 1);
  };
  auto spg_check = [&](uint32_t pg) -> uint32_t {
    const bool bad = pg >= (uint32_t)p.num_pages;
    if (bad) atomicOr(err, kErrPage);
    return bad ? ((int)pg < 0 ? 0u : (uint32_t)(p.num_pages - 1)) : pg;
  };
  auto srow = [&](uint32_t sid, uint32_t pg) -> const char* {
    return reinterpret_cast<const char*>(kc) + ((long long)pg * (1 << p.log2_page) + (sid & page_mask)) * kRowBytes;
  };
  // transfer q of a tile whose checked row ids and pages are sid, spg (per lane)
  auto sparse_piece = [&](uint32_t sid, uint32_t spg, int q, char* dst) __attribute__((always_inline)) {
    if (q < kRowsPerWave) {
      const uint32_t id = __builtin_amdgcn_readlane(sid, 8 * q), pg = __builtin_amdgcn_readlane(spg, 8 * q);
      lds_dma16s(srow(id, pg), 16 * lane, dst + row_lds(kRowsPerWave * wave + q));
    } else {
      lds_dma16(srow(sid, spg) + 1024 + 16 * rchunk, dst + kRopeOff + 1024 * wave);
    }
  };

  // LDS read addresses of the MFMA operands: one base per operand, the rest immediate
  //   K, k-step ks < 32: token n, dims 16 ks + 8 g -> row_lds(n) + 16 g + 32 ks
  //   rope, k-step 32 + r: token n, chunk c = 2 r + g at slot c ^ ((n / 2) % 8)
  //   V^T (transposed reads, 16-lane groups G = lane / 16, j = lane % 16): block d
  //     of 32 dv, k-block b, half c: lane supplies token 16 b + 8 c + 4 g + j / 4,
  //     dv 32 d + 16 (G % 2) + 4 (j % 4) .. +3, and receives row dv 32 d + (lane % 32)
  //     at tokens 16 b + 8 c + 4 g + e; row_lds of those tokens is lane-constant
  //     apart: + 17408 b + 8736 c (the 4-token groups keep their slot pattern)
  const uint32_t kbase = row_lds(n) + 16 * g;
  uint32_t rope_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rope_off[r] = kRopeOff + 128 * n + 16 * ((2 * r + g) ^ ((n >> 1) & 7));
  const uint32_t vbase = row_lds(4 * g + ((lane & 15) >> 2)) + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

  // Q^T operand: lane holds head 32 wave + n, dims 16 ks + 8 g .. +8.  The
  // first kQReg k-steps stay in registers (108 VGPRs) for the whole item; the
  // other 9 go to the wave's own LDS area in the same lane order (one transfer
  // per k-step, read back conflict free), which leaves the register file room
  // for the operand pipeline.  The register part is loaded with untracked
  // loads (load16_async): every q load is issued before the transfers of the
  // next tile fetch, so the vmcnt(kDmaPerWave) wait at the top of the next
  // step covers it, and the score loop carries no wait for q.
  u32x4 qv[kQReg] = {};
  char* qlds_w = qlds[wave];
  auto load_q = [&](int unit) {
    const size_t row = (size_t)unit * p.hq + kHW * wave + n;
    const uint16_t* qp = qg + row * kDqk + 8 * g;
    unroll<kQReg>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      load16_async<32 * j>(qv[j], qp);
    });
#pragma unroll
    for (int r = 0; r < kKSteps - kQReg; ++r)
      lds_dma16(reinterpret_cast<const char*>(qp + 16 * (kQReg + r)), qlds_w + 1024 * r);
  };

  // ------------------------------------------------ the block stream
  // Every iteration issues exactly one tile fetch (kDmaPerWave transfers per
  // wave) as its last memory operations: among the score products, or after
  // the next item's q loads when the item ends.  So the loads outstanding at
  // the top of iteration k are, oldest first: tile k, [the page / row-id
  // prefetches and q loads of iteration k-1], tile k+1.  Past the last block
  // the fetch re-reads a block of the chunk into the free stage (never read
  // again).
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
  // The page of the tile after the one being fetched is loaded asynchronously
  // (into pg_pref) before that fetch's transfers, so the wait at the top of
  // the next iteration covers it and the fetch never waits on the block table.
  auto page_now = [&](const Item& I, int j) { return uni(*bt_entry(I, j)); };
  uint32_t pg_pref = 0;
  // index-sparse pipeline: at the top of step k, sid2 holds the checked row
  // ids of tile k+2; in flight (landed once the top wait is passed) are the
  // row ids of tile k+3 (sid_fl) and the block-table entries of tile k+2
  // (spg_fl); c3, c4 are the cursors of tiles k+3, k+4
  struct Cursor {
    Item I;
    int it, j, nb;
  };
  auto adv = [&](Cursor& c) { advance(c.I, c.it, c.j, c.nb); };
  Cursor c3{cur, i0, 0, cur_nb}, c4 = c3;
  uint32_t sid2 = 0, sid_fl = 0, spg_fl = 0;
  if constexpr (SPARSE) {
    // tiles 0 and 1 and the state of step 0 with ordinary loads (once): q
    // first (untracked, it lands behind everything below), then the row ids
    // of tiles 0..3 in one round of loads and the block-table entries of
    // tiles 0..2 in a second, every load of a round issued before any check
    // (the checks' error atomics would otherwise order each load behind the
    // previous tile's)
    load_q(cur.unit);
    Cursor t1 = c3;
    adv(t1);
    Cursor t2 = t1;
    adv(t2);
    Cursor t3 = t2;
    adv(t3);
    const uint32_t r0 = (uint32_t)*sid_ptr(c3.I, c3.j), r1 = (uint32_t)*sid_ptr(t1.I, t1.j);
    const uint32_t r2 = (uint32_t)*sid_ptr(t2.I, t2.j);
    sid_fl = (uint32_t)*sid_ptr(t3.I, t3.j);
    const uint32_t s0 = sid_check(c3.I, r0), s1 = sid_check(t1.I, r1);
    sid2 = sid_check(t2.I, r2);
    const uint32_t g0 = (uint32_t)*spg_ptr(c3.I, s0), g1 = (uint32_t)*spg_ptr(t1.I, s1);
    spg_fl = (uint32_t)*spg_ptr(t2.I, sid2);
    const uint32_t p0 = spg_check(g0), p1 = spg_check(g1);
    c3 = t3;
    c4 = t3;
    adv(c4);
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) sparse_piece(s0, p0, q, ring[0]);
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) sparse_piece(s1, p1, q, ring[1]);
  } else {
    load_q(cur.unit);
    auto fetch_now = [&](const Item& I, int j, int sidx, int pg) {
      const DenseFetch F = dense_prep(I, j, pg);
      unroll<kDmaPerWave>([&](auto qc) { dense_piece(F, qc, ring_lds + sidx * kStageBytes); });
    };
    fetch_now(pI, p_j, 0, page_now(pI, p_j));
    advance(pI, p_it, p_j, p_nb);
    if (nblk > 1) {
      const int pg1 = page_now(pI, p_j);
      Item nI = pI;
      int n_it = p_it, n_j = p_j, n_nb = p_nb;
      advance(nI, n_it, n_j, n_nb);
      pg_pref = load_dword_async(nblk > 2 ? bt_entry(nI, n_j) : bt);
      fetch_now(pI, p_j, 1, pg1);
      pI = nI;
      p_it = n_it;
      p_j = n_j;
      p_nb = n_nb;
    } else {
      fetch_now(cur, 0, 1, 0);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;  // head n of the wave (lanes n and n + 32 agree on m_run)
  // O^T block d: rows dv 32 d + row, columns heads (in a[16 d .. 16 d + 15])
  acc_reserve();
  acc_zero();
  bool fresh = true;  // no block of the current item seen yet
  // split pieces this workgroup published (only a chunk's first and last
  // items can be split), one word each: unit << 11 | split << 2 | arrived
  // last << 1 | 1 (0: none; the arrival bit is set after the stream); the
  // host keeps units below 2^20 and split indices below 2^9
  int pend0 = 0, pend1 = 0;

  // one block: tile k in stage st = k % 3; the fetch two blocks ahead goes to stage (k + 2) % 3
  int st = 0, st2 = 2;
  auto step = [&](int k) __attribute__((always_inline)) {
    // tile k (and any q loads, issued before tile k+1's transfers) has landed
    // for every wave; every wave is done with tile k-1's stage
    wait_vmcnt<kDmaPerWave>();
    wait_lds();
    barrier();
    const char* tile = ring[st];
    const int tok0 = cur.tb + cur_j * kBlk;
    const int nv = min(kBlk, cur.te - tok0);
    if constexpr (!SPARSE) {
      if (nv < kBlk) {
        // rows past the item end hold whatever the page holds there: zero
        // their V columns (their probabilities are exactly 0, and 0 times a
        // non-finite value would not be)
        char* zt = ring[st];
        for (int i = tid; i < (kBlk - nv) * 64; i += kThreads)
          *reinterpret_cast<u32x4*>(zt + row_lds(nv + (i >> 6)) + 16 * (i & 63)) = u32x4{0u, 0u, 0u, 0u};
        wait_lds();
        barrier();
      }
    }

    // The fetch of the tile two blocks ahead (a filler past the end): its
    // transfers go between the score MFMAs, unless this tile ends an item and
    // the next item's q loads have to be issued before them (the vmcnt waits
    // count on that order).
    const bool item_ends = cur_j == cur_nb - 1;
    const bool q_next = item_ends && k + 1 < nblk;
    DenseFetch F = {nullptr, nullptr, nullptr};
    uint32_t fsid = 0, fspg = 0;  // index-sparse: checked row ids and pages of the fetched tile
    if constexpr (SPARSE) {
      const uint32_t sid3 = sid_check(c3.I, take_vgpr(sid_fl));  // ids of tile k+3
      fspg = spg_check(take_vgpr(spg_fl));                       // pages of tile k+2
      fsid = sid2;
      spg_fl = load_dword_async(spg_ptr(c3.I, sid3));  // pages of tile k+3
      sid_fl = load_dword_async(sid_ptr(c4.I, c4.j));  // ids of tile k+4
      sid2 = sid3;
      c3 = c4;
      adv(c4);
    } else {
      const Item fI = k + 2 < nblk ? pI : cur;
      const int fj = k + 2 < nblk ? p_j : cur_j;
      int fpg = 0;  // page of the fetched block (the filler reads page 0, never used)
      if (k + 2 < nblk) {
        fpg = take_dword(pg_pref);
        Item nI = pI;
        int n_it = p_it, n_j = p_j, n_nb = p_nb;
        advance(nI, n_it, n_j, n_nb);
        pg_pref = load_dword_async(k + 3 < nblk ? bt_entry(nI, n_j) : bt);
        pI = nI;
        p_it = n_it;
        p_j = n_j;
        p_nb = n_nb;
      }
      F = dense_prep(fI, fj, fpg);
    }
    char* fdst = ring[st2];
    const uint32_t fst_lds = ring_lds + st2 * kStageBytes;
    auto piece = [&](auto qc) __attribute__((always_inline)) {
      if constexpr (SPARSE)
        sparse_piece(fsid, fspg, decltype(qc)::value, fdst);
      else
        dense_piece(F, qc, fst_lds);
    };

    // S^T = K Q^T, 36 k-steps, operands read kPreS k-steps ahead
    f32x16 s;
    auto scores = [&](auto inter_c) __attribute__((always_inline)) {
      constexpr bool kInter = decltype(inter_c)::value;
      u32x4 kop[kKSteps], qop[kKSteps];  // K^T operands; Q^T operands of the LDS k-steps
      auto kload = [&](int ks) {
        kop[ks] = *reinterpret_cast<const u32x4*>(tile + (ks < kLatentSteps ? kbase + 32 * ks : rope_off[ks - kLatentSteps]));
        if (ks >= kQReg) qop[ks] = *reinterpret_cast<const u32x4*>(qlds_w + 1024 * (ks - kQReg) + 16 * lane);
      };
#pragma unroll
      for (int ks = 0; ks < kPreS; ++ks) kload(ks);
      unroll<kKSteps>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        if (ks + kPreS < kKSteps) kload(ks + kPreS);
        if (ks == 0)
          mfma32_v_first(s, kop[0], qv[0]);
        else if (ks < kQReg)
          mfma32_v(s, kop[ks], qv[ks]);
        else
          mfma32_v(s, kop[ks], qop[ks]);
        if constexpr (kInter && (ks & 3) == 2) piece(std::integral_constant<int, (ks >> 2)>{});
      });
    };
    if (!q_next)
      scores(std::true_type{});
    else
      scores(std::false_type{});
    mfma32_v_drain();
    if (q_next) {
      // q of the next item replaces this one as soon as the scores no longer need it
      load_q(uni(items[cur_it + 1].x));
    }
    if (q_next) unroll<kDmaPerWave>([&](auto qc) { piece(qc); });

    // scores (base 2), masked past the item end; register r is token 8 (r / 4) + 4 g + r % 4
    float x[16];
    if (nv == kBlk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = s[r] * scale_log2;
    } else {
      const int lim = nv - 4 * g;  // register r holds a valid token when 8 (r / 4) + r % 4 < lim
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (8 * (r >> 2) + (r & 3) < lim) ? s[r] * scale_log2 : -INFINITY;
    }
    float bmax = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) bmax = fmaxf(bmax, x[r]);
    {  // max with the other half of the wave (lanes n and n + 32 hold the same head)
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, bmax),
                                                      __builtin_bit_cast(uint32_t, bmax), false, false);
      bmax = fmaxf(__builtin_bit_cast(float, sw[0]), __builtin_bit_cast(float, sw[1]));
    }
    // move the reference max only when some head needs it
    const bool need = bmax > m_run + kLazy;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float mnew = fmaxf(m_run, bmax);
      const float alpha = fast_exp2(m_run - mnew);
      l_run *= alpha;
      m_run = mnew;
      if (!fresh) acc_scale(alpha);  // every accumulator of this lane belongs to head n
    }
    fresh = false;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = fast_exp2(x[r] - m_run);
      psum += x[r];
    }
    l_run += psum;
    // P^T operand of k-block b: tokens {16 b + 4 g + i, 16 b + 8 + 4 g + i} = registers 8 b .. 8 b + 7
    u32x4 pb[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
      pb[b] = u32x4{pack_bf16(x[8 * b], x[8 * b + 1]), pack_bf16(x[8 * b + 2], x[8 * b + 3]),
                    pack_bf16(x[8 * b + 4], x[8 * b + 5]), pack_bf16(x[8 * b + 6], x[8 * b + 7])};

    // O^T += V^T P^T.  Rows past the item end are zero (see the top of the
    // step) and their probabilities are exactly 0, so they add nothing.
    // 32 MFMAs m = 16 b + d (k-block b, dv block d), V^T operands read kPreV ahead
    {
      u32x4 vop[32];
      auto vload = [&](int m) -> u32x4 {
        const char* a = tile + vbase + 64 * (m & 15) + 17408 * (m >> 4);
        const u32x2 lo = lds_read_tr16(a), hi = lds_read_tr16(a + 8736);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
#pragma unroll
      for (int m = 0; m < kPreV; ++m) vop[m] = vload(m);
      unroll<32>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr (m + kPreV < 32) vop[m + kPreV] = vload(m + kPreV);
        pv1<m & 15>(vop[m], pb[m >> 4]);
      });
    }

    if (item_ends) {
      // -------- finish the item: this workgroup holds the whole piece
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const size_t qrow = (size_t)cur.unit * kHeads;  // first head of the unit: (b Tq + t) Hq
      const int hh = kHW * wave + n;                  // this lane's head in the unit
      // register 4 jj + i of block d is dv 32 d + 8 jj + 4 g + i
      const bool whole = cur.nsplit == 1;
      float* ps = partials + (size_t)(cur.pbase + cur.split) * p.slot_floats;
      const float scale = whole ? 1.f / l_tot : 1.f;
      float* orow = out + (qrow + hh) * kDv + 4 * g;
      wait_xdl_result();
      if (whole) {
        if (g == 0) lse[qrow + hh] = (m_run + __log2f(l_tot)) * kLn2;
        unroll<16>([&](auto dc) {
          constexpr int d = decltype(dc)::value;
          unroll<4>([&](auto jc) {
            constexpr int jj = decltype(jc)::value;
            *reinterpret_cast<f32x4*>(orow + 32 * d + 8 * jj) =
                f32x4{acc_read<16 * d + 4 * jj>(), acc_read<16 * d + 4 * jj + 1>(), acc_read<16 * d + 4 * jj + 2>(),
                      acc_read<16 * d + 4 * jj + 3>()} *
                scale;
          });
        });
      } else {
        // row scale r = max |o| over the head's 512 columns (this lane holds
        // 256 of them, lane n ^ 32 the rest), then o / r in fp16
        float r = acc_absmax();
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, r),
                                                          __builtin_bit_cast(uint32_t, r), false, false);
          r = fmaxf(__builtin_bit_cast(float, sw[0]), __builtin_bit_cast(float, sw[1]));
        }
        const float rinv = r > 0.f ? 1.f / r : 0.f;
        if (g == 0) {
          partial_store(ps + hh, m_run);
          partial_store(ps + kPartL + hh, l_tot);
          partial_store(ps + kPartR + hh, r);
        }
        // The halves go out as whole 256-byte row segments with device-coherent
        // stores (they reach memory before vmcnt clears, so the arrival below
        // needs no L2-wide write-back).  A lane holds 4-half pieces of one
        // head row, so each quarter of the row (4 dv blocks) is transposed
        // through this wave's 8.5 KB of the stage of the tile just consumed
        // (every wave is past its last read of it after the barrier).
        __syncthreads();
        char* tw = ring[st] + kPartRowLds * kHW * wave;
        char* prow = reinterpret_cast<char*>(ps + kPartO) + (size_t)(kHW * wave) * (kDv * 2);
        unroll<4>([&](auto qc) {
          constexpr int R = decltype(qc)::value;
          unroll<4>([&](auto dc) {
            constexpr int d = 4 * R + decltype(dc)::value;
            unroll<4>([&](auto jc) {
              constexpr int jj = decltype(jc)::value;
              const f16x2 lo = __builtin_convertvector(
                  f32x2{acc_read<16 * d + 4 * jj>() * rinv, acc_read<16 * d + 4 * jj + 1>() * rinv}, f16x2);
              const f16x2 hi = __builtin_convertvector(
                  f32x2{acc_read<16 * d + 4 * jj + 2>() * rinv, acc_read<16 * d + 4 * jj + 3>() * rinv}, f16x2);
              *reinterpret_cast<u32x2*>(tw + kPartRowLds * n + 2 * (32 * (d - 4 * R) + 8 * jj + 4 * g)) =
                  u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            });
          });
          wait_lds();
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int row = 4 * t + (lane >> 4);
            const u32x4 v = *reinterpret_cast<const u32x4*>(tw + kPartRowLds * row + 16 * (lane & 15));
            store16_coherent(prow + (size_t)row * (kDv * 2) + 256 * R + 16 * (lane & 15), v);
          }
        });
      }
      if (!whole) {
        if (p.reduce == CC_REDUCE_FUSED) {
          // the piece arrives after the stream (so the stream never waits for
          // its stores), and the unit is merged then
          const int word = (cur.unit << 11) | (cur.split << 2) | 1;
          if (pend0 == 0) {
            pend0 = word;
          } else {
            pend1 = word;
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
        acc_zero();
        fresh = true;
      }
    } else {
      ++cur_j;
    }
  };
  for (int k = 0; k < nblk; ++k) {
    step(k);
    st = st == 2 ? 0 : st + 1;
    st2 = st2 == 2 ? 0 : st2 + 1;
  }
  if (tl && tid == 0) tl[1] = tl[2] = __builtin_amdgcn_s_memrealtime();
  if (pend0) {
    // every wave's partial stores are complete (device-coherent stores reach
    // memory before vmcnt clears), then one arrival per piece, both in flight
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const int u0 = pend0 >> 11, u1 = pend1 >> 11;
      const int o0 = atomicAdd(&counters[kCounterStride * u0], 1);
      const int o1 = pend1 ? atomicAdd(&counters[kCounterStride * u1], 1) : 0;
      sh_pend[0] = pend0 | ((o0 & kArriveMask) == unit_nsplit[u0] - 1 ? 2 : 0);
      sh_pend[1] = pend1 ? pend1 | ((o1 & kArriveMask) == unit_nsplit[u1] - 1 ? 2 : 0) : 0;
    }
    __syncthreads();
    pend0 = uni(sh_pend[0]);
    pend1 = uni(sh_pend[1]);
  }
  // Merge of the split units this workgroup published pieces of (no q or
  // accumulators live here).  A unit's 128 heads form nsl = min(nsplit,
  // kSlices) slices of whole 8-head blocks.  Once every piece of a unit has
  // arrived, each of its pieces claims slice "split index" if that is still
  // free, merges it, and then claims and merges any slice still free until
  // none is left; a claim is an atomic OR on the unit's claim mask, so each
  // slice is merged exactly once, by whichever workgroup claims it.  A
  // workgroup polls its (at most two) units in turn and works on whichever is
  // complete.  The last arriver never waits, so every slice is merged even
  // when other pieces stop polling (after kSpinLimit polls): no piece's
  // progress depends on another workgroup being resident.  Each piece then
  // leaves (the counter's upper half); the last to leave clears the counter
  // and the mask, so the workspace is left zeroed.
  int todo = (pend0 ? 1 : 0) | (pend1 ? 2 : 0);
  const int poll_limit = todo ? uni(__hip_atomic_load(&g_merge_poll_limit, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)) : 0;
  for (int spin = 0; todo; ++spin) {
    const bool give_up = spin >= poll_limit;
    for (int e = 0; e < 2; ++e) {
      if (!((todo >> e) & 1)) continue;
      const int word = uni(e == 0 ? pend0 : pend1);
      const int unit = word >> 11;
      const int split = (word >> 2) & 511;
      const int ns = uni(unit_nsplit[unit]);
      const int nsl = min(ns, kSlices);
      int32_t* cnt = counters + kCounterStride * unit;
      uint32_t* claim = reinterpret_cast<uint32_t*>(cnt + 1);
      __syncthreads();  // every thread has read sh_claim
      if (tid == 0) {
        bool ready = (word >> 1) & 1;  // arrived last
        if (!ready) ready = (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kArriveMask) == ns;
        if (ready) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        sh_claim = ready;
      }
      __syncthreads();
      const bool ready = uni((int)sh_claim) != 0;
      if (!ready && !give_up) continue;
      if (ready) {
        const float* pb = partials + (size_t)uni(unit_pbase[unit]) * p.slot_floats;
        float* ou = out + (size_t)unit * kHeads * kDv;
        float* lu = lse + (size_t)unit * kHeads;
        const uint32_t every = (1u << nsl) - 1u;
        int want = split < nsl ? split : -1;
        uint32_t seen = 0;  // claim bits known to be taken
        for (;;) {
          __syncthreads();  // every thread has read sh_claim
          if (tid == 0) {
            int got = -1;
            while (got < 0) {
              if (want < 0) {
                const uint32_t free = every & ~seen;
                if (!free) break;
                want = __builtin_ctz(free);
              }
              const uint32_t bit = 1u << want;
              const uint32_t old = atomicOr(claim, bit);
              seen |= old | bit;
              if (!(old & bit)) got = want;
              want = -1;
            }
            sh_claim = (uint32_t)got;
          }
          __syncthreads();
          const int r = uni((int)sh_claim);
          if (r < 0) break;
          const int h0 = slice_head(r, nsl);
          merge_unit(pb, in_vgpr(ns), in_vgpr(p.slot_floats), ou, lu,
                     reinterpret_cast<float*>(ring[0]), h0, slice_head(r + 1, nsl) - h0);
        }
      }
      __syncthreads();  // sh_claim is rewritten next
      if (tid == 0) {
        const int old = atomicAdd(cnt, kLeave);
        if ((old >> kLeaveShift) == ns - 1) {
          __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(claim, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      todo &= ~(1 << e);
    }
    if (todo && tid == 0) __builtin_amdgcn_s_sleep(kPollSleep);
  }
  if (tl && tid == 0) tl[3] = tl[4] = __builtin_amdgcn_s_memrealtime();
}

// Split-then-combine comparison launch: the decode kernel only writes the
// pieces' partials; this kernel merges them, one workgroup per (unit, group
// of kCombineHeads heads), with the same merge as the fused path.
constexpr int kCombineHeads = 16;
__global__ void __launch_bounds__(kThreads)
mla_combine_kernel(int slot_floats, const int32_t* __restrict__ unit_nsplit, const int32_t* __restrict__ unit_pbase,
                   const float* __restrict__ partials, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) float lds[merge_lds_floats_mla(kCombineHeads)];
  const int u = blockIdx.x;
  const int ns = unit_nsplit[u];
  if (ns <= 1) return;
  merge_unit(partials + (size_t)unit_pbase[u] * slot_floats, ns, slot_floats, out + (size_t)u * kHeads * kDv,
             lse + (size_t)u * kHeads, lds, blockIdx.y * kCombineHeads, kCombineHeads);
}

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

}  // namespace mla

hipError_t launch_mla_combine(const DecodeArgs& a, hipStream_t s) {
  hipExtLaunchKernelGGL(mla::mla_combine_kernel, dim3(a.units, mla::kHeads / mla::kCombineHeads),
                        dim3(mla::kThreads), 0u, s, a.ev_start, a.ev_stop, 0u, a.slot_floats, a.unit_nsplit,
                        a.unit_pbase, a.partials, a.out, a.lse);
  return hipGetLastError();
}

hipError_t set_mla_merge_poll_limit(int polls) {
  const int v = polls < 0 ? mla::kSpinLimit : polls;
  return hipMemcpyToSymbol(HIP_SYMBOL(mla::g_merge_poll_limit), &v, sizeof v);
}

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
    hipExtLaunchKernelGGL(mla::mla_decode_kernel<true>, dim3(a.workers), dim3(mla::kThreads), 0u, s, a.ev_start,
        a.ev_stop, 0u, p, a.wg_off, a.items, a.unit_nsplit, a.unit_pbase, a.q, a.k, a.block_table, a.seqlens, a.indices,
        a.out, a.lse, a.err, a.counters, a.partials, a.timeline);
  } else {
    hipExtLaunchKernelGGL(mla::mla_decode_kernel<false>, dim3(a.workers), dim3(mla::kThreads), 0u, s, a.ev_start,
        a.ev_stop, 0u, p, a.wg_off, a.items, a.unit_nsplit, a.unit_pbase, a.q, a.k, a.block_table, a.seqlens, a.indices,
        a.out, a.lse, a.err, a.counters, a.partials, a.timeline);
  }
  return hipGetLastError();
}

}  // namespace cc
