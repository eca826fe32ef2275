// Log-sum-exp merge of a unit's split partials, run by one whole workgroup.
//
// Each split piece s of a unit left (m_s, l_s, o_s) per head: the running max
// of its scores (base 2), the sum of exp2(score - m_s) and the un-normalised
// output.  The exact result over the union of the pieces is
//   M = max_s m_s,  c_s = exp2(m_s - M) / sum_s l_s exp2(m_s - M),
//   out = sum_s c_s o_s,  lse = ln2 * (M + log2 sum_s l_s exp2(m_s - M)).
// This is the reduction a split-KV decode hands its partial outputs to
// (MeldKernel summary, "Core method": partial outputs feed the reduction).
//
// The merge sits on the critical path of the last piece to arrive, so every
// load is issued independently: one wave per head for (M, L), then float4
// reads of o_s with several splits in flight per thread and, when the unit is
// small, the splits spread over thread groups and summed through LDS.
// Splits are combined in index order with fixed groupings: the result does not
// depend on which piece arrived last.
#pragma once

#include <hip/hip_runtime.h>

namespace cc {

constexpr int kMergeCoef = 2048;  // split coefficients held in LDS per pass
constexpr int kMergeInflight = 8; // o_s loads in flight per thread

// Small partials (a GQA group: a few KB per piece) cross compute units (and
// XCDs, whose L2 caches are not coherent with each other) inside one launch
// as relaxed agent-scope atomics: those accesses carry the device-scope cache
// policy and are coherent across the XCDs by themselves, so neither the
// writer nor the reader has to write back or invalidate a whole L2 (what an
// agent-scope release/acquire fence does for ordinary data).  The writer makes
// the stores complete (s_waitcnt vmcnt(0)) before its arrival on the unit's
// counter; the reader issues its loads after observing the last arrival.
// Large partials (MLA: 128 KB per piece) are written with device-coherent
// 16-byte stores, which write through the XCD's L2, so the writer needs no
// release fence either; every workgroup that merges a slice of them issues an
// agent-scope acquire fence (its L2 may hold stale lines of the slots from an
// earlier call) and then reads them with ordinary 16-byte loads, which cost
// less there than per-element device-scope loads.
__device__ __forceinline__ void partial_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float partial_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Offset (floats) of o inside a partial slot.
__host__ __device__ constexpr int partial_o_offset(int hpu) { return (2 * hpu + 3) & ~3; }

// LDS floats merge_splits needs for NT threads and hpu heads.
__host__ __device__ constexpr int merge_lds_floats(int nt, int hpu) {
  return ((2 * hpu + kMergeCoef + 3) & ~3) + 4 * nt;
}

// partials: slot s at pb + s * slot_floats holds m[hpu] at 0, l[hpu] at hpu and
// o[hpu][dv] at partial_o_offset(hpu) (16-byte aligned), written with ordinary
// stores and published by an agent-scope release (or a kernel boundary); the
// caller has performed the matching acquire.
// out: head hh of the unit at out + hh * dv; lse: lse[hh].  dv % 4 == 0.
template <int NT>
__device__ void merge_splits(const float* pb, int ns, int slot_floats, int hpu, int dv, float* out,
                             float* lse, float* lds) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  constexpr int kWavesM = NT / 64;
  float* ml = lds;                         // M[hpu], 1/L[hpu]
  float* coef = lds + 2 * hpu;             // [split in pass][hpu]
  f4* red = reinterpret_cast<f4*>(lds + ((2 * hpu + kMergeCoef + 3) & ~3));
  constexpr float kLn2 = 0.69314718055994531f;

  // (M, L) per head: one wave per head, lanes over splits.  With at most 64
  // splits whose coefficients all fit in LDS (the common case) each lane keeps
  // its split's (m, l) in registers and writes c_s right away, so the whole
  // merge is two rounds of loads: (m, l), then o.
  const bool one_pass = ns <= 64 && ns * hpu <= kMergeCoef;
  for (int hh = wave; hh < hpu; hh += kWavesM) {
    if (one_pass) {
      const bool on = lane < ns;
      const float* ps = pb + (size_t)(on ? lane : 0) * slot_floats;
      const float m = on ? ps[hh] : -INFINITY;
      const float l = on ? ps[hpu + hh] : 0.f;
      float mx = m;
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float w = on ? __builtin_amdgcn_exp2f(m - mx) : 0.f;
      float L = l * w;
      for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
      if (on) coef[lane * hpu + hh] = w / L;
      if (lane == 0) lse[hh] = (mx + __log2f(L)) * kLn2;
      continue;
    }
    float mx = -INFINITY;
    for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, pb[(size_t)s * slot_floats + hh]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float L = 0.f;
    for (int s = lane; s < ns; s += 64) {
      const float* ps = pb + (size_t)s * slot_floats;
      L += ps[hpu + hh] * __builtin_amdgcn_exp2f(ps[hh] - mx);
    }
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    if (lane == 0) {
      ml[hh] = mx;
      ml[hpu + hh] = 1.f / L;
      lse[hh] = (mx + __log2f(L)) * kLn2;
    }
  }
  __syncthreads();

  const int EG = hpu * dv / 4;  // float4 groups of the output
  const int chunk = kMergeCoef / hpu > 0 ? kMergeCoef / hpu : 1;
  // small units: split the splits over TG thread groups and add through LDS
  int TG = NT / EG;
  TG = TG < 1 ? 1 : (TG > 8 ? 8 : TG);
  const int EPT = NT / TG;      // threads per split group
  const int q = tid / EPT, e = tid - (tid / EPT) * EPT;
  f4 acc_small = {0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < ns; c0 += chunk) {
    const int c1 = min(ns, c0 + chunk);
    if (!one_pass) {
      for (int i = tid; i < (c1 - c0) * hpu; i += NT) {
        const int s = c0 + i / hpu, hh = i - (i / hpu) * hpu;
        coef[i] = __builtin_amdgcn_exp2f(pb[(size_t)s * slot_floats + hh] - ml[hh]) * ml[hpu + hh];
      }
      __syncthreads();
    }
    if (TG > 1) {
      if (q < TG && e < EG) {
        const int hh = (4 * e) / dv, col = 4 * e - hh * dv;
        const float* base = pb + partial_o_offset(hpu) + hh * dv + col;
        for (int s = c0 + q; s < c1; s += kMergeInflight * TG) {
          f4 v[kMergeInflight];
          float cf[kMergeInflight];
#pragma unroll
          for (int u = 0; u < kMergeInflight; ++u) {
            const int ss = s + u * TG;
            const bool ok = ss < c1;
            v[u] = ok ? *reinterpret_cast<const f4*>(base + (size_t)ss * slot_floats) : f4{0.f, 0.f, 0.f, 0.f};
            cf[u] = ok ? coef[(ss - c0) * hpu + hh] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < kMergeInflight; ++u) acc_small += cf[u] * v[u];
        }
      }
    } else {
      for (int eg = tid; eg < EG; eg += NT) {
        const int hh = (4 * eg) / dv, col = 4 * eg - hh * dv;
        const float* base = pb + partial_o_offset(hpu) + hh * dv + col;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = c0; s < c1; s += kMergeInflight) {
          f4 v[kMergeInflight];
          float cf[kMergeInflight];
#pragma unroll
          for (int u = 0; u < kMergeInflight; ++u) {
            const int ss = s + u;
            const bool ok = ss < c1;
            v[u] = ok ? *reinterpret_cast<const f4*>(base + (size_t)ss * slot_floats) : f4{0.f, 0.f, 0.f, 0.f};
            cf[u] = ok ? coef[(ss - c0) * hpu + hh] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < kMergeInflight; ++u) acc += cf[u] * v[u];
        }
        f4* dst = reinterpret_cast<f4*>(out + hh * dv + col);
        if (c0 > 0) acc += *dst;
        *dst = acc;
      }
    }
    __syncthreads();  // coefficients of this pass consumed
  }
  if (TG > 1) {
    if (q < TG && e < EG) red[q * EPT + e] = acc_small;
    __syncthreads();
    if (q == 0 && e < EG) {
      f4 acc = red[e];
      for (int g = 1; g < TG; ++g) acc += red[g * EPT + e];
      const int hh = (4 * e) / dv, col = 4 * e - hh * dv;
      *reinterpret_cast<f4*>(out + hh * dv + col) = acc;
    }
    __syncthreads();
  }
}

// Single-round merge of one unit: thread e owns output element e and issues
// the loads of m, l and o of CH splits at a time before using any of them,
// combining the chunks online in split order (so the result does not depend
// on which piece arrived last).  The shared-prefix kernel's waves use it with
// CH = 4, the same chunking as merge_units_batched, so both give the same bits.
constexpr int kDirectChunk = 32;
// ns splits from partial slot pb on, output
// rows row0 .. row0 + hpu - 1; thread t of NT; CH splits' loads in flight.
template <int NT, int CH = kDirectChunk>
__device__ __forceinline__ void merge_unit_direct(const float* pb, int ns, size_t row0, int slot_floats, int hpu,
                                                  int dv, float* out, float* lse, int t) {
  constexpr float kLn2 = 0.69314718055994531f;
  const int E = hpu * dv;
  const int o_off = partial_o_offset(hpu);
  for (int e = t; e < E; e += NT) {
    const int hh = e / dv, col = e - (e / dv) * dv;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int s0 = 0; s0 < ns; s0 += CH) {
      float mt[CH], lt[CH], ot[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const bool ok = s0 + i < ns;
        const float* ps = pb + (size_t)(ok ? s0 + i : 0) * slot_floats;
        mt[i] = ok ? partial_load(ps + hh) : -INFINITY;
        lt[i] = ok ? partial_load(ps + hpu + hh) : 0.f;
        ot[i] = ok ? partial_load(ps + o_off + e) : 0.f;
      }
      float Mc = M;
#pragma unroll
      for (int i = 0; i < CH; ++i) Mc = fmaxf(Mc, mt[i]);
      // 0 on the first chunk (M = -inf); the same guard as merge_units_batched,
      // so both give the same bits for the same splits and chunk
      const float a = Mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
      L *= a;
      O *= a;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const float f = __builtin_amdgcn_exp2f(mt[i] - Mc);
        L += lt[i] * f;
        O += ot[i] * f;
      }
      M = Mc;
    }
    const size_t row = row0 + hh;
    out[row * dv + col] = O / L;
    if (col == 0) lse[row] = (M + __log2f(L)) * kLn2;
  }
}

// merge_unit_direct for many units at once: the (unit, column quad) pairs
// of all nu units are spread over the NT threads, each thread merging UB
// pairs together with CH splits' loads of every pair in flight (m, l and the
// quad's four o values as two 8-byte loads), so a workgroup that completes
// many small units (a few splits each) pays a few load round trips in all
// rather than one or more per unit.  dv must be a multiple of 4 (slots and o
// are 16-byte aligned).  Splits are combined in index order and each element
// gets the operations of merge_unit_direct<., CH>, so both give the same bits.
template <int NT, int UB, int CH>
__device__ void merge_units_batched(const float* partials, const int (*units)[3], int nu, int slot_floats, int hpu,
                                    int dv, float* out, float* lse) {
  constexpr float kLn2 = 0.69314718055994531f;
  const int E4 = hpu * dv / 4;  // column quads per unit
  const int o_off = partial_o_offset(hpu);
  const int total = nu * E4;
  for (int base = threadIdx.x; base < total; base += NT * UB) {
    const float* pb[UB];
    int ns[UB], hh[UB], ee[UB], nsmax = 0;
    float M[UB], L[UB], O[UB][4];
#pragma unroll
    for (int k = 0; k < UB; ++k) {
      const int pr = base + k * NT;
      const bool ok = pr < total;
      const int u = ok ? pr / E4 : 0;
      ee[k] = ok ? 4 * (pr - u * E4) : 0;  // first element of the quad
      hh[k] = ee[k] / dv;
      ns[k] = ok ? units[u][1] : 0;
      pb[k] = partials + (size_t)units[u][0] * slot_floats;
      nsmax = max(nsmax, ns[k]);
      M[k] = -INFINITY;
      L[k] = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) O[k][c] = 0.f;
    }
    for (int s0 = 0; s0 < nsmax; s0 += CH) {
      float mt[UB][CH], lt[UB][CH], ot[UB][CH][4];
#pragma unroll
      for (int k = 0; k < UB; ++k) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const bool ok = s0 + i < ns[k];
          const float* ps = pb[k] + (size_t)(ok ? s0 + i : 0) * slot_floats;
          mt[k][i] = ok ? partial_load(ps + hh[k]) : -INFINITY;
          lt[k][i] = ok ? partial_load(ps + hpu + hh[k]) : 0.f;
          const uint64_t* po = reinterpret_cast<const uint64_t*>(ps + o_off + ee[k]);
          const uint64_t lo = __hip_atomic_load(po, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t hi = __hip_atomic_load(po + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ot[k][i][0] = ok ? __builtin_bit_cast(float, (uint32_t)lo) : 0.f;
          ot[k][i][1] = ok ? __builtin_bit_cast(float, (uint32_t)(lo >> 32)) : 0.f;
          ot[k][i][2] = ok ? __builtin_bit_cast(float, (uint32_t)hi) : 0.f;
          ot[k][i][3] = ok ? __builtin_bit_cast(float, (uint32_t)(hi >> 32)) : 0.f;
        }
      }
#pragma unroll
      for (int k = 0; k < UB; ++k) {
        float Mc = M[k];
#pragma unroll
        for (int i = 0; i < CH; ++i) Mc = fmaxf(Mc, mt[k][i]);
        const float a = Mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[k] - Mc);
        L[k] *= a;
#pragma unroll
        for (int c = 0; c < 4; ++c) O[k][c] *= a;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const float f = __builtin_amdgcn_exp2f(mt[k][i] - Mc);
          L[k] += lt[k][i] * f;
#pragma unroll
          for (int c = 0; c < 4; ++c) O[k][c] += ot[k][i][c] * f;
        }
        M[k] = Mc;
      }
    }
#pragma unroll
    for (int k = 0; k < UB; ++k) {
      const int pr = base + k * NT;
      if (pr < total) {
        const int u = pr / E4;
        const size_t row = (size_t)units[u][2] + hh[k];
        const int col = ee[k] - hh[k] * dv;
#pragma unroll
        for (int c = 0; c < 4; ++c) out[row * dv + col + c] = O[k][c] / L[k];
        if (col == 0) lse[row] = (M[k] + __log2f(L[k])) * kLn2;
      }
    }
  }
}


// The units a workgroup completed, one after another, each in one round of
// loads with the splits spread over thread groups.  Thread t takes column quad
// q = t mod E4 (E4 = hpu dv / 4 quads) for group g = t / E4, and group g the
// splits g, g + TG, g + 2 TG, ... (TG = min(8, NT / E4) groups), merged online
// in that order with kGroupChunk splits' loads in flight; the groups' (M, L, O)
// then meet in LDS and group 0 combines them in group order.  A split costs a
// thread four loads (m, l and its o quad as two 8-byte halves) for four output
// elements, against three per element in merge_unit_direct.  The grouping is
// fixed, so the bits do not depend on which piece arrived last.  lds: at least
// 24 NT bytes; dv a multiple of 4; out rows 16-byte aligned.
constexpr int kGroupChunk = 8;
template <int NT>
__device__ void merge_units_grouped(const float* partials, const int (*units)[3], int nu, int slot_floats,
                                    int hpu, int dv, float* out, float* lse, float* lds) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr float kLn2 = 0.69314718055994531f;
  const int tid = threadIdx.x;
  const int E4 = hpu * dv / 4;
  int TG = NT / E4;
  TG = TG < 1 ? 1 : (TG > 8 ? 8 : TG);
  const int g = TG > 1 ? tid / E4 : 0;
  const int o_off = partial_o_offset(hpu);
  f4* lo = reinterpret_cast<f4*>(lds);  // [TG][E4] group outputs, then M and L
  float* lm = lds + 4 * NT;
  float* ll = lm + NT;
  for (int u = 0; u < nu; ++u) {
    const int ns = __builtin_amdgcn_readfirstlane(units[u][1]);
    const float* pb = partials + (size_t)__builtin_amdgcn_readfirstlane(units[u][0]) * slot_floats;
    const size_t row0 = (size_t)__builtin_amdgcn_readfirstlane(units[u][2]);
    for (int q0 = 0; q0 < E4; q0 += NT) {  // one pass unless E4 > NT (then TG = 1)
      const int q = q0 + (TG > 1 ? tid - g * E4 : tid);
      const bool on = g < TG && q < E4;
      const int hh = on ? (4 * q) / dv : 0;
      float M = -INFINITY, L = 0.f;
      f4 O = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = g; on && s0 < ns; s0 += TG * kGroupChunk) {
        float mt[kGroupChunk], lt[kGroupChunk];
        f4 ot[kGroupChunk];
#pragma unroll
        for (int i = 0; i < kGroupChunk; ++i) {
          const int sp = s0 + i * TG;
          const bool ok = sp < ns;
          const float* ps = pb + (size_t)(ok ? sp : 0) * slot_floats;
          const float m = partial_load(ps + hh), l = partial_load(ps + hpu + hh);
          const uint64_t* po = reinterpret_cast<const uint64_t*>(ps + o_off + 4 * q);
          const uint64_t lo8 = __hip_atomic_load(po, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t hi8 = __hip_atomic_load(po + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          mt[i] = ok ? m : -INFINITY;
          lt[i] = ok ? l : 0.f;
          ot[i] = ok ? f4{__builtin_bit_cast(float, (uint32_t)lo8), __builtin_bit_cast(float, (uint32_t)(lo8 >> 32)),
                          __builtin_bit_cast(float, (uint32_t)hi8), __builtin_bit_cast(float, (uint32_t)(hi8 >> 32))}
                     : f4{0.f, 0.f, 0.f, 0.f};
        }
        float Mc = M;
#pragma unroll
        for (int i = 0; i < kGroupChunk; ++i) Mc = fmaxf(Mc, mt[i]);
        const float a = Mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
        L *= a;
        O *= a;
#pragma unroll
        for (int i = 0; i < kGroupChunk; ++i) {
          const float f = __builtin_amdgcn_exp2f(mt[i] - Mc);
          L += lt[i] * f;
          O += ot[i] * f;
        }
        M = Mc;
      }
      if (TG > 1) {
        if (on) {
          lo[g * E4 + q] = O;
          lm[g * E4 + q] = M;
          ll[g * E4 + q] = L;
        }
        __syncthreads();
        if (on && g == 0) {
          for (int gg = 1; gg < TG; ++gg) {  // group order
            const float Mg = lm[gg * E4 + q], Lg = ll[gg * E4 + q];
            const f4 Og = lo[gg * E4 + q];
            const float Mc = fmaxf(M, Mg);
            const float a = Mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
            const float b = Mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mg - Mc);
            L = L * a + Lg * b;
            O = O * a + Og * b;
            M = Mc;
          }
        }
        __syncthreads();  // the LDS is free for the next unit
      }
      if (on && g == 0) {
        const int col = 4 * q - hh * dv;
        const size_t row = row0 + hh;
        *reinterpret_cast<f4*>(out + row * dv + col) = O / L;
        if (col == 0) lse[row] = (M + __log2f(L)) * kLn2;
      }
    }
  }
}

}  // namespace cc
