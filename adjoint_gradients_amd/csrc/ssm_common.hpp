// ssm_common.hpp -- device helpers shared by the gfx950 kernels of the
// selective-SSM adjoint-gradient library.
//
// Lane layout of every scan kernel (one 64-wide wavefront):
//   G  = N / NL lane groups, each group holds NL consecutive states n;
//   CH = 64 / G channels per wavefront;
//   lane = grp * CH + pl  (grp in [0,G), pl in [0,CH)),  channel p = cb*CH + pl.
// Per-channel values (s, x, g) are therefore read by G lanes at the same
// address (served by L1 as a broadcast), per-token state values (b_t, c_t)
// by the CH lanes of a group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grid_order.hpp"

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float -> bfloat16, round to nearest, ties to even (NaN kept quiet): one
// v_cvt_pk_bf16_f32 on gfx950, in the default round-to-nearest mode.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f)); }

template <typename T> __device__ __forceinline__ float load_io(const T* p);
template <> __device__ __forceinline__ float load_io<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_io<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

// An io element as held in a register between its load and its use: the
// bf16 bits (zero-extended) or the float itself.  Converting at the use keeps
// a wait for the load out of the code that issues it (a conversion right
// after a prefetching load would wait for that load at once).
template <typename T> struct IoRaw;
template <> struct IoRaw<float> { typedef float type; };
template <> struct IoRaw<bf16_t> { typedef uint32_t type; };
template <typename T> __device__ __forceinline__ typename IoRaw<T>::type load_raw(const T* p) { return *p; }
__device__ __forceinline__ float raw_to_f32(float v) { return v; }
__device__ __forceinline__ float raw_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ void store_io(T* p, float v);
template <> __device__ __forceinline__ void store_io<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_io<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// Fourth word of a raw buffer resource on gfx9 parts (offsets in bytes,
// range-checked against the record count: a store at or past it is dropped),
// and a lane offset past any row the kernels store into.  Kernels store
// through such resources where some lanes or some iterations store nothing,
// so that no lane mask or branch splits their loop bodies.
constexpr int kBufWord3 = 0x00020000;
constexpr int kBufOutside = 0x7ffffff0;

// 2^x on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// softplus(d) = max(d,0) + log(1 + e) with e = e^{-|d|} in (0, 1], on the
// hardware exp2/log2 units.  For e < 1/16 the series e - e^2/2 + e^3/3 - e^4/4
// (relative truncation < e^4/5 < 2e-6 of the smallest term kept... overall
// < 1e-7) keeps full relative accuracy where 1 + e would round away e.
__device__ __forceinline__ float softplus_f(float d) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(d) * kLog2e);
  const float big = __builtin_amdgcn_logf(1.0f + e) * 0.69314718055994531f;
  const float small = e * (1.0f - e * (0.5f - e * ((1.0f / 3.0f) - e * 0.25f)));
  return fmaxf(d, 0.0f) + (e < 0.0625f ? small : big);
}

// 1 - e^{-s} for s >= 0, i.e. the logistic sigmoid of Delta when s = softplus(Delta).
// Below 0.25 the series s sum_k (-s)^k / (k+1)!, cut after k = 6 (remainder
// < s^7/8! < 2e-9 relative), avoids the cancellation of 1 - e^{-s}; above
// it, 1 - e^{-s} >= 0.22 loses under 5e-7 relative to the rounding of
// e^{-s}.  Both branches are evaluated and selected (no divergence, no
// divisions); the series is one Horner fma per term.
__device__ __forceinline__ float one_minus_exp_neg(float s) {
  const float big = 1.0f - fast_exp2(-s * kLog2e);
  const float z = -s;
  float t = 1.0f / 5040.0f;
  t = fmaf(t, z, 1.0f / 720.0f);
  t = fmaf(t, z, 1.0f / 120.0f);
  t = fmaf(t, z, 1.0f / 24.0f);
  t = fmaf(t, z, 1.0f / 6.0f);
  t = fmaf(t, z, 0.5f);
  t = fmaf(t, z, 1.0f);
  const float small = s * t;
  return s > 0.25f ? big : small;
}

// Sums over the two 32-lane halves of two values with one lane exchange:
// lanes 0..31 get u(l) + u(l + 32), lanes 32..63 get v(l - 32) + v(l).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second, leaving [u_lo | v_lo] and [u_hi | v_hi].
__device__ __forceinline__ float half_sums_pair(float u, float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(u), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v + v(lane ^ D) for a compile-time lane distance D: DPP for 1 and 2,
// v_permlane32_swap for 32 (it exchanges the two 32-lane halves: the sum of
// its two results is the pairwise sum on every lane), ds_bpermute otherwise.
template <int D>
__device__ __forceinline__ float xor_sum(float v) {
  if constexpr (D == 1) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  } else if constexpr (D == 2) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  } else if constexpr (D == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    return v + __shfl_xor(v, D, 64);
  }
}

// Sum over the G lane groups of one channel (lanes pl, pl+CH, pl+2CH, ...).
template <int G, int CH>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (CH <= 32 && G >= 2) v = xor_sum<CH>(v);
  if constexpr (CH <= 16 && G >= 4) v = xor_sum<2 * CH>(v);
  if constexpr (CH <= 8 && G >= 8) v = xor_sum<4 * CH>(v);
  return v;
}

// Segmented scan of an affine recurrence over chunks, x <- d_k x + u_k, one
// value per lane: chunks k_lo .. k_hi - 1 in order (REV: k_hi - 1 down to
// k_lo), entering with x = cin; store(k, x) receives the value entering chunk
// k and the return value is the one leaving the range.
//
// Chunks are grouped in segments of L at fixed positions (segment j: chunks
// [j L, (j + 1) L)).  A segment maps the value entering it to the value
// leaving it by x -> A x + B (A the product of its d_k, B its walk from zero).
// A workgroup of S wavefronts (its lanes the same 64 independent recurrences
// in every wavefront) takes S segments at a time: each wavefront loads its
// segment through load(k, &u, &d) (all L loads in flight together) and forms
// the segment's map; the maps meet in LDS; each wavefront passes the group's
// entry value through the maps of the segments before its own and walks its
// segment from there, calling store.  The dependent chain is L + S steps per
// group instead of one per chunk.  Empty slots of a partial segment are the
// identity map (d = 1, u = 0), applied exactly, so launches that split a
// range at multiples of L give the same values, bit for bit, as one launch.
// Every wavefront of the workgroup must call this (it holds barriers).
template <int L, int S, bool REV, class Load, class Store>
__device__ __forceinline__ float seg_affine_scan(int64_t k_lo, int64_t k_hi, float cin, float (&sA)[S][64],
                                                 float (&sB)[S][64], int sg, int lane, Load load, Store store) {
  constexpr int64_t GL = static_cast<int64_t>(S) * L;
  const int64_t g_first = REV ? (k_hi - 1) / GL : k_lo / GL;
  const int64_t g_last = REV ? k_lo / GL : (k_hi - 1) / GL;
  for (int64_t g = g_first; REV ? g >= g_last : g <= g_last; g += REV ? -1 : 1) {
    int64_t s0 = g * GL + static_cast<int64_t>(sg) * L;
    int64_t s1 = s0 + L;
    s0 = s0 > k_lo ? s0 : k_lo;
    s1 = s1 < k_hi ? s1 : k_hi;
    float u[L], d[L];
#pragma unroll
    for (int r = 0; r < L; r++) {
      const int64_t k = REV ? s1 - 1 - r : s0 + r;
      const bool valid = REV ? k >= s0 : k < s1;
      float uk, dk;
      load(valid ? k : k_lo, &uk, &dk);
      u[r] = valid ? uk : 0.0f;
      d[r] = valid ? dk : 1.0f;
    }
    float A = 1.0f, B = 0.0f;
#pragma unroll
    for (int r = 0; r < L; r++) {
      B = fmaf(d[r], B, u[r]);
      A *= d[r];
    }
    sA[sg][lane] = A;
    sB[sg][lane] = B;
    __syncthreads();
    float x = cin;
    if (REV) {
      for (int j = S - 1; j > sg; j--) x = fmaf(sA[j][lane], x, sB[j][lane]);
    } else {
      for (int j = 0; j < sg; j++) x = fmaf(sA[j][lane], x, sB[j][lane]);
    }
#pragma unroll
    for (int r = 0; r < L; r++) {
      const int64_t k = REV ? s1 - 1 - r : s0 + r;
      if (REV ? k >= s0 : k < s1) store(k, x);
      x = fmaf(d[r], x, u[r]);
    }
    float xn = cin;
    if (REV) {
      for (int j = S - 1; j >= 0; j--) xn = fmaf(sA[j][lane], xn, sB[j][lane]);
    } else {
      for (int j = 0; j < S; j++) xn = fmaf(sA[j][lane], xn, sB[j][lane]);
    }
    cin = xn;
    __syncthreads();  // the next group overwrites the maps
  }
  return cin;
}

// Launch grid and workgroup -> (chunk, channel group) of the chunked scans
// (order in grid_order.hpp).
inline dim3 chunk_group_grid(int64_t nk, int64_t ng) {
  uint32_t gx = 0, gy = 0;
  chunk_group_dims(nk, ng, &gx, &gy);
  return dim3(gx, gy);
}
__device__ __forceinline__ void chunk_and_group(uint32_t* c, uint32_t* g) {
  chunk_group_of(blockIdx.x, blockIdx.y, gridDim.x, c, g);
}

}  // namespace ssm
