// scan_bwd.hip -- windowed reverse adjoint scan fused with the local VJPs, on gfx950.
//
// Source: review of "Adjoint sharding for very long context training of state
// space models" -- "What carries the argument" (adjoint state
// lambda_{t,i} = C_t A_t ... A_{i+1}; Proposition 1) and "Core claim"
// (Proposition 2 and truncated adjoint sharding over the last W tokens).
//
// For one channel p and state n, every VJP term of token i is multiplied by
//   mu_i = sum_{t=i}^{min(T,i+W)-1} g_t c_t prod_{j=i+1}^{t} a_j ,
// the cotangent-weighted sum of adjoint states.  mu obeys the reverse
// recurrence
//   mu_i = a_{i+1} mu_{i+1} + g_i c_i - g_{i+W} c_{i+W} D_i,
//   D_i  = prod_{j=i+1}^{i+W} a_j = exp(-alpha sum_{j=i+1}^{i+W} s_j)
// (the last term drops the token leaving the window; it is absent when
// W >= T or i+W >= T).  The recurrence is Proposition 1 with df/dh = diag(a)
// and a source that is local in time, so it parallelises over chunks exactly
// like the forward scan: affine chunk maps, a carry pass, then a final pass.
// The window sums of s are kept in fp64, so D needs no subtraction of
// rounded products.
//
// The local VJPs of token i (Proposition 2's vjp^{A_i}, vjp^{B_i}, vjp^{C_t}):
//   da_i     = mu_i h_{i-1}                  dDelta_i = sigmoid(Delta_i) sum_n da_i (-alpha a_i)
//   dalpha  += da_i (-s_i a_i)               dbias   += dDelta_i
//   db_i[n]  = sum_p mu_i x_i[p]             dxdir_i = sum_n mu_i b_i[n]
//   dc_i[n]  = sum_p g_i h_i[p]   (no time sum, hence no window)
// h_{i-1} is recomputed inside each chunk from the checkpoint h_{kC-1}
// (review of "Training Deep Nets with Sublinear Memory Cost": recompute
// inside segments): a forward walk stores h at the start of every S-token
// sub-chunk in a workspace region that holds one slab of chunks, then each
// sub-chunk is recomputed into registers and walked in reverse.
// Sums over channels (db, dc) go through an LDS transpose per wavefront, an
// LDS sum over the wavefronts of the workgroup, and a deterministic final sum
// over workgroups in a separate kernel.
#include <type_traits>

#include "ssm_common.hpp"
#include "ssm_kernels.hpp"
#include "red_layout.hpp"

namespace ssm {

namespace {

template <int NL>
__device__ __forceinline__ void load_row(const float* __restrict__ src, float (&dst)[NL]) {
  if constexpr (NL % 4 == 0) {
#pragma unroll
    for (int j = 0; j < NL; j += 4) {
      float4 v = *reinterpret_cast<const float4*>(src + j);
      dst[j] = v.x; dst[j + 1] = v.y; dst[j + 2] = v.z; dst[j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NL; j++) dst[j] = src[j];
  }
}

// Orders this wavefront's LDS writes before its following LDS reads of other
// lanes' data (and prevents the compiler from moving accesses across it).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

constexpr int kWpb = 4;  // wavefronts per workgroup of the main kernel and of the sub-chunk pass

// LDS floats of k_bwd_main (NL states per lane, G groups): two staging
// buffers of 3 row kinds x kSub tokens x NN states, and per wavefront the
// channel-sum transpose area, the token sums [kSub][2 NN] and two buffers of
// 5 per-lane quantities [kSub][CH] (each padded by 32 floats).  The kernel
// checks its own layout against this at compile time.
constexpr size_t bwd_main_lds_floats(int NL, int G) {
  return static_cast<size_t>(2 * 3 * kSub * NL * G) +
         static_cast<size_t>(kWpb) * (redl::floats(NL, G) + kSub * 2 * NL * G + 2 * 5 * (kSub * (64 / G) + 32));
}

}  // namespace

// Exclusive prefix over chunks of the per-chunk sums of s, in fp64:
// ps64[0] = 0, ps64[k + 1] = ps64[k] + ssum[k].  A workgroup of kPrefixRanges
// wavefronts takes 64 channels; wavefront w owns the w-th of kPrefixRanges
// contiguous ranges of chunks.  Each wavefront sums its range, the range
// totals meet in LDS, and each wavefront then writes its range's prefix
// starting from the sum of the totals before it (in range order), so the
// dependent chain is K / kPrefixRanges additions instead of K.
constexpr int kPrefixRanges = 16;

__global__ __launch_bounds__(64 * kPrefixRanges) void k_bwd_prefix(int64_t K, int64_t P,
                                                                   const double* __restrict__ ssum,
                                                                   double* __restrict__ ps64) {
  __shared__ double tot[kPrefixRanges][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const bool live = p < P;
  const int64_t pc = live ? p : P - 1;  // clamped for reads
  const int64_t k0 = K * w / kPrefixRanges, k1 = K * (w + 1) / kPrefixRanges;
  double acc = 0.0;
#pragma unroll 8
  for (int64_t k = k0; k < k1; k++) acc += ssum[k * P + pc];
  tot[w][lane] = acc;
  __syncthreads();
  double run = 0.0;
  for (int j = 0; j < w; j++) run += tot[j][lane];
  if (live && w == 0) ps64[p] = 0.0;
#pragma unroll 8
  for (int64_t k = k0; k < k1; k++) {
    run += ssum[k * P + pc];
    if (live) ps64[(k + 1) * P + p] = run;
  }
}

// Local reverse scan of every chunk with zero carry: writes
//   umu[k] = a_{t0} mu^loc_{t0}   (the chunk's contribution to the carry leaving it),
// and for a window W < T the fp64 sum of s over the W tokens after the chunk.
template <typename IO, int NL, int G, bool WIN>
__global__ __launch_bounds__(64) void k_bwd_local(BwdArgs a) {
  constexpr int CH = 64 / G;
  constexpr int NN = NL * G;
  const int lane = threadIdx.x;
  const int grp = lane / CH, pl = lane % CH;
  const int64_t T = a.T, P = a.P, W = a.W;
  const int C = a.C;
  const int64_t K = (T + C - 1) / C;
  const int64_t k = blockIdx.x;
  const int64_t p = static_cast<int64_t>(blockIdx.y) * CH + pl;
  const bool valid = p < P;
  const int64_t pc = valid ? p : P - 1;
  const int n0 = grp * NL;
  float al2[NL], inc[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) {
    al2[j] = a.alpha[pc * NN + n0 + j] * kLog2e;
    inc[j] = 0.0f;
  }
  const int64_t t0 = k * C;
  const int64_t t1 = (t0 + C < T) ? t0 + C : T;
  double H = 0.0, sigma = 0.0, suffix = 0.0;
  if constexpr (WIN) {
    // H = sum of s over tokens (t1 .. t1+W-1) clipped to T: whole chunks
    // k+1 .. k+q, then the first w0 tokens of chunk k+q+1.
    const int64_t q = W / C, w0 = W % C;
    const int64_t kb = (k + q + 1 < K) ? k + q + 1 : K;
    const int64_t ka = (k + 1 < K) ? k + 1 : K;
    H = a.ps64[kb * P + pc] - a.ps64[ka * P + pc];
    if (k + q + 1 < K) {
      const int64_t h0 = (k + q + 1) * C;
      const int64_t h1 = (h0 + w0 < T) ? h0 + w0 : T;
      for (int64_t t = h0; t < h1; t++) H += static_cast<double>(a.s[t * P + pc]);
    }
    if (valid && grp == 0) a.hwin[k * P + p] = H;
  }
  const IO* x = static_cast<const IO*>(a.x);
  (void)x;
  for (int64_t i = t1 - 1; i >= t0; i--) {
    const float s = a.s[i * P + pc];
    const float gv = a.g[i * P + pc];
    float ct[NL];
    load_row<NL>(a.c + i * NN + n0, ct);
    float mu[NL], av[NL];
#pragma unroll
    for (int j = 0; j < NL; j++) {
      av[j] = fast_exp2(-s * al2[j]);
      mu[j] = fmaf(gv, ct[j], inc[j]);
    }
    if constexpr (WIN) {
      const int64_t m = i + W;
      if (m < T) {
        const float sm = a.s[m * P + pc];
        const float gm = a.g[m * P + pc];
        float cm[NL];
        load_row<NL>(a.c + m * NN + n0, cm);
        const float E = static_cast<float>(sigma + H - suffix);
#pragma unroll
        for (int j = 0; j < NL; j++) {
          const float D = fast_exp2(-E * al2[j]);
          mu[j] = fmaf(-gm * cm[j], D, mu[j]);
        }
        suffix += static_cast<double>(sm);
      }
      sigma += static_cast<double>(s);
    }
#pragma unroll
    for (int j = 0; j < NL; j++) inc[j] = av[j] * mu[j];
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < NL; j++) a.umu[(k * P + p) * NN + n0 + j] = inc[j];
  }
}

// Staged variant of k_bwd_local (N >= 4, rows of a chunk fit in LDS): a
// 4-wavefront workgroup takes 4 channel blocks of one chunk; the chunk's c
// rows and its window-partner rows c_{t+W} are staged once into LDS, and the
// per-lane s, g and partner s, g come through an 8-token register ring,
// walked right to left.
constexpr int kBwdLocWpb = 4;
constexpr int kBwdLocRing = 8;
constexpr size_t kBwdLocRowLds = 32 * 1024;
// The sub-chunk pass stages only b rows; up to 64 KB of them (C = 256 at
// N = 64) still leaves room for two workgroups per CU.
constexpr size_t kHsubRowLds = 64 * 1024;

template <typename IO, int NL, int G, bool WIN>
__global__ __launch_bounds__(256) void k_bwd_local_staged(BwdArgs a, int64_t NB) {
  constexpr int CH = 64 / G;
  constexpr int NN = NL * G;
  constexpr int D = kBwdLocRing;
  extern __shared__ float rows[];  // [WIN ? 2 : 1][C][NN]: c rows, then partner c rows
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int grp = lane / CH, pl = lane % CH;
  const int64_t T = a.T, P = a.P, W = a.W;
  const int C = a.C;
  const int64_t K = (T + C - 1) / C;
  const int64_t k = blockIdx.x;
  const int64_t cb = static_cast<int64_t>(blockIdx.y) * kBwdLocWpb + w;
  const int64_t p = cb * CH + pl;
  const bool valid = cb < NB && p < P;
  const int64_t pc = p < P ? p : P - 1;
  const int n0 = grp * NL;
  const int64_t t0 = k * C;
  const int64_t t1 = (t0 + C < T) ? t0 + C : T;
  const int len = static_cast<int>(t1 - t0);
  // stage rows: c[t0 .. t1) and (window) c[t0 + W .. t1 + W) clipped to T
  {
    const int per = len * NN / 4;
    const float4* s4 = reinterpret_cast<const float4*>(a.c + t0 * NN);
    float4* d4 = reinterpret_cast<float4*>(rows);
    for (int e = tid; e < per; e += 64 * kBwdLocWpb) d4[e] = s4[e];
    if constexpr (WIN) {
      const int64_t m1 = (t1 + W < T) ? t1 + W : T;
      const int plen = (t0 + W < m1) ? static_cast<int>(m1 - (t0 + W)) : 0;
      const int pper = plen * NN / 4;
      const float4* m4 = reinterpret_cast<const float4*>(a.c + (t0 + W) * NN);
      float4* e4 = reinterpret_cast<float4*>(rows + static_cast<size_t>(C) * NN);
      for (int e = tid; e < pper; e += 64 * kBwdLocWpb) e4[e] = m4[e];
    }
  }
  float al2[NL], inc[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) {
    al2[j] = a.alpha[pc * NN + n0 + j] * kLog2e;
    inc[j] = 0.0f;
  }
  double sigma = 0.0, suffix = 0.0;
  if constexpr (WIN) {
    // window sum of s after the chunk (see k_bwd_local); sigma starts there
    const int64_t q = W / C, w0 = W % C;
    const int64_t kb = (k + q + 1 < K) ? k + q + 1 : K;
    const int64_t ka = (k + 1 < K) ? k + 1 : K;
    double H = a.ps64[kb * P + pc] - a.ps64[ka * P + pc];
    if (k + q + 1 < K) {
      const int64_t h0 = (k + q + 1) * C;
      const int64_t h1 = (h0 + w0 < T) ? h0 + w0 : T;
      for (int64_t t = h0; t < h1; t++) H += static_cast<double>(a.s[t * P + pc]);
    }
    if (valid && grp == 0) a.hwin[k * P + p] = H;
    sigma = H;
  }
  const uint32_t ob4 = static_cast<uint32_t>(pc) * 4u;
  float rs[D], rg[D], rsm[D], rgm[D];
  // ring slot r holds token t1 - 1 - (index), index = position in the reverse walk
  auto ld = [&](int slot, int64_t i) {
    rs[slot] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.s + i * P) + ob4);
    rg[slot] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.g + i * P) + ob4);
    if constexpr (WIN) {
      // partner token; the walk reads these only where i + W < T
      const int64_t m = i + W;
      const int64_t mm = m < T ? m : i;
      rsm[slot] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.s + mm * P) + ob4);
      rgm[slot] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.g + mm * P) + ob4);
    }
  };
#pragma unroll
  for (int q = 0; q < D - 1; q++)
    if (q < len) ld(q, t1 - 1 - q);
  __syncthreads();  // staged rows visible
  // one token of the walk at position idx; the ring fetches position ahead
  auto tok = [&](int r, int idx, bool fetch, int ahead) {
    if (fetch) ld((r + D - 1) % D, t1 - 1 - ahead);
    const int tau = len - 1 - idx;  // token i = t0 + tau
    const int64_t i = t0 + tau;
    const float sv = rs[r], gv = rg[r];
    float ct[NL];
    const float* rc = rows + tau * NN + n0;
#pragma unroll
    for (int j = 0; j < NL; j += 4) {
      const float4 v = *reinterpret_cast<const float4*>(rc + j);
      ct[j] = v.x; ct[j + 1] = v.y; ct[j + 2] = v.z; ct[j + 3] = v.w;
    }
    float mu[NL], av[NL];
#pragma unroll
    for (int j = 0; j < NL; j++) {
      av[j] = fast_exp2(-sv * al2[j]);
      mu[j] = fmaf(gv, ct[j], inc[j]);
    }
    if constexpr (WIN) {
      if (i + W < T) {
        float cm[NL];
        const float* rm = rows + static_cast<size_t>(C) * NN + tau * NN + n0;
#pragma unroll
        for (int j = 0; j < NL; j += 4) {
          const float4 v = *reinterpret_cast<const float4*>(rm + j);
          cm[j] = v.x; cm[j + 1] = v.y; cm[j + 2] = v.z; cm[j + 3] = v.w;
        }
        const float E = static_cast<float>(sigma - suffix);
        const float gm = rgm[r];
#pragma unroll
        for (int j = 0; j < NL; j++) {
          const float Dw = fast_exp2(-E * al2[j]);
          mu[j] = fmaf(-gm * cm[j], Dw, mu[j]);
        }
        suffix += static_cast<double>(rsm[r]);
      }
      sigma += static_cast<double>(sv);
    }
#pragma unroll
    for (int j = 0; j < NL; j++) inc[j] = av[j] * mu[j];
  };
  if (len % D == 0) {
    // whole ring turns: no per-token branches (fetches past the chunk start
    // re-read its first token), so no merge of paths makes the compiler wait
    // for the ring's loads in flight
    for (int q8 = 0; q8 < len; q8 += D) {
#pragma unroll
      for (int r = 0; r < D; r++) {
        const int idx = q8 + r;
        tok(r, idx, true, (idx + D - 1 < len) ? idx + D - 1 : len - 1);
      }
    }
  } else {
    for (int q8 = 0; q8 < len; q8 += D) {
#pragma unroll
      for (int r = 0; r < D; r++) {
        const int idx = q8 + r;  // position in the reverse walk
        if (idx < len) tok(r, idx, idx + D - 1 < len, idx + D - 1);
      }
    }
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < NL; j++) a.umu[(k * P + p) * NN + n0 + j] = inc[j];
  }
}

// Sub-chunk start states for the main kernel (N >= 4, a chunk's b rows fit in
// LDS): the forward walk from the chunk checkpoint, as in the main kernel's
// first phase, with the workgroup layout of the main kernel (4 wavefronts =
// 4 channel blocks of one chunk, the same per-wavefront scratch layout), the
// chunk's b rows staged in LDS and s, x through an 8-token register ring.
template <typename IO, int NL, int G>
__global__ __launch_bounds__(256) void k_bwd_hsub(BwdArgs a, int64_t NB) {
  constexpr int CH = 64 / G;
  constexpr int NN = NL * G;
  constexpr int D = kBwdLocRing;
  constexpr int S = kSub;
  extern __shared__ float rows[];  // [C][NN] b rows
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int grp = lane / CH, pl = lane % CH;
  const int64_t T = a.T, P = a.P;
  const int C = a.C;
  const int64_t k = a.k_lo + blockIdx.x;  // chunk (the launch covers one slab)
  const int64_t cb = static_cast<int64_t>(blockIdx.y) * kWpb + w;
  const bool wave_live = cb < NB;
  const int64_t p = cb * CH + pl;
  const int64_t pc = p < P ? p : P - 1;
  const int n0 = grp * NL;
  const int64_t t0 = k * C;
  const int64_t t1 = (t0 + C < T) ? t0 + C : T;
  const int len = static_cast<int>(t1 - t0);
  const int nsub_max = (C + S - 1) / S;
  float* hsg = a.hsub + hsub_offset(k - a.hsub_k0, wave_live ? cb : 0, 0, NB, nsub_max, NL);
  {
    const int per = len * NN / 4;
    const float4* s4 = reinterpret_cast<const float4*>(a.b + t0 * NN);
    float4* d4 = reinterpret_cast<float4*>(rows);
    for (int e = tid; e < per; e += 64 * kWpb) d4[e] = s4[e];
  }
  float al2[NL], h[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) {
    al2[j] = a.alpha[pc * NN + n0 + j] * kLog2e;
    h[j] = a.h_ckpt[(k * P + pc) * NN + n0 + j];
  }
  const IO* xp = static_cast<const IO*>(a.x);
  const uint32_t ob4 = static_cast<uint32_t>(pc) * 4u;
  const uint32_t obx = static_cast<uint32_t>(pc) * static_cast<uint32_t>(sizeof(IO));
  float rs[D];
  typename IoRaw<IO>::type rx[D];
  auto ld = [&](int slot, int64_t t) {
    rs[slot] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.s + t * P) + ob4);
    rx[slot] = load_raw(reinterpret_cast<const IO*>(reinterpret_cast<const char*>(xp + t * P) + obx));
  };
#pragma unroll
  for (int q = 0; q < D - 1; q++)
    if (q < len) ld(q, t0 + q);
  __syncthreads();  // staged rows visible
  static_assert(D % S == 0 || S % D == 0, "ring and sub-chunk sizes");
  for (int q8 = 0; q8 < len; q8 += D) {
#pragma unroll
    for (int r = 0; r < D; r++) {
      const int tau = q8 + r;
      if (tau < len) {
        if (tau % S == 0 && wave_live) {
#pragma unroll
          for (int j = 0; j < NL; j++) hsg[((tau / S) * NL + j) * 64 + lane] = h[j];
        }
        if (tau + D - 1 < len) ld((r + D - 1) % D, t0 + tau + D - 1);
        const float ns = -rs[r];
        const float xv = raw_to_f32(rx[r]);
        const float* rb = rows + tau * NN + n0;
#pragma unroll
        for (int j = 0; j < NL; j += 4) {
          const float4 v = *reinterpret_cast<const float4*>(rb + j);
          const float bq[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int jj = 0; jj < 4; jj++)
            h[j + jj] = fmaf(fast_exp2(ns * al2[j + jj]), h[j + jj], bq[jj] * xv);
        }
      }
    }
  }
}

// The chunk-local reverse aggregate and the sub-chunk start states in one
// forward walk over the chunk (exact aggregates: no window term inside the
// walk), for slabs processed right to left.  The aggregate of chunk k with a
// zero carry entering from its right,
//   umu[k] = a_{t0} mu^loc_{t0} = sum_{t in k} g_t c_t prod_{j=t0}^{t} a_j ,
// is accumulated in token order with the running product
// Q_t = prod_{j=t0}^{t} a_j, so the same decay factors serve the state
// recurrence h_t = a_t h_{t-1} + b_t x_t, whose value entering every kSub-th
// token goes to the sub-chunk-state slab (layout of k_bwd_hsub).  A 4-wavefront
// workgroup takes 4 channel blocks of one chunk; the chunk's b and c rows are
// staged once into LDS, s, x and g come through an 8-token register ring.
template <typename IO, int NL, int G, bool PARTS>
__global__ __launch_bounds__(256) void k_bwd_local_hsub(BwdArgs a, int64_t NB) {
  constexpr int CH = 64 / G;
  constexpr int NN = NL * G;
  constexpr int D = kBwdLocRing;
  constexpr int S = kSub;
  // The chunk's b and c rows are staged in parts of TP tokens (the whole
  // chunk when its rows fit the staging area): [TP][NN] b rows, then [TP][NN]
  // c rows.
  constexpr int TP = static_cast<int>(kHsubRowLds / (2 * NN * 4)) / D * D;
  static_assert(TP >= D, "a ring turn of rows fits the staging area");
  extern __shared__ float rows[];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int grp = lane / CH, pl = lane % CH;
  const int64_t T = a.T, P = a.P;
  const int C = a.C;
  // one workgroup per (chunk of the slab, channel group): chunk_group_grid
  uint32_t kc, kg;
  chunk_and_group(&kc, &kg);
  const int64_t k = a.k_lo + kc;  // chunk (the launch covers one slab)
  const int64_t cb = static_cast<int64_t>(kg) * kWpb + w;
  const bool wave_live = cb < NB;
  const int64_t p = cb * CH + pl;
  const bool valid = wave_live && p < P;
  const int64_t pc = p < P ? p : P - 1;
  const int n0 = grp * NL;
  const int64_t t0 = k * C;
  const int64_t t1 = (t0 + C < T) ? t0 + C : T;
  const int len = static_cast<int>(t1 - t0);
  const int nsub_max = (C + S - 1) / S;
  // The sub-chunk start states go through a buffer resource over this
  // wavefront's region (covering no bytes for a wavefront past the last
  // channel block), at this lane's offset plus the sub-chunk's, both in the
  // range-checked vector offset (the scalar offset is not range-checked): no
  // branch and no 64-bit address per store.  The state entering sub-chunk
  // u + 1 is stored right after the token that ends sub-chunk u (a chunk's
  // last one lands past the region and is dropped), the chunk checkpoint
  // before the walk, so the walk never stores a state still being loaded and
  // its ring's loads are not drained at every sub-chunk.
  const __amdgpu_buffer_rsrc_t rsub = __builtin_amdgcn_make_buffer_rsrc(
      a.hsub + hsub_offset(k - a.hsub_k0, wave_live ? cb : 0, 0, NB, nsub_max, NL), 0,
      wave_live ? static_cast<int>(static_cast<int64_t>(nsub_max) * NL * 64 * 4) : 0, kBufWord3);
  const int voff_lane = lane * 4;
  const int tp = len < TP ? len : TP;  // tokens per staged part
  float* crow = rows + static_cast<size_t>(tp) * NN;
  // rows of tokens [lo, lo + n) -> the staging area (the caller synchronises)
  auto stage = [&](int lo, int n) {
    const int per = n * NN / 4;
    const float4* b4 = reinterpret_cast<const float4*>(a.b + (t0 + lo) * NN);
    const float4* c4 = reinterpret_cast<const float4*>(a.c + (t0 + lo) * NN);
    float4* db4 = reinterpret_cast<float4*>(rows);
    float4* dc4 = reinterpret_cast<float4*>(crow);
    for (int e = tid; e < per; e += 64 * kWpb) {
      db4[e] = b4[e];
      dc4[e] = c4[e];
    }
  };
  stage(0, tp);
  float al2[NL], h[NL], Q[NL], U[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) {
    al2[j] = a.alpha[pc * NN + n0 + j] * kLog2e;
    h[j] = a.h_ckpt[(k * P + pc) * NN + n0 + j];
    Q[j] = 1.0f;
    U[j] = 0.0f;
  }
  const IO* xp = static_cast<const IO*>(a.x);
  const uint32_t ob4 = static_cast<uint32_t>(pc) * 4u;
  const uint32_t obx = static_cast<uint32_t>(pc) * static_cast<uint32_t>(sizeof(IO));
  float rs[D], rg[D];
  typename IoRaw<IO>::type rx[D];
  auto ld = [&](int slot, int64_t t) {
    rs[slot] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.s + t * P) + ob4);
    rg[slot] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.g + t * P) + ob4);
    rx[slot] = load_raw(reinterpret_cast<const IO*>(reinterpret_cast<const char*>(xp + t * P) + obx));
  };
#pragma unroll
  for (int q = 0; q < D - 1; q++)
    if (q < len) ld(q, t0 + q);
  // the state entering sub-chunk 0: the checkpoint
#pragma unroll
  for (int j = 0; j < NL; j++)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(h[j]), rsub, voff_lane + j * 256, 0, 0);
  __syncthreads();  // staged rows visible
  static_assert(D % S == 0 || S % D == 0, "ring and sub-chunk sizes");
  int plo = 0;  // first token of the staged part
  {
    constexpr bool MULTI = PARTS;
    auto tok = [&](int r, int tau, bool fetch, int ahead) {
      if (fetch) ld((r + D - 1) % D, t0 + ahead);
      const float ns = -rs[r];
      const float xv = raw_to_f32(rx[r]);
      const float gv = rg[r];
      const float* rb = rows + (MULTI ? tau - plo : tau) * NN + n0;
      const float* rc = crow + (MULTI ? tau - plo : tau) * NN + n0;
#pragma unroll
      for (int j = 0; j < NL; j += 4) {
        const float4 vb = *reinterpret_cast<const float4*>(rb + j);
        const float4 vc = *reinterpret_cast<const float4*>(rc + j);
        const float bq[4] = {vb.x, vb.y, vb.z, vb.w};
        const float cq[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const float av = fast_exp2(ns * al2[j + jj]);
          h[j + jj] = fmaf(av, h[j + jj], bq[jj] * xv);
          Q[j + jj] *= av;
          U[j + jj] = fmaf(gv * cq[jj], Q[j + jj], U[j + jj]);
        }
      }
      if ((tau + 1) % S == 0) {
#pragma unroll
        for (int j = 0; j < NL; j++)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(h[j]), rsub,
                                                voff_lane + ((tau + 1) / S) * (NL * 256) + j * 256, 0, 0);
      }
    };
    // the next part's rows, once every wavefront is done with this part's
    // (parts are whole ring turns)
    auto next_part = [&](int q8) {
      if (MULTI && q8 > plo && q8 - plo == tp) {
        __syncthreads();
        plo = q8;
        stage(plo, len - plo < tp ? len - plo : tp);
        __syncthreads();
      }
    };
    if (len % D == 0) {
      // whole ring turns: fetches past the chunk end re-read its last token,
      // so the ring body has no per-token branch
      for (int q8 = 0; q8 < len; q8 += D) {
        next_part(q8);
#pragma unroll
        for (int r = 0; r < D; r++) {
          const int tau = q8 + r;
          tok(r, tau, true, (tau + D - 1 < len) ? tau + D - 1 : len - 1);
        }
      }
    } else {
      for (int q8 = 0; q8 < len; q8 += D) {
        next_part(q8);
#pragma unroll
        for (int r = 0; r < D; r++) {
          const int tau = q8 + r;
          if (tau < len) tok(r, tau, tau + D - 1 < len, tau + D - 1);
        }
      }
    }
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < NL; j++) a.umu[(k * P + p) * NN + n0 + j] = U[j];
  }
}

// Carry of the adjoint sums between chunks, right to left:
//   carry[K-1] = 0,  carry[k-1] = A_k carry[k] + u_k,  A_k = exp(-alpha sum_{t in k} s_t),
// with u_k the aggregate of chunk k.  carry[k] is a_{e+1} mu_{e+1} for the
// last token e of chunk k.
//
// Windows of a whole number q = W / C of chunks: the window term of chunk k's
// aggregate is then the exact aggregate of chunk k + q scaled by the decay
// across the W tokens in between,
//   sum_{i in k} g_{i+W} c_{i+W} prod_{j=t0}^{i+W} a_j
//     = exp(-alpha sum_{t=t0}^{t0+W-1} s_t) * umu_exact[k+q],
// because the tokens i + W of a full chunk k are exactly chunk k + q (a
// partial chunk is the last one, and has no partner inside the sequence).
// The local pass then runs without window terms, and with q > 0 this kernel
// forms each windowed aggregate from the exact ones as it reads them; lanes
// of state 0 also write the fp64 sum of s over the W tokens that follow each
// chunk, for the main kernel.  With q = 0 umu holds the aggregates as they
// are.
//
// The walk is a segmented scan (seg_affine_scan): segments of kSegLen chunks
// at fixed positions, kSegs wavefronts per workgroup, 64 (channel, state)
// pairs per wavefront.  A launch over [k_lo, k_hi) starts from `edge` (zero
// at the right end of the sequence) and leaves the carry entering chunk
// k_lo - 1 in `edge`.  Slabs that start at multiples of kSegLen give the
// same carries, bit for bit, as one launch over all chunks.
constexpr int kSegs = 16;

template <int L>
__global__ __launch_bounds__(64 * kSegs) void k_bwd_carry_seg(int64_t K, int64_t P, int64_t N, int64_t q,
                                                              int64_t k_lo, int64_t k_hi,
                                                              const float* __restrict__ alpha,
                                                              const double* __restrict__ ssum,
                                                              const double* __restrict__ ps64,
                                                              const float* __restrict__ umu,
                                                              float* __restrict__ carry, float* __restrict__ edge,
                                                              double* __restrict__ hwin) {
  __shared__ float sA[kSegs][64], sB[kSegs][64];
  const int64_t PN = P * N;
  const int lane = threadIdx.x & 63;
  const int sg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const bool live = e < PN;
  const int64_t ee = live ? e : PN - 1;  // clamped for reads
  const int64_t p = ee / N;
  const float al2 = alpha[ee] * kLog2e;
  const float cin = k_hi < K ? edge[ee] : 0.0f;
  auto load = [&](int64_t k, float* u, float* d) {
    float v = umu[k * PN + ee];
    if (q > 0 && k + q < K) {
      const float Ew = static_cast<float>(ps64[(k + q) * P + p] - ps64[k * P + p]);
      v = fmaf(-fast_exp2(-Ew * al2), umu[(k + q) * PN + ee], v);
    }
    *u = v;
    *d = fast_exp2(-static_cast<float>(ssum[k * P + p]) * al2);
  };
  auto store = [&](int64_t k, float x) {
    if (live) carry[k * PN + e] = x;
  };
  const float out = seg_affine_scan<L, kSegs, true>(k_lo, k_hi, cin, sA, sB, sg, lane, load, store);
  if (k_lo > 0 && live && sg == 0) edge[e] = out;
  if (q > 0 && live && ee - p * N == 0) {
    for (int64_t k = k_lo + sg; k < k_hi; k += kSegs) {
      const int64_t kb = (k + q + 1 < K) ? k + q + 1 : K;
      const int64_t ka = (k + 1 < K) ? k + 1 : K;
      hwin[k * P + p] = ps64[kb * P + p] - ps64[ka * P + p];
    }
  }
}

#include "bwd_main.inl"

// db, dc: deterministic sum of the per-workgroup partials, written as the
// io-typed columns [P, P+2N) of dY (the weight-gradient GEMM operand).
template <typename IO>
__global__ __launch_bounds__(256) void k_bwd_reduce_dbdc(int64_t T, int64_t P, int OUT, int64_t NBW,
                                                         const float* __restrict__ part, IO* __restrict__ dY,
                                                         int64_t ldy) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= T * OUT) return;
  const int64_t t = e / OUT;
  const int o = static_cast<int>(e % OUT);
  const float* src = part + t * NBW * OUT + o;
  float v = 0.0f;
  for (int64_t wb = 0; wb < NBW; wb++) v += src[wb * OUT];
  store_io(dY + t * ldy + P + o, v);
}

// The same sums, four outputs per thread (OUT a multiple of 4): the NBW
// partials of a token come as 16-byte loads, all in flight together, and
// each output is summed over the workgroups in the same order as above.
template <typename IO>
__global__ __launch_bounds__(256) void k_bwd_reduce_dbdc4(int64_t T, int64_t P, int OUT, int64_t NBW,
                                                          const float* __restrict__ part, IO* __restrict__ dY,
                                                          int64_t ldy) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int Q = OUT / 4;
  if (e >= T * Q) return;
  const int64_t t = e / Q;
  const int o = static_cast<int>(e % Q) * 4;
  const float4* src = reinterpret_cast<const float4*>(part + t * NBW * OUT + o);
  const int64_t step = OUT / 4;
  float4 v = src[0];
  int64_t wb = 1;
  for (; wb + 4 <= NBW; wb += 4) {
    float4 r[4];
#pragma unroll
    for (int i = 0; i < 4; i++) r[i] = src[(wb + i) * step];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v.x += r[i].x;
      v.y += r[i].y;
      v.z += r[i].z;
      v.w += r[i].w;
    }
  }
  for (; wb < NBW; wb++) {
    const float4 r = src[wb * step];
    v.x += r.x;
    v.y += r.y;
    v.z += r.z;
    v.w += r.w;
  }
  IO* dst = dY + t * ldy + P + o;
  store_io(dst, v.x);
  store_io(dst + 1, v.y);
  store_io(dst + 2, v.z);
  store_io(dst + 3, v.w);
}

// dalpha and dbias: sums over chunks in a fixed order, in two stages so the
// loads are spread over many threads: stage 1 sums KS slices of the chunk
// range into tmp[KS][P*N + P], stage 2 adds the KS slice sums.
__global__ __launch_bounds__(256) void k_bwd_reduce_chunks1(int64_t K, int64_t P, int64_t N, int KS,
                                                            const float* __restrict__ dal_part,
                                                            const float* __restrict__ dbias_part,
                                                            float* __restrict__ tmp) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int s = blockIdx.y;
  const int64_t PN = P * N;
  const int64_t k0 = (K * s) / KS, k1 = (K * (s + 1)) / KS;
  if (e < PN) {
    float v = 0.0f;
    for (int64_t k = k0; k < k1; k++) v += dal_part[k * PN + e];
    tmp[static_cast<int64_t>(s) * (PN + P) + e] = v;
  } else if (e < PN + P) {
    const int64_t q = e - PN;
    float v = 0.0f;
    for (int64_t k = k0; k < k1; k++) v += dbias_part[k * P + q];
    tmp[static_cast<int64_t>(s) * (PN + P) + e] = v;
  }
}

__global__ __launch_bounds__(256) void k_bwd_reduce_chunks2(int64_t P, int64_t N, int KS, const float* __restrict__ tmp,
                                                            float* __restrict__ dalpha, float* __restrict__ dbias) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t PN = P * N;
  if (e >= PN + P) return;
  float v = 0.0f;
  for (int s = 0; s < KS; s++) v += tmp[static_cast<int64_t>(s) * (PN + P) + e];
  if (e < PN) {
    if (dalpha) dalpha[e] = v;
  } else if (dbias) {
    dbias[e - PN] = v;
  }
}

// ----------------------------------------------------------------- planning

static void nl_g_for(int64_t N, int* NL, int* G) {
  if (N <= 8) { *NL = static_cast<int>(N); *G = 1; }
  else { *NL = 8; *G = static_cast<int>(N / 8); }
}

bool bwd_plan(int64_t P, int64_t N, int C, BwdPlan* pl) {
  int NL, G;
  nl_g_for(N, &NL, &G);
  const int CH = 64 / G;
  const int S = kSub;
  const int wpb = kWpb;
  const size_t floats = bwd_main_lds_floats(NL, G);
  if (floats * 4 > 160 * 1024) return false;
  (void)C;
  const int64_t NB = (P + CH - 1) / CH;
  pl->NL = NL; pl->G = G; pl->CH = CH; pl->S = S; pl->wpb = wpb;
  pl->NB = NB;
  pl->NBW = (NB + wpb - 1) / wpb;
  pl->lds_bytes = floats * 4;
  return true;
}

size_t bwd_hsub_floats_chunks(int64_t chunks, int64_t P, int64_t N, int C) {
  BwdPlan pl;
  if (!bwd_plan(P, N, C, &pl)) return 0;
  const int64_t nsub = (C + pl.S - 1) / pl.S;
  return static_cast<size_t>(chunks * pl.NB * nsub) * pl.NL * 64;
}

size_t bwd_hsub_floats(int64_t T, int64_t P, int64_t N, int C) {
  return bwd_hsub_floats_chunks((T + C - 1) / C, P, N, C);
}

size_t bwd_hall_floats(int64_t T, int64_t P, int64_t N, int C) {
  BwdPlan pl;
  if (!bwd_plan(P, N, C, &pl)) return 0;
  return static_cast<size_t>((T + C - 1) / C * pl.NB * C) * pl.NL * 64;
}

int64_t bwd_hsub_slab_chunks(int64_t T, int64_t P, int64_t N, int C) {
  const int64_t K = (T + C - 1) / C;
  const size_t per = bwd_hsub_floats_chunks(1, P, N, C) * sizeof(float);
  if (per == 0) return K;
  int64_t n = static_cast<int64_t>(kHsubSlabBytes / per);
  if (n >= 32) n -= n % 32;  // whole rounds of resident workgroups when the channel blocks allow
  else if (n >= kSegLen) n -= n % kSegLen;
  if (n < 1) n = 1;
  return n < K ? n : K;
}

// ----------------------------------------------------------------- launchers

template <typename IO, int NL, int G, bool WIN>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  constexpr int CH = 64 / G;
  BwdPlan pl;
  if (!bwd_plan(a.P, a.N, a.C, &pl)) return hipErrorInvalidValue;
  const int64_t K = (a.T + a.C - 1) / a.C;
  const int64_t NB = pl.NB;
  hipError_t e;
  if constexpr (WIN) {
    k_bwd_prefix<<<static_cast<unsigned>((a.P + 63) / 64), 64 * kPrefixRanges, 0, st>>>(K, a.P, a.ssum, a.ps64);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // A window of whole chunks is composed from exact chunk aggregates in the
  // carry pass; otherwise the local pass walks the window term itself.
  const bool compose = WIN && (a.W % a.C) == 0;
  const bool wl = WIN && !compose;
  constexpr int NNc = NL * G;
  // Without sub-chunk states from the forward, exact local aggregates and a
  // chunk's b and c rows in LDS: the aggregates are formed in the same
  // forward walk that rebuilds the sub-chunk states, slab by slab from the
  // right (the carry enters each chunk from its right, so a slab needs only
  // the aggregates of itself and of the slabs already done).
  // (b and c rows in LDS, in parts of at most kHsubRowLds bytes)
  const size_t rows_f = std::min(static_cast<size_t>(2) * a.C * NNc * 4, kHsubRowLds / (2 * NNc * 4) / kBwdLocRing *
                                                                           kBwdLocRing * 2 * NNc * 4);
  const bool fused = !(a.hsub_given || a.hall != nullptr) && !wl && NNc % 4 == 0;
  if (!fused) {
    const size_t rows_b = static_cast<size_t>(wl ? 2 : 1) * a.C * NNc * 4;
    const dim3 gs(static_cast<unsigned>(K), static_cast<unsigned>((NB + kBwdLocWpb - 1) / kBwdLocWpb));
    const dim3 g1(static_cast<unsigned>(K), static_cast<unsigned>(NB));
    const bool staged = NNc % 4 == 0 && rows_b <= kBwdLocRowLds;
    if constexpr (WIN) {
      if (wl) {
        if (staged) k_bwd_local_staged<IO, NL, G, true><<<gs, 64 * kBwdLocWpb, rows_b, st>>>(a, NB);
        else k_bwd_local<IO, NL, G, true><<<g1, 64, 0, st>>>(a);
      }
    }
    if (!wl) {
      if (staged) k_bwd_local_staged<IO, NL, G, false><<<gs, 64 * kBwdLocWpb, rows_b, st>>>(a, NB);
      else k_bwd_local<IO, NL, G, false><<<g1, 64, 0, st>>>(a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  a.marks.rec(1, st);
  const int64_t PN = a.P * a.N;
  // States kept by the forward: nothing is rebuilt, and the carries run over
  // all chunks at once.
  const bool given = a.hsub_given || a.hall != nullptr;
  // Segment length of the carry's scan: short segments when the default slab
  // is short, so that the kSegs wavefronts of a workgroup all hold chunks of
  // it (a carry over all chunks at once keeps the long ones).  It depends on
  // the shapes only (not on the slab size a caller picks), and both lengths
  // divide kSegLen: slabs at multiples of kSegLen give the same carries, bit
  // for bit.
  const int64_t nseg = fused ? bwd_hsub_slab_chunks(a.T, a.P, a.N, a.C) : K;
  const bool short_seg = nseg <= static_cast<int64_t>(kSegs) * kSegLenShort;
  // carries of chunks [lo, hi) (windowed aggregates composed on the way)
  auto carry_range = [&](int64_t lo, int64_t hi) -> hipError_t {
    auto ck = short_seg ? k_bwd_carry_seg<kSegLenShort> : k_bwd_carry_seg<kSegLen>;
    ck<<<static_cast<unsigned>((PN + 63) / 64), 64 * kSegs, 0, st>>>(
        K, a.P, a.N, compose ? a.W / a.C : 0, lo, hi, a.alpha, a.ssum, a.ps64, a.umu, a.carry, a.edge, a.hwin);
    return hipGetLastError();
  };
  if (!fused && (e = carry_range(0, K)) != hipSuccess) return e;
  a.marks.rec(2, st);
  // Sub-chunk start states and the fused reverse walk.  States kept by the
  // forward cover every chunk: one launch.  Otherwise the gradient rebuilds
  // them slab by slab into a region that holds a.hsub_chunks chunks, each
  // slab's rebuild followed by the reverse walk over the same chunks, so the
  // region's size does not grow with T.
  auto kern = a.hall ? k_bwd_main<IO, NL, G, WIN, true> : k_bwd_main<IO, NL, G, WIN, false>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(pl.lds_bytes));
  if (e != hipSuccess) return e;
  const size_t rows_h = static_cast<size_t>(a.C) * NNc * 4;
  const bool hpass = !given && !fused && NNc % 4 == 0 && rows_h <= kHsubRowLds;
  if (hpass) {
    auto hk = k_bwd_hsub<IO, NL, G>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(hk), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(rows_h));
    if (e != hipSuccess) return e;
  }
  // rows staged in parts when a chunk's do not fit the staging area at once
  const bool parts = static_cast<size_t>(2) * a.C * NNc * 4 > kHsubRowLds;
  auto fk = parts ? k_bwd_local_hsub<IO, NL, G, true> : k_bwd_local_hsub<IO, NL, G, false>;
  if (fused) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(fk), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(rows_f));
    if (e != hipSuccess) return e;
  }
  const int64_t slab = given ? K : a.hsub_chunks;
  if (slab < 1) return hipErrorInvalidValue;
  const int64_t nslab = (K + slab - 1) / slab;
  for (int64_t q = 0; q < nslab; q++) {
    // slabs right to left when the aggregates are formed slab by slab
    const int64_t si = fused ? nslab - 1 - q : q;
    const int64_t k_lo = si * slab;
    const int64_t nk = (K - k_lo < slab) ? K - k_lo : slab;
    BwdArgs am = a;  // arguments of this slab's launches
    am.k_lo = k_lo;
    am.hsub_k0 = given ? 0 : k_lo;
    am.hsub_ready = given ? 1 : 0;
    const dim3 grid(static_cast<unsigned>(nk), static_cast<unsigned>(pl.NBW));
    if (fused) {
      fk<<<chunk_group_grid(nk, pl.NBW), 64 * kWpb, rows_f, st>>>(am, NB);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = carry_range(k_lo, k_lo + nk)) != hipSuccess) return e;
      am.hsub_ready = 1;
    } else if (hpass) {
      k_bwd_hsub<IO, NL, G><<<grid, 64 * kWpb, rows_h, st>>>(am, NB);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      am.hsub_ready = 1;
    }
    a.marks.rec_slab(static_cast<int>(2 * q), st);
    kern<<<grid, pl.wpb * 64, pl.lds_bytes, st>>>(am, pl.NB, pl.NBW);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    a.marks.rec_slab(static_cast<int>(2 * q + 1), st);
  }
  a.marks.rec(3, st);
  const int OUT = 2 * static_cast<int>(a.N);
  if (OUT % 4 == 0)
    k_bwd_reduce_dbdc4<IO><<<static_cast<unsigned>((a.T * (OUT / 4) + 255) / 256), 256, 0, st>>>(
        a.T, a.P, OUT, pl.NBW, a.part, static_cast<IO*>(a.dY), a.ldy);
  else
    k_bwd_reduce_dbdc<IO><<<static_cast<unsigned>((a.T * OUT + 255) / 256), 256, 0, st>>>(
        a.T, a.P, OUT, pl.NBW, a.part, static_cast<IO*>(a.dY), a.ldy);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.dalpha || a.dbias) {
    // the chunk aggregates (umu) are dead after the carry pass: reuse them as scratch
    int KS = static_cast<int>(K < 64 ? K : 64);
    while (KS > 1 && static_cast<int64_t>(KS) * (PN + a.P) > K * PN + a.P) KS--;
    const unsigned nb = static_cast<unsigned>((PN + a.P + 255) / 256);
    k_bwd_reduce_chunks1<<<dim3(nb, static_cast<unsigned>(KS)), 256, 0, st>>>(K, a.P, a.N, KS, a.dal_part,
                                                                             a.dbias_part, a.umu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_bwd_reduce_chunks2<<<nb, 256, 0, st>>>(a.P, a.N, KS, a.umu, a.dalpha, a.dbias);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  (void)CH;
  a.marks.rec(4, st);
  return hipSuccess;
}

template <typename IO, bool WIN>
static hipError_t launch_bwd_w(const BwdArgs& a, hipStream_t st) {
  switch (a.N) {
    case 1: return launch_bwd_t<IO, 1, 1, WIN>(a, st);
    case 2: return launch_bwd_t<IO, 2, 1, WIN>(a, st);
    case 4: return launch_bwd_t<IO, 4, 1, WIN>(a, st);
    case 8: return launch_bwd_t<IO, 8, 1, WIN>(a, st);
    case 16: return launch_bwd_t<IO, 8, 2, WIN>(a, st);
    case 32: return launch_bwd_t<IO, 8, 4, WIN>(a, st);
    case 64: return launch_bwd_t<IO, 8, 8, WIN>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_backward_scan(const BwdArgs& a, bool bf16, hipStream_t st) {
  const bool win = a.W < a.T;
  if (bf16) return win ? launch_bwd_w<bf16_t, true>(a, st) : launch_bwd_w<bf16_t, false>(a, st);
  return win ? launch_bwd_w<float, true>(a, st) : launch_bwd_w<float, false>(a, st);
}

}  // namespace ssm
