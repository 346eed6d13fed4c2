// scan_fwd.hip -- chunked, time-parallel forward scan of the selective SSM
// recurrence on gfx950.
//
// Recurrence (review of "Adjoint sharding for very long context training of
// state space models", Assumptions / Section 3.1), diagonal per channel p:
//   a_t[p][n] = exp(-s_t[p] alpha[p][n]),   s = softplus(Delta)
//   h_t[p][n] = a_t[p][n] h_{t-1}[p][n] + b_t[n] x_t[p]
//   y_t[p]    = sum_n c_t[n] h_t[p][n]
// Time is cut into chunks of C tokens.  Three launches:
//   1. k_fwd_local : every (chunk, channel block) scans its chunk from h = 0
//                    and records the end state and sum_t s_t (fp64).
//   2. k_fwd_carry : per (p, n), a segmented scan over the chunks in order
//                    composes the affine chunk maps h -> A_k h + hloc_k with
//                    A_k = exp(-alpha sum_{t in k} s_t); it writes the state
//                    entering every chunk, h_{kC-1}, which is also the saved
//                    checkpoint (store at segment boundaries, recompute inside:
//                    review of "Training Deep Nets with Sublinear Memory Cost",
//                    What carries the argument).
//   3. k_fwd_final : every (chunk, channel block) rescans its chunk from the
//                    exact entering state and writes y.
#include <type_traits>

#include "ssm_common.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

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

template <typename IO, int NL, int G>
__global__ __launch_bounds__(64) void k_fwd_local(int64_t T, int64_t P, int64_t N, int C,
                                                  const float* __restrict__ sp, const IO* __restrict__ x,
                                                  const float* __restrict__ b, const float* __restrict__ alpha,
                                                  float* __restrict__ hloc, double* __restrict__ ssum) {
  constexpr int CH = 64 / G;
  const int lane = threadIdx.x;
  const int grp = lane / CH, pl = lane % CH;
  const int64_t k = blockIdx.x;
  const int64_t p = static_cast<int64_t>(blockIdx.y) * CH + pl;
  const bool valid = p < P;
  const int64_t pc = valid ? p : P - 1;
  const int n0 = grp * NL;
  float al2[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) al2[j] = alpha[pc * N + n0 + j] * kLog2e;
  float h[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) h[j] = 0.0f;
  double ss = 0.0;
  const int64_t t0 = k * C;
  const int64_t t1 = (t0 + C < T) ? t0 + C : T;
  for (int64_t t = t0; t < t1; t++) {
    const float ns = -sp[t * P + pc];
    const float xv = load_io(x + t * P + pc);
    float bt[NL];
    load_row<NL>(b + t * N + n0, bt);
#pragma unroll
    for (int j = 0; j < NL; j++) {
      const float a = fast_exp2(ns * al2[j]);
      h[j] = fmaf(a, h[j], bt[j] * xv);
    }
    ss -= static_cast<double>(ns);
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < NL; j++) hloc[(k * P + p) * N + n0 + j] = h[j];
    if (grp == 0) ssum[k * P + p] = ss;
  }
}

// The carry as a segmented scan (seg_affine_scan): segments of kSegLen chunks,
// kFwdSegs wavefronts per workgroup, 64 (channel, state) pairs per wavefront,
// so the dependent chain is kSegLen + kFwdSegs steps per kSegLen kFwdSegs
// chunks instead of one per chunk.
constexpr int kFwdSegs = 16;

__global__ __launch_bounds__(64 * kFwdSegs) void k_fwd_carry(int64_t K, int64_t P, int64_t N,
                                                            const float* __restrict__ alpha,
                                                            const double* __restrict__ ssum,
                                                            const float* __restrict__ hloc,
                                                            float* __restrict__ h_ckpt) {
  __shared__ float sA[kFwdSegs][64], sB[kFwdSegs][64];
  const int64_t PN = P * N;
  const int lane = threadIdx.x & 63;
  const int sg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const bool live = e < PN;
  const int64_t ee = live ? e : PN - 1;  // clamped for reads
  const int64_t p = ee / N;
  const float al2 = alpha[ee] * kLog2e;
  auto load = [&](int64_t k, float* u, float* d) {
    *u = hloc[k * PN + ee];
    *d = fast_exp2(-static_cast<float>(ssum[k * P + p]) * al2);
  };
  auto store = [&](int64_t k, float x) {
    if (live) h_ckpt[k * PN + e] = x;
  };
  seg_affine_scan<kSegLen, kFwdSegs, false>(0, K, 0.0f, sA, sB, sg, lane, load, store);
}

template <typename IO, int NL, int G>
__global__ __launch_bounds__(64) void k_fwd_final(int64_t T, int64_t P, int64_t N, int C,
                                                  const float* __restrict__ sp, const IO* __restrict__ x,
                                                  const float* __restrict__ b, const float* __restrict__ c,
                                                  const float* __restrict__ alpha,
                                                  const float* __restrict__ h_ckpt, float* __restrict__ y,
                                                  float* __restrict__ hsub, float* __restrict__ hall) {
  constexpr int CH = 64 / G;
  const int lane = threadIdx.x;
  const int grp = lane / CH, pl = lane % CH;
  const int64_t k = blockIdx.x;
  const int64_t p = static_cast<int64_t>(blockIdx.y) * CH + pl;
  const bool valid = p < P;
  const int64_t pc = valid ? p : P - 1;
  const int n0 = grp * NL;
  float al2[NL], h[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) {
    al2[j] = alpha[pc * N + n0 + j] * kLog2e;
    h[j] = h_ckpt[(k * P + pc) * N + n0 + j];
  }
  const int64_t t0 = k * C;
  const int64_t t1 = (t0 + C < T) ? t0 + C : T;
  // sub-chunk start states for the gradient, when kept
  const int64_t NB = (P + CH - 1) / CH, nsub_max = (C + kSub - 1) / kSub;
  float* hsg = hsub ? hsub + hsub_offset(k, blockIdx.y, 0, NB, nsub_max, NL) + lane : nullptr;
  // every state, when kept (the store-everything baseline): h_t after token t
  float* hag = hall ? hall + hsub_offset(k, blockIdx.y, 0, NB, C, NL) + lane : nullptr;
  for (int64_t t = t0; t < t1; t++) {
    if (hsg && (t - t0) % kSub == 0) {
#pragma unroll
      for (int j = 0; j < NL; j++) hsg[((t - t0) / kSub * NL + j) * 64] = h[j];
    }
    const float ns = -sp[t * P + pc];
    const float xv = load_io(x + t * P + pc);
    float bt[NL], ct[NL];
    load_row<NL>(b + t * N + n0, bt);
    load_row<NL>(c + t * N + n0, ct);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NL; j++) {
      const float a = fast_exp2(ns * al2[j]);
      h[j] = fmaf(a, h[j], bt[j] * xv);
      acc = fmaf(ct[j], h[j], acc);
    }
    if (hag) {
#pragma unroll
      for (int j = 0; j < NL; j++) hag[((t - t0) * NL + j) * 64] = h[j];
    }
    acc = group_sum<G, CH>(acc);
    if (valid && grp == 0) y[t * P + p] = acc;
  }
}

// ---------------------------------------------------------- staged variants
// For N >= 4 and chunks whose rows fit in LDS: a 4-wavefront workgroup takes
// 4 channel blocks of one chunk.  The chunk's per-token rows (b, and c for
// the final pass), shared by all channels, are staged once into LDS by the
// whole workgroup; the per-lane s and x come through an 8-token register
// ring, so every load is issued 7 tokens before its use.
constexpr int kFwdWpb = 4;
constexpr int kFwdRing = 8;
constexpr size_t kFwdRowLds = 32 * 1024;  // LDS bytes for staged rows

template <int NQ>
__device__ __forceinline__ void stage_rows(float* rows, const float* __restrict__ const (&src)[NQ], int64_t t0,
                                          int len, int NN, int stride, int tid) {
  // rows[q][tau][n] = src[q][(t0 + tau) * NN + n], tau < len, with `stride`
  // tokens per row kind; float4 granularity
  const int per = len * NN / 4;
#pragma unroll
  for (int q = 0; q < NQ; q++) {
    const float4* s4 = reinterpret_cast<const float4*>(src[q] + t0 * NN);
    float4* d4 = reinterpret_cast<float4*>(rows + static_cast<size_t>(q) * stride * NN);
    for (int e = tid; e < per; e += 64 * kFwdWpb) d4[e] = s4[e];
  }
}

// The staged forward walk.  PARTS: the chunk's rows are staged in parts (the
// launcher picks this instantiation when a chunk's rows exceed the staging
// area); otherwise the whole chunk is staged at once.
template <typename IO, int NL, int G, bool FINAL, bool PARTS, bool KEEP = false>
__global__ __launch_bounds__(256) void k_fwd_staged(int64_t T, int64_t P, int64_t N, int C, int64_t NB,
                                                    const float* __restrict__ sp, const IO* __restrict__ x,
                                                    const float* __restrict__ b, const float* __restrict__ c,
                                                    const float* __restrict__ alpha,
                                                    const float* __restrict__ h_ckpt, float* __restrict__ y,
                                                    float* __restrict__ hloc, double* __restrict__ ssum,
                                                    float* __restrict__ hsub, float* __restrict__ hall) {
  constexpr int CH = 64 / G;
  constexpr int NN = NL * G;
  constexpr int D = kFwdRing;
  constexpr int NQ = FINAL ? 2 : 1;  // staged row kinds: b (, c)
  // The chunk's rows are staged in parts of TP tokens (the whole chunk when
  // its rows fit the staging area): [NQ][TP][NN].
  constexpr int TP = static_cast<int>(kFwdRowLds / (NQ * NN * 4)) / D * D;
  static_assert(TP >= D, "a ring turn of rows fits the staging area");
  extern __shared__ float rows[];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int grp = lane / CH, pl = lane % CH;
  // one workgroup per (chunk, channel group): chunk_group_grid
  uint32_t kc, kg;
  chunk_and_group(&kc, &kg);
  const int64_t k = kc;
  const int64_t cb = static_cast<int64_t>(kg) * kFwdWpb + w;
  const int64_t p = cb * CH + pl;
  const bool valid = cb < NB && p < P;
  const int64_t pc = p < P ? p : P - 1;
  const int n0 = grp * NL;
  const int64_t t0 = k * C;
  const int64_t t1 = (t0 + C < T) ? t0 + C : T;
  const int len = static_cast<int>(t1 - t0);
  const int tp = len < TP ? len : TP;  // tokens per staged part
  auto stage = [&](int lo, int n) {
    if constexpr (FINAL) {
      const float* __restrict__ srcs[2] = {b, c};
      stage_rows<2>(rows, srcs, t0 + lo, n, NN, tp, tid);
    } else {
      const float* __restrict__ srcs[1] = {b};
      stage_rows<1>(rows, srcs, t0 + lo, n, NN, tp, tid);
    }
  };
  stage(0, tp);
  float al2[NL], h[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) {
    al2[j] = alpha[pc * NN + n0 + j] * kLog2e;
    h[j] = FINAL ? h_ckpt[(k * P + pc) * NN + n0 + j] : 0.0f;
  }
  const uint32_t ob4 = static_cast<uint32_t>(pc) * 4u;
  const uint32_t obx = static_cast<uint32_t>(pc) * static_cast<uint32_t>(sizeof(IO));
  float rs[D];
  typename IoRaw<IO>::type rx[D];
  auto ld = [&](int slot, int64_t t) {
    rs[slot] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(sp + t * P) + ob4);
    rx[slot] = load_raw(reinterpret_cast<const IO*>(reinterpret_cast<const char*>(x + t * P) + obx));
  };
#pragma unroll
  for (int q = 0; q < D - 1; q++)
    if (q < len) ld(q, t0 + q);
  __syncthreads();  // staged rows visible
  // sub-chunk start states for the gradient, when kept (final pass only)
  const int64_t nsub_max = (C + kSub - 1) / kSub;
  // (KEEP: the final pass may store states; without it the pass stores y only)
  float* hsg = (FINAL && KEEP && hsub && cb < NB) ? hsub + hsub_offset(k, cb, 0, NB, nsub_max, NL) + lane : nullptr;
  // every state, when kept (the store-everything baseline): h_t after token t
  float* hag = (FINAL && KEEP && hall && cb < NB) ? hall + hsub_offset(k, cb, 0, NB, C, NL) + lane : nullptr;
  // y rows are stored through buffer resources: lanes that store nothing
  // carry an offset past the row, so the store needs no branch
  const int voff_y = (valid && grp == 0) ? static_cast<int>(ob4) : kBufOutside;
  static_assert(D % kSub == 0, "ring length a multiple of the sub-chunk");
  double ss = 0.0;
  int plo = 0;  // first token of the staged part
  {
    constexpr bool MULTI = PARTS;
    // One token of the walk; `ahead` is the token whose s and x the ring
    // fetches now (D - 1 tokens on).
    auto token = [&](int r, int tau, bool fetch, int64_t ahead) {
      // one token's work stays together (left alone, the scheduler hoists
      // later tokens' loads and exps and multiplies the live registers)
      if constexpr (FINAL && !KEEP) __builtin_amdgcn_sched_barrier(0);
      if (FINAL && KEEP && r % kSub == 0 && hsg) {
#pragma unroll
        for (int j = 0; j < NL; j++) hsg[(tau / kSub * NL + j) * 64] = h[j];
      }
      if (fetch) ld((r + D - 1) % D, ahead);
      const float ns = -rs[r];
      const float xv = raw_to_f32(rx[r]);
      const float* rb = rows + (MULTI ? tau - plo : tau) * NN + n0;
      float bt[NL];
#pragma unroll
      for (int j = 0; j < NL; j += 4) {
        const float4 v = *reinterpret_cast<const float4*>(rb + j);
        bt[j] = v.x; bt[j + 1] = v.y; bt[j + 2] = v.z; bt[j + 3] = v.w;
      }
      if constexpr (FINAL) {
        const float* rc = rows + static_cast<size_t>(tp) * NN + (MULTI ? tau - plo : tau) * NN + n0;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NL; j += 4) {
          const float4 cv = *reinterpret_cast<const float4*>(rc + j);
          const float cq[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            const float a = fast_exp2(ns * al2[j + jj]);
            h[j + jj] = fmaf(a, h[j + jj], bt[j + jj] * xv);
            acc = fmaf(cq[jj], h[j + jj], acc);
          }
        }
        if (KEEP && hag) {
#pragma unroll
          for (int j = 0; j < NL; j++) hag[(tau * NL + j) * 64] = h[j];
        }
        acc = group_sum<G, CH>(acc);
        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc(y + (t0 + tau) * P, 0, static_cast<int>(P * 4), kBufWord3);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc), ry, voff_y, 0, 0);
      } else {
#pragma unroll
        for (int j = 0; j < NL; j++) {
          const float a = fast_exp2(ns * al2[j]);
          h[j] = fmaf(a, h[j], bt[j] * xv);
        }
        ss -= static_cast<double>(ns);
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
    if ((!FINAL || !KEEP) && len % D == 0) {
      // whole ring turns: no per-token bounds branches (the fetches past the
      // chunk end re-read its last token), so the state stays in place rather
      // than being copied back at every token, and with no branch in the ring
      // turn the waits for its loads count them one by one.  (A final pass
      // that stores states keeps the checked loop.)
      for (int q8 = 0; q8 < len; q8 += D) {
        next_part(q8);
#pragma unroll
        for (int r = 0; r < D; r++) {
          const int tau = q8 + r;
          const int ahead = (tau + D - 1 < len) ? tau + D - 1 : len - 1;
          token(r, tau, true, t0 + ahead);
        }
      }
    } else {
      for (int q8 = 0; q8 < len; q8 += D) {
        next_part(q8);
#pragma unroll
        for (int r = 0; r < D; r++) {
          const int tau = q8 + r;
          if (tau < len) token(r, tau, tau + D - 1 < len, t0 + tau + D - 1);
        }
      }
    }
  }
  if constexpr (!FINAL) {
    if (valid) {
#pragma unroll
      for (int j = 0; j < NL; j++) hloc[(k * P + p) * NN + n0 + j] = h[j];
      if (grp == 0) ssum[k * P + p] = ss;
    }
  }
}

// ----------------------------------------------------------------- launchers

template <typename IO, int NL, int G>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  constexpr int CH = 64 / G;
  constexpr int NN = NL * G;
  const int64_t NB = (a.P + CH - 1) / CH;
  const int64_t K = (a.T + a.C - 1) / a.C;
  // staged kernels: rows of a chunk (b, c) in LDS, in parts of at most
  // kFwdRowLds bytes, 4 channel blocks per workgroup
  auto part_bytes = [&](int nq) {
    const size_t tp = kFwdRowLds / (nq * NN * 4) / kFwdRing * kFwdRing;
    return static_cast<size_t>(nq) * std::min<size_t>(a.C, tp) * NN * 4;
  };
  const size_t rows_local = part_bytes(1), rows_final = part_bytes(2);
  const bool staged = NN % 4 == 0;
  // rows staged in parts when a chunk's do not fit at once
  const bool parts_local = static_cast<size_t>(a.C) * NN * 4 > kFwdRowLds;
  const bool parts_final = static_cast<size_t>(2) * a.C * NN * 4 > kFwdRowLds;
  const dim3 grid(static_cast<unsigned>(K), static_cast<unsigned>(NB));
  const dim3 grid_s = chunk_group_grid(K, (NB + kFwdWpb - 1) / kFwdWpb);
  hipError_t e;
  if (staged) {
    auto kl = parts_local ? k_fwd_staged<IO, NL, G, false, true> : k_fwd_staged<IO, NL, G, false, false>;
    kl<<<grid_s, 64 * kFwdWpb, rows_local, st>>>(a.T, a.P, a.N, a.C, NB, a.s, static_cast<const IO*>(a.x), a.b, a.c,
                                                 a.alpha, a.h_ckpt, a.y, a.hloc, a.ssum, nullptr, nullptr);
  } else {
    k_fwd_local<IO, NL, G><<<grid, 64, 0, st>>>(a.T, a.P, a.N, a.C, a.s, static_cast<const IO*>(a.x), a.b,
                                                a.alpha, a.hloc, a.ssum);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  a.marks.rec(2, st);
  const int64_t PN = a.P * a.N;
  k_fwd_carry<<<static_cast<unsigned>((PN + 63) / 64), 64 * kFwdSegs, 0, st>>>(K, a.P, a.N, a.alpha, a.ssum,
                                                                              a.hloc, a.h_ckpt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  a.marks.rec(3, st);
  if (staged) {
    // states kept by the forward: the variant that stores them
    const bool keep = a.hsub || a.hall;
    auto kf = parts_final ? (keep ? k_fwd_staged<IO, NL, G, true, true, true> : k_fwd_staged<IO, NL, G, true, true>)
                          : (keep ? k_fwd_staged<IO, NL, G, true, false, true> : k_fwd_staged<IO, NL, G, true, false>);
    kf<<<grid_s, 64 * kFwdWpb, rows_final, st>>>(a.T, a.P, a.N, a.C, NB, a.s, static_cast<const IO*>(a.x), a.b, a.c,
                                                 a.alpha, a.h_ckpt, a.y, a.hloc, a.ssum, a.hsub, a.hall);
  } else {
    k_fwd_final<IO, NL, G><<<grid, 64, 0, st>>>(a.T, a.P, a.N, a.C, a.s, static_cast<const IO*>(a.x), a.b, a.c,
                                                a.alpha, a.h_ckpt, a.y, a.hsub, a.hall);
  }
  e = hipGetLastError();
  a.marks.rec(4, st);
  return e;
}

template <typename IO>
static hipError_t launch_fwd_io(const FwdArgs& a, hipStream_t st) {
  switch (a.N) {
    case 1: return launch_fwd_t<IO, 1, 1>(a, st);
    case 2: return launch_fwd_t<IO, 2, 1>(a, st);
    case 4: return launch_fwd_t<IO, 4, 1>(a, st);
    case 8: return launch_fwd_t<IO, 8, 1>(a, st);
    case 16: return launch_fwd_t<IO, 8, 2>(a, st);
    case 32: return launch_fwd_t<IO, 8, 4>(a, st);
    case 64: return launch_fwd_t<IO, 8, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_forward_scan(const FwdArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_fwd_io<bf16_t>(a, st) : launch_fwd_io<float>(a, st);
}

}  // namespace ssm
