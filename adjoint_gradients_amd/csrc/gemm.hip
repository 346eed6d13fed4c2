// gemm.hip -- MFMA GEMMs for the dense contractions of the layer (gfx950).
//
//   projections      [Delta | b | c]_t = W_cat x_t            (C = X W_cat^T)
//   weight gradient  dW_cat = sum_t [dDelta | db | dc]_t x_t^T (the time sum of
//                    Proposition 2's per-token VJPs through the linear maps,
//                    review of "Adjoint sharding for very long context
//                    training of state space models", Core claim)
//   input cotangent  dx_t = W_cat^T [dDelta | db | dc]_t + dxdir_t
//
// One kernel template: 128x128 output tile per 256-thread workgroup (2x2
// wavefronts of 64x64, each 2x2 tiles of v_mfma_f32_32x32x16_bf16 or
// v_mfma_f32_32x32x2f32), K staged through LDS in steps of 32.  Operands whose
// reduction index is not contiguous in memory are transposed while being
// written to LDS, so the MFMA operand fetch is always a contiguous read.
// Lane layouts (verified on gfx950): A operand lane l holds row l%32 and
// k = (l/32)*8 .. +7 (bf16) or k = l/32 (f32); B likewise with column l%32;
// the 32x32 result holds column l%32, rows (r/4)*8 + (l/32)*4 + r%4 in
// register r.
#include "ssm_common.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

namespace {

constexpr int BM = 128, BN = 128, BK = 32;

template <typename TI> struct Tr;
template <> struct Tr<bf16_t> {
  static constexpr int VEC = 8;   // elements per 16-byte chunk
  static constexpr int PAD = 8;   // LDS row padding (elements)
};
template <> struct Tr<float> {
  static constexpr int VEC = 4;
  static constexpr int PAD = 1;
};

// Epilogues: operator() for the small-tile kernel; prep(col) + apply() for the
// large-tile kernel (the column-dependent choice is made once per column, so
// the unrolled per-element code has no branches).
struct EpiProj {
  // its last tile column holds the 2N projection columns past the P of Delta:
  // the direct-to-LDS kernel skips the blocks past them
  static constexpr bool kSkipTail = true;
  // eight wavefronts per workgroup in the direct-to-LDS kernel (measured at
  // 1M x 2080 x 2048: 10.65 -> 10.20 ms)
  static constexpr int kWaveCols = 4;
  EpiProjArgs e;
  __device__ __forceinline__ void operator()(int64_t row, int64_t col, float v, int) const {
    if (col < e.P) {
      e.s[row * e.P + col] = softplus_f(v + (e.bias ? e.bias[col] : 0.0f));
    } else if (col < e.P + e.N) {
      e.b[row * e.N + (col - e.P)] = v;
    } else {
      e.c[row * e.N + (col - e.P - e.N)] = v;
    }
  }
  struct Prep {
    float* base;
    int64_t ld;
    float bias;
    bool sp;
  };
  __device__ __forceinline__ Prep prep(int64_t col, int) const {
    Prep q;
    if (col < e.P) {
      q.base = e.s + col; q.ld = e.P; q.bias = e.bias ? e.bias[col] : 0.0f; q.sp = true;
    } else if (col < e.P + e.N) {
      q.base = e.b + (col - e.P); q.ld = e.N; q.bias = 0.0f; q.sp = false;
    } else {
      q.base = e.c + (col - e.P - e.N); q.ld = e.N; q.bias = 0.0f; q.sp = false;
    }
    return q;
  }
  __device__ __forceinline__ void apply(const Prep& q, int64_t row, float v) const { at(q, row * q.ld, v); }
  // element at row offset `off` (= row * q.ld) of the prepared column
  __device__ __forceinline__ void at(const Prep& q, int64_t off, float v) const {
    const float w = v + q.bias;
    const float sp = softplus_f(w);
    q.base[off] = q.sp ? sp : w;
  }
};

struct EpiPart {
  float* part;
  int64_t M, Nc;
  __device__ __forceinline__ void operator()(int64_t row, int64_t col, float v, int z) const {
    part[(static_cast<int64_t>(z) * M + row) * Nc + col] = v;
  }
  struct Prep {
    float* base;
    int64_t ld;
  };
  __device__ __forceinline__ Prep prep(int64_t col, int z) const {
    return Prep{part + static_cast<int64_t>(z) * M * Nc + col, Nc};
  }
  __device__ __forceinline__ void apply(const Prep& q, int64_t row, float v) const { q.base[row * Nc] = v; }
  __device__ __forceinline__ void at(const Prep& q, int64_t off, float v) const { q.base[off] = v; }
};

struct EpiAdd {
  static constexpr int kWaveCols = 4;
  EpiAddArgs e;
  int64_t Nc;
  __device__ __forceinline__ void operator()(int64_t row, int64_t col, float v, int) const {
    const int64_t idx = row * Nc + col;
    float r = v + e.add0[idx];
    if (e.add1) r += e.add1[idx];
    e.out[idx] = r;
  }
  struct Prep {
    int64_t col;
    int64_t ld;
  };
  __device__ __forceinline__ Prep prep(int64_t col, int) const { return Prep{col, Nc}; }
  __device__ __forceinline__ void apply(const Prep& q, int64_t row, float v) const { at(q, row * Nc, v); }
  __device__ __forceinline__ void at(const Prep& q, int64_t off, float v) const {
    const int64_t idx = off + q.col;
    float r = v + e.add0[idx];
    if (e.add1) r += e.add1[idx];
    e.out[idx] = r;
  }
  // NV outputs at element offsets off[]: every addend is loaded before any
  // result is stored.  out may be add1 (an in-place update), so the compiler
  // cannot move a later element's loads above an earlier element's store by
  // itself; element by element, each would wait a full memory round trip.
  template <int NV>
  __device__ __forceinline__ void at_batch(const Prep& q, const int64_t (&off)[NV], const float (&v)[NV]) const {
    // same rounding as at(): (v + add0) + add1
    float r[NV];
#pragma unroll
    for (int k = 0; k < NV; k++) r[k] = v[k] + e.add0[off[k] + q.col];
    if (e.add1) {
      float a1[NV];
#pragma unroll
      for (int k = 0; k < NV; k++) a1[k] = e.add1[off[k] + q.col];
#pragma unroll
      for (int k = 0; k < NV; k++) r[k] += a1[k];
    }
#pragma unroll
    for (int k = 0; k < NV; k++) e.out[off[k] + q.col] = r[k];
  }
};

// Stage a BR x BK tile of operand X (rows r0.., k0..) into LDS as [BR][BK+PAD].
// kc: X(r,k) = X[r*ld + k]; otherwise X(r,k) = X[k*ld + r].
template <typename TI, int BR>
__device__ __forceinline__ void stage(TI* __restrict__ lds, const TI* __restrict__ X, int64_t ld, bool kc,
                                      int64_t R, int64_t Kend, int64_t r0, int64_t k0, int tid) {
  constexpr int VEC = Tr<TI>::VEC;
  constexpr int LDR = BK + Tr<TI>::PAD;
  if (kc) {
    constexpr int CPR = BK / VEC;          // chunks per row
    constexpr int NCH = BR * CPR;
    const bool vec_ok = (ld % VEC) == 0;
    for (int c = tid; c < NCH; c += 256) {
      const int r = c / CPR, kk = (c % CPR) * VEC;
      const int64_t gr = r0 + r, gk = k0 + kk;
      alignas(16) TI vals[VEC];
      if (gr < R && gk + VEC <= Kend && vec_ok) {
        const uint4 v = *reinterpret_cast<const uint4*>(X + gr * ld + gk);
        *reinterpret_cast<uint4*>(vals) = v;
      } else {
#pragma unroll
        for (int e = 0; e < VEC; e++) vals[e] = (gr < R && gk + e < Kend) ? X[gr * ld + gk + e] : TI(0);
      }
      if constexpr ((LDR * sizeof(TI)) % 16 == 0) {
        *reinterpret_cast<uint4*>(lds + r * LDR + kk) = *reinterpret_cast<uint4*>(vals);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; e++) lds[r * LDR + kk + e] = vals[e];
      }
    }
  } else {
    constexpr int CPK = BR / VEC;          // chunks per k-row
    constexpr int NCH = BK * CPK;
    const bool vec_ok = (ld % VEC) == 0;
    for (int c = tid; c < NCH; c += 256) {
      const int kk = c / CPK, r = (c % CPK) * VEC;
      const int64_t gk = k0 + kk, gr = r0 + r;
      alignas(16) TI vals[VEC];
      if (gk < Kend && gr + VEC <= R && vec_ok) {
        const uint4 v = *reinterpret_cast<const uint4*>(X + gk * ld + gr);
        *reinterpret_cast<uint4*>(vals) = v;
      } else {
#pragma unroll
        for (int e = 0; e < VEC; e++) vals[e] = (gk < Kend && gr + e < R) ? X[gk * ld + gr + e] : TI(0);
      }
#pragma unroll
      for (int e = 0; e < VEC; e++) lds[(r + e) * LDR + kk] = vals[e];
    }
  }
}

template <typename TI, class Epi>
__global__ __launch_bounds__(256) void k_gemm(int64_t M, int64_t Nc, int64_t K, const TI* __restrict__ A,
                                              int64_t lda, bool a_kc, const TI* __restrict__ B, int64_t ldb,
                                              bool b_kc, int64_t k_per_split, Epi epi) {
  constexpr int LDR = BK + Tr<TI>::PAD;
  __shared__ __attribute__((aligned(16))) TI As[BM * LDR];
  __shared__ __attribute__((aligned(16))) TI Bs[BN * LDR];
  const int tid = threadIdx.x;
  const int wave = tid / 64, l = tid % 64;
  const int wm = wave / 2, wn = wave % 2;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int z = blockIdx.z;
  const int64_t kbeg = static_cast<int64_t>(z) * k_per_split;
  const int64_t kend = (kbeg + k_per_split < K) ? kbeg + k_per_split : K;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    stage<TI, BM>(As, A, lda, a_kc, M, kend, m0, k0, tid);
    stage<TI, BN>(Bs, B, ldb, b_kc, Nc, kend, n0, k0, tid);
    __syncthreads();
    if constexpr (sizeof(TI) == 2) {
#pragma unroll
      for (int kk = 0; kk < BK; kk += 16) {
        bf16x8_t af[2], bfv[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
          const TI* pa = As + (wm * 64 + i * 32 + l % 32) * LDR + kk + (l / 32) * 8;
          af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(pa));
          const TI* pb = Bs + (wn * 64 + i * 32 + l % 32) * LDR + kk + (l / 32) * 8;
          bfv[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(pb));
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
          for (int j = 0; j < 2; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < BK; kk += 2) {
        float af[2], bfv[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
          af[i] = As[(wm * 64 + i * 32 + l % 32) * LDR + kk + l / 32];
          bfv[i] = Bs[(wn * 64 + i * 32 + l % 32) * LDR + kk + l / 32];
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
          for (int j = 0; j < 2; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bfv[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t row = m0 + wm * 64 + i * 32 + (r / 4) * 8 + (l / 32) * 4 + (r % 4);
        const int64_t col = n0 + wn * 64 + j * 32 + l % 32;
        if (row < M && col < Nc) epi(row, col, acc[i][j][r], z);
      }
}

template <typename TI, class Epi>
hipError_t run(const GemmOperands& op, int splits, int64_t kps, Epi epi, hipStream_t st) {
  dim3 grid(static_cast<unsigned>((op.Nc + BN - 1) / BN), static_cast<unsigned>((op.M + BM - 1) / BM),
            static_cast<unsigned>(splits));
  k_gemm<TI, Epi><<<grid, 256, 0, st>>>(op.M, op.Nc, op.K, static_cast<const TI*>(op.A), op.lda, op.a_kc,
                                       static_cast<const TI*>(op.B), op.ldb, op.b_kc, kps, epi);
  return hipGetLastError();
}

}  // namespace

#include "gemm_bf16.inl"
#include "gemm_dl.inl"

namespace {

__global__ __launch_bounds__(256) void k_reduce_wgrad(const float* __restrict__ part, int splits, int64_t P,
                                                      int64_t N, float* __restrict__ dWd, float* __restrict__ dWb,
                                                      float* __restrict__ dWc) {
  const int64_t M = P + 2 * N;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= M * P) return;
  float v = 0.0f;
  for (int z = 0; z < splits; z++) v += part[static_cast<int64_t>(z) * M * P + e];
  const int64_t row = e / P, col = e % P;
  if (row < P) dWd[row * P + col] = v;
  else if (row < P + N) dWb[(row - P) * P + col] = v;
  else dWc[(row - P - N) * P + col] = v;
}

__global__ __launch_bounds__(256) void k_residual_update(int64_t n, float* r, const float* __restrict__ y,
                                                         void* __restrict__ xio, int bf16, float* rout) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float v = r[e];
  if (y) {
    v += y[e];
    rout[e] = v;
  }
  if (!xio) return;
  if (bf16) static_cast<bf16_t*>(xio)[e] = f32_to_bf16(v);
  else static_cast<float*>(xio)[e] = v;
}

__global__ __launch_bounds__(256) void k_residual_init(int64_t n, const void* __restrict__ x0, int bf16,
                                                       float* __restrict__ r) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= n) return;
  r[e] = bf16 ? bf16_to_f32(static_cast<const bf16_t*>(x0)[e]) : static_cast<const float*>(x0)[e];
}

}  // namespace

// bf16 GEMMs take the direct-to-LDS kernel where its shape conditions hold,
// the register-staged one otherwise.
template <class Epi>
static hipError_t run_bf16(const GemmOperands& op, int splits, int64_t kps, Epi epi, hipStream_t st) {
  if (gdl::supports(op, kps)) return gdl::run(op, splits, kps, epi, st);
  return gbf::run(op, splits, kps, epi, st);
}

hipError_t gemm_projection(const GemmOperands& op, bool bf16, const EpiProjArgs& e, hipStream_t st) {
  EpiProj epi{e};
  return bf16 ? run_bf16(op, 1, op.K, epi, st) : run<float>(op, 1, op.K, epi, st);
}

hipError_t gemm_splitk(const GemmOperands& op, bool bf16, int splits, float* part, hipStream_t st) {
  int64_t kps = (op.K + splits - 1) / splits;
  kps = ((kps + BK - 1) / BK) * BK;
  EpiPart epi{part, op.M, op.Nc};
  if (bf16) {
    int64_t kpb = (op.K + splits - 1) / splits;
    kpb = ((kpb + gbf::BK - 1) / gbf::BK) * gbf::BK;
    return run_bf16(op, splits, kpb, epi, st);
  }
  return run<float>(op, splits, kps, epi, st);
}

hipError_t gemm_add(const GemmOperands& op, bool bf16, const EpiAddArgs& e, hipStream_t st) {
  EpiAdd epi{e, op.Nc};
  return bf16 ? run_bf16(op, 1, op.K, epi, st) : run<float>(op, 1, op.K, epi, st);
}

hipError_t reduce_weight_grads(const float* part, int splits, int64_t P, int64_t N, float* dWd, float* dWb,
                               float* dWc, hipStream_t st) {
  const int64_t tot = (P + 2 * N) * P;
  k_reduce_wgrad<<<static_cast<unsigned>((tot + 255) / 256), 256, 0, st>>>(part, splits, P, N, dWd, dWb, dWc);
  return hipGetLastError();
}

hipError_t residual_update(int64_t n, float* r, const float* y, void* xio, bool bf16, hipStream_t st, float* rout) {
  k_residual_update<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(n, r, y, xio, bf16 ? 1 : 0,
                                                                             rout ? rout : r);
  return hipGetLastError();
}

hipError_t residual_init(int64_t n, const void* x0, bool bf16, float* r, hipStream_t st) {
  k_residual_init<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(n, x0, bf16 ? 1 : 0, r);
  return hipGetLastError();
}

}  // namespace ssm
