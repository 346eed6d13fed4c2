// norm.hip -- RMS normalisation of the residual stream before each layer of
// the stack, and its vector-Jacobian product.
//
// The review of "Adjoint sharding for very long context training of state
// space models" (Algorithm 1, the memory analysis) has every layer read a
// normalised input x-hat without defining the norm; the reading taken is RMS
// normalisation with a per-channel scale gamma:
//   rinv_t = 1 / sqrt(mean_p r[t][p]^2 + eps),  x[t][p] = io(gamma[p] r[t][p] rinv_t).
// Its VJP for the cotangent d of x (the io cast taken as the identity), with
// xh = r rinv and u = gamma d:
//   dr[t][p] = rinv_t (u[p] - xh[p] m_t),  m_t = mean_q(u[q] xh[q]),
//   dgamma[p] = sum_t d[t][p] xh[t][p].
// Row reductions run one wavefront per token; the update of the cotangent
// stream and dgamma run on column tiles (coalesced), with per-row-block
// partial sums of dgamma reduced in a fixed order: deterministic.
#include "ssm_common.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

namespace {

constexpr int kNormRowsPerWg = 4;   // one wavefront per row
constexpr int kNormTileRows = 256;  // rows per column tile of the VJP

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__global__ __launch_bounds__(64 * kNormRowsPerWg) void k_rmsnorm_fwd(int64_t T, int64_t P,
                                                                    const float* __restrict__ r,
                                                                    const float* __restrict__ gamma, float eps,
                                                                    void* __restrict__ xio, int bf16,
                                                                    float* __restrict__ rinv,
                                                                    float* __restrict__ rcopy) {
  const int lane = threadIdx.x % 64;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kNormRowsPerWg + threadIdx.x / 64;
  if (t >= T) return;  // whole wavefronts only: T rows, one each
  const float* row = r + t * P;
  float ss = 0.0f;
  for (int64_t p = lane; p < P; p += 64) ss = fmaf(row[p], row[p], ss);
  ss = wave_sum(ss);
  const float ri = 1.0f / sqrtf(ss / static_cast<float>(P) + eps);
  if (lane == 0) rinv[t] = ri;
  for (int64_t p = lane; p < P; p += 64) {
    const float v = row[p];
    const float o = gamma[p] * (v * ri);
    if (bf16) static_cast<bf16_t*>(xio)[t * P + p] = f32_to_bf16(o);
    else static_cast<float*>(xio)[t * P + p] = o;
    rcopy[t * P + p] = v;
  }
}

// m_t = mean_p(gamma d xh) per row
__global__ __launch_bounds__(64 * kNormRowsPerWg) void k_rmsnorm_dot(int64_t T, int64_t P,
                                                                    const float* __restrict__ r,
                                                                    const float* __restrict__ rinv,
                                                                    const float* __restrict__ gamma,
                                                                    const float* __restrict__ d,
                                                                    float* __restrict__ m) {
  const int lane = threadIdx.x % 64;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kNormRowsPerWg + threadIdx.x / 64;
  if (t >= T) return;
  const float ri = rinv[t];
  float acc = 0.0f;
  for (int64_t p = lane; p < P; p += 64) acc = fmaf(gamma[p] * d[t * P + p], r[t * P + p] * ri, acc);
  acc = wave_sum(acc);
  if (lane == 0) m[t] = acc / static_cast<float>(P);
}

// delta[t][p] += rinv_t (gamma[p] d[t][p] - xh[t][p] m_t) on a column tile;
// part[rb][p] = sum over the tile's rows of d xh
__global__ __launch_bounds__(256) void k_rmsnorm_vjp(int64_t T, int64_t P, const float* __restrict__ r,
                                                    const float* __restrict__ rinv,
                                                    const float* __restrict__ gamma,
                                                    const float* __restrict__ d, const float* __restrict__ m,
                                                    float* __restrict__ delta, float* __restrict__ part) {
  // blockIdx.x: row block (up to 2^23 of them), blockIdx.y: column tile
  const int64_t p = static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x;
  if (p >= P) return;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kNormTileRows;
  const int64_t t1 = (t0 + kNormTileRows < T) ? t0 + kNormTileRows : T;
  const float gp = gamma[p];
  float dg = 0.0f;
  for (int64_t t = t0; t < t1; t++) {
    const float ri = rinv[t];
    const float xh = r[t * P + p] * ri;
    const float dv = d[t * P + p];
    delta[t * P + p] += ri * (gp * dv - xh * m[t]);
    dg = fmaf(dv, xh, dg);
  }
  part[static_cast<int64_t>(blockIdx.x) * P + p] = dg;
}

__global__ __launch_bounds__(256) void k_reduce_rows(int64_t nb, int64_t P, const float* __restrict__ part,
                                                    float* __restrict__ out) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (p >= P) return;
  float s = 0.0f;
  for (int64_t b = 0; b < nb; b++) s += part[b * P + p];
  out[p] = s;
}

}  // namespace

int64_t norm_row_blocks(int64_t T) { return (T + kNormTileRows - 1) / kNormTileRows; }

hipError_t rmsnorm_forward(int64_t T, int64_t P, const float* r, const float* gamma, float eps, void* xio,
                           bool bf16, float* rinv, float* rcopy, hipStream_t st) {
  const unsigned blocks = static_cast<unsigned>((T + kNormRowsPerWg - 1) / kNormRowsPerWg);
  k_rmsnorm_fwd<<<blocks, 64 * kNormRowsPerWg, 0, st>>>(T, P, r, gamma, eps, xio, bf16 ? 1 : 0, rinv, rcopy);
  return hipGetLastError();
}

hipError_t rmsnorm_vjp(int64_t T, int64_t P, const float* r, const float* rinv, const float* gamma, const float* d,
                       float* m, float* delta, float* part, float* dgamma, hipStream_t st) {
  const unsigned rb = static_cast<unsigned>((T + kNormRowsPerWg - 1) / kNormRowsPerWg);
  k_rmsnorm_dot<<<rb, 64 * kNormRowsPerWg, 0, st>>>(T, P, r, rinv, gamma, d, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nb = norm_row_blocks(T);
  const dim3 grid(static_cast<unsigned>(nb), static_cast<unsigned>((P + 255) / 256));
  k_rmsnorm_vjp<<<grid, 256, 0, st>>>(T, P, r, rinv, gamma, d, m, delta, part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (dgamma) {
    k_reduce_rows<<<static_cast<unsigned>((P + 255) / 256), 256, 0, st>>>(nb, P, part, dgamma);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace ssm
