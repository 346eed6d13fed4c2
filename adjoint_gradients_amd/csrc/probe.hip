// probe.hip -- issue-rate probes of single gfx950 units (declared in ssm_probe.h).
//
// The scans of this library are priced against the fp32 VALU issue rate,
// counting a hardware exp2 as two issue slots; the GEMMs against the dense
// bf16 MFMA rate.  These kernels measure those rates directly: each lane (or
// wavefront, for MFMA) runs independent dependency chains of one kind of
// instruction, enough of them that the unit's throughput, not an
// instruction's latency, bounds the loop.  The shader clock and the constant
// wall clock are read at the loop's start and end of every wavefront, so the
// caller can relate the rate to the clock the chip actually ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssm_adjoint.h"
#include "../../include/ssm_probe.h"
#include "ssm_common.hpp"

namespace ssm {
namespace {

constexpr int kChains = 8;      // independent chains a lane (VALU probes)
constexpr int kMfmaChains = 4;  // independent accumulators a wavefront (MFMA probe)

__device__ __forceinline__ void record_clocks(uint64_t* clk, int64_t wave, uint64_t c0, uint64_t c1, uint64_t w0,
                                              uint64_t w1) {
  clk[wave * 4 + 0] = c0;
  clk[wave * 4 + 1] = c1;
  clk[wave * 4 + 2] = w0;
  clk[wave * 4 + 3] = w1;
}

// FMA: x <- x a + b (a < 1, so x stays near b / (1 - a)).  EXP: x <- 2^-x
// (x stays in (0, 1]).  EXP_FMA: one of each a chain and iteration.
template <int KIND>
__global__ __launch_bounds__(256) void k_probe_valu(int64_t iters, float* __restrict__ sink,
                                                    uint64_t* __restrict__ clk) {
  const int lane = threadIdx.x & 63;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  float x[kChains], y[kChains];
#pragma unroll
  for (int i = 0; i < kChains; i++) {
    x[i] = 0.5f + 0.001f * static_cast<float>(lane + i);
    y[i] = x[i];
  }
  const float a = 0.9990234375f, b = 0.0009765625f;
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t c0 = clock64(), w0 = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);
  for (int64_t it = 0; it < iters; it++) {
#pragma unroll
    for (int i = 0; i < kChains; i++) {
      if constexpr (KIND == SSM_PROBE_FMA) {
        x[i] = fmaf(x[i], a, b);
      } else if constexpr (KIND == SSM_PROBE_EXP) {
        x[i] = __builtin_amdgcn_exp2f(-x[i]);
      } else {
        x[i] = __builtin_amdgcn_exp2f(-x[i]);
        y[i] = fmaf(y[i], a, b);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t c1 = clock64(), w1 = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChains; i++) s += (KIND == SSM_PROBE_EXP_FMA) ? x[i] + y[i] : x[i];
  sink[gid] = s;
  if (lane == 0) record_clocks(clk, gid >> 6, c0, c1, w0, w1);
}

// kMfmaChains accumulators, each acc <- A B + acc with the same operands
// (A and B hold 2^-6 and 2^-5: an accumulator grows by 2^-7 a step).
__global__ __launch_bounds__(256) void k_probe_mfma(int64_t iters, float* __restrict__ sink,
                                                    uint64_t* __restrict__ clk) {
  const int lane = threadIdx.x & 63;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  bf16x8_t av, bv;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    av[e] = static_cast<__bf16>(0.015625f);
    bv[e] = static_cast<__bf16>(0.03125f);
  }
  f32x16_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; c++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[c][r] = 0.0f;
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t c0 = clock64(), w0 = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);
  for (int64_t it = 0; it < iters; it++) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[c], 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t c1 = clock64(), w1 = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; c++)
#pragma unroll
    for (int r = 0; r < 16; r++) s += acc[c][r];
  sink[gid] = s;
  if (lane == 0) record_clocks(clk, gid >> 6, c0, c1, w0, w1);
}

}  // namespace
}  // namespace ssm

extern "C" int ssm_probe_units(int kind, int64_t wgs, int64_t iters, float* sink, uint64_t* clk, void* stream) {
  if (kind < SSM_PROBE_FMA || kind > SSM_PROBE_MFMA) return SSM_ERR_ARG;
  if (wgs < 1 || wgs > (int64_t(1) << 20) || iters < 1 || iters >= (int64_t(1) << 31)) return SSM_ERR_ARG;
  if (!sink || !clk) return SSM_ERR_ARG;
  static_assert(SSM_PROBE_WAVES_PER_WG * 64 == 256, "workgroups of 256 lanes");
  const dim3 grid(static_cast<unsigned>(wgs));
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (kind) {
    case SSM_PROBE_FMA:
      ssm::k_probe_valu<SSM_PROBE_FMA><<<grid, 256, 0, st>>>(iters, sink, clk);
      break;
    case SSM_PROBE_EXP:
      ssm::k_probe_valu<SSM_PROBE_EXP><<<grid, 256, 0, st>>>(iters, sink, clk);
      break;
    case SSM_PROBE_EXP_FMA:
      ssm::k_probe_valu<SSM_PROBE_EXP_FMA><<<grid, 256, 0, st>>>(iters, sink, clk);
      break;
    default:
      ssm::k_probe_mfma<<<grid, 256, 0, st>>>(iters, sink, clk);
      break;
  }
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" int ssm_probe_wall_clock_khz(int* khz) {
  if (!khz) return SSM_ERR_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SSM_ERR_HIP;
  return hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}
