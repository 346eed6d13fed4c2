/* ssm_probe.h -- issue-rate probes of single gfx950 units.
 *
 * Not part of the gradient path.  These calls measure the rates the
 * library's kernels are priced against: the fp32 VALU rate (one FMA a lane),
 * the rate of v_exp_f32 on the transcendental unit, the two interleaved, and
 * the dense bf16 MFMA rate (v_mfma_f32_32x32x16_bf16).  Each probe kernel
 * also reads the shader clock and the constant wall clock at its start and
 * end, so the caller can tell the effective clock the chip ran that load at
 * (it falls below 2.4 GHz when the chip is held by its power limit).
 *
 * Status codes are those of ssm_adjoint.h.
 */
#ifndef SSM_PROBE_H
#define SSM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_PROBE_FMA = 0,      /* 8 independent fp32 FMA chains a lane (v_fma_f32, packed forms off) */
  SSM_PROBE_EXP = 1,      /* 8 independent chains x <- 2^-x a lane (v_exp_f32) */
  SSM_PROBE_EXP_FMA = 2,  /* both of the above in the same loop, one exp per FMA */
  SSM_PROBE_MFMA = 3      /* 4 independent bf16 MFMA 32x32x16 accumulators a wavefront */
} ssm_probe_kind;

/* Wavefronts per workgroup of every probe (workgroups of 256 lanes). */
#define SSM_PROBE_WAVES_PER_WG 4

/* Launches one probe: `wgs` workgroups of 256 lanes, each lane running
 * `iters` iterations of its kind's loop.  Asynchronous on `stream` (a
 * hipStream_t; null = the default stream); the caller times it.
 *   sink: device, wgs * 256 floats -- per lane the sum of its chains, stored
 *         so the loop cannot be optimised away (values are meaningless);
 *   clk:  device, wgs * SSM_PROBE_WAVES_PER_WG * 4 uint64 -- per wavefront
 *         the shader clock at the loop's start and end, then the wall clock
 *         at its start and end (rate: ssm_probe_wall_clock_khz).
 * Both buffers belong to the caller.  Returns SSM_OK, SSM_ERR_ARG (unknown
 * kind, wgs outside [1, 2^20], iters outside [1, 2^31), a null buffer) or
 * SSM_ERR_HIP (the launch failed). */
int ssm_probe_units(int kind, int64_t wgs, int64_t iters, float* sink, uint64_t* clk, void* stream);

/* The wall clock's rate in kHz (hipDeviceAttributeWallClockRate of the
 * current device) into *khz.  Returns SSM_OK, SSM_ERR_ARG (null khz) or
 * SSM_ERR_HIP. */
int ssm_probe_wall_clock_khz(int* khz);

#ifdef __cplusplus
}
#endif

#endif /* SSM_PROBE_H */
