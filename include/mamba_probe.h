/*
 * Measurement probes of libmambascan.so (gfx950).
 *
 * Not part of the selective scan: these kernels measure the ceilings the scan's kernels are
 * compared with -- the HBM bandwidth a plain device copy reaches, and the rates at which
 * the chip issues the VALU forms the scan's state update is made of (one v_exp_f32 and four
 * fp32 multiply/FMA per state element, "Understanding Mamba" sections 4.4 and 7: the fused
 * discretisation Abar = exp(Delta A), Bbar u = Delta B u and the recurrence).  The pages
 * measure their kernels the same way, by the share of the hardware's bandwidth and compute
 * a kernel attains ("State space models and the Mamba series" section 4.2).
 *
 * Conventions as in mamba_scan.h: device pointers, caller-owned buffers, asynchronous on
 * `stream` (a hipStream_t; NULL = null stream), argument checks on the host before any
 * launch.  Time the calls with events on the same stream.
 */
#ifndef MAMBA_PROBE_H
#define MAMBA_PROBE_H

#include "mamba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copies `bytes` (a multiple of 16) from src to dst with `blocks` workgroups of 256 threads,
 * 16 bytes per thread per iteration (grid-stride).  src and dst 16-byte aligned
 * (MAMBA_ERR_MISALIGNED), not overlapping (MAMBA_ERR_ALIASING).  Moves 2 x bytes through
 * HBM. */
MAMBA_API mamba_status_t mamba_probe_copy(const void *src, void *dst, size_t bytes,
                                          int32_t blocks, void *stream);

/* Instruction forms of mamba_probe_issue. */
#define MAMBA_PROBE_FMA_VGPR 0 /* v_fmac_f32, all operands in vector registers          */
#define MAMBA_PROBE_FMA_SGPR 1 /* v_fmac_f32 with a scalar-register operand            */
#define MAMBA_PROBE_EXP 2      /* v_exp_f32                                             */
#define MAMBA_PROBE_UPDATE 3   /* the scan's state update: FMA, v_exp_f32, multiply by
                                  a scalar B, FMA (recurrence), FMA by a scalar C        */
#define MAMBA_PROBE_FMA_DPP 4  /* v_fmac_f32 whose first operand is a DPP row broadcast
                                  (row_newbcast) of a vector register                     */
#define MAMBA_PROBE_UPDATE_DPP 5 /* the state update with B and C one value per lane of
                                  a vector register, taken by DPP row broadcasts folded
                                  into the multiply and the readout FMA                  */

/* Runs compute_units x waves_per_simd workgroups of 256 threads (one wave per SIMD each),
 * every lane issuing `iters` iterations of 8 independent instructions of the given form
 * (MAMBA_PROBE_UPDATE, _UPDATE_DPP: 8 steps x 2 states of the update per iteration).
 * *wave_instr (host) receives the wave-level instructions of the launch (for the updates: wave-level
 * state updates), so that instructions / elapsed time is the chip's issue rate of that form.
 * sink: device float buffer of compute_units x waves_per_simd x 256 entries (written, not
 * meaningful).  waves_per_simd in 1..8, iters >= 1, compute_units >= 1 (MAMBA_ERR_BAD_SHAPE),
 * unknown kind MAMBA_ERR_UNSUPPORTED. */
MAMBA_API mamba_status_t mamba_probe_issue(int32_t kind, int32_t waves_per_simd, int32_t iters,
                                           int32_t compute_units, float *sink,
                                           uint64_t *wave_instr, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_PROBE_H */
