/*
 * muonclip_probe.h - measurement aids exported by libmuonclip.so.
 *
 * Not part of the optimizer step.  They measure, on the GPU at hand, the two
 * ceilings the step's kernels are judged against besides the data-sheet
 * peaks (2.5 PFLOP/s dense bf16 MFMA, 8 TB/s HBM3E on MI355X): the MFMA rate
 * the chip sustains at the clock it holds under full matrix load, and the
 * rate of a plain device-to-device copy.  Conventions (device pointers,
 * stream as void*, checks before launch, status codes) are those of
 * muonclip.h.
 */
#ifndef MUONCLIP_PROBE_H
#define MUONCLIP_PROBE_H

#include "muonclip.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * MFMA ceiling: `workgroups` workgroups of 256 threads (4 waves, one per
 * SIMD) each run `iters` iterations of 16 independent
 * v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic in the
 * loop).  Work: workgroups * 4 * iters * 16 * 32768 flop.  Operands are
 * random bf16 with exponents near 1 (zero_operands = 0) or all zero
 * (zero_operands != 0; less switching, so the chip clocks higher).
 *   out: device float32 [workgroups * 256], one checksum per thread (keeps
 *        the work from being optimised away; its value has no meaning).
 * Errors: MC_EINVAL for workgroups < 1 or > 65536, iters < 1 or > 2^30, or
 * a NULL / misaligned out; MC_EHIP on a failed launch.
 */
MC_API mc_status_t mc_probe_mfma_bf16(int64_t workgroups, int64_t iters, int zero_operands, float* out,
                                      void* stream);

/*
 * Stream ceiling: dst[0 .. bytes) = src[0 .. bytes) with 16-byte
 * non-temporal loads and stores, one vector per thread.  The buffers must
 * not overlap.  Errors: MC_EINVAL for bytes < 0, not a multiple of 16, or a
 * NULL pointer with bytes > 0; MC_EALIGN for pointers not 16-byte aligned;
 * MC_EHIP on a failed launch.
 */
MC_API mc_status_t mc_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MUONCLIP_PROBE_H */
