/*
 * efla_peaks.h - reference kernels for the machine peaks the EFLA kernels are
 * measured against.
 *
 * The operator's roofline fractions are stated against MI355X's published
 * peaks (HBM 8 TB/s; dense bf16 MFMA 2.5 PFLOP/s; fp32 MFMA 157.3 TFLOP/s)
 * and, beside them, against what these two kernels reach on the same GPU in
 * the same process: a streaming device copy and a loop of independent MFMAs
 * with operands held in registers.  They compute nothing of the method.
 *
 * Same conventions as efla.h: device pointers owned by the caller,
 * asynchronous on `stream` (a hipStream_t; NULL = the null stream), arguments
 * validated before any HIP call, no allocation, no printing.
 */
#ifndef EFLA_PEAKS_H
#define EFLA_PEAKS_H

#include <stddef.h>

#include "efla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0 .. bytes) = src[0 .. bytes): 16-byte loads and non-temporal 16-byte
 * stores, a grid of 8 workgroups per CU striding over the buffer.  src and
 * dst 16-byte aligned, bytes a multiple of 16, the two ranges disjoint;
 * otherwise EFLA_ERR_INVALID_ARG.  The bandwidth is 2 * bytes / time. */
efla_status_t efla_peak_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Matrix-core throughput: `blocks` workgroups of four waves (one per SIMD),
 * each wave running `iters` rounds of eight independent MFMAs on register
 * operands -- v_mfma_f32_16x16x32_bf16 for EFLA_BF16, v_mfma_f32_16x16x4_f32
 * for EFLA_F32 -- and writing one float per wave to sink[blocks * 4] so that
 * nothing is elided.  *flops (if not NULL) receives the floating-point
 * operations of one launch.  blocks, iters >= 1, else EFLA_ERR_INVALID_ARG. */
efla_status_t efla_peak_mfma(float *sink, int blocks, int iters, efla_dtype_t dt,
                             double *flops, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EFLA_PEAKS_H */
