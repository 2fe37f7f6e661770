/*
 * dsa_peak.h - peak probes of the device the DSA library runs on (libpeak.so).
 *
 * Measurement helpers, not part of the attention path: each call enqueues one kernel on
 * `stream` that runs only the named work, so that its duration (timed by the caller with
 * events on the same stream) gives the device's sustained rate under load.  The caller owns
 * all memory; `sink` is a device buffer of at least 16 * (number of compute units) floats that
 * the kernels may write (never read back meaningfully).  Return 0 on success, 1 for an invalid
 * argument, 4 for a failed launch.
 */
#ifndef DSA_PEAK_H_
#define DSA_PEAK_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Independent chains of v_mfma_f32_32x32x16_bf16 in every wave of four workgroups of 512
 * threads per compute unit, iters rounds of 8 per wave; *flops receives the FLOPs enqueued. */
int dsa_peak_mfma_bf16(int iters, float* sink, hipStream_t stream, double* flops);

/* The same with v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3 operands with unit scales. */
int dsa_peak_mfma_fp8(int iters, float* sink, hipStream_t stream, double* flops);

/* A streaming read of bytes bytes at src (16-byte aligned) by 16 workgroups per compute unit. */
int dsa_peak_read(const void* src, size_t bytes, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_PEAK_H_ */
