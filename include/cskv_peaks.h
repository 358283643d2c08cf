/*
 * cskv_peaks.h - measurement helpers of libcskv_peaks.so (not part of the method).
 *
 * Two microbenchmarks that give the measured ceilings the roofline fractions are also quoted
 * against, beside the published MI355X peaks: a streaming HBM read and a loop of independent
 * MFMA chains. They compute nothing of use; their only output is a value that is written only
 * if a never-met condition holds (so the loads and products cannot be removed).
 *
 * Return codes as in cskv.h (CSKV_OK, CSKV_EINVAL, CSKV_EHIP); cskv_peaks_last_error gives the
 * text of the last error on the calling thread.
 */
#ifndef CSKV_PEAKS_H_
#define CSKV_PEAKS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define CSKV_PEAKS_API __attribute__((visibility("default")))
#else
#define CSKV_PEAKS_API
#endif

/*
 * cskv_peak_hbm_read - reads bytes bytes of device memory at buf (16-byte aligned, bytes a
 * multiple of 16) once, with blocks workgroups of 256 threads (1 <= blocks <= 65536), each
 * thread keeping eight non-temporal 16-byte loads in flight. sink: device array of blocks uint32 (written
 * only if a never-met condition holds). Enqueued on stream (a hipStream_t, NULL = default).
 * Errors: CSKV_EINVAL (null or misaligned pointer, bad size or block count), CSKV_EHIP.
 */
CSKV_PEAKS_API int cskv_peak_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream);

/*
 * cskv_peak_mfma - blocks workgroups of 4 waves; each wave issues iters rounds of 4 independent
 * MFMA chains of kind 0: v_mfma_f32_32x32x16_bf16 (32768 flops each), 1:
 * v_mfma_scale_f32_32x32x64_f8f6f4 with e2m1 A and B (131072 flops each), 2: the same with
 * e4m3 A and B. A launch performs blocks * 4 * iters * 4 such instructions. sink: device array
 * of blocks floats (written only if a never-met condition holds).
 * Errors: CSKV_EINVAL (kind outside [0, 2], iters < 1, blocks outside [1, 65536], null sink),
 * CSKV_EHIP.
 */
CSKV_PEAKS_API int cskv_peak_mfma(int kind, int iters, int blocks, float* sink, void* stream);

CSKV_PEAKS_API const char* cskv_peaks_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CSKV_PEAKS_H_ */
