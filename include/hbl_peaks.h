/*
 * hbl_peaks.h -- C ABI of libhbl_peaks.so: ceilings of one gfx950 GPU
 * measured by plain probe kernels, so that a benchmark can state its kernels'
 * fractions against what the chip delivers beside the published peaks.  The
 * probes are not part of the H-BitLinear layer and compute nothing of it.
 *
 * Conventions: pointers are DEVICE pointers owned by the caller; `stream` is
 * a hipStream_t passed as void* (NULL = the default stream); work is queued
 * and the call returns at once; arguments are checked on the host first and a
 * bad one queues nothing.  Return values: 0 = queued, 1 = invalid argument,
 * 2 = the launch failed.
 */
#ifndef HBL_PEAKS_H
#define HBL_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core instruction looped by hbl_peak_mfma. */
enum {
    HBL_PEAK_MFMA_I8 = 0,   /* v_mfma_i32_32x32x32_i8: 65536 ops per instruction */
    HBL_PEAK_MFMA_F6F4 = 1, /* v_mfma_scale_f32_32x32x64_f8f6f4, FP6 E3M2 x FP4 E2M1: 131072 ops */
    HBL_PEAK_MFMA_BF16 = 2  /* v_mfma_f32_32x32x16_bf16: 32768 ops */
};

/* Streaming copy of `bytes` (a multiple of 16, >= 0) from src to dst, 16 bytes
 * per lane and load; both 16-byte aligned, non-overlapping.  It moves 2*bytes
 * of HBM traffic (read + write). */
int hbl_peak_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* `blocks` workgroups of 256 threads (4 waves); every wave issues `iters`
 * rounds of four independent instructions of kind `kind` on register
 * operands, then writes one 32-bit value per thread to out[0 .. blocks*256)
 * (so the work cannot be discarded).  out_len is out's length in elements;
 * blocks in [1, 2^20], iters in [1, 2^24]. */
int hbl_peak_mfma(int kind, int32_t* out, int64_t out_len, int blocks, int iters, void* stream);

/* Dense operations one hbl_peak_mfma launch performs (2 per multiply-add),
 * or -1 for an invalid argument. */
int64_t hbl_peak_mfma_ops(int kind, int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* HBL_PEAKS_H */
