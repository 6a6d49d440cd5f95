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

/* Streaming write of `bytes` (a multiple of 16, >= 0) to dst (16-byte
 * aligned), 16 bytes per lane and store, four stores per thread, nothing
 * read: the burst of output one wave of GEMM tiles leaves behind. */
int hbl_peak_write(void* dst, int64_t bytes, void* stream);

/* Streaming read of `bytes` (a multiple of 16, > 0) from src (16-byte
 * aligned), 16 bytes per lane and load, four loads per thread; nothing is
 * written unless the data's folded words hit a fixed value, so the traffic
 * is the read alone.  sink (device, sink_len 32-bit words) must hold
 * hbl_peak_read_sink_len(bytes) words. */
int hbl_peak_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_len, void* stream);
int64_t hbl_peak_read_sink_len(int64_t bytes);

/* An empty kernel of `blocks` workgroups of 256 threads (blocks in
 * [1, 2^20]): the fixed cost of one launch. */
int hbl_peak_empty(int blocks, void* stream);

/* `blocks` workgroups of 256 threads (4 waves); every wave issues `iters`
 * rounds of four independent instructions of kind `kind` on register
 * operands, then writes one 32-bit value per thread to out[0 .. blocks*256)
 * (so the work cannot be discarded).  out_len is out's length in elements;
 * blocks in [1, 2^20], iters in [1, 2^24]. */
int hbl_peak_mfma(int kind, int32_t* out, int64_t out_len, int blocks, int iters, void* stream);

/* Dense operations one hbl_peak_mfma launch performs (2 per multiply-add),
 * or -1 for an invalid argument. */
int64_t hbl_peak_mfma_ops(int kind, int blocks, int iters);

/* Data-path probe of hbl_peak_lds: the work of one wave in one round. */
enum {
    HBL_PEAK_LDS_READ = 0,      /* 14 LDS reads of 16 bytes per lane (14 KiB per wave) */
    HBL_PEAK_LDS_DIRECT = 1,    /* 5 LDS-direct loads (buffer_load ... lds) of 1 KiB from src */
    HBL_PEAK_LDS_KSTEP = 2,     /* 5 LDS-direct loads, 14 LDS reads, 16 FP6 x FP4 32x32x64
                                   matrix-core instructions, one workgroup barrier: the per-wave
                                   work of one 128-deep K step of a 256 x 256 FP6 x FP4 tile */
    HBL_PEAK_LDS_KSTEP_NOBAR = 3, /* the same without the barrier */
    HBL_PEAK_LDS_KSTEP_NOLOAD = 4 /* HBL_PEAK_LDS_KSTEP without the LDS-direct loads */
};

/* `blocks` workgroups of 8 waves, each holding 96 KiB of LDS so that no two
 * share a compute unit (launch one per compute unit); every wave runs `iters`
 * rounds of the work of `kind`, with its LDS-direct loads two rounds ahead.
 * src (device, 16-byte aligned) holds src_bytes, a power of two in
 * [64 KiB, 1 GiB]; the loads walk it round robin (a small src stays in the
 * L2 caches).  Kinds HBL_PEAK_LDS_READ and HBL_PEAK_LDS_KSTEP_NOLOAD ignore
 * src (it may be NULL).
 * clk (device, clk_len >= 2 * blocks 64-bit words) receives, per workgroup,
 * the shader-clock cycles (s_memtime) and the 100 MHz real-time ticks
 * (s_memrealtime) that its first wave spent in the loop: their ratio is the
 * shader clock.  sink (device, sink_len >= blocks words) is written only if
 * the folded data hit a fixed value, so nothing can be discarded.
 * blocks in [1, 2^20], iters in [2, 2^24]. */
int hbl_peak_lds(int kind, const void* src, int64_t src_bytes, int blocks, int iters, int64_t* clk,
                 int64_t clk_len, uint32_t* sink, int64_t sink_len, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HBL_PEAKS_H */
