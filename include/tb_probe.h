/*
 * tb_probe.h - measurement probes of libtb_probe (not part of the product
 * path): kernels that measure what the device the benchmark runs on
 * achieves, against which the product kernels' figures are read.
 *
 * Conventions as in tb.h: device pointers, work enqueued on `stream` (a
 * hipStream_t passed as a plain pointer), nothing allocated, a return of 0
 * when the launch was accepted (else the HIP error code).
 */
#ifndef TB_PROBE_H
#define TB_PROBE_H

#include <stddef.h>
#include <stdint.h>

#define TBP_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read of `bytes` bytes at `src` (16-byte aligned; bytes a multiple
 * of 4096): `grid` workgroups of four waves walk the buffer in 4 KB steps per
 * wave, four 16-byte loads per lane in flight, and fold what they read into
 * one word per lane.  `sink` (grid * 256 uint32) receives a word only when the
 * fold hits a fixed pattern, so the loads cannot be dropped; it is not read
 * back.  The achievable HBM read bandwidth is bytes / kernel time.
 */
TBP_API int tbp_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, void* stream);

/*
 * A loop of v_mfma_f32_16x16x32_bf16 on register operands: `grid`
 * workgroups of four waves, each wave `iters` iterations of four independent
 * matrix instructions (16 x 16 x 32 each, 2 * 16 * 16 * 32 flops).  One float
 * per lane goes to `sink` (grid * 256 floats).  The achievable dense bf16
 * matrix rate is grid * 4 * iters * 4 * 16384 flops / kernel time.
 */
TBP_API int tbp_mfma_bf16(float* sink, int iters, int grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TB_PROBE_H */
