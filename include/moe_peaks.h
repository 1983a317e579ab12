/*
 * moe_peaks.h -- measurement probes of libmoepeaks.so (not part of the layer).
 *
 * Two microbenchmarks give the machine limits that the MoE kernels' measured
 * rates are compared with, next to MI355X's datasheet peaks (HBM3E 8 TB/s,
 * dense bf16 MFMA 2.5 PFLOP/s):
 *   peak_stream_read  reads `bytes` of device memory once with plain 16-byte
 *                     vector loads (8 in flight per thread; `blocks`
 *                     workgroups of 256 threads take contiguous 32 KB pieces
 *                     in turn): bytes / kernel time
 *                     is the achievable HBM read rate when the buffer is much
 *                     larger than the caches.
 *   peak_mfma_loop    runs `iters` (a multiple of 4) rounds of 8 independent
 *                     v_mfma_f32_32x32x16_bf16 per wave on random register
 *                     operands (`data`: peak_mfma_data_bytes of random bits),
 *                     4 waves per workgroup: peak_mfma_flops(iters, blocks) /
 *                     kernel time is the achievable dense bf16 rate.
 * All pointers are device pointers, 16-byte aligned, owned by the caller;
 * `sink` receives peak_stream_sink_words / peak_mfma_sink_words values that
 * keep the work from being optimised away.  Calls enqueue one kernel on
 * `stream` (a hipStream_t) and return 0, or 1 for a bad argument, 2 for a
 * failed launch.
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int peak_stream_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, void* stream);
size_t peak_stream_sink_words(int blocks);
int peak_mfma_loop(const void* data, int iters, int blocks, float* sink, void* stream);
size_t peak_mfma_data_bytes(void);
size_t peak_mfma_sink_words(int blocks);
double peak_mfma_flops(int iters, int blocks);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAKS_H */
