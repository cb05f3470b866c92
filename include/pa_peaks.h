/*
 * pa_peaks.h — achievable-peak probes of libpa_peaks (MI355X, gfx950).
 *
 * Not part of the attention path: bench.py runs these next to the path's
 * kernels to place their rates against what the chip delivers on the same
 * kind of work, beside the published peaks ("大模型推理优化学习笔记",
 * "计算密集与访存密集": decode is bound by memory bandwidth, prefill by
 * compute). All pointers are device pointers owned by the caller; each call
 * only enqueues one kernel on `stream` and returns 0, or a HIP error code if
 * the launch fails (nothing is checked on the device).
 */
#ifndef PA_PEAKS_H
#define PA_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* pa_stream_t;

/*
 * Reads `ntiles` tiles of 4 KiB, tile t at byte offset 4096 * tile_ids[t] of
 * buf (every id in [0, buf_bytes / 4096)), as a paged gather does: one wave
 * per tile, 16-byte nontemporal loads. mode 0: each load instruction covers
 * 1 KiB contiguous; mode 1: the decode kernel's key pattern (64 bytes from
 * each of 16 rows of 256 bytes). grid_blocks workgroups of 256 threads
 * stride over the tiles. sink: >= grid_blocks uint32, written only to keep
 * the loads alive.
 */
int32_t pa_peak_read_tiles(const void* buf, const int32_t* tile_ids, int32_t ntiles, int32_t mode,
                           int32_t grid_blocks, uint32_t* sink, pa_stream_t stream);

/*
 * Back-to-back dense matrix-core work: every wave of grid_blocks workgroups
 * of 256 threads runs `iters` rounds of 4 independent 32x32x16 MFMAs
 * (kind 0: bf16, kind 1: fp16), i.e. 4 * 32768 flops per wave per round.
 * sink: >= 256 * grid_blocks floats.
 */
int32_t pa_peak_mfma(int32_t kind, int32_t iters, int32_t grid_blocks, float* sink, pa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PEAKS_H */
