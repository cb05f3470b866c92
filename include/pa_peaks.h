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
 * buf (every id in [0, buf_bytes / 4096)), as a paged gather does. mode 0:
 * one wave per tile, 16-byte nontemporal loads, each load instruction
 * covering 1 KiB contiguous; mode 1: the same with the decode kernel's key
 * pattern (64 bytes from each of 16 rows of 256 bytes); mode 2: 16-byte
 * nontemporal global -> LDS copies, each wave a contiguous range of the list
 * with one tile in flight while it reads the previous one back from LDS.
 * grid_blocks workgroups of 256 threads share the tiles; another mode
 * returns hipErrorInvalidValue. sink: >= grid_blocks uint32, written only to
 * keep the loads alive.
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

/*
 * LDS bandwidth of one compute unit: grid_blocks workgroups of 512 threads
 * (8 waves; 96 KiB of LDS each, so one per compute unit) run `iters` rounds
 * of 8 LDS accesses per lane; kind 0: 16-byte reads, consecutive lanes on
 * consecutive addresses (no bank conflicts); kind 1: the same with a 32-byte
 * lane stride (two-way conflicts); kind 2: 8-byte writes of consecutive
 * lanes. Bytes per workgroup: iters * 8 * 512 * (16, 16 or 8).
 * cycles: >= grid_blocks int64, each workgroup's loop time in shader-clock
 * cycles (s_memtime). sink: >= 512 * grid_blocks uint32.
 */
int32_t pa_peak_lds(int32_t kind, int32_t iters, int32_t grid_blocks, uint32_t* sink, int64_t* cycles,
                    pa_stream_t stream);

/*
 * Issue mix of one SIMD: grid_blocks workgroups of 64 * waves threads (waves
 * 4 or 8: one or two waves per SIMD; 96 KiB of LDS each, so one per compute
 * unit), each wave running `iters` rounds of 16 32x32x16 bf16 MFMAs and 64
 * fp32 FMAs plus 16 exp2 (the softmax of a 32-key step), as mode 0: matrix
 * work only, 1: vector work only, 2: both, interleaved (one MFMA, then 5
 * vector instructions). cycles: >= grid_blocks * 8 int64, each wave's loop
 * time in shader-clock cycles. sink: >= 512 * grid_blocks floats.
 */
int32_t pa_peak_issue(int32_t mode, int32_t waves, int32_t iters, int32_t grid_blocks, float* sink,
                      int64_t* cycles, pa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PEAKS_H */
