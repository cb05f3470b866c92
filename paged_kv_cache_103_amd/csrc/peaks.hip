// Achievable-peak probes (include/pa_peaks.h): a paged gather of random
// 4 KiB tiles, and back-to-back MFMAs. Built as libpa_peaks.so, apart from
// the attention library.
#include "pa_peaks.h"

#include <hip/hip_runtime.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int MODE>
__global__ __launch_bounds__(256) void read_tiles(const u32x4* __restrict__ p, const int* __restrict__ ids,
                                                  int ntiles, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nw = (gridDim.x * blockDim.x) >> 6;
  uint32_t acc = 0;
  for (int t = wave; t < ntiles; t += nw) {
    const u32x4* base = p + (size_t)ids[t] * 256;
    u32x4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = MODE == 0 ? 64 * j + lane : (lane & 15) * 16 + 4 * j + (lane >> 4);
      a[j] = __builtin_nontemporal_load(base + off);
    }
    // every component is used, so that each load stays a 16-byte load (a
    // partly used vector is narrowed to 4-byte loads by the compiler)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc ^= a[j].x ^ a[j].y ^ a[j].z ^ a[j].w;
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop(int iters, float* sink) {
  const uint32_t t = threadIdx.x;
  const u32x4 a = {t, t * 3u, t * 5u, t * 7u}, b = {t * 11u, t * 13u, t, t * 17u};
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    if constexpr (KIND == 0) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c3, 0, 0, 0);
    } else {
      const f16x8 x = __builtin_bit_cast(f16x8, a), y = __builtin_bit_cast(f16x8, b);
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c3, 0, 0, 0);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) r += c0[v] + c1[v] + c2[v] + c3[v];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

}  // namespace

extern "C" int32_t pa_peak_read_tiles(const void* buf, const int32_t* tile_ids, int32_t ntiles, int32_t mode,
                                      int32_t grid_blocks, uint32_t* sink, pa_stream_t stream) {
  if (ntiles <= 0 || grid_blocks <= 0) return 0;
  const u32x4* p = static_cast<const u32x4*>(buf);
  if (mode == 0)
    hipLaunchKernelGGL(read_tiles<0>, dim3(grid_blocks), dim3(256), 0, (hipStream_t)stream, p, tile_ids, ntiles, sink);
  else
    hipLaunchKernelGGL(read_tiles<1>, dim3(grid_blocks), dim3(256), 0, (hipStream_t)stream, p, tile_ids, ntiles, sink);
  return (int32_t)hipGetLastError();
}

extern "C" int32_t pa_peak_mfma(int32_t kind, int32_t iters, int32_t grid_blocks, float* sink, pa_stream_t stream) {
  if (iters <= 0 || grid_blocks <= 0) return 0;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_loop<0>, dim3(grid_blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_loop<1>, dim3(grid_blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return (int32_t)hipGetLastError();
}
