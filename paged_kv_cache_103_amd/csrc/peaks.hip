// Achievable-peak probes (include/pa_peaks.h): a paged gather of random
// 4 KiB tiles, and back-to-back MFMAs. Built as libpa_peaks.so, apart from
// the attention library.
#include "pa_peaks.h"

#include <hip/hip_runtime.h>

#include "pa_device.h"

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

// The same gather by direct global -> LDS copies (nontemporal), as the
// side-by-side decode stages its tiles: each wave takes a contiguous range
// of the tile list and keeps one tile in flight while it reads the other
// from a ring of two (every copied byte is read back from LDS).
__global__ __launch_bounds__(256) void read_tiles_lds(const uint8_t* p, const int* ids, int ntiles, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][2][4096];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int per = (ntiles + nw - 1) / nw;
  const int x0 = (blockIdx.x * 4 + wave) * per;
  const int n = min(ntiles, x0 + per) - x0;
  typedef __attribute__((address_space(4))) const int cint;
  const cint* tc = (const cint*)ids;
  const uint32_t ring_lds = pa::lds_addr(&ring[wave][0][0]);
  auto issue = [&](int u) {  // tile x0 + u into slot u % 2
    const uint8_t* src = p + (size_t)(uint32_t)tc[x0 + u] * 4096;
#pragma unroll
    for (int j = 0; j < 4; ++j) pa::copy16_to_lds<true>(src + 1024 * j, 16u * lane, ring_lds + (u & 1) * 4096 + 1024 * j);
  };
  uint32_t acc = 0;
  if (n > 0) {
    issue(0);
    for (int u = 0; u < n; ++u) {
      if (u + 1 < n) {
        issue(u + 1);
        pa::wait_vmcnt<4>();
      } else {
        pa::wait_vmcnt<0>();
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 v = pa::lds_read16(ring_lds + (u & 1) * 4096 + 1024 * j + 16 * lane);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
      pa::wait_lgkmcnt0();  // the slot's reads are done before the next copy into it
    }
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

// (both probes take kHoldLds bytes of dynamic LDS: one workgroup per compute
// unit)
constexpr size_t kHoldLds = 96 * 1024;

template <int KIND>
__global__ __launch_bounds__(512) void lds_loop(int iters, uint32_t* sink, long long* cycles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t buf[];  // 64 KiB used
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 65536 / 4; i += 512) reinterpret_cast<uint32_t*>(buf)[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const uint32_t stride = KIND == 1 ? 32u : (KIND == 2 ? 8u : 16u);
  const uint32_t step = KIND == 2 ? 512u : 1024u;  // bytes one access instruction of a wave covers (kinds 0, 2)
  const uint32_t mask = KIND == 2 ? 0xfff8u : 0xfff0u;
  uint32_t acc = 0;
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t addr = ((uint32_t)lane * stride + (uint32_t)(wave * 8 + u) * step) & mask;
      if constexpr (KIND == 2) {
        *reinterpret_cast<uint2*>(buf + addr) = uint2{acc + (uint32_t)it, (uint32_t)u};
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(buf + addr);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
    __asm__ volatile("" ::: "memory");
  }
  __syncthreads();
  const long long t1 = __builtin_amdgcn_s_memtime();
  if constexpr (KIND == 2) acc ^= reinterpret_cast<const uint32_t*>(buf)[tid];
  sink[blockIdx.x * 512 + tid] = acc;
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

template <int MODE>
__global__ __launch_bounds__(512) void issue_loop(int iters, float* sink, long long* cycles) {
  extern __shared__ uint8_t hold[];
  const uint32_t t = threadIdx.x;
  const int wave = threadIdx.x >> 6;
  const u32x4 a = {t, t * 3u, t * 5u, t * 7u}, b = {t * 11u, t * 13u, t, t * 17u};
  const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
  f32x16 c[4] = {};
  float v[16], e[16];
  for (int i = 0; i < 16; ++i) {
    v[i] = 0.01f * (float)(t + i);
    e[i] = -0.001f * (float)(t + i);
  }
  hold[t] = 0;
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE != 1) {
#pragma unroll
      for (int k = 0; k < 16; ++k) c[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c[k & 3], 0, 0, 0);
    }
    if constexpr (MODE != 0) {
#pragma unroll
      for (int k = 0; k < 64; ++k) v[k & 15] = fmaf(v[k & 15], 0.999f, 0.001f);
#pragma unroll
      for (int k = 0; k < 16; ++k) e[k] = __builtin_amdgcn_exp2f(e[k]);
    }
    if constexpr (MODE == 2) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float r = 0.f;
  for (int q = 0; q < 4; ++q)
    for (int i = 0; i < 16; ++i) r += c[q][i];
  for (int i = 0; i < 16; ++i) r += v[i] + e[i];
  sink[blockIdx.x * 512 + t] = r + (float)hold[(t + 1) & 511];
  if ((t & 63) == 0) cycles[blockIdx.x * 8 + wave] = t1 - t0;
}

}  // namespace

extern "C" int32_t pa_peak_lds(int32_t kind, int32_t iters, int32_t grid_blocks, uint32_t* sink, int64_t* cycles,
                               pa_stream_t stream) {
  if (iters <= 0 || grid_blocks <= 0) return 0;
  long long* cyc = reinterpret_cast<long long*>(cycles);
  auto go = [&](auto kernel) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHoldLds);
    if (e != hipSuccess) return (int32_t)e;
    hipLaunchKernelGGL(kernel, dim3(grid_blocks), dim3(512), kHoldLds, (hipStream_t)stream, iters, sink, cyc);
    return (int32_t)hipGetLastError();
  };
  if (kind == 0) return go(lds_loop<0>);
  if (kind == 1) return go(lds_loop<1>);
  return go(lds_loop<2>);
}

extern "C" int32_t pa_peak_issue(int32_t mode, int32_t waves, int32_t iters, int32_t grid_blocks, float* sink,
                                 int64_t* cycles, pa_stream_t stream) {
  if (iters <= 0 || grid_blocks <= 0 || (waves != 4 && waves != 8)) return 0;
  long long* cyc = reinterpret_cast<long long*>(cycles);
  auto go = [&](auto kernel) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHoldLds);
    if (e != hipSuccess) return (int32_t)e;
    hipLaunchKernelGGL(kernel, dim3(grid_blocks), dim3(64 * waves), kHoldLds, (hipStream_t)stream, iters, sink, cyc);
    return (int32_t)hipGetLastError();
  };
  if (mode == 0) return go(issue_loop<0>);
  if (mode == 1) return go(issue_loop<1>);
  return go(issue_loop<2>);
}

extern "C" int32_t pa_peak_read_tiles(const void* buf, const int32_t* tile_ids, int32_t ntiles, int32_t mode,
                                      int32_t grid_blocks, uint32_t* sink, pa_stream_t stream) {
  if (ntiles <= 0 || grid_blocks <= 0) return 0;
  const u32x4* p = static_cast<const u32x4*>(buf);
  if (mode == 0)
    hipLaunchKernelGGL(read_tiles<0>, dim3(grid_blocks), dim3(256), 0, (hipStream_t)stream, p, tile_ids, ntiles, sink);
  else if (mode == 1)
    hipLaunchKernelGGL(read_tiles<1>, dim3(grid_blocks), dim3(256), 0, (hipStream_t)stream, p, tile_ids, ntiles, sink);
  else if (mode == 2)
    hipLaunchKernelGGL(read_tiles_lds, dim3(grid_blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint8_t*>(buf), tile_ids, ntiles, sink);
  else
    return (int32_t)hipErrorInvalidValue;
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
