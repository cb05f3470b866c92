// Merge of attention results computed over disjoint key ranges
// (pa_merge_partials, include/pa.h). Decode context parallelism splits a
// sequence's cached positions into contiguous ranges, one per GPU; each range
// yields a normalised output o_r and the log of its softmax denominator
// lse_r, and the exact result is sum_r e^(lse_r - M) o_r / sum_r e^(lse_r - M)
// with M = max_r lse_r ("宣稱省下 106 倍成本…", "DCP 的切法：照「序列位置」切，
// 不照「頭」切" and the online-softmax Q&A of "中：Kimi K3 的 DCP 選擇與 DEP 轉折").
//
// One wave per (token, head) row; lane l holds dimensions l, l + 64, ...
// The ranges' weights are computed once per row; every load is a coalesced
// 64-wide row segment.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void store_elem(T* p, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, float x) { *p = f32_to_bf16(x); }

template <typename T, int DL>
__global__ __launch_bounds__(256) void merge_lse_kernel(T* out, float* lse_out, const T* parts,
                                                        const float* parts_lse, int num_parts, int num_rows) {
  constexpr int D = 64 * DL;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= num_rows) return;
  float M = -INFINITY;
  for (int r = lane; r < num_parts; r += 64) M = fmaxf(M, parts_lse[(size_t)r * num_rows + row]);
  M = strided_max<1>(M);
  float acc[DL];
#pragma unroll
  for (int k = 0; k < DL; ++k) acc[k] = 0.f;
  float den = 0.f;
  if (M > -INFINITY) {
    for (int r = 0; r < num_parts; ++r) {
      const float w = __expf(parts_lse[(size_t)r * num_rows + row] - M);
      den += w;
      const T* src = parts + ((size_t)r * num_rows + row) * D + lane;
#pragma unroll
      for (int k = 0; k < DL; ++k) acc[k] = fmaf(w, load_elem<T>(src + 64 * k), acc[k]);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  T* dst = out + (size_t)row * D + lane;
#pragma unroll
  for (int k = 0; k < DL; ++k) store_elem<T>(dst + 64 * k, acc[k] * inv);
  if (lse_out != nullptr && lane == 0) lse_out[row] = M + logf(den);
}

template <typename T>
static hipError_t run_merge_lse(void* out, float* lse_out, const void* parts, const float* parts_lse, int num_parts,
                                int num_rows, int head_size, hipStream_t st) {
  const dim3 grid((unsigned)((num_rows + 3) / 4));
  T* o = static_cast<T*>(out);
  const T* p = static_cast<const T*>(parts);
  switch (head_size) {
    case 64: hipLaunchKernelGGL((merge_lse_kernel<T, 1>), grid, dim3(256), 0, st, o, lse_out, p, parts_lse, num_parts, num_rows); break;
    case 128: hipLaunchKernelGGL((merge_lse_kernel<T, 2>), grid, dim3(256), 0, st, o, lse_out, p, parts_lse, num_parts, num_rows); break;
    case 512: hipLaunchKernelGGL((merge_lse_kernel<T, 8>), grid, dim3(256), 0, st, o, lse_out, p, parts_lse, num_parts, num_rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge_lse(void* out, float* lse_out, const void* parts, const float* parts_lse, int num_parts,
                            int num_rows, int head_size, int kind, hipStream_t stream) {
  if (num_rows == 0) return hipSuccess;
  if (kind == KF32) return run_merge_lse<float>(out, lse_out, parts, parts_lse, num_parts, num_rows, head_size, stream);
  if (kind == KBF16)
    return run_merge_lse<uint16_t>(out, lse_out, parts, parts_lse, num_parts, num_rows, head_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
