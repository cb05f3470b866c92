// Copy-on-write of whole physical blocks (pa_copy_blocks, include/pa_blocks.h):
// before a branch appends to a shared block that is not full, the block is
// copied to a block of its own ("从静态批处理到状态化推理集群", "Prefix reuse").
// One workgroup per (pair, KV head) moves that head's K tile and V tile with
// 16-byte loads and stores; the first head's workgroup also copies the fp8
// block scales. A pair naming a block outside the pool is skipped.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* k_cache, uint8_t* v_cache, float* k_scale,
                                                          float* v_scale, const int32_t* pairs,
                                                          uint32_t tile_bytes, int num_kv_heads, int num_blocks) {
  const int p = blockIdx.x / num_kv_heads, h = blockIdx.x % num_kv_heads;
  const int32_t s32 = pairs[2 * p], d32 = pairs[2 * p + 1];
  if (s32 < 0 || s32 >= num_blocks || d32 < 0 || d32 >= num_blocks) return;
  const size_t src = (size_t)s32, dst = (size_t)d32;
  const size_t block_bytes = (size_t)num_kv_heads * tile_bytes;
  const size_t so = src * block_bytes + (size_t)h * tile_bytes, d0 = dst * block_bytes + (size_t)h * tile_bytes;
  for (uint32_t i = threadIdx.x * 16u; i < tile_bytes; i += 256u * 16u) {
    *reinterpret_cast<u32x4*>(k_cache + d0 + i) = *reinterpret_cast<const u32x4*>(k_cache + so + i);
    *reinterpret_cast<u32x4*>(v_cache + d0 + i) = *reinterpret_cast<const u32x4*>(v_cache + so + i);
  }
  if (h == 0 && threadIdx.x == 0 && k_scale != nullptr) {
    k_scale[dst] = k_scale[src];
    v_scale[dst] = v_scale[src];
  }
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const int32_t* pairs,
                              int num_pairs, size_t tile_bytes, int num_kv_heads, int num_blocks,
                              hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs * (unsigned)num_kv_heads), dim3(256), 0, stream,
                     static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), k_scale, v_scale, pairs,
                     (uint32_t)tile_bytes, num_kv_heads, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
