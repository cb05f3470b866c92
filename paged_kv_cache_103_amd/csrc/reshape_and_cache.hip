// KV write: scatter the new tokens' K/V rows into the paged pool.
//
// slot = physical_block * 16 + offset (the slot_mapping the model runner
// builds while preparing inputs — vLLM architecture summary, "第一部分：LLM
// 引擎核心"); K/V are written at prefill and appended at each decode step
// ("大模型推理优化学习笔记", "KV Cache"). K rows keep their [head_size] order;
// V is stored transposed inside the block ([head_size][16]), so one token's
// value row becomes a column of its block.
//
// One thread moves 8 consecutive elements of one (token, KV head) row. Same
// dtype in and out is a bit copy; an fp8 cache takes a quantising write with
// the caller's per-block scale.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <typename IT, int CK>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const IT* __restrict__ key, const IT* __restrict__ value,
    typename CacheElem<CK>::T* __restrict__ k_cache, typename CacheElem<CK>::T* __restrict__ v_cache,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads, int head_size) {
  typedef typename CacheElem<CK>::T CT;
  const int cshift = head_size == 128 ? 4 : 3;  // 8-element chunks per row: 16 or 8
  const int chunks = 1 << cshift;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks;
  if (idx >= total) return;
  const int c = (int)(idx & (chunks - 1));
  int h;
  int64_t t;
  if (total <= 0x7fffffff) {  // uniform; 32-bit division (64-bit is a long emulated sequence)
    const uint32_t r = (uint32_t)idx >> cshift;
    h = (int)(r % (uint32_t)num_kv_heads);
    t = r / (uint32_t)num_kv_heads;
  } else {
    h = (int)((idx >> cshift) % num_kv_heads);
    t = (idx >> cshift) / num_kv_heads;
  }
  // the row loads below do not depend on the slot: each branch issues them
  // before it tests the slot, so the two memory latencies overlap (rows of
  // skipped tokens are read too: they are inside key and value)
  const int64_t slot = slot_mapping[t];
  const bool skip = slot < 0;
  const int64_t blk = slot >> 4;
  const int off = (int)(slot & 15);
  const int d0 = c << 3;

  const IT* ksrc = key + ((t * num_kv_heads + h) * head_size + d0);
  const IT* vsrc = value + ((t * num_kv_heads + h) * head_size + d0);
  const int64_t tile = (blk * num_kv_heads + h) * (int64_t)(16 * head_size);
  CT* kdst = k_cache + tile + (int64_t)off * head_size + d0;  // [16][D] row-major
  CT* vdst = v_cache + tile + (int64_t)d0 * 16 + off;          // [D][16]

  if constexpr (sizeof(IT) == sizeof(CT)) {
    // bit copy
    if constexpr (sizeof(IT) == 4) {
      u32x4 a = load16(ksrc), b = load16(ksrc + 4);
      u32x4 va = load16(vsrc), vb = load16(vsrc + 4);
      __asm__ volatile("" ::"v"(a), "v"(b), "v"(va), "v"(vb));  // keeps the loads above the test
      if (skip) return;
      *reinterpret_cast<u32x4*>(kdst) = a;
      *reinterpret_cast<u32x4*>(kdst + 4) = b;
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&va);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vb);
#pragma unroll
      for (int e = 0; e < 4; ++e) reinterpret_cast<uint32_t*>(vdst)[e * 16] = w[e];
#pragma unroll
      for (int e = 0; e < 4; ++e) reinterpret_cast<uint32_t*>(vdst)[(e + 4) * 16] = w2[e];
    } else if constexpr (sizeof(IT) == 2) {
      u32x4 a = load16(ksrc);
      u32x4 v = load16(vsrc);
      __asm__ volatile("" ::"v"(a), "v"(v));  // keeps the loads above the test
      if (skip) return;
      *reinterpret_cast<u32x4*>(kdst) = a;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vdst[(2 * e) * 16] = (CT)(v[e] & 0xffffu);
        vdst[(2 * e + 1) * 16] = (CT)(v[e] >> 16);
      }
    } else {
      uint2 a = *reinterpret_cast<const uint2*>(ksrc);
      uint2 v = *reinterpret_cast<const uint2*>(vsrc);
      __asm__ volatile("" ::"v"(a.x), "v"(a.y), "v"(v.x), "v"(v.y));  // keeps the loads above the test
      if (skip) return;
      *reinterpret_cast<uint2*>(kdst) = a;
#pragma unroll
      for (int e = 0; e < 4; ++e) vdst[e * 16] = (CT)((v.x >> (8 * e)) & 0xff);
#pragma unroll
      for (int e = 0; e < 4; ++e) vdst[(e + 4) * 16] = (CT)((v.y >> (8 * e)) & 0xff);
    }
  } else {
    // quantising write into e4m3fn: byte = e4m3(x / scale[block]), RNE,
    // saturated to +-448; the quotient is an IEEE (correctly rounded) division.
    static_assert(CK == KFP8, "quantising write targets fp8 only");
    float kx[8], vx[8];
    if constexpr (sizeof(IT) == 4) {
#pragma unroll
      for (int e = 0; e < 8; ++e) { kx[e] = ksrc[e]; vx[e] = vsrc[e]; }
    } else {
      u32x4 a = load16(ksrc), b = load16(vsrc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kx[2 * e] = bf16_lo(a[e]); kx[2 * e + 1] = bf16_hi(a[e]);
        vx[2 * e] = bf16_lo(b[e]); vx[2 * e + 1] = bf16_hi(b[e]);
      }
    }
    if (skip) return;
    const float ks = k_scale[blk], vs = v_scale[blk];
    uint8_t kb[8], vb[8];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float k0 = sat_e4m3(kx[e] / ks), k1 = sat_e4m3(kx[e + 1] / ks);
      float v0 = sat_e4m3(vx[e] / vs), v1 = sat_e4m3(vx[e + 1] / vs);
      uint32_t kp = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(k0, k1, 0, false);
      uint32_t vp = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
      kb[e] = kp & 0xff; kb[e + 1] = (kp >> 8) & 0xff;
      vb[e] = vp & 0xff; vb[e + 1] = (vp >> 8) & 0xff;
    }
    uint2 kw;
    kw.x = kb[0] | (kb[1] << 8) | (kb[2] << 16) | ((uint32_t)kb[3] << 24);
    kw.y = kb[4] | (kb[5] << 8) | (kb[6] << 16) | ((uint32_t)kb[7] << 24);
    *reinterpret_cast<uint2*>(kdst) = kw;
#pragma unroll
    for (int e = 0; e < 8; ++e) vdst[e * 16] = vb[e];
  }
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_size, int in_kind, int cache_kind, hipStream_t stream) {
  const int64_t total = (int64_t)num_tokens * num_kv_heads * (head_size / 8);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
#define PA_RC_LAUNCH(IT, CK)                                                                 \
  hipLaunchKernelGGL((reshape_and_cache_kernel<IT, CK>), dim3((unsigned)blocks), dim3(threads), 0, \
                     stream, (const IT*)key, (const IT*)value,                                \
                     (typename CacheElem<CK>::T*)k_cache, (typename CacheElem<CK>::T*)v_cache, \
                     k_scale, v_scale, slot_mapping, num_tokens, num_kv_heads, head_size)
  if (in_kind == KF32 && cache_kind == KF32) PA_RC_LAUNCH(float, KF32);
  else if (in_kind == KBF16 && cache_kind == KBF16) PA_RC_LAUNCH(uint16_t, KBF16);
  else if (in_kind == KFP8 && cache_kind == KFP8) PA_RC_LAUNCH(uint8_t, KFP8);
  else if (in_kind == KF32 && cache_kind == KFP8) PA_RC_LAUNCH(float, KFP8);
  else if (in_kind == KBF16 && cache_kind == KFP8) PA_RC_LAUNCH(uint16_t, KFP8);
  else return hipErrorInvalidValue;
#undef PA_RC_LAUNCH
  return hipGetLastError();
}

}  // namespace pa
