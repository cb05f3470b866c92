// Paged decode attention on matrix cores for grouped-query heads (gfx950).
//
// Same computation and split-K plan as decode.hip (one query token per
// sequence, keys read through the block table, partitions merged by their
// softmax summaries), but the G query heads that share a KV head are treated
// as the columns of a small matrix: per pair of 16-token blocks the scores of
// all G heads are S^T = K Q^T (32 keys x 16 columns, bf16 16x16x32 MFMA, fp32
// accumulate) and the values are accumulated as O^T += V^T P^T. Grouped-query
// decode is a dense (G x d)(d x keys) contraction per block; on the VALU the
// dot products, cross-lane sums and the 16 exponentials per lane cost ~580
// instructions per bf16 block, more than the HBM time of the block, while
// here a block costs ~50 VALU instructions and 12 MFMAs, leaving the kernel
// bound by HBM (columns beyond G are padding).
//
// Layout tricks:
//  * key rows are fed to the score MFMA in a permuted order (tile kt, row i
//    holds key 8*(i/4) + 4*kt + i%4 of the 32-key pair), so that the score
//    accumulator of lane group q (lanes 16q..16q+15) ends up holding keys
//    8q..8q+7 — exactly the k-slice the PV MFMA wants from that lane group,
//    and a contiguous 16-byte run of the transposed V block;
//  * probabilities never leave their lane: the score accumulator (column =
//    head, 8 keys per lane) is the B operand of O^T = V^T P^T as it stands;
//  * P enters PV as bf16 hi + lo (two MFMAs), keeping ~16 bits of p;
//  * fp8 e4m3fn bytes are widened to bf16 exactly; the block's K scale
//    multiplies the score, its V scale the probability used in PV.
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 mfma_bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mfma_bf16x8_t, a),
                                                  __builtin_bit_cast(mfma_bf16x8_t, b), c, 0, 0, 0);
}

template <int CK, int D>
struct MfmaDecodeShape {
  static constexpr int E = CacheElem<CK>::bytes;   // 2 (bf16) or 1 (fp8)
  static constexpr int DS = D / 32;                // score MFMA k-steps over head_size
  static constexpr int DT = D / 16;                // 16-row tiles of head_size in O^T
  static constexpr int TILE = 16 * D * E;          // bytes of one (block, head) tile
  // K registers per block pair: bf16 one 16-byte load per (kt, k-step);
  // fp8 one 16-byte load per (kt, two k-steps)
  static constexpr int KL = (E == 2) ? 2 * DS : DS;
};

// Physical head dim of the first of the 8 values lane group q feeds to
// k-step j (the same map for K and Q, so the contraction is unchanged).
template <int E>
__device__ __forceinline__ int kstep_d0(int j, int q) {
  return (E == 2) ? 32 * j + 8 * q : 64 * (j >> 1) + 16 * q + 8 * (j & 1);
}

template <int CK, int D>
struct PairRegs {
  u32x4 k[MfmaDecodeShape<CK, D>::KL];
  // V^T fragments: bf16 16 bytes per 16-row tile of head_size; fp8 8 bytes
  u32x4 v[(CacheElem<CK>::bytes == 2) ? D / 16 : D / 32];
};

// Loads one pair of blocks (b, b+1). When b+1 is past the context the pair's
// second half re-reads block b (valid memory); those keys are >= ctx and are
// masked out of the scores and zeroed in V.
template <int CK, int D>
__device__ __forceinline__ void load_pair(PairRegs<CK, D>& r, const uint8_t* kcache, const uint8_t* vcache,
                                          size_t phys0, size_t phys1, size_t head_stride, int c16, int q4) {
  using S = MfmaDecodeShape<CK, D>;
  constexpr int E = S::E;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int kp = 8 * (c16 >> 2) + 4 * kt + (c16 & 3);  // this lane's key row in score tile kt
    const size_t phys = (kp >> 4) ? phys1 : phys0;
    const uint8_t* row = kcache + phys * head_stride + (size_t)(kp & 15) * (D * E);
    if constexpr (E == 2) {
#pragma unroll
      for (int j = 0; j < S::DS; ++j) r.k[kt * S::DS + j] = load16(row + kstep_d0<E>(j, q4) * 2);
    } else {
#pragma unroll
      for (int c = 0; c < S::DS / 2; ++c) r.k[kt * (S::DS / 2) + c] = load16(row + 64 * c + 16 * q4);
    }
  }
  // V^T: lane group q reads keys 8q..8q+7 = block q/2, keys 8(q&1)..+8
  const size_t vphys = (q4 >> 1) ? phys1 : phys0;
  const uint8_t* vt = vcache + vphys * head_stride + 8 * (q4 & 1) * E;
  if constexpr (E == 2) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) r.v[dt] = load16(vt + (size_t)(dt * 16 + c16) * 32);
  } else {
#pragma unroll
    for (int dp = 0; dp < D / 32; ++dp) {
      const uint2 a = *reinterpret_cast<const uint2*>(vt + (size_t)((2 * dp) * 16 + c16) * 16);
      const uint2 c = *reinterpret_cast<const uint2*>(vt + (size_t)((2 * dp + 1) * 16 + c16) * 16);
      r.v[dp] = u32x4{a.x, a.y, c.x, c.y};
    }
  }
}

template <int CK, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_mfma_kernel(DecodeArgs a) {
  using S = MfmaDecodeShape<CK, D>;
  constexpr int E = S::E, DS = S::DS, DT = S::DT;
  __shared__ float w_m[4][16], w_l[4][16];
  __shared__ float w_o[4][16][D];

  const int part = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, q4 = lane >> 4;
  const int G = a.num_heads / a.num_kv_heads;

  int qrow = s;
  if (a.cu_seqlens != nullptr) {
    const int q0 = a.cu_seqlens[s];
    if (a.cu_seqlens[s + 1] - q0 != 1) return;
    qrow = q0;
  }
  const int ctx = a.context_lens[s];
  const int lo = a.window > 0 ? max(0, ctx - a.window) : 0;
  const int b_first = lo >> 4, b_last = (ctx - 1) >> 4;
  const int nparts = (b_last - b_first + a.pb) / a.pb;
  if (part >= nparts) return;
  const int blk0 = b_first + part * a.pb;
  const int blk1 = min(blk0 + a.pb, b_last + 1);

  u32x4 qf[DS];
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  const size_t head_stride = (size_t)a.num_kv_heads * S::TILE;
  const uint8_t* kcache = reinterpret_cast<const uint8_t*>(a.k_cache) + (size_t)g * S::TILE;
  const uint8_t* vcache = reinterpret_cast<const uint8_t*>(a.v_cache) + (size_t)g * S::TILE;
  const int* bt = a.block_table + (size_t)s * a.bt_stride;

  // wave-strided pairs of blocks; several waves per SIMD keep loads in flight
  // (pairs that straddle the window start or the context end take the
  // masked variant of the step; interior pairs carry no masking code)
  auto step = [&](auto edge_tag, const PairRegs<CK, D>& r, size_t phys0, size_t phys1, int b) {
    constexpr bool EDGE = decltype(edge_tag)::value;

    // ---- scores S^T (2 tiles of 16 permuted keys x 16 heads) ----
    f32x4 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < DS; ++j) {
        u32x4 kf;
        if constexpr (E == 2) {
          kf = r.k[kt * DS + j];
        } else {
          const u32x4& w = r.k[kt * (DS / 2) + (j >> 1)];
          kf = (j & 1) ? fp8x8_to_bf16x8(w[2], w[3]) : fp8x8_to_bf16x8(w[0], w[1]);
        }
        st[kt] = mfma_bf16_16x16x32(kf, qf[j], st[kt]);
      }
    }
    // this lane's keys: b*16 + 8*q4 + 4*kt + r, all in block b + q4/2
    float ks = a.scale_log2, vs = 1.f;
    if constexpr (CK == KFP8) {
      const size_t phys = (q4 >> 1) ? phys1 : phys0;
      ks *= a.k_scale[phys];
      vs = a.v_scale[phys];
    }
    const int key0 = b * 16 + 8 * q4;
    float x[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float v = st[kt][rr] * ks;
        if constexpr (EDGE) {
          const int kp = key0 + 4 * kt + rr;
          v = (kp >= lo && kp < ctx) ? v : -INFINITY;
        }
        x[kt][rr] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = strided_max<16>(tmax);
    const float mn = fmaxf(m, tmax);  // finite: every pair has a key in [lo, ctx)
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    float ps = 0.f, pv[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float p = __builtin_amdgcn_exp2f(x[kt][rr] - mn);
        ps += p;
        pv[kt][rr] = p * vs;
      }
    lsum = lsum * alpha + ps;
    if (__any(alpha != 1.f)) {  // the running max rarely moves after the first blocks
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[dt][0] *= alpha; o[dt][1] *= alpha; o[dt][2] *= alpha; o[dt][3] *= alpha;
      }
    }
    // P^T operand: logical k 8*q4 + e <-> key 8*q4 + e (e = 4*kt + rr)
    u32x4 ph, pl;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float a0 = pv[t >> 1][(t & 1) * 2], a1 = pv[t >> 1][(t & 1) * 2 + 1];
      const uint32_t hi = pack_bf16x2(a0, a1);
      ph[t] = hi;
      pl[t] = pack_bf16x2(a0 - bf16_lo(hi), a1 - bf16_hi(hi));
    }
    // value slices of keys >= ctx may hold anything (even NaN): zero them
    uint32_t vmask[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    if constexpr (EDGE) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k0 = key0 + 2 * t;
        vmask[t] = (k0 < ctx ? 0x0000ffffu : 0u) | (k0 + 1 < ctx ? 0xffff0000u : 0u);
      }
    }
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x4 vf;
      if constexpr (E == 2) {
        vf = r.v[dt];
      } else {
        const u32x4& w = r.v[dt >> 1];
        vf = (dt & 1) ? fp8x8_to_bf16x8(w[2], w[3]) : fp8x8_to_bf16x8(w[0], w[1]);
      }
      if constexpr (EDGE) {
        vf[0] &= vmask[0]; vf[1] &= vmask[1]; vf[2] &= vmask[2]; vf[3] &= vmask[3];
      }
      o[dt] = mfma_bf16_16x16x32(vf, ph, o[dt]);
      o[dt] = mfma_bf16_16x16x32(vf, pl, o[dt]);
    }
  };
  auto run = [&](const PairRegs<CK, D>& r, size_t p0, size_t p1, int b) {
    if (b * 16 < lo || b * 16 + 32 > ctx) step(std::true_type{}, r, p0, p1, b);
    else step(std::false_type{}, r, p0, p1, b);
  };
  // The wave's next pair is always in flight while one is computed (two
  // register buffers, alternating).
  PairRegs<CK, D> ra, rb;
  size_t a0 = 0, a1 = 0, b0 = 0, b1 = 0;
  int b = blk0 + 2 * wave;
  if (b < blk1) {
    a0 = (size_t)bt[b];
    a1 = (b + 1 < blk1) ? (size_t)bt[b + 1] : a0;
    load_pair<CK, D>(ra, kcache, vcache, a0, a1, head_stride, c16, q4);
  }
  // queries of the group as the B operand (column = head; columns >= G are 0)
#pragma unroll
  for (int j = 0; j < DS; ++j) {
    if (c16 < G) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.query) +
                           ((size_t)qrow * a.num_heads + g * G + c16) * D + kstep_d0<E>(j, q4);
      qf[j] = load16(qp);
    } else {
      qf[j] = u32x4{0, 0, 0, 0};
    }
  }

  while (b < blk1) {
    const int bn = b + 8;
    if (bn < blk1) {
      b0 = (size_t)bt[bn];
      b1 = (bn + 1 < blk1) ? (size_t)bt[bn + 1] : b0;
      load_pair<CK, D>(rb, kcache, vcache, b0, b1, head_stride, c16, q4);
    }
    run(ra, a0, a1, b);
    if (bn >= blk1) break;
    const int bnn = bn + 8;
    if (bnn < blk1) {
      a0 = (size_t)bt[bnn];
      a1 = (bnn + 1 < blk1) ? (size_t)bt[bnn + 1] : a0;
      load_pair<CK, D>(ra, kcache, vcache, a0, a1, head_stride, c16, q4);
    }
    run(rb, b0, b1, bn);
    b = bnn;
  }

  // ---- merge the 4 waves; write the output or this partition's summary ----
  lsum = strided_sum<16>(lsum);
  if (q4 == 0) { w_m[wave][c16] = m; w_l[wave][c16] = lsum; }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) w_o[wave][c16][dt * 16 + 4 * q4 + rr] = o[dt][rr];
  __syncthreads();

  const bool single = (nparts == 1);
  for (int e = threadIdx.x; e < G * D; e += 256) {
    const int h = e / D, d = e % D;
    float M = w_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, w_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float c = __builtin_amdgcn_exp2f(w_m[w][h] - M);
      L += w_l[w][h] * c;
      O += w_o[w][h][d] * c;
    }
    const int hq = g * G + h;
    if (single) {
      reinterpret_cast<uint16_t*>(a.out)[((size_t)qrow * a.num_heads + hq) * D + d] = f32_to_bf16(O / L);
    } else {
      const size_t slot = ((size_t)s * a.num_heads + hq) * a.max_parts + part;
      a.part_o[slot * D + d] = O;
      if (d == 0) {
        a.part_ml[slot * 2] = M;
        a.part_ml[slot * 2 + 1] = L;
      }
    }
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int cache_kind, int head_size, hipStream_t st) {
  dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
  if (cache_kind == KBF16 && head_size == 128)
    hipLaunchKernelGGL((decode_mfma_kernel<KBF16, 128>), grid, dim3(256), 0, st, a);
  else if (cache_kind == KBF16 && head_size == 64)
    hipLaunchKernelGGL((decode_mfma_kernel<KBF16, 64>), grid, dim3(256), 0, st, a);
  else if (cache_kind == KFP8 && head_size == 128)
    hipLaunchKernelGGL((decode_mfma_kernel<KFP8, 128>), grid, dim3(256), 0, st, a);
  else if (cache_kind == KFP8 && head_size == 64)
    hipLaunchKernelGGL((decode_mfma_kernel<KFP8, 64>), grid, dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
