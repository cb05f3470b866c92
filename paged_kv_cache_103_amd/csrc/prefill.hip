// Chunked-prefill paged attention on gfx950 matrix cores (MFMA) for fp8
// caches (bf16 caches take the kernel of prefill_bf16.hip).
//
// What it computes: every query row of a chunk longer than one token attends
// causally to its sequence's cached keys, read through the block table: the
// chunk sits on top of a cached prefix, and query row r of a chunk of q_len
// rows in a context of ctx tokens is at position ctx - q_len + r
// ("大模型推理优化学习笔记", "Chunked Prefill"; "从静态批处理到状态化推理集群",
// "Chunked prefill：在共置引擎里治理阶段干扰"). Prefill reuses each K/V row across
// many queries and is compute-bound ("大模型推理优化学习笔记", "计算密集与访存密集"),
// so QK^T and PV run on MFMA with fp32 accumulation.
//
// Tiling (one workgroup = 4 waves):
//  * a tile is 128 query columns of one KV head: 128/G tokens x the G query
//    heads of the group, so each staged K/V tile serves the whole group;
//  * keys advance 32 at a time (two 16-token blocks), gathered through the
//    block table into LDS — K as [32][head_size] (padded rows), V as the
//    cache's own transposed [head_size][16] block tiles — with the next two
//    blocks loaded into registers while the current ones are used;
//  * each wave owns 32 columns and computes S^T = K Q^T (16x16x32 bf16 MFMA,
//    queries as the B operand held in registers), so the score accumulator
//    of a lane holds 4 keys x 1 column; exactly that layout is the B operand
//    of O^T = V^T P^T, so probabilities never leave the lane, and the column
//    statistics (running max and sum) need no shuffles to rescale O^T;
//  * P enters PV as two bf16 operands (hi = bf16(p), lo = bf16(p - hi)), two
//    MFMAs per tile: a single bf16 rounding of p would move an output that a
//    few keys dominate by up to 2^-8 |v|, beyond the parity tolerance;
//  * causal / window masks are applied only to key tiles that cross a
//    column's boundary; keys past the context are zeroed in V while staging.
//
// Tiles are handed out heaviest-first (the last query tile of a sequence sees
// the most keys), and the KV head is the fastest-varying part of the
// workgroup index so that the tiles of one head land on the same XCD.
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 mfma_bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mfma_bf16x8, a),
                                                  __builtin_bit_cast(mfma_bf16x8, b), c, 0, 0, 0);
}

template <int CK, int D>
struct PrefillShape {
  static constexpr int KT = 64;                   // keys per tile (four 16-token blocks)
  static constexpr int K_LDS = KT * D;            // bf16 elements of one K tile ([64][D], swizzled)
  static constexpr int V_LDS = 4 * D * 16;        // four transposed V block tiles ([D][16], swizzled)
  static constexpr int BUF = K_LDS + V_LDS;       // one stage
  static constexpr int E = CacheElem<CK>::bytes;
  static constexpr int BLK_BYTES = 16 * D * E;    // global bytes of one (block, head) tile
  static constexpr int CHUNKS16 = 4 * BLK_BYTES / 16;       // 16-byte global chunks per tile (K or V)
  static constexpr int CHUNKS = (CHUNKS16 + 255) / 256;     // per thread
};

// LDS bank swizzles (16-byte chunk index XOR a function of the row). A K row
// holds D bf16 = D/8 chunks; the score MFMA reads, per 16-lane group, one
// chunk from each of the rows 8q + 4kt + r (q, r in 0..3): the XOR spreads
// those 16 reads over all 64 banks. A V^T row holds 16 keys = 2 chunks; the
// PV MFMA reads one chunk from 16 consecutive rows: flipping the chunk for
// rows 8..15 separates rows d and d+8.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (D == 128) return (row & 3) | (((row >> 3) & 3) << 2);
  else return ((row >> 1) & 1) | (((row >> 3) & 3) << 1);
}
__device__ __forceinline__ int v_swz(int row) { return (row >> 3) & 1; }

template <int CK, int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillArgs a) {
  using S = PrefillShape<CK, D>;
  constexpr int TQ = 128 / G;  // tokens per tile
  constexpr int DS = D / 32;   // MFMA k-steps over head_size
  constexpr int DT = D / 16;   // 16-row tiles of head_size in O^T
  constexpr int E = S::E;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * S::BUF];
  __shared__ int sh_scan[256];
  __shared__ int sh_found[3];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x % a.num_kv_heads;
  const int t = blockIdx.x / a.num_kv_heads;

  // ---- which (sequence, query tile) this workgroup owns ----
  if (tid == 0) { sh_found[0] = -1; sh_found[1] = 0; sh_found[2] = 0; }
  __syncthreads();
  int running = 0;
  for (int base = 0; base < a.num_seqs; base += 256) {
    const int s = base + tid;
    int n = 0;
    if (s < a.num_seqs) {
      const int ql = a.cu_seqlens[s + 1] - a.cu_seqlens[s];
      n = ql > 1 ? (ql + TQ - 1) / TQ : 0;
    }
    sh_scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = tid >= off ? sh_scan[tid - off] : 0;
      __syncthreads();
      sh_scan[tid] += v;
      __syncthreads();
    }
    const int incl = sh_scan[tid];
    if (n > 0 && t >= running + incl - n && t < running + incl) {
      sh_found[0] = s;
      sh_found[1] = t - (running + incl - n);
      sh_found[2] = n;
    }
    running += sh_scan[255];
    __syncthreads();
    if (sh_found[0] >= 0) break;
  }
  const int s = sh_found[0];
  if (s < 0) return;
  const int qt = sh_found[2] - 1 - sh_found[1];  // heaviest tile first

  const int q0 = a.cu_seqlens[s];
  const int qlen = a.cu_seqlens[s + 1] - q0;
  const int ctx = a.context_lens[s];
  const int tok0 = qt * TQ;
  const int ntok = min(TQ, qlen - tok0);
  const int qpos_first = ctx - qlen + tok0;
  const int qpos_last = qpos_first + ntok - 1;
  const int lo_first = a.window > 0 ? max(0, qpos_first - a.window + 1) : 0;
  const int b_last = (ctx - 1) >> 4;
  const int* bt = a.block_table + (size_t)s * a.bt_stride;

  // ---- queries of this wave's 32 columns as B operands (registers) ----
  u32x4 qf[2][DS];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int col = wave * 32 + ct * 16 + (lane & 15);
    const int tok = col / G, h = col % G;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      if (tok < ntok) {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.query) +
                             ((size_t)(q0 + tok0 + tok) * a.num_heads + g * G + h) * D + ds * 32 +
                             (lane >> 4) * 8;
        qf[ct][ds] = load16(qp);
      } else {
        qf[ct][ds] = u32x4{0, 0, 0, 0};
      }
    }
  }

  f32x4 o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) o[dt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};

  // ---- staging: global (four blocks) -> registers -> LDS ----
  const size_t head_stride = (size_t)a.num_kv_heads * S::BLK_BYTES;
  const uint8_t* kcache = reinterpret_cast<const uint8_t*>(a.k_cache) + (size_t)g * S::BLK_BYTES;
  const uint8_t* vcache = reinterpret_cast<const uint8_t*>(a.v_cache) + (size_t)g * S::BLK_BYTES;
  u32x4 kreg[S::CHUNKS], vreg[S::CHUNKS];

  // Blocks past the context are not read (their chunks stay zero).
  auto load_tile = [&](int j) {
    const int b0 = j >> 4;
#pragma unroll
    for (int r = 0; r < S::CHUNKS; ++r) {
      const int c = tid + 256 * r;                 // 16-byte chunk within the four blocks
      const int blk = c / (S::BLK_BYTES / 16);
      const int off = (c % (S::BLK_BYTES / 16)) * 16;
      if (c < S::CHUNKS16 && b0 + blk <= b_last) {
        const size_t phys = (size_t)bt[b0 + blk];
        kreg[r] = load16(kcache + phys * head_stride + off);
        vreg[r] = load16(vcache + phys * head_stride + off);
      } else {
        kreg[r] = u32x4{0, 0, 0, 0};
        vreg[r] = u32x4{0, 0, 0, 0};
      }
    }
  };
  // K rows keep key order in LDS ([64][D]); V keeps the cache's per-block
  // [D][16] tiles; 16-byte chunks are placed by the bank swizzles. Values of
  // keys past the context are zeroed.
  auto store_tile = [&](int j, uint16_t* buf) {
    uint16_t* ks = buf;
    uint16_t* vs = buf + S::K_LDS;
#pragma unroll
    for (int r = 0; r < S::CHUNKS; ++r) {
      const int c = tid + 256 * r;
      if (c >= S::CHUNKS16) continue;
      const int blk = c / (S::BLK_BYTES / 16);
      const int off = (c % (S::BLK_BYTES / 16)) * 16;  // byte offset inside the block tile
      const int el = off / E;
      const int krow = blk * 16 + el / D, kchunk = (el % D) / 8;
      const int vd = el / 16, vchunk = (el % 16) / 8;
      const int key_base = j + blk * 16 + (el % 16);
      uint16_t* kdst = ks + krow * D;
      uint16_t* vdst = vs + (blk * D + vd) * 16;
      if constexpr (CK == KBF16) {
        *reinterpret_cast<u32x4*>(kdst + 8 * (kchunk ^ k_swz<D>(krow))) = kreg[r];
        u32x4 v = vreg[r];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] &= ((key_base + 2 * e < ctx) ? 0x0000ffffu : 0u) | ((key_base + 2 * e + 1 < ctx) ? 0xffff0000u : 0u);
        *reinterpret_cast<u32x4*>(vdst + 8 * (vchunk ^ v_swz(vd))) = v;
      } else {
        const u32x4 k0 = fp8x8_to_bf16x8(kreg[r][0], kreg[r][1]);
        const u32x4 k1 = fp8x8_to_bf16x8(kreg[r][2], kreg[r][3]);
        *reinterpret_cast<u32x4*>(kdst + 8 * (kchunk ^ k_swz<D>(krow))) = k0;
        *reinterpret_cast<u32x4*>(kdst + 8 * ((kchunk + 1) ^ k_swz<D>(krow))) = k1;
        u32x4 v0 = fp8x8_to_bf16x8(vreg[r][0], vreg[r][1]);
        u32x4 v1 = fp8x8_to_bf16x8(vreg[r][2], vreg[r][3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v0[e] &= ((key_base + 2 * e < ctx) ? 0x0000ffffu : 0u) | ((key_base + 2 * e + 1 < ctx) ? 0xffff0000u : 0u);
          v1[e] &= ((key_base + 8 + 2 * e < ctx) ? 0x0000ffffu : 0u) |
                   ((key_base + 8 + 2 * e + 1 < ctx) ? 0xffff0000u : 0u);
        }
        *reinterpret_cast<u32x4*>(vdst + 8 * (0 ^ v_swz(vd))) = v0;
        *reinterpret_cast<u32x4*>(vdst + 8 * (1 ^ v_swz(vd))) = v1;
      }
    }
  };

  // bf16 caches skip the register staging: each wave copies one block's K
  // rows and V^T tile straight from global memory into LDS (one 16-byte chunk
  // per lane, lane i to byte 16*i of a 1 KiB region), choosing per lane the
  // global chunk that the bank swizzle wants at that LDS position. Blocks past
  // the context re-read the last block; their keys are masked (scores) and
  // zeroed (values) in the masked tiles.
  typedef __attribute__((address_space(3))) void lds_void_t;
  typedef __attribute__((address_space(1))) void glob_void_t;
  auto dma_tile = [&](int j, uint16_t* buf) {
    const int b = min((j >> 4) + wave, b_last);
    const size_t phys = (size_t)bt[b];
    const uint8_t* kb = kcache + phys * head_stride;
    const uint8_t* vb = vcache + phys * head_stride;
    uint16_t* kdst = buf + wave * 16 * D;
    uint16_t* vdst = buf + S::K_LDS + wave * D * 16;
    constexpr int RPR = D / 8;            // 16-byte chunks per K row
    constexpr int ROWS_PER_KB = 64 / RPR;  // K rows per 1 KiB region
    constexpr int REGIONS = 16 * D * 2 / 1024;
#pragma unroll
    for (int n = 0; n < REGIONS; ++n) {
      const int rr = n * ROWS_PER_KB + lane / RPR;
      const int c = (lane % RPR) ^ k_swz<D>(16 * wave + rr);
      __builtin_amdgcn_global_load_lds((glob_void_t*)(kb + rr * (2 * D) + c * 16), (lds_void_t*)(kdst + n * 512),
                                       16, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < REGIONS; ++n) {
      const int d = n * 32 + lane / 2;
      const int c = (lane & 1) ^ v_swz(d);
      __builtin_amdgcn_global_load_lds((glob_void_t*)(vb + d * 32 + c * 16), (lds_void_t*)(vdst + n * 512), 16,
                                       0, 0);
    }
  };

  const int jstart = (lo_first >> 6) << 6;
  const int jend = qpos_last;  // last key any column of the tile can see
  int cur = 0;
  if constexpr (CK == KBF16) {
    dma_tile(jstart, lds);
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    load_tile(jstart);
    store_tile(jstart, lds);
  }
  __syncthreads();

  const int c16 = lane & 15, q4 = lane >> 4;
  const int col_l = wave * 32 + c16;  // column of ct = 0; ct = 1 adds 16
  // Score rows are fed in a permuted key order: in each 32-key step, tile kt
  // row i holds key 8*(i/4) + 4*kt + i%4, so that lane group q ends up with
  // keys 8q..8q+7 — the k-slice PV wants from it, and a contiguous 16-byte
  // run of the transposed V block.
  const int kperm0 = 8 * (c16 >> 2) + (c16 & 3);
  int qpos_c[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) qpos_c[ct] = qpos_first + (col_l + ct * 16) / G;

  // One 64-key tile. MASKED tiles cross a column's causal or window edge or
  // the context end; interior tiles carry no masking code.
  auto tile = [&](auto masked_tag, int j, const uint16_t* ks, const uint16_t* vs) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float ksc[2] = {a.scale_log2, a.scale_log2};  // per 32-key step: this lane group's block
    float vsc[2] = {1.f, 1.f};
    if constexpr (CK == KFP8) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int blk = (j >> 4) + 2 * st + (q4 >> 1);
        if (blk <= b_last) {
          const int phys = bt[blk];
          ksc[st] *= a.k_scale[phys];
          vsc[st] = a.v_scale[phys];
        }
      }
    }
#pragma unroll 1
    for (int st = 0; st < 2; ++st) {  // two 32-key steps
      // ---- S^T = K Q^T : 2 key tiles x 2 column tiles ----
      f32x4 sc[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sc[kt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sc[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int row = 32 * st + kperm0 + 4 * kt;
        const uint16_t* krow = ks + row * D;
        const int sw = k_swz<D>(row);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(krow + 8 * ((4 * ds + q4) ^ sw));
          sc[kt][0] = mfma16x16x32(kf, qf[0][ds], sc[kt][0]);
          sc[kt][1] = mfma16x16x32(kf, qf[1][ds], sc[kt][1]);
        }
      }
      // ---- scale, mask, online softmax per column ----
      const int kbase = j + 32 * st + 8 * q4;  // this lane's keys: kbase + 4*kt + r
      u32x4 ph[2], pl[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        float x[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = sc[kt][ct][r] * ksc[st];
            if constexpr (MASKED) {
              const int kp = kbase + 4 * kt + r;
              const int qpos = qpos_c[ct];
              const bool ok = kp <= qpos && kp < ctx && (a.window <= 0 || kp > qpos - a.window);
              v = ok ? v : -INFINITY;
            }
            x[kt][r] = v;
            tmax = fmaxf(tmax, v);
          }
        tmax = strided_max<16>(tmax);
        // Lazy rescaling: the running max moves only when the tile's max
        // exceeds it by more than 2^8 (p stays below 256 otherwise), so the
        // O^T rescale is rare; the final division uses the same max.
        const bool up = tmax > m[ct] + 8.f;
        if (__any(up)) {
          const float alpha = up ? __builtin_amdgcn_exp2f(m[ct] - tmax) : 1.f;  // 0 when m was -inf
          m[ct] = up ? tmax : m[ct];
          lsum[ct] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            o[dt][ct][0] *= alpha; o[dt][ct][1] *= alpha; o[dt][ct][2] *= alpha; o[dt][ct][3] *= alpha;
          }
        }
        const float base = (m[ct] == -INFINITY) ? 0.f : m[ct];
        float ps = 0.f;
        float pv[2][4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(x[kt][r] - base);
            ps += p;
            pv[kt][r] = (CK == KFP8) ? p * vsc[st] : p;
          }
        lsum[ct] += ps;
        // P^T operand, logical k 8*q4 + e <-> key kbase + e (e = 4*kt + r);
        // p = hi + lo, both bf16
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float a0 = pv[t >> 1][(t & 1) * 2], a1 = pv[t >> 1][(t & 1) * 2 + 1];
          const uint32_t hi = pack_bf16x2(a0, a1);
          ph[ct][t] = hi;
          pl[ct][t] = pack_bf16x2(a0 - bf16_lo(hi), a1 - bf16_hi(hi));
        }
      }
      // ---- O^T += V^T P^T over these 32 keys ----
      // (values of keys past the context may hold anything, even NaN: the
      // masked tiles zero this lane's 8 keys kbase..kbase+7 that are >= ctx)
      uint32_t vmask[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        vmask[t] = (kbase + 2 * t < ctx ? 0x0000ffffu : 0u) | (kbase + 2 * t + 1 < ctx ? 0xffff0000u : 0u);
      (void)vmask;
      const uint16_t* vblk = vs + (2 * st + (q4 >> 1)) * D * 16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 16 + c16;
        u32x4 vf = *reinterpret_cast<const u32x4*>(vblk + d * 16 + 8 * ((q4 & 1) ^ v_swz(d)));
        if constexpr (MASKED && CK == KBF16) {
          vf[0] &= vmask[0]; vf[1] &= vmask[1]; vf[2] &= vmask[2]; vf[3] &= vmask[3];
        }
        o[dt][0] = mfma16x16x32(vf, ph[0], o[dt][0]);
        o[dt][1] = mfma16x16x32(vf, ph[1], o[dt][1]);
        o[dt][0] = mfma16x16x32(vf, pl[0], o[dt][0]);
        o[dt][1] = mfma16x16x32(vf, pl[1], o[dt][1]);
      }
    }
  };

  for (int j = jstart; j <= jend; j += S::KT) {
    const bool more = j + S::KT <= jend;
    if constexpr (CK == KBF16) {
      if (more) dma_tile(j + S::KT, lds + (cur ^ 1) * S::BUF);
    } else {
      if (more) load_tile(j + S::KT);
    }
    const uint16_t* ks = lds + cur * S::BUF;
    const uint16_t* vs = ks + S::K_LDS;
    const bool need_mask = (j + S::KT - 1 > qpos_first) || (a.window > 0 && j < qpos_last - a.window + 1);
    if (need_mask) tile(std::true_type{}, j, ks, vs);
    else tile(std::false_type{}, j, ks, vs);
    if constexpr (CK == KBF16) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies into the other stage are done
    } else {
      if (more) store_tile(j + S::KT, lds + (cur ^ 1) * S::BUF);
    }
    __syncthreads();
    cur ^= 1;
  }

  // ---- normalise and write this wave's columns ----
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const float L = strided_sum<16>(lsum[ct]);
    const float inv = 1.f / L;
    const int col = col_l + ct * 16;
    const int tok = col / G, h = col % G;
    if (tok < ntok) {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) +
                     ((size_t)(q0 + tok0 + tok) * a.num_heads + g * G + h) * D + (lane >> 4) * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint2 w;
        w.x = pack_bf16x2(o[dt][ct][0] * inv, o[dt][ct][1] * inv);
        w.y = pack_bf16x2(o[dt][ct][2] * inv, o[dt][ct][3] * inv);
        *reinterpret_cast<uint2*>(op + dt * 16) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
int prefill_tokens_per_tile(int cache_kind, int group) {
  return cache_kind == KBF16 ? prefill_bf16_tokens_per_tile(group) : 128 / group;
}

bool prefill_supported(int q_kind, int cache_kind, int head_size, int group) {
  if (head_size != 64 && head_size != 128) return false;
  if (!(group == 1 || group == 2 || group == 4 || group == 8 || group == 16)) return false;
  return q_kind == KBF16 && (cache_kind == KBF16 || cache_kind == KFP8);
}

template <int CK, int D, int G>
static hipError_t run_prefill(const PrefillArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)a.num_tiles * (unsigned)a.num_kv_heads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<CK, D, G>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int CK, int D>
static hipError_t run_prefill_g(const PrefillArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return run_prefill<CK, D, 1>(a, st);
    case 2: return run_prefill<CK, D, 2>(a, st);
    case 4: return run_prefill<CK, D, 4>(a, st);
    case 8: return run_prefill<CK, D, 8>(a, st);
    case 16: return run_prefill<CK, D, 16>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, int cache_kind, int head_size, hipStream_t stream) {
  const int G = a.num_heads / a.num_kv_heads;
  if (cache_kind == KBF16) {
    return launch_prefill_bf16(a, head_size, stream);
  } else if (cache_kind == KFP8) {
    if (head_size == 64) return run_prefill_g<KFP8, 64>(a, G, stream);
    if (head_size == 128) return run_prefill_g<KFP8, 128>(a, G, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
