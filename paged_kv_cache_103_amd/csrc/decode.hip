// Paged decode attention for gfx950: one query token per sequence.
//
// What it computes: for each sequence s and query head h, softmax over the
// sequence's cached keys (read through its block table) of scale * q.K,
// times V ("从静态批处理到状态化推理集群", "PagedAttention：把逻辑连续与物理连续分开":
// the kernel reads K/V through the block table). Decode is bandwidth-bound —
// every step re-reads all history K/V ("大模型推理优化学习笔记", "计算密集与访存
// 密集" and "Decode") — so the design aims at streaming each (block, KV head)
// tile from HBM exactly once per step:
//
//  * grid (partition, KV head, sequence): a workgroup owns one contiguous run
//    of `pb` blocks of one sequence and one KV head, and serves all G query
//    heads of that group from the same tile (grouped-query sharing);
//  * the 4 waves of a workgroup take every 4th block of the run; a (block,
//    head) tile is contiguous (K: 16 rows x head_size, V: head_size rows x 16
//    keys), so each wave reads it with 16-byte loads that cover 1 KiB per
//    instruction, and the next block is in flight while this one is computed;
//  * scores: packed-bf16 dot2 (fp32 accumulate) over each lane's 16-byte slice
//    of a key row, then a DPP sum across the lanes of the row;
//  * online softmax per head (running max and sum, rescale of the
//    accumulators when the max grows — the "local max, correction factor"
//    of the online-softmax Q&A in "宣稱省下 106 倍成本…", "中：Kimi K3 的 DCP
//    選擇與 DEP 轉折");
//  * PV: probabilities go through a few bytes of LDS from the key-row lanes
//    to the value-row lanes; the transposed V tile gives bf16 pairs along keys
//    that meet the probability pairs in dot2. A probability is sent as two
//    bf16 numbers (hi = bf16(p), lo = bf16(p - hi)) so that PV keeps about 16
//    significant bits of p: one bf16 rounding of p alone would move an output
//    dominated by a few keys by up to 2^-8 |v|;
//  * the 4 waves merge through LDS; a sequence with several partitions writes
//    (max, sum, unnormalised output) per partition and a second kernel merges
//    them with the same correction factors (flash-decoding split).
//
// fp8 (e4m3fn) caches: bytes are widened to bf16 exactly with the hardware
// conversion; the block's K scale multiplies the score and the V scale the
// probability used in PV (the running sum keeps the unscaled one).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <int CK, int D>
struct DecodeShape {
  static constexpr int E = CacheElem<CK>::bytes;  // bytes per cache element
  static constexpr int EPL = 16 / E;              // elements in a lane's 16-byte slice
  static constexpr int LPR = D * E / 16;          // lanes per K row (one token)
  static constexpr int RPI = 64 / LPR;            // K rows per 1 KiB load
  static constexpr int NI = 16 / RPI;             // loads per tile = tokens (and V rows) per lane
  static constexpr int VR = 64 / E;               // V^T rows (head dims) per 1 KiB load
  static constexpr int TILE = 16 * D * E;         // bytes of one (block, head) tile
  static_assert(LPR >= 4 && LPR <= 64, "unsupported head size / element size");
};

template <typename QT, int CK, int D, int G>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeArgs a) {
  using S = DecodeShape<CK, D>;
  constexpr int NI = S::NI, LPR = S::LPR, RPI = S::RPI, EPL = S::EPL, E = S::E;
  constexpr bool F32 = (CK == KF32);
  // probabilities exchanged through LDS: fp32 for an fp32 cache, bf16 otherwise
  // bf16 probabilities are carried as hi + lo (p = hi + lo to ~2^-16), so
  // the PV products keep nearly fp32 precision while still using dot2
  constexpr int PBYTES = F32 ? 4 : 2;
  constexpr int PLANES = F32 ? 1 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[4][PLANES][G][16 * PBYTES];
  __shared__ float w_m[4][G], w_l[4][G];
  __shared__ float w_o[4][G][D];

  const int part = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

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

  // ---- this lane's query slices (all G heads of the group) ----
  const int dq = (lane % LPR) * EPL;
  constexpr int QW = F32 ? EPL : EPL / 2;  // floats, or packed bf16 pairs
  uint32_t q[G][QW];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const QT* qp = reinterpret_cast<const QT*>(a.query) +
                   ((size_t)qrow * a.num_heads + g * G + h) * D + dq;
#pragma unroll
    for (int j = 0; j < QW; j += 4) {
      u32x4 v = load16(qp + j * (F32 ? 1 : 2));
      q[h][j] = v[0]; q[h][j + 1] = v[1]; q[h][j + 2] = v[2]; q[h][j + 3] = v[3];
    }
  }

  float m[G], lsum[G], acc[NI][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int n = 0; n < NI; ++n) acc[n][h] = 0.f;
  }

  const size_t head_stride = (size_t)a.num_kv_heads * S::TILE;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache) + (size_t)g * S::TILE + lane * 16;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache) + (size_t)g * S::TILE + lane * 16;
  const int* bt = a.block_table + (size_t)s * a.bt_stride;
  const int kk0 = (lane % E) * EPL;  // first key of this lane's V^T slice

  int b = blk0 + wave;
  // K/V tiles are read once per call: nontemporal loads (3.41 -> 3.91 TB/s
  // on 64 sequences of 1K-8K keys, 32/8 heads, bf16)
  u32x4 kr[NI], vr[NI];
  int phys = 0;
  if (b < blk1) {
    phys = bt[b];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      kr[i] = load16_stream(kbase + phys * head_stride + i * 1024);
      vr[i] = load16_stream(vbase + phys * head_stride + i * 1024);
    }
  }
  for (; b < blk1; b += 4) {
    // prefetch the wave's next block while this one is computed
    const int bn = b + 4;
    u32x4 kn[NI], vn[NI];
    int physn = 0;
    if (bn < blk1) {
      physn = bt[bn];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        kn[i] = load16_stream(kbase + physn * head_stride + i * 1024);
        vn[i] = load16_stream(vbase + physn * head_stride + i * 1024);
      }
    }

    // ---- scores of this lane's NI tokens for the G heads ----
    float sc[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (CK == KBF16) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float x = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) x = dot2_bf16(q[h][j], kr[i][j], x);
          sc[i][h] = x;
        }
      } else if constexpr (CK == KFP8) {
        uint32_t kp[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) fp8x4_to_bf16x4(kr[i][j], kp[2 * j], kp[2 * j + 1]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float x = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) x = dot2_bf16(q[h][j], kp[j], x);
          sc[i][h] = x;
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float x = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) x = fmaf(__uint_as_float(q[h][j]), __uint_as_float(kr[i][j]), x);
          sc[i][h] = x;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) sc[i][h] = group_sum<LPR>(sc[i][h]);
    }

    float kscale = a.scale_log2;
    float vscale = 1.f;
    if constexpr (CK == KFP8) {
      kscale *= a.k_scale[phys];
      vscale = a.v_scale[phys];
    }
    const int key0 = b * 16;
    const bool edge = (key0 < lo) || (key0 + 16 > ctx);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int pos = key0 + i * RPI + lane / LPR;
      const bool ok = !edge || (pos >= lo && pos < ctx);
#pragma unroll
      for (int h = 0; h < G; ++h) sc[i][h] = ok ? sc[i][h] * kscale : -INFINITY;
    }

    // ---- online softmax ----
    float p[NI][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) bm = fmaxf(bm, sc[i][h]);
      bm = strided_max<LPR>(bm);
      const float mn = fmaxf(m[h], bm);
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
      m[h] = mn;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        p[i][h] = __builtin_amdgcn_exp2f(sc[i][h] - mn);
        ps += p[i][h];
      }
      lsum[h] = lsum[h] * alpha + ps;
#pragma unroll
      for (int n = 0; n < NI; ++n) acc[n][h] *= alpha;
    }

    // ---- probabilities: key-row lanes -> LDS -> value-row lanes ----
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if ((lane % LPR) == (h % LPR)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int t = i * RPI + lane / LPR;
          const float pv = p[i][h] * vscale;
          if constexpr (F32) {
            reinterpret_cast<float*>(p_lds[wave][0][h])[t] = pv;
          } else {
            const uint16_t hi = f32_to_bf16(pv);
            reinterpret_cast<uint16_t*>(p_lds[wave][0][h])[t] = hi;
            reinterpret_cast<uint16_t*>(p_lds[wave][1][h])[t] = f32_to_bf16(pv - bf16_to_f32(hi));
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();

    // value slices of keys outside [lo, ctx) may hold anything (even NaN):
    // zero them in edge blocks so that a zero probability stays zero
    if (edge) {
#pragma unroll
      for (int n = 0; n < NI; ++n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t mask = 0;
#pragma unroll
          for (int e = 0; e < 4 / E; ++e) {
            // word j holds keys kk0 + j*(4/E) + e, each E bytes wide
            const int pos = key0 + kk0 + j * (4 / E) + e;
            const bool ok = pos >= lo && pos < ctx;
            const uint32_t em = (E == 4) ? 0xffffffffu : (E == 2 ? 0xffffu : 0xffu);
            if (ok) mask |= em << (8 * E * e);
          }
          vr[n][j] &= mask;
        }
      }
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      if constexpr (CK == KBF16) {
        const u32x4 ph = *reinterpret_cast<const u32x4*>(p_lds[wave][0][h] + kk0 * 2);
        const u32x4 pl = *reinterpret_cast<const u32x4*>(p_lds[wave][1][h] + kk0 * 2);
#pragma unroll
        for (int n = 0; n < NI; ++n) {
          float x = acc[n][h];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x = dot2_bf16(ph[j], vr[n][j], x);
            x = dot2_bf16(pl[j], vr[n][j], x);
          }
          acc[n][h] = x;
        }
      } else if constexpr (CK == KFP8) {
        uint32_t ph[8], pl[8];
#pragma unroll
        for (int q4 = 0; q4 < 2; ++q4) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(p_lds[wave][0][h] + 16 * q4);
          const u32x4 c = *reinterpret_cast<const u32x4*>(p_lds[wave][1][h] + 16 * q4);
#pragma unroll
          for (int j = 0; j < 4; ++j) { ph[4 * q4 + j] = a[j]; pl[4 * q4 + j] = c[j]; }
        }
#pragma unroll
        for (int n = 0; n < NI; ++n) {
          float x = acc[n][h];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t v01, v23;
            fp8x4_to_bf16x4(vr[n][j], v01, v23);
            x = dot2_bf16(ph[2 * j], v01, x);
            x = dot2_bf16(pl[2 * j], v01, x);
            x = dot2_bf16(ph[2 * j + 1], v23, x);
            x = dot2_bf16(pl[2 * j + 1], v23, x);
          }
          acc[n][h] = x;
        }
      } else {
        const f32x4 pp = *reinterpret_cast<const f32x4*>(p_lds[wave][0][h] + kk0 * 4);
#pragma unroll
        for (int n = 0; n < NI; ++n) {
          float x = acc[n][h];
#pragma unroll
          for (int j = 0; j < 4; ++j) x = fmaf(pp[j], __uint_as_float(vr[n][j]), x);
          acc[n][h] = x;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();

    phys = physn;
#pragma unroll
    for (int i = 0; i < NI; ++i) { kr[i] = kn[i]; vr[i] = vn[i]; }
  }

  // ---- per-wave totals -> LDS ----
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = strided_sum<LPR>(lsum[h]);
#pragma unroll
    for (int n = 0; n < NI; ++n) acc[n][h] = group_sum<E>(acc[n][h]);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { w_m[wave][h] = m[h]; w_l[wave][h] = lsum[h]; }
  }
  if ((lane % E) == 0) {
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int d = n * S::VR + lane / E;
#pragma unroll
      for (int h = 0; h < G; ++h) w_o[wave][h][d] = acc[n][h];
    }
  }
  __syncthreads();

  // ---- merge the 4 waves; write the output or this partition's summary ----
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
      const float r = O / L;
      if constexpr (sizeof(QT) == 4) {
        reinterpret_cast<float*>(a.out)[((size_t)qrow * a.num_heads + hq) * D + d] = r;
      } else {
        reinterpret_cast<uint16_t*>(a.out)[((size_t)qrow * a.num_heads + hq) * D + d] = f32_to_bf16(r);
      }
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

// One wave per (sequence, query head): exact merge of the partitions'
// summaries, M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L.
template <typename QT, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= a.num_seqs * a.num_heads) return;
  const int s = idx / a.num_heads, hq = idx % a.num_heads;
  int qrow = s;
  if (a.cu_seqlens != nullptr) {
    const int q0 = a.cu_seqlens[s];
    if (a.cu_seqlens[s + 1] - q0 != 1) return;
    qrow = q0;
  }
  const int ctx = a.context_lens[s];
  const int lo = a.window > 0 ? max(0, ctx - a.window) : 0;
  const int nparts = (((ctx - 1) >> 4) - (lo >> 4) + a.pb) / a.pb;
  if (nparts <= 1) return;
  const size_t base = ((size_t)s * a.num_heads + hq) * a.max_parts;
  const float* ml = a.part_ml + base * 2;
  const float* po = a.part_o + base * D;

  float M = -INFINITY;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ml[2 * p]);
  M = strided_max<1>(M);

  constexpr int DL = D / 64;
  float o[DL];
#pragma unroll
  for (int k = 0; k < DL; ++k) o[k] = 0.f;
  float L = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    const int p = p0 + lane;
    const float w = (p < nparts) ? __builtin_amdgcn_exp2f(ml[2 * p] - M) : 0.f;
    if (p < nparts) L += ml[2 * p + 1] * w;
    const int cnt = min(64, nparts - p0);
    // eight partitions' rows in flight at a time
    for (int j0 = 0; j0 < cnt; j0 += 8) {
      float v[8][DL];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* row = po + (size_t)(p0 + j0 + u) * D;
#pragma unroll
        for (int k = 0; k < DL; ++k) v[u][k] = (j0 + u < cnt) ? row[k * 64 + lane] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), (j0 + u) & 63));
#pragma unroll
        for (int k = 0; k < DL; ++k) o[k] = fmaf(wj, v[u][k], o[k]);
      }
    }
  }
  L = strided_sum<1>(L);
  const float inv = 1.f / L;
#pragma unroll
  for (int k = 0; k < DL; ++k) {
    const size_t oi = ((size_t)qrow * a.num_heads + hq) * D + k * 64 + lane;
    if constexpr (sizeof(QT) == 4) {
      reinterpret_cast<float*>(a.out)[oi] = o[k] * inv;
    } else {
      reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(o[k] * inv);
    }
  }
}

// ---------------------------------------------------------------------------
// host side: plan and dispatch
// ---------------------------------------------------------------------------
// Compute units of the calling thread's current device, asked once per
// device (the grids of the split plans are sized by it).
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int device_lds_per_cu() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess || n <= 0)
    return 0;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Which decode kernel serves a request: the matrix-core kernel for bf16/fp8
// caches (any group up to 16 query heads per KV head), the VALU kernel for
// fp32 caches (and for every cache type when the caller asks for it:
// pa_decode_valu, kept for side-by-side measurement).
bool decode_uses_mfma(int q_kind, int cache_kind, int group) {
  return q_kind == KBF16 && (cache_kind == KBF16 || cache_kind == KFP8) && group <= 16;
}

DecodePlan plan_decode(int num_seqs, int max_context_len, int num_heads, int num_kv_heads, int head_size,
                       int q_kind, int cache_kind, int sliding_window, bool force_valu) {
  DecodePlan plan{};
  const int G = std::max(1, num_heads / std::max(1, num_kv_heads));
  // (the matrix-core kernel keeps per-sequence prefix sums in LDS: up to
  // kMfmaMaxSeqs sequences per launch; pa_decode splits larger batches, other
  // callers' larger batches take the VALU kernel)
  int max_blocks = (max_context_len + 15) / 16;
  if (sliding_window > 0) max_blocks = std::min(max_blocks, (sliding_window + 15) / 16 + 1);
  if (max_blocks < 1) max_blocks = 1;
  if (!force_valu && decode_uses_mfma(q_kind, cache_kind, G) && num_seqs <= kMfmaMaxSeqs) {
    // two resident workgroups of four waves per CU
    plan.split_waves = 8 * device_cu_count();
    plan.pb = 0;
    plan.max_parts = 0;
    // every (sequence, KV head) stream at most 16 blocks (a short context or
    // a sliding window): one wave per stream finishes it in place, with no
    // summaries and no merge launch; a split would leave each wave a pair or
    // two and cost more in summaries, merge and launch than it saves
    plan.one_per_stream = max_blocks <= kOnePerStreamMaxBlocks ? 1 : 0;
    return plan;
  }
  // VALU kernel: a workgroup per (sequence, KV head, partition of pb blocks);
  // the largest partition (16..256 blocks) that still leaves about 16 work
  // items per CU, assuming contexts average half the maximum.
  const long long target = 4096;
  int pb = 16;
  for (int cand = 256; cand >= 16; cand /= 2) {
    const long long half = (max_blocks + 1) / 2;
    const long long items = (long long)num_seqs * num_kv_heads * ((half + cand - 1) / cand);
    if (items >= target) { pb = cand; break; }
  }
  plan.pb = pb;
  plan.max_parts = (max_blocks + pb - 1) / pb;
  plan.split_waves = 0;
  return plan;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(const DecodePlan& plan, int num_seqs, int num_heads, int num_kv_heads,
                              int head_size) {
  if (plan.split_waves > 0 && plan.one_per_stream) return 0;
  if (plan.split_waves > 0) {
    const int G = num_heads / num_kv_heads;
    const size_t slots = (size_t)plan.split_waves + (size_t)num_seqs * num_kv_heads;
    return align256((size_t)(num_seqs + 2) * sizeof(int)) + align256(slots * G * head_size * sizeof(float)) +
           slots * G * 2 * sizeof(float);
  }
  if (plan.max_parts <= 1) return 0;
  const size_t slots = (size_t)num_seqs * num_heads * plan.max_parts;
  return slots * head_size * sizeof(float) + slots * 2 * sizeof(float);
}

size_t decode_shared_prefix_workspace_bytes(int num_seqs, int num_groups, int num_heads, int num_kv_heads,
                                            int head_size) {
  // records of 16 query columns; at most 2 * num_seqs streams per KV head
  const size_t slots = (size_t)(8 * device_cu_count()) + (size_t)2 * num_seqs * num_kv_heads;
  (void)num_heads;
  return align256((size_t)shared_prefix_meta_ints(num_seqs, num_groups) * sizeof(int)) +
         align256(slots * 16 * head_size * sizeof(float)) + slots * 16 * 2 * sizeof(float);
}

static bool group_ok(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

bool decode_supported(int q_kind, int cache_kind, int head_size, int group) {
  if (head_size != 64 && head_size != 128) return false;
  if (!group_ok(group)) return false;
  return (q_kind == KF32 && cache_kind == KF32) || (q_kind == KBF16 && cache_kind == KBF16) ||
         (q_kind == KBF16 && cache_kind == KFP8);
}

template <typename QT, int CK, int D, int G>
static hipError_t run_decode(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<QT, CK, D, G>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename QT, int D>
static hipError_t run_merge(const DecodeArgs& a, hipStream_t st) {
  const int waves = a.num_seqs * a.num_heads;
  hipLaunchKernelGGL((decode_merge_kernel<QT, D>), dim3((waves + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename QT, int CK, int D>
static hipError_t run_decode_g(const DecodeArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return run_decode<QT, CK, D, 1>(a, st);
    case 2: return run_decode<QT, CK, D, 2>(a, st);
    case 4: return run_decode<QT, CK, D, 4>(a, st);
    case 8: return run_decode<QT, CK, D, 8>(a, st);
    case 16: return run_decode<QT, CK, D, 16>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename QT, int CK>
static hipError_t run_decode_d(const DecodeArgs& a, int D, int G, hipStream_t st) {
  if (D == 64) return run_decode_g<QT, CK, 64>(a, G, st);
  if (D == 128) return run_decode_g<QT, CK, 128>(a, G, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int cache_kind, int head_size, hipStream_t st);


hipError_t launch_decode(const DecodeArgs& a, int q_kind, int cache_kind, int head_size,
                         hipStream_t stream) {
  const int G = a.num_heads / a.num_kv_heads;
  hipError_t e;
  if (a.split_waves > 0) return launch_decode_mfma(a, cache_kind, head_size, stream);
  if (q_kind == KF32 && cache_kind == KF32) e = run_decode_d<float, KF32>(a, head_size, G, stream);
  else if (q_kind == KBF16 && cache_kind == KBF16) e = run_decode_d<uint16_t, KBF16>(a, head_size, G, stream);
  else if (q_kind == KBF16 && cache_kind == KFP8) e = run_decode_d<uint16_t, KFP8>(a, head_size, G, stream);
  else return hipErrorInvalidValue;
  if (e != hipSuccess || a.max_parts <= 1) return e;
  if (q_kind == KF32) return head_size == 64 ? run_merge<float, 64>(a, stream) : run_merge<float, 128>(a, stream);
  return head_size == 64 ? run_merge<uint16_t, 64>(a, stream) : run_merge<uint16_t, 128>(a, stream);
}

}  // namespace pa
