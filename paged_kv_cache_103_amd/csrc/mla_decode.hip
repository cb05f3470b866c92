// Decode over a paged latent (MLA) cache on matrix cores (pa_mla_decode,
// include/pa.h).
//
// Multi-head latent attention keeps one row c per token for every head; with
// the up-projections folded into the queries each head scores its absorbed
// query directly against c, and the values are the rows' first 512 elements
// ("宣稱省下 106 倍成本…", "MLA(Multi-head Latent Attention)是什麼、為什麼讓 TP
// 沒效率" and its Q&As). One row read from memory therefore serves all H
// heads: per 32 keys the work is an (H x dk)(dk x 32) score product and an
// (H x 32)(32 x 512) value product, dense enough that the rows have to be
// read once per workgroup and shared through LDS.
//
// Workgroup: 8 waves, one per CU (the LDS holds a 3-slot ring of 32-key row
// tiles plus a transposed value tile). Wave w serves the 16 heads of head
// group w / NDP and the 512 / NDP output dims of part w % NDP (NDP = 128 / H:
// with fewer heads the value dims are split so that every wave has work;
// the score product is then repeated by the waves of a head group).
// Per step of 32 keys (two blocks):
//  * the tile arrives by global->LDS copies issued two steps ahead, row
//    major with a per-row XOR swizzle of its 16-byte chunks (conflict-free
//    score-operand reads); the copies are nontemporal, as every row is read
//    once per call (measured: 16 heads 0.35 -> 0.26 ms, 128 heads ~5% faster
//    on 64 sequences of 4K-32K keys);
//  * one pass by all 512 threads writes the value part again, transposed and
//    converted to fp16 ([512 dims][32 keys], 64-byte rows with a chunk
//    swizzle), zeroing keys past the context: the value product needs 8
//    consecutive keys of one dim per lane, the score product 8 consecutive
//    dims of one key;
//  * scores S^T = C Q^T on 16x16x32 bf16 MFMAs (queries held in registers as
//    the B operand, keys in the permuted row order that makes each lane's
//    score accumulator its own P^T operand), online softmax with lazy
//    rescaling, O^T += V^T P^T on 16x16x32 fp16 MFMAs with P scaled by 2^7.
//    (128 heads take mla_decode_wide below: the same steps, the value
//    product on 32x32 tiles, one barrier per step.)
//    A value beyond fp16's range (65504) becomes infinity in the tile and
//    leaves inf or NaN in the outputs of every head; the merge kernel finds
//    such rows and computes them again exactly (fp32, from the bf16 rows), so
//    every finite cached value is in the call's domain.
// The concatenated (sequence, pair of blocks) streams are split evenly over
// the workgroups; a sequence covered by one workgroup is finished in place,
// others leave (max, sum, unnormalised output) summaries that a second kernel
// merges exactly.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int MLA_DV = 512;
constexpr int MLA_VT_ROW = 64;  // bytes per transposed value row: 32 keys in fp16
// 16-byte chunk c (8 keys) of transposed value row d sits at chunk
// c ^ vt_swizzle(d): 16 consecutive rows read at one chunk column hit 16
// distinct bank groups.
__device__ __forceinline__ int vt_swizzle(int d) { return (d >> 2) & 3; }
__device__ __forceinline__ uint32_t vt_offset(int d, int chunk) {
  return (uint32_t)(d * MLA_VT_ROW + 16 * (chunk ^ vt_swizzle(d)));
}

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                  0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ uint32_t f16x2_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}

// Chunk swizzle of a tile row (key 0..31 of the step): 16 lanes reading one
// chunk column of 16 permuted keys hit 16 distinct 16-byte bank groups.
template <int DK>
__device__ __forceinline__ int row_swizzle(int key) {
  if constexpr (DK == 576) return ((key >> 1) & 1) | (((key >> 3) & 3) << 1);  // rows of 72 chunks
  else return (key & 3) | (((key >> 3) & 3) << 2);                              // rows of 64 chunks
}




}  // namespace

// Units of work of every sequence (pairs of blocks, UNIT = 2, or blocks,
// UNIT = 1) and their exclusive prefix sums, by all NT threads of the
// workgroup, into psum[0..num_seqs]; returns the total.
template <int NT, int UNIT>
__device__ __forceinline__ int unit_prefix_sums(const MlaArgs& a, int* psum, int* scan) {
  const int tid = threadIdx.x, NS = a.num_seqs;
  int running = 0;
  for (int base = 0; base < NS; base += NT) {
    const int i = base + tid;
    const int ctx = i < NS ? a.context_lens[i] : 0;
    const int nb = ctx > 0 ? (ctx + 15) >> 4 : 0;
    const int n = UNIT == 2 ? (nb + 1) >> 1 : nb;
    scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    if (i < NS) psum[i] = running + scan[tid] - n;
    running += scan[NT - 1];
    __syncthreads();
  }
  if (tid == 0) psum[NS] = running;
  __syncthreads();
  return psum[NS];
}

// For the merge: units per worker and the prefix sums (workgroup 0).
template <int NT>
__device__ __forceinline__ void write_meta(const MlaArgs& a, const int* psum, int C) {
  if (blockIdx.x != 0) return;
  if (threadIdx.x == 0) a.meta[0] = C;
  for (int i = threadIdx.x; i <= a.num_seqs; i += NT) a.meta[1 + i] = psum[i];
}

template <int DK, int NW>
struct MlaShape {
  static constexpr int NT = 64 * NW;
  static constexpr int ROWB = DK * 2;            // bytes of one cached row
  static constexpr int BLKB = 16 * ROWB;         // bytes of one block
  static constexpr int TILEB = 32 * ROWB;        // bytes of one 32-key tile
  static constexpr int PIECES = TILEB / 1024;    // 1 KiB copies per tile (36 or 32)
  static constexpr int MAXP = (PIECES + NW - 1) / NW;  // copies per wave
  static constexpr int KS = DK / 32;             // score k-steps
  static constexpr int SLOTS = 3;
  static constexpr int TITEMS = 8 * (MLA_DV / 8);  // transposition items: (key quad, 8-dim chunk)
};

constexpr int kMlaMaxSeqs = 2048;

// NW waves; each wave serves HG groups of 16 heads (the groups share every
// LDS operand fragment) and DVW of the 512 value dims.
template <int DK, int H, int NW, int HG>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void mla_decode_split(MlaArgs a) {
  using S = MlaShape<DK, NW>;
  constexpr int NT = S::NT;
  constexpr int NHG = H / (16 * HG);   // head groups of the workgroup
  static_assert(NHG >= 1 && NW % NHG == 0, "waves must cover the heads");
  constexpr int NDP = NW / NHG;        // value-dim parts
  constexpr int DVW = MLA_DV / NDP;    // value dims per wave
  constexpr int DTW = DVW / 16;        // 16-dim output tiles per wave
  __shared__ __attribute__((aligned(16))) uint8_t ring[S::SLOTS * S::TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t vt[MLA_DV * MLA_VT_ROW];
  __shared__ int psum[kMlaMaxSeqs + 1];
  __shared__ int scan[NT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, q4 = lane >> 4;
  const int hg = wave / NDP, dp = wave % NDP;
  const int NS = a.num_seqs;

  const int T = unit_prefix_sums<NT, 2>(a, psum, scan);
  const int C = max(1, (T + (int)gridDim.x - 1) / (int)gridDim.x);
  write_meta<NT>(a, psum, C);

  // ---- per-lane constant offsets ----
  // copies: piece k of a tile = bytes [1024 k, 1024 k + 1024), wholly inside
  // block k / (PIECES / 2); this lane's source offset inside that block
  auto src_off = [&](int k, int ln) {  // (unsigned: division by a constant is a multiply)
    const uint32_t P = 1024u * (uint32_t)k + 16u * (uint32_t)ln;
    const uint32_t row = P / (uint32_t)S::ROWB, pch = (P - row * (uint32_t)S::ROWB) >> 4;
    return (row & 15u) * (uint32_t)S::ROWB + 16u * (pch ^ (uint32_t)row_swizzle<DK>((int)row));
  };
  const int npieces = (S::PIECES - wave + NW - 1) / NW;  // uniform per wave
  const uint32_t ring_lds = lds_addr(ring), vt_lds = lds_addr(vt);
  // score operand rows: tile kt, MFMA row c16 holds key 8 (c16 / 4) + 4 kt + c16 % 4
  // (addresses computed in the loop); value operand rows: dim dp * DVW +
  // 16 dt + c16, keys 8 q4 .. 8 q4 + 7

  const uint8_t* cache = reinterpret_cast<const uint8_t*>(a.cache);
  const long long x_end = min<long long>((long long)(blockIdx.x + 1) * C, T);
  long long x = (long long)blockIdx.x * C;
  while (x < x_end) {
    // sequence holding pair x: last s with psum[s] <= x (uniform)
    int lo = 0, hi = NS - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (psum[mid] <= x) lo = mid;
      else hi = mid - 1;
    }
    const int s = __builtin_amdgcn_readfirstlane(lo);
    const int sp0 = __builtin_amdgcn_readfirstlane(psum[s]);
    const int np = psum[s + 1] - sp0;
    const int p0 = (int)(x - sp0);
    const int p1 = (int)(min<long long>(x_end, (long long)sp0 + np) - sp0);
    const int n = p1 - p0;
    // uniform metadata by scalar loads (constant address space): a vector
    // load would make the compiler wait for every copy in flight
    typedef __attribute__((address_space(4))) const int cint;
    const int ctx = ((const cint*)a.context_lens)[s];
    const int nblk = (ctx + 15) >> 4;
    const cint* bt = (const cint*)(a.block_table + (size_t)s * a.bt_stride);

    // queries of this wave's heads (B operand of the score product)
    u32x4 qf[HG][S::KS];
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.query) +
                          ((size_t)s * H + 16 * (HG * hg + g) + c16) * S::ROWB + 16 * q4;
#pragma unroll
      for (int j = 0; j < S::KS; ++j) qf[g][j] = load16(qp + 64 * j);
    }
    f32x4 o[HG][DTW];
#pragma unroll
    for (int g = 0; g < HG; ++g)
#pragma unroll
      for (int t = 0; t < DTW; ++t) o[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m[HG], lsum[HG];
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      m[g] = -INFINITY;
      lsum[g] = 0.f;
    }

    // block ids of the segment's pair i (scalar loads)
    auto pair_blocks = [&](int i, int& b0, int& b1) {
      const int pb = 2 * (p0 + i);
      b0 = bt[pb];
      b1 = bt[min(pb + 1, nblk - 1)];  // (a last odd block pairs with itself)
    };
    auto issue = [&](int i, int ln, int b0, int b1) {  // copies of the segment's pair i into slot i % 3
      const uint32_t slot = ring_lds + (uint32_t)((i % S::SLOTS) * S::TILEB);
#pragma unroll
      for (int c = 0; c < S::MAXP; ++c) {
        if (c < npieces) {
          const int k = wave + NW * c;
          const int blk = k < S::PIECES / 2 ? b0 : b1;
          copy16_to_lds<true>(cache + (size_t)(uint32_t)blk * S::BLKB, src_off(k, ln), slot + 1024u * (uint32_t)k);
        }
      }
    };
    // the queries have landed before any copy is issued: the compiler cannot
    // count the copies, and a wait it placed for the queries inside the loop
    // would drain every copy in flight each step
    wait_vmcnt<0>();
    int b0, b1;
    pair_blocks(0, b0, b1);
    issue(0, H >= 128 ? lane_id_here() : lane, b0, b1);
    if (n > 1) {
      pair_blocks(1, b0, b1);
      issue(1, H >= 128 ? lane_id_here() : lane, b0, b1);
    }
    // the block ids of the next pair to copy are loaded one step ahead
    if (n > 2) pair_blocks(2, b0, b1);

    for (int i = 0; i < n; ++i) {
      // the copies of pair i have landed (those of pair i + 1 may be in flight)
      if (i + 1 < n) {
        if (npieces == S::MAXP) wait_vmcnt<S::MAXP>();
        else wait_vmcnt<S::MAXP - 1>();
      } else {
        wait_vmcnt<0>();
      }
      barrier_keep_loads();  // every wave is done with pair i - 1
      // with 128 heads the registers are full: lane-derived addresses are
      // recomputed once per step (see lane_id_here) instead of kept live
      const int ln = H >= 128 ? lane_id_here() : lane;
      if (i + 2 < n) {
        issue(i + 2, ln, b0, b1);
        if (i + 3 < n) pair_blocks(i + 3, b0, b1);
      }
      const int key0 = 32 * (p0 + i);
      const int kend = ctx - key0;  // keys of this tile at or past kend are masked
      const uint32_t slot = ring_lds + (uint32_t)((i % S::SLOTS) * S::TILEB);

      // ---- transposed fp16 value tile: item = (key quad tq, 8-dim chunk tc);
      // done after the score product's reads are issued, so that its reads
      // wait behind the last score MFMAs ----
      constexpr int TI = S::TITEMS / NT;  // items per thread
      static_assert(S::TITEMS % NT == 0, "whole items per thread");
      u32x4 th[TI][4];  // th[c][t][w]: bf16, then fp16, pair (dims 2w, 2w+1) of key 4 tq + t
      auto transpose_load = [&]() {
#pragma unroll
        for (int c = 0; c < TI; ++c) {
          const int it = NT * c + 64 * wave + ln;
          const int tq = it & 7, tc = it >> 3;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int key = 4 * tq + t;
            th[c][t] = lds_read16(slot + (uint32_t)(key * S::ROWB + 16 * (tc ^ row_swizzle<DK>(key))));
          }
        }
      };
      auto transpose_store = [&]() {
#pragma unroll
        for (int c = 0; c < TI; ++c) {
          const int it = NT * c + 64 * wave + ln;
          const int tq = it & 7, tc = it >> 3;
          u32x4 (&h)[4] = th[c];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t keep = 4 * tq + t < kend ? 0xffffffffu : 0u;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint32_t b = h[t][w];
              h[t][w] = f16x2_bits(__uint_as_float(b << 16), __uint_as_float(b & 0xffff0000u)) & keep;
            }
          }
#pragma unroll
          for (int d = 0; d < 8; ++d) {
            // dim 8 tc + d: keys 4 tq .. 4 tq + 3
            const int w = d >> 1;
            const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
            const uint32_t lo2 = __builtin_amdgcn_perm(h[1][w], h[0][w], sel);
            const uint32_t hi2 = __builtin_amdgcn_perm(h[3][w], h[2][w], sel);
            lds_write8(vt_lds + vt_offset(8 * tc + d, tq >> 1) + 8 * (tq & 1), lo2, hi2);
          }
        }
      };

      // ---- scores S^T: per head group, 2 tiles of 16 permuted keys x 16 heads ----
      // Operand chunk of k-step j: (4 j + rq) ^ swz. The swizzle only touches
      // the low NB * 4 chunks' bits, so the address is one of NB per-lane
      // bases plus a constant: bases[j % NB] + 64 NB (j / NB) bytes.
      constexpr int NB = DK == 576 ? 2 : 4;
      uint32_t kb[2][NB];
      {
        const int r16 = ln & 15, rq = ln >> 4;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int key = 8 * (r16 >> 2) + 4 * kt + (r16 & 3);
          const int swz = row_swizzle<DK>(key);
#pragma unroll
          for (int b = 0; b < NB; ++b)
            kb[kt][b] = slot + (uint32_t)(key * S::ROWB + 16 * (((b << 2) | rq) ^ swz));
        }
      }
      f32x4 st[HG][2];
#pragma unroll
      for (int g = 0; g < HG; ++g) st[g][0] = st[g][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      // k-step j of key tile kt is read PD reads ahead of its MFMAs
      constexpr int NKR = 2 * S::KS, PD = 4;
      auto kread = [&](int r) {
        const int j = r >> 1, kt = r & 1;
        return lds_read16(kb[kt][j % NB] + (uint32_t)(64 * NB * (j / NB)));
      };
      __builtin_amdgcn_sched_barrier(0);
      u32x4 kbuf[PD];
#pragma unroll
      for (int r = 0; r < PD; ++r) kbuf[r] = kread(r);
#pragma unroll
      for (int r = 0; r < NKR; ++r) {
        const u32x4 kf = kbuf[r % PD];
        if (r + PD < NKR) kbuf[r % PD] = kread(r + PD);
#pragma unroll
        for (int g = 0; g < HG; ++g) st[g][r & 1] = mfma_bf16(kf, qf[g][r >> 1], st[g][r & 1]);
      }
      transpose_load();
      // keep PD reads in flight: reads, then (MFMAs of one read, next read);
      // the transposition's reads go out behind the last score reads
      __builtin_amdgcn_sched_group_barrier(0x100, PD, 0);
#pragma unroll
      for (int r = 0; r < NKR - PD; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, HG, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * TI, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, HG * PD, 0);
      __builtin_amdgcn_sched_barrier(0);
      transpose_store();
      u32x4 pf[HG];
#pragma unroll
      for (int g = 0; g < HG; ++g) {
        // this lane's keys: 8 q4 + 4 kt + r of the tile
        float xv[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = st[g][kt][r] * a.scale_log2;
            v = (8 * q4 + 4 * kt + r < kend) ? v : -INFINITY;
            xv[kt][r] = v;
            tmax = fmaxf(tmax, v);
          }
        tmax = strided_max<16>(tmax);  // key 0 of the tile is always valid
        const bool up = tmax > m[g] + 8.f;
        if (__any(up)) {
          const float alpha = up ? __builtin_amdgcn_exp2f(m[g] - tmax) : 1.f;
          m[g] = up ? tmax : m[g];
          lsum[g] *= alpha;
#pragma unroll
          for (int t = 0; t < DTW; ++t) {
            o[g][t][0] *= alpha; o[g][t][1] *= alpha; o[g][t][2] *= alpha; o[g][t][3] *= alpha;
          }
        }
        // p scaled by 2^7 (at most 2^15): fp16 keeps small weights normal
        const float mb = m[g] - 7.f;
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(xv[e >> 2][e & 3] - mb);
          lsum[g] += pv[e];
        }
        pf[g][0] = f16x2_bits(pv[0], pv[1]);
        pf[g][1] = f16x2_bits(pv[2], pv[3]);
        pf[g][2] = f16x2_bits(pv[4], pv[5]);
        pf[g][3] = f16x2_bits(pv[6], pv[7]);
      }

      barrier_keep_loads();  // the transposed value tile is complete
      // ---- O^T += V^T P^T ----
      const uint32_t pv_base = vt_lds + vt_offset(dp * DVW + (ln & 15), ln >> 4);
      // (value fragments read VD ahead of their MFMAs; rows 16 t apart keep
      // the swizzle)
      constexpr int VD = 4;
      u32x4 vbuf[VD];
#pragma unroll
      for (int t = 0; t < VD && t < DTW; ++t) vbuf[t] = lds_read16(pv_base + (uint32_t)(16 * t * MLA_VT_ROW));
#pragma unroll
      for (int t = 0; t < DTW; ++t) {
        const u32x4 vf = vbuf[t % VD];
        if (t + VD < DTW) vbuf[t % VD] = lds_read16(pv_base + (uint32_t)(16 * (t + VD) * MLA_VT_ROW));
#pragma unroll
        for (int g = 0; g < HG; ++g) o[g][t] = mfma_f16(vf, pf[g], o[g][t]);
      }
      if constexpr (DTW > VD) {
        __builtin_amdgcn_sched_group_barrier(0x100, VD, 0);
#pragma unroll
        for (int t = 0; t < DTW - VD; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, HG, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, HG * VD, 0);
      }
    }
    // ---- result of the segment ----
    const bool single = (sp0 / C) == ((sp0 + np - 1) / C);
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      const float L = strided_sum<16>(lsum[g]);
      const int head = 16 * (HG * hg + g) + c16;
      if (single) {
        const float inv = 1.f / L;
        uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((size_t)s * H + head) * MLA_DV + dp * DVW + 4 * q4;
#pragma unroll
        for (int t = 0; t < DTW; ++t) {
          uint2 w;
          w.x = pack_bf16x2(o[g][t][0] * inv, o[g][t][1] * inv);
          w.y = pack_bf16x2(o[g][t][2] * inv, o[g][t][3] * inv);
          *reinterpret_cast<uint2*>(op + 16 * t) = w;
        }
      } else {
        const size_t rec = (size_t)(blockIdx.x + s) * H + head;
        float* op = a.part_o + rec * MLA_DV + dp * DVW + 4 * q4;
#pragma unroll
        for (int t = 0; t < DTW; ++t) *reinterpret_cast<f32x4*>(op + 16 * t) = o[g][t];
        if (dp == 0 && q4 == 0) {
          a.part_ml[rec * 2] = m[g] - 7.f;
          a.part_ml[rec * 2 + 1] = L;
        }
      }
    }
    barrier_keep_loads();  // the ring is reused by the next segment
    x = (long long)sp0 + p1;
  }
}

// ---- 128 heads: one barrier per step, the value product a step behind ----
//
// Per step i of 32 keys, after the step's one barrier: the value product of
// tile i - 1 (32x32x16 fp16 tiles of 32 heads x 256 dims per wave, its
// weights P and rescale factors left in LDS by the waves that scored those
// heads), with the copies of tile i + 1 (a ring of two tile slots) issued
// between its MFMAs; the score product of tile i (16 heads per wave, as
// above) with the transposition of tile i's values; the softmax of tile i,
// whose P^T rows and rescale factors go to LDS. The transposed values, P and the rescale
// factors are double-buffered by step parity, so that nothing written in
// step i is read before the next barrier. The prefix sums live in the ring
// during setup only: a workgroup finds its first sequence by them and then
// walks the sequences by their context lengths.
template <int DK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_decode_wide(MlaArgs a) {
  using S = MlaShape<DK, 8>;
  constexpr int H = 128, NW = 8, NT = 512, WDT = 8;
  static_assert(S::TITEMS == NT, "one transposition item per thread");
  static_assert((kMlaMaxSeqs + 1 + NT) * 4 <= 2 * S::TILEB, "setup arrays fit the ring");
  __shared__ __attribute__((aligned(16))) uint8_t ring[2 * S::TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t vt[2][MLA_DV * MLA_VT_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][H * 64];  // P^T rows (heads) of 32 fp16 keys
  __shared__ float alpha_sh[2][H];  // per head: the rescale of the step's P
  __shared__ float lsum_sh[H];      // per head: the segment's sum

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, q4 = lane >> 4;
  const int NS = a.num_seqs;
  typedef __attribute__((address_space(4))) const int cint;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  typedef __attribute__((address_space(3))) const u32x4 lds_cu32x4;

  long long x, x_end;
  int s = 0, sp0 = 0, C;
  {
    int* psum = reinterpret_cast<int*>(ring);
    int* scan = psum + kMlaMaxSeqs + 1;
    const int T = unit_prefix_sums<NT, 2>(a, psum, scan);
    C = max(1, (T + (int)gridDim.x - 1) / (int)gridDim.x);
    write_meta<NT>(a, psum, C);
    x = (long long)blockIdx.x * C;
    x_end = min<long long>((long long)(blockIdx.x + 1) * C, T);
    if (x < x_end) {  // first sequence: last s with psum[s] <= x
      int lo = 0, hi = NS - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (psum[mid] <= x) lo = mid;
        else hi = mid - 1;
      }
      s = __builtin_amdgcn_readfirstlane(lo);
      sp0 = __builtin_amdgcn_readfirstlane(psum[s]);
    }
    __syncthreads();  // the ring is free from here on
  }
  const int npieces = (S::PIECES - wave + NW - 1) / NW;  // uniform per wave
  const uint32_t ring_lds = lds_addr(ring), vt_lds = lds_addr(vt), pb_lds = lds_addr(pbuf);
  auto src_off = [&](int k, int ln) {
    const uint32_t P = 1024u * (uint32_t)k + 16u * (uint32_t)ln;
    const uint32_t row = P / (uint32_t)S::ROWB, pch = (P - row * (uint32_t)S::ROWB) >> 4;
    return (row & 15u) * (uint32_t)S::ROWB + 16u * (pch ^ (uint32_t)row_swizzle<DK>((int)row));
  };
  const uint8_t* cache = reinterpret_cast<const uint8_t*>(a.cache);

  while (x < x_end && s < NS) {
    // pairs of sequence s, as the prefix sums count them (x lies in
    // [sp0, sp0 + np) of the first non-empty one from s on)
    const int cx = ((const cint*)a.context_lens)[s];
    const int np = cx > 0 ? (((cx + 15) >> 4) + 1) >> 1 : 0;
    if (np == 0) {
      ++s;
      continue;
    }
    const int p0 = (int)(x - sp0);
    const int p1 = (int)(min<long long>(x_end, (long long)sp0 + np) - sp0);
    const int n = p1 - p0;
    const int ctx = ((const cint*)a.context_lens)[s];
    const int nblk = (ctx + 15) >> 4;
    const cint* bt = (const cint*)(a.block_table + (size_t)s * a.bt_stride);

    // queries of this wave's 16 heads (B operand of the score product)
    u32x4 qf[S::KS];
    {
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.query) + ((size_t)s * H + 16 * wave + c16) * S::ROWB +
                          16 * q4;
#pragma unroll
      for (int j = 0; j < S::KS; ++j) qf[j] = load16(qp + 64 * j);
    }
    f32x16 ow[WDT];  // dims 256 (wave / 4) + 32 t .. of heads 32 (wave % 4) ..
#pragma unroll
    for (int t = 0; t < WDT; ++t) ow[t] = f32x16{};
    float m = -INFINITY, lsum = 0.f;

    auto pair_blocks = [&](int i, int& b0, int& b1) {
      const int pb = 2 * (p0 + i);
      b0 = bt[pb];
      b1 = bt[min(pb + 1, nblk - 1)];  // (a last odd block pairs with itself)
    };
    // copy c of this wave's share of the segment's pair i, into slot i % 2
    auto copy_piece = [&](int i, int c, int ln, int b0, int b1) __attribute__((always_inline)) {
      if (c < npieces) {
        const uint32_t slot = ring_lds + (uint32_t)((i & 1) * S::TILEB);
        const int k = wave + NW * c;
        const int blk = k < S::PIECES / 2 ? b0 : b1;
        copy16_to_lds<true>(cache + (size_t)(uint32_t)blk * S::BLKB, src_off(k, ln), slot + 1024u * (uint32_t)k);
      }
    };
    auto issue = [&](int i, int ln, int b0, int b1) {  // all of them
#pragma unroll
      for (int c = 0; c < S::MAXP; ++c) copy_piece(i, c, ln, b0, b1);
    };
    // the queries have landed before any copy is issued (a wait the compiler
    // placed for them later would drain the copies in flight)
    wait_vmcnt<0>();
    int b0, b1;
    pair_blocks(0, b0, b1);
    issue(0, lane_id_here(), b0, b1);
    if (n > 1) pair_blocks(1, b0, b1);  // (the next pair's ids, a step ahead)

    for (int i = 0; i <= n; ++i) {
      // tile i has landed (the only copies in flight); every wave is done
      // with step i - 1
      wait_vmcnt<0>();
      barrier_keep_loads();
      const int ln = lane_id_here();  // (lane-derived values recomputed: the registers are full)
      // the copies of tile i + 1: here in the first step, else between the
      // value product's MFMAs (one every third), where their issue overlaps
      // matrix work instead of holding up all waves at once (~4% faster)
      const bool do_issue = i + 1 < n;
      if (i == 0 && do_issue) issue(i + 1, ln, b0, b1);

      // ---- value product of tile i - 1: lane's head 32 (wave % 4) + ln % 32,
      // dims 256 (wave / 4) + 32 t + (ln % 32) of the A operand; k-step ks
      // covers keys 16 ks + 8 (ln / 32) .. + 7 ----
      if (i > 0) {
        const int pp = (i - 1) & 1;
        const int l32 = ln & 31, kh = ln >> 5;
        const int head = 32 * (wave & 3) + l32;
        const float al = alpha_sh[pp][head];
        if (__any(al != 1.f)) {
#pragma unroll
          for (int t = 0; t < WDT; ++t) ow[t] *= al;
        }
        u32x4 pw[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          pw[ks] = *(lds_cu32x4*)(uintptr_t)(pb_lds + (uint32_t)(pp * H * 64 + head * 64 +
                                                                 16 * ((2 * ks + kh) ^ vt_swizzle(head))));
        const uint32_t vbase = vt_lds + (uint32_t)(pp * MLA_DV * MLA_VT_ROW);
        const int d0 = 256 * (wave >> 2) + l32;
        uint32_t vb[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vb[ks] = vbase + vt_offset(d0, 2 * ks + kh);
        constexpr int NVR = 2 * WDT, VD = 4;  // value reads (tile t, k-step ks) = read 2 t + ks
        auto vread = [&](int r) { return lds_read16(vb[r & 1] + (uint32_t)(32 * MLA_VT_ROW * (r >> 1))); };
        __builtin_amdgcn_sched_barrier(0);
        u32x4 vbuf[VD];
#pragma unroll
        for (int r = 0; r < VD; ++r) vbuf[r] = vread(r);
#pragma unroll
        for (int r = 0; r < NVR; ++r) {
          const u32x4 vf = vbuf[r % VD];
          if (r + VD < NVR) vbuf[r % VD] = vread(r + VD);
          ow[r >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, vf),
                                                             __builtin_bit_cast(f16x8_t, pw[r & 1]), ow[r >> 1], 0, 0, 0);
          if (do_issue && r % 3 == 1 && r / 3 < S::MAXP) copy_piece(i + 1, r / 3, lane_id_here(), b0, b1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (do_issue && i + 2 < n) pair_blocks(i + 2, b0, b1);
      if (i == n) break;

      // ---- score product and transposition of tile i ----
      const int cp = i & 1;
      const int kend = ctx - 32 * (p0 + i);  // keys of this tile at or past kend are masked
      const uint32_t slot = ring_lds + (uint32_t)(cp * S::TILEB);
      const uint32_t vdst = vt_lds + (uint32_t)(cp * MLA_DV * MLA_VT_ROW);
      u32x4 th[4];  // th[t][w]: bf16, then fp16, pair (dims 2w, 2w+1) of key 4 tq + t
      const int tq = (64 * wave + ln) & 7, tc = (64 * wave + ln) >> 3;
      constexpr int NB = DK == 576 ? 2 : 4;  // (see the score reads above)
      uint32_t kb[2][NB];
      {
        const int r16 = ln & 15, rq = ln >> 4;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int key = 8 * (r16 >> 2) + 4 * kt + (r16 & 3);
          const int swz = row_swizzle<DK>(key);
#pragma unroll
          for (int b = 0; b < NB; ++b)
            kb[kt][b] = slot + (uint32_t)(key * S::ROWB + 16 * (((b << 2) | rq) ^ swz));
        }
      }
      f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      constexpr int NKR = 2 * S::KS, PD = 4;
      auto kread = [&](int r) {
        const int j = r >> 1, kt = r & 1;
        return lds_read16(kb[kt][j % NB] + (uint32_t)(64 * NB * (j / NB)));
      };
      __builtin_amdgcn_sched_barrier(0);
      u32x4 kbuf[PD];
#pragma unroll
      for (int r = 0; r < PD; ++r) kbuf[r] = kread(r);
#pragma unroll
      for (int r = 0; r < NKR; ++r) {
        const u32x4 kf = kbuf[r % PD];
        if (r + PD < NKR) kbuf[r % PD] = kread(r + PD);
        st[r & 1] = mfma_bf16(kf, qf[r >> 1], st[r & 1]);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int key = 4 * tq + t;
        th[t] = lds_read16(slot + (uint32_t)(key * S::ROWB + 16 * (tc ^ row_swizzle<DK>(key))));
      }
      __builtin_amdgcn_sched_group_barrier(0x100, PD, 0);
#pragma unroll
      for (int r = 0; r < NKR - PD; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, PD, 0);
      __builtin_amdgcn_sched_barrier(0);
      const bool tail = kend < 32;  // (uniform) the context ends inside this tile
      {  // transposed fp16 values of tile i, keys past the context zeroed
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t b = th[t][w];
            th[t][w] = f16x2_bits(__uint_as_float(b << 16), __uint_as_float(b & 0xffff0000u));
          }
        }
        if (tail) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t keep = 4 * tq + t < kend ? 0xffffffffu : 0u;
#pragma unroll
            for (int w = 0; w < 4; ++w) th[t][w] &= keep;
          }
        }
#pragma unroll
        for (int d = 0; d < 8; ++d) {  // dim 8 tc + d: keys 4 tq .. 4 tq + 3
          const int w = d >> 1;
          const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
          const uint32_t lo2 = __builtin_amdgcn_perm(th[1][w], th[0][w], sel);
          const uint32_t hi2 = __builtin_amdgcn_perm(th[3][w], th[2][w], sel);
          lds_write8(vdst + vt_offset(8 * tc + d, tq >> 1) + 8 * (tq & 1), lo2, hi2);
        }
      }

      // ---- softmax of tile i: this lane's keys 8 q4 + 4 kt + r, head
      // 16 wave + c16; P^T row and rescale factor to LDS ----
      {
        const int rq = ln >> 4, h16 = 16 * wave + (ln & 15);
        float xv[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) xv[kt][r] = st[kt][r] * a.scale_log2;
        if (tail) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) xv[kt][r] = (8 * rq + 4 * kt + r < kend) ? xv[kt][r] : -INFINITY;
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, xv[kt][r]);
        tmax = strided_max<16>(tmax);  // key 0 of the tile is always valid
        const bool up = tmax > m + 8.f;
        const float alpha = up ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;
        m = up ? tmax : m;
        lsum *= alpha;
        if (rq == 0) alpha_sh[cp][h16] = alpha;
        // p scaled by 2^7 (at most 2^15): fp16 keeps small weights normal
        const float mb = m - 7.f;
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(xv[e >> 2][e & 3] - mb);
          lsum += pv[e];
        }
        const u32x4 pf = {f16x2_bits(pv[0], pv[1]), f16x2_bits(pv[2], pv[3]), f16x2_bits(pv[4], pv[5]),
                          f16x2_bits(pv[6], pv[7])};
        *(lds_u32x4*)(uintptr_t)(pb_lds + (uint32_t)(cp * H * 64 + h16 * 64 + 16 * (rq ^ vt_swizzle(h16)))) = pf;
      }
    }

    // ---- result of the segment: the scoring waves publish each head's sum
    // (and leave the summary's max and sum); the owners of the outputs
    // normalise or store them ----
    const bool single = (sp0 / C) == ((sp0 + np - 1) / C);
    {
      const int ln = lane_id_here();
      const float L = strided_sum<16>(lsum);
      if ((ln >> 4) == 0) {
        lsum_sh[16 * wave + (ln & 15)] = L;
        if (!single) {
          const size_t rec = (size_t)(blockIdx.x + s) * H + 16 * wave + (ln & 15);
          a.part_ml[rec * 2] = m - 7.f;
          a.part_ml[rec * 2 + 1] = L;
        }
      }
      barrier_keep_loads();
      // lane: head 32 (wave % 4) + ln % 32; ow[t][4 j + r] is dim
      // 256 (wave / 4) + 32 t + 8 j + 4 (ln / 32) + r
      const int head = 32 * (wave & 3) + (ln & 31);
      const int d0 = 256 * (wave >> 2) + 4 * (ln >> 5);
      if (single) {
        const float inv = 1.f / lsum_sh[head];
        uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((size_t)s * H + head) * MLA_DV + d0;
#pragma unroll
        for (int t = 0; t < WDT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint2 w;
            w.x = pack_bf16x2(ow[t][4 * j] * inv, ow[t][4 * j + 1] * inv);
            w.y = pack_bf16x2(ow[t][4 * j + 2] * inv, ow[t][4 * j + 3] * inv);
            *reinterpret_cast<uint2*>(op + 32 * t + 8 * j) = w;
          }
      } else {
        const size_t rec = (size_t)(blockIdx.x + s) * H + head;
        float* op = a.part_o + rec * MLA_DV + d0;
#pragma unroll
        for (int t = 0; t < WDT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f32x4*>(op + 32 * t + 8 * j) =
                f32x4{ow[t][4 * j], ow[t][4 * j + 1], ow[t][4 * j + 2], ow[t][4 * j + 3]};
      }
      barrier_keep_loads();  // the ring and the head sums are reused by the next segment
    }
    x = (long long)sp0 + p1;
    if (p1 == np) {  // the sequence is done: the next segment starts the next one
      sp0 += np;
      ++s;
    }
  }
}

// ---- 16 heads: the waves split the keys ----------------------------------
//
// With 16 heads a 32-key step holds too little work for 8 waves to share:
// the kernel above would repeat the 16-head score product in every wave.
// Here each of a workgroup's 4 waves (one per SIMD) walks its own even share
// of the concatenated blocks, as the grouped-query decode does, and stages
// its blocks by global->LDS copies in a ring of its own (no workgroup
// barrier in the loop), with the copies of the next NSL - 1 blocks in flight. Per 16-key block: scores S^T = C Q^T on
// 16x16x32 bf16 MFMAs (the 16 heads are the MFMA columns; a lane's four
// score values are keys 4 (lane / 16) + r of head lane % 16, exactly its
// P^T operand for a 16x16x16 MFMA over the 16 keys), online softmax with
// lazy rescaling, O^T += V^T P^T on 16x16x16 bf16 MFMAs with P split into
// bf16 hi + lo (2^-16 relative), the value operand read transposed straight
// from the row-major block with gfx950's transposing LDS read.
typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_bf16_k16(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, a), __builtin_bit_cast(v4i16, b), c, 0,
                                                   0, 0);
}
// ds_read_b64_tr_b16: in each 16-lane group, lane j receives element j % 4 of
// the four-element pieces that lanes j / 4, j / 4 + 4, j / 4 + 8 and
// j / 4 + 12 of the group point at.
__device__ __forceinline__ u32x2 lds_read_tr8(uint32_t addr) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)addr));
}
// Chunk swizzle of a block row (key 0..15), chosen so that the score reads
// (16 lanes: 16 rows, one chunk column) and the transposed value reads (32
// lanes: 8 rows x 2 chunks) hit distinct banks.
template <int DK>
__device__ __forceinline__ int narrow_swizzle(int row) {
  const int r = row & 15;
  if constexpr (DK == 576) return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);  // rows of 72 chunks
  else return ((r & 7) << 1) | (r >> 3);                                   // rows of 64 chunks
}

#ifndef MLA_NARROW_WAVES
#define MLA_NARROW_WAVES 4
#endif
constexpr int kNarrowWaves = MLA_NARROW_WAVES;          // waves per workgroup
constexpr int kNarrowSlots = 8 / MLA_NARROW_WAVES;      // ring slots per wave (the LDS holds 8 blocks)

// At most `ahead` blocks of this wave's copies (COPIES each) still in flight.
template <int COPIES, int NSL>
__device__ __forceinline__ void wait_blocks(int ahead) {
  if constexpr (NSL >= 4) {
    if (ahead >= 3) { wait_vmcnt<3 * COPIES>(); return; }
  }
  if constexpr (NSL >= 3) {
    if (ahead >= 2) { wait_vmcnt<2 * COPIES>(); return; }
  }
  if (ahead >= 1) { wait_vmcnt<COPIES>(); return; }
  wait_vmcnt<0>();
}

template <int DK>
struct MlaNarrowShape {
  static constexpr int ROWB = DK * 2;
  static constexpr int BLKB = 16 * ROWB;       // one block = one slot
  static constexpr int COPIES = BLKB / 1024;   // 1 KiB copies per block (18 or 16)
  static constexpr int KS = DK / 32;           // score MFMAs per block
  static constexpr int DTV = MLA_DV / 16;      // 16-dim output tiles
};

template <int DK>
__global__ __launch_bounds__(64 * kNarrowWaves) __attribute__((amdgpu_waves_per_eu(1, 1))) void mla_decode_narrow(
    MlaArgs a) {
  using S = MlaNarrowShape<DK>;
  constexpr int H = 16, NW = kNarrowWaves, NT = 64 * NW, NSL = kNarrowSlots;
  static_assert((NSL & (NSL - 1)) == 0 && NSL >= 2 && NSL <= 4, "2 or 4 slots");
  __shared__ __attribute__((aligned(16))) uint8_t ring[NW * NSL * S::BLKB];
  __shared__ int psum[kMlaMaxSeqs + 1];
  __shared__ int scan[NT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, q4 = lane >> 4;
  const int NS = a.num_seqs;
  const int T = unit_prefix_sums<NT, 1>(a, psum, scan);
  const int workers = NW * (int)gridDim.x;
  const int C = max(1, (T + workers - 1) / workers);  // blocks per wave
  write_meta<NT>(a, psum, C);

  // copies: piece k of a block = bytes [1024 k, 1024 k + 1024) of its slot;
  // this lane's source offset in the block for each piece
  uint32_t src[S::COPIES];
#pragma unroll
  for (int k = 0; k < S::COPIES; ++k) {
    const int P = 1024 * k + 16 * lane;
    const int row = P / S::ROWB, pch = (P % S::ROWB) / 16;
    src[k] = (uint32_t)(row * S::ROWB + 16 * (pch ^ narrow_swizzle<DK>(row)));
  }
  const uint32_t ring_lds = lds_addr(ring) + (uint32_t)(wave * NSL * S::BLKB);
  // score operand: key c16, dims 32 j + 8 q4 .. + 7 (chunk 4 j + q4)
  const int kswz = narrow_swizzle<DK>(c16);
  // value operand: lane (group q4, j = c16) points at key 4 q4 + j / 4, dims
  // 16 t + 4 (j % 4) .. + 3, i.e. chunk 2 t + (j % 4) / 2, half j % 2
  const int vrow = 4 * q4 + (c16 >> 2);
  const int vswz = narrow_swizzle<DK>(vrow);
  const uint32_t vbase = (uint32_t)(vrow * S::ROWB + 8 * (c16 & 1));
  const int vch = (c16 & 3) >> 1;

  const uint8_t* cache = reinterpret_cast<const uint8_t*>(a.cache);
  const int w = (int)blockIdx.x * NW + wave;
  const long long x_end = min<long long>((long long)(w + 1) * C, T);
  long long x = (long long)w * C;
  while (x < x_end) {
    int lo = 0, hi = NS - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (psum[mid] <= x) lo = mid;
      else hi = mid - 1;
    }
    const int s = __builtin_amdgcn_readfirstlane(lo);
    const int sp0 = __builtin_amdgcn_readfirstlane(psum[s]);
    const int nbs = psum[s + 1] - sp0;
    const int b0 = (int)(x - sp0);
    const int b1 = (int)(min<long long>(x_end, (long long)sp0 + nbs) - sp0);
    const int n = b1 - b0;
    typedef __attribute__((address_space(4))) const int cint;
    const int ctx = ((const cint*)a.context_lens)[s];
    const cint* bt = (const cint*)(a.block_table + (size_t)s * a.bt_stride);

    u32x4 qf[S::KS];
    {
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.query) + ((size_t)s * H + c16) * S::ROWB + 16 * q4;
#pragma unroll
      for (int j = 0; j < S::KS; ++j) qf[j] = load16(qp + 64 * j);
    }
    f32x4 o[S::DTV];
#pragma unroll
    for (int t = 0; t < S::DTV; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;

    auto issue = [&](int i) {  // copies of the segment's block i into slot i % NSL
      const uint8_t* base = cache + (size_t)(uint32_t)bt[b0 + i] * S::BLKB;
      const uint32_t slot = ring_lds + (uint32_t)((i & (NSL - 1)) * S::BLKB);
#pragma unroll
      for (int k = 0; k < S::COPIES; ++k) copy16_to_lds<true>(base, src[k], slot + 1024u * (uint32_t)k);
    };
    // the queries have landed before any copy is issued (a wait the compiler
    // placed for them later would drain the copies in flight)
    wait_vmcnt<0>();
#pragma unroll
    for (int j = 0; j < NSL - 1; ++j)
      if (j < n) issue(j);
    for (int i = 0; i < n; ++i) {
      // block i + NSL - 1 into the slot block i - 1 left; block i has landed
      // once at most the blocks after it are in flight
      if (i + NSL - 1 < n) issue(i + NSL - 1);
      wait_blocks<S::COPIES, NSL>(min(n - 1 - i, NSL - 1));
      const uint32_t slot = ring_lds + (uint32_t)((i & (NSL - 1)) * S::BLKB);
      const int kend = ctx - 16 * (b0 + i);  // keys at or past kend are masked (last block only)

      // ---- scores: lane holds keys 4 q4 + r of head c16. All operand reads
      // are issued before the MFMAs, and the value operands right after
      // them, so that one wave per SIMD does not wait out each read ----
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
      const uint32_t kb = slot + (uint32_t)(c16 * S::ROWB);
      u32x4 kf[S::KS];
#pragma unroll
      for (int j = 0; j < S::KS; ++j) kf[j] = lds_read16(kb + (uint32_t)(16 * ((4 * j + q4) ^ kswz)));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < S::KS; ++j) st = mfma_bf16(kf[j], qf[j], st);
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t vb = slot + vbase;
      u32x2 vf[S::DTV];
#pragma unroll
      for (int t = 0; t < S::DTV; ++t) vf[t] = lds_read_tr8(vb + (uint32_t)(16 * ((2 * t + vch) ^ vswz)));
      __builtin_amdgcn_sched_barrier(0);
      float xv[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = st[r] * a.scale_log2;
        v = 4 * q4 + r < kend ? v : -INFINITY;
        xv[r] = v;
        tmax = fmaxf(tmax, v);
      }
      tmax = strided_max<16>(tmax);  // key 0 of a block is always valid
      const bool up = tmax > m + 8.f;
      if (__any(up)) {
        const float alpha = up ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;
        m = up ? tmax : m;
        lsum *= alpha;
#pragma unroll
        for (int t = 0; t < S::DTV; ++t) {
          o[t][0] *= alpha; o[t][1] *= alpha; o[t][2] *= alpha; o[t][3] *= alpha;
        }
      }
      // p = 2^(x - m) <= 2^8 as bf16 hi + lo
      uint32_t ph[2], pl[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(xv[2 * e] - m);
        const float p1 = __builtin_amdgcn_exp2f(xv[2 * e + 1] - m);
        lsum += p0 + p1;
        ph[e] = pack_bf16x2(p0, p1);
        pl[e] = pack_bf16x2(p0 - bf16_lo(ph[e]), p1 - bf16_hi(ph[e]));
      }
      const u32x2 phv = {ph[0], ph[1]}, plv = {pl[0], pl[1]};
      // values of keys past the context may be anything (NaN): zero them
      const bool edge = kend < 16;
      uint32_t vmask[2] = {0xffffffffu, 0xffffffffu};
      if (edge) {
        vmask[0] = (4 * q4 < kend ? 0x0000ffffu : 0u) | (4 * q4 + 1 < kend ? 0xffff0000u : 0u);
        vmask[1] = (4 * q4 + 2 < kend ? 0x0000ffffu : 0u) | (4 * q4 + 3 < kend ? 0xffff0000u : 0u);
      }
      // ---- O^T += V^T P^T over the 16 keys ----
#pragma unroll
      for (int t = 0; t < S::DTV; ++t) {
        vf[t][0] &= vmask[0];
        vf[t][1] &= vmask[1];
        o[t] = mfma_bf16_k16(vf[t], phv, o[t]);
        o[t] = mfma_bf16_k16(vf[t], plv, o[t]);
      }
    }
    // ---- result of the segment: lane holds dims 16 t + 4 q4 + r of head c16 ----
    const float L = strided_sum<16>(lsum);
    const bool single = (sp0 / C) == ((sp0 + nbs - 1) / C);
    if (single) {
      const float inv = 1.f / L;
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((size_t)s * H + c16) * MLA_DV + 4 * q4;
#pragma unroll
      for (int t = 0; t < S::DTV; ++t) {
        uint2 wv;
        wv.x = pack_bf16x2(o[t][0] * inv, o[t][1] * inv);
        wv.y = pack_bf16x2(o[t][2] * inv, o[t][3] * inv);
        *reinterpret_cast<uint2*>(op + 16 * t) = wv;
      }
    } else {
      const size_t rec = (size_t)(w + s) * H + c16;
      float* op = a.part_o + rec * MLA_DV + 4 * q4;
#pragma unroll
      for (int t = 0; t < S::DTV; ++t) *reinterpret_cast<f32x4*>(op + 16 * t) = o[t];
      if (q4 == 0) {
        a.part_ml[rec * 2] = m;
        a.part_ml[rec * 2 + 1] = L;
      }
    }
    x = (long long)sp0 + b1;
  }
}

// One (sequence, head) row computed directly, by one wave, in fp32 from the
// bf16 rows: online softmax over every key of the sequence (lane l holds
// dims l + 64 k). Slow; it serves the rows whose fp16 value tiles overflowed.
template <int DK, int H>
__device__ void mla_row_exact(const MlaArgs& a, int s, int h, int lane) {
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.query) + ((size_t)s * H + h) * DK;
  float qv[DK / 64];
#pragma unroll
  for (int k = 0; k < DK / 64; ++k) qv[k] = bf16_to_f32(q[64 * k + lane]);
  const int ctx = a.context_lens[s];
  const int* bt = a.block_table + (size_t)s * a.bt_stride;
  float m = -INFINITY, l = 0.f, acc[MLA_DV / 64];
#pragma unroll
  for (int k = 0; k < MLA_DV / 64; ++k) acc[k] = 0.f;
  for (int j = 0; j < ctx; ++j) {
    const uint16_t* row =
        reinterpret_cast<const uint16_t*>(a.cache) + ((size_t)(uint32_t)bt[j >> 4] * 16 + (j & 15)) * DK;
    float c[DK / 64];
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < DK / 64; ++k) {
      c[k] = bf16_to_f32(row[64 * k + lane]);
      d = fmaf(qv[k], c[k], d);
    }
    const float x = group_sum<64>(d) * a.scale_log2;
    const float mn = fmaxf(m, x);
    const float corr = exp2f(m - mn), p = exp2f(x - mn);
    l = l * corr + p;
#pragma unroll
    for (int k = 0; k < MLA_DV / 64; ++k) acc[k] = fmaf(p, c[k], acc[k] * corr);
    m = mn;
  }
  uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((size_t)s * H + h) * MLA_DV;
#pragma unroll
  for (int k = 0; k < MLA_DV / 64; ++k) o[64 * k + lane] = f32_to_bf16(acc[k] / l);
}

// Exact merge of a (sequence, head)'s summaries, one wave each: the
// workgroups w0..w1 covering the sequence left theirs in slot w + s. With
// fp16 value tiles (more than 16 heads) a row that comes out non-finite is
// computed again exactly (mla_row_exact).
template <int DK, int H>
__global__ __launch_bounds__(256) void mla_merge(MlaArgs a) {
  constexpr bool FP16_TILES = H > 16;
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= a.num_seqs * H) return;
  const int s = idx / H, h = idx % H;
  const int C = a.meta[0];
  const int* psum = a.meta + 1;
  const int np = psum[s + 1] - psum[s];
  if (np == 0) {
    for (int d = lane; d < MLA_DV; d += 64) reinterpret_cast<uint16_t*>(a.out)[((size_t)s * H + h) * MLA_DV + d] = 0;
    return;
  }
  const int w0 = psum[s] / C, w1 = (psum[s] + np - 1) / C;
  if (w0 == w1) {  // finished in place
    if constexpr (FP16_TILES) {
      const uint16_t* o = reinterpret_cast<const uint16_t*>(a.out) + ((size_t)s * H + h) * MLA_DV;
      bool bad = false;
#pragma unroll
      for (int k = 0; k < MLA_DV / 64; ++k) bad |= (o[64 * k + lane] & 0x7f80u) == 0x7f80u;
      if (__any(bad)) mla_row_exact<DK, H>(a, s, h, lane);
    }
    return;
  }
  const int n = w1 - w0 + 1;
  auto rec = [&](int i) { return (size_t)(w0 + i + s) * H + h; };
  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, a.part_ml[rec(i) * 2]);
  M = strided_max<1>(M);
  float acc[MLA_DV / 64];
#pragma unroll
  for (int k = 0; k < MLA_DV / 64; ++k) acc[k] = 0.f;
  float L = 0.f;
  // records in batches of RB, every load of a batch issued before the first
  // is used (one memory round trip per batch instead of per record); the
  // sums run in record order as one at a time would
  constexpr int RB = 8;
  for (int i0 = 0; i0 < n; i0 += RB) {
    float ml[RB][2], v[RB][MLA_DV / 64];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const size_t r = rec(min(i0 + u, n - 1));  // (past the end: a valid record, not summed)
      ml[u][0] = a.part_ml[r * 2];
      ml[u][1] = a.part_ml[r * 2 + 1];
      const float* row = a.part_o + r * MLA_DV;
#pragma unroll
      for (int k = 0; k < MLA_DV / 64; ++k) v[u][k] = row[64 * k + lane];
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if (i0 + u < n) {
        const float w = __builtin_amdgcn_exp2f(ml[u][0] - M);
        L += w * ml[u][1];
#pragma unroll
        for (int k = 0; k < MLA_DV / 64; ++k) acc[k] = fmaf(w, v[u][k], acc[k]);
      }
    }
  }
  const float inv = 1.f / L;
  if constexpr (FP16_TILES) {
    bool bad = false;
#pragma unroll
    for (int k = 0; k < MLA_DV / 64; ++k) bad |= !(fabsf(acc[k] * inv) <= 3.4028235e38f);
    if (__any(bad)) {
      mla_row_exact<DK, H>(a, s, h, lane);
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < MLA_DV / 64; ++k)
    reinterpret_cast<uint16_t*>(a.out)[((size_t)s * H + h) * MLA_DV + 64 * k + lane] = f32_to_bf16(acc[k] * inv);
}

// Summary slots: one per worker (a workgroup; a wave for 16 heads) plus one
// per sequence (a worker's segments each advance the sequence or the worker).
static size_t mla_slots(int num_seqs, int num_heads, int grid) {
  const size_t workers = (size_t)grid * (num_heads == 16 ? kNarrowWaves : 1);
  return workers + (size_t)num_seqs;
}

size_t mla_workspace_bytes(int num_seqs, int num_heads, int grid) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t slots = mla_slots(num_seqs, num_heads, grid);
  return al((size_t)(num_seqs + 2) * sizeof(int)) + al(slots * num_heads * MLA_DV * sizeof(float)) +
         al(slots * num_heads * 2 * sizeof(float));
}

void mla_bind_workspace(MlaArgs& a, void* workspace, int num_seqs, int num_heads, int grid) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t slots = mla_slots(num_seqs, num_heads, grid);
  char* ws = static_cast<char*>(workspace);
  a.meta = reinterpret_cast<int*>(ws);
  ws += al((size_t)(num_seqs + 2) * sizeof(int));
  a.part_o = reinterpret_cast<float*>(ws);
  ws += al(slots * num_heads * MLA_DV * sizeof(float));
  a.part_ml = reinterpret_cast<float*>(ws);
}

int mla_max_seqs() { return kMlaMaxSeqs; }

template <int DK, int H>
static hipError_t run_mla(const MlaArgs& a, int grid, hipStream_t st) {
  // 8 waves of one 16-head group each. (Four waves of two groups, which
  // halves the LDS operand reads, measured slower: one wave per SIMD hides
  // the LDS latency worse, and at 128 heads the registers spill.)
  constexpr int NW = 8, HG = 1;
  if constexpr (H == 16)  // the waves split the keys
    hipLaunchKernelGGL((mla_decode_narrow<DK>), dim3((unsigned)grid), dim3(64 * kNarrowWaves), 0, st, a);
  else if constexpr (H == 128)
    hipLaunchKernelGGL((mla_decode_wide<DK>), dim3((unsigned)grid), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((mla_decode_split<DK, H, NW, HG>), dim3((unsigned)grid), dim3(64 * NW), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mla_merge<DK, H>), dim3((unsigned)((a.num_seqs * H + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_mla_decode(const MlaArgs& a, int head_dim_k, int grid, hipStream_t st) {
  const int H = a.num_heads;
  if (head_dim_k == 576) {
    if (H == 16) return run_mla<576, 16>(a, grid, st);
    if (H == 32) return run_mla<576, 32>(a, grid, st);
    if (H == 64) return run_mla<576, 64>(a, grid, st);
    if (H == 128) return run_mla<576, 128>(a, grid, st);
  } else if (head_dim_k == 512) {
    if (H == 16) return run_mla<512, 16>(a, grid, st);
    if (H == 32) return run_mla<512, 32>(a, grid, st);
    if (H == 64) return run_mla<512, 64>(a, grid, st);
    if (H == 128) return run_mla<512, 128>(a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
