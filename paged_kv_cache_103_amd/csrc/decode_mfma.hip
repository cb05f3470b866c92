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

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "sparse_pick.h"

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
  // K/V tiles are read once per call: nontemporal loads (on the fp8 batch of
  // 128 sequences x 8K-131K keys: 2.82 ms against 3.10 ms with ordinary
  // loads; bf16 tiles likewise faster on scattered tiles)
  auto ld16 = [](const void* p) { return load16_stream(p); };
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int kp = 8 * (c16 >> 2) + 4 * kt + (c16 & 3);  // this lane's key row in score tile kt
    const size_t phys = (kp >> 4) ? phys1 : phys0;
    const uint8_t* row = kcache + phys * head_stride + (size_t)(kp & 15) * (D * E);
    if constexpr (E == 2) {
#pragma unroll
      for (int j = 0; j < S::DS; ++j) r.k[kt * S::DS + j] = ld16(row + kstep_d0<E>(j, q4) * 2);
    } else {
#pragma unroll
      for (int c = 0; c < S::DS / 2; ++c) r.k[kt * (S::DS / 2) + c] = ld16(row + 64 * c + 16 * q4);
    }
  }
  // V^T: lane group q reads keys 8q..8q+7 = block q/2, keys 8(q&1)..+8
  const size_t vphys = (q4 >> 1) ? phys1 : phys0;
  const uint8_t* vt = vcache + vphys * head_stride + 8 * (q4 & 1) * E;
  if constexpr (E == 2) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) r.v[dt] = ld16(vt + (size_t)(dt * 16 + c16) * 32);
  } else {
#pragma unroll
    for (int dp = 0; dp < D / 32; ++dp) {
      const u32x2 a = load8_stream(vt + (size_t)((2 * dp) * 16 + c16) * 16);
      const u32x2 c = load8_stream(vt + (size_t)((2 * dp + 1) * 16 + c16) * 16);
      r.v[dp] = u32x4{a[0], a[1], c[0], c[1]};
    }
  }
}

// Running state of one wave over its keys: O^T (column = head), the running
// max m (log2 units, uniform over the lane groups) and the partial sum of
// exponentials of this lane's keys.
template <int D>
struct WaveAcc {
  f32x4 o[D / 16];
  float m, lsum;
};

// Scores, online softmax and PV for one pair of blocks (b, b+1). EDGE pairs
// straddle the window start or the context end and carry the masking code.
// Keys of the pair outside [lo, kend) are masked: kend is the end of the
// wave's segment of the stream (at most the context end), so a pair whose
// second block belongs to the next segment, or lies past the context (and
// then re-reads the first block), contributes only its own keys.
template <int CK, int D, bool EDGE>
__device__ __forceinline__ void pair_step(WaveAcc<D>& acc, const PairRegs<CK, D>& r, const u32x4* qf,
                                          size_t phys0, size_t phys1, int b, int lo, int ctx,
                                          const DecodeArgs& a, int c16, int q4) {
  // (ctx is the segment's exclusive key end here)
  using S = MfmaDecodeShape<CK, D>;
  constexpr int E = S::E, DS = S::DS, DT = S::DT;
  f32x4* o = acc.o;
  float& m = acc.m;
  float& lsum = acc.lsum;

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
  // the pair's two blocks' scales by scalar loads (uniform ids), then per lane
  typedef __attribute__((address_space(4))) const float cfloat;
  const cfloat* kss = (const cfloat*)(a.k_scale);
  const cfloat* vss = (const cfloat*)(a.v_scale);
  const float k0 = kss[phys0], k1 = kss[phys1], v0 = vss[phys0], v1 = vss[phys1];
  ks *= (q4 >> 1) ? k1 : k0;
  vs = (q4 >> 1) ? v1 : v0;
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
  // Lazy rescaling: the running max moves only when this pair's max exceeds
  // it by more than 2^8 (p stays below 256 otherwise); the final division
  // uses the same max. tmax is finite: every pair has a key in [lo, ctx).
  const bool up = tmax > m + 8.f;
  if (__any(up)) {
    const float alpha = up ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;
    m = up ? tmax : m;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt][0] *= alpha; o[dt][1] *= alpha; o[dt][2] *= alpha; o[dt][3] *= alpha;
    }
  }
  float ps = 0.f, pv[2][4];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float p = __builtin_amdgcn_exp2f(x[kt][rr] - m);
      ps += p;
      pv[kt][rr] = p * vs;
    }
  lsum += ps;
  // P^T operand: logical k 8*q4 + e <-> key 8*q4 + e (e = 4*kt + rr)
  u32x4 ph, pl;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
  const float a0 = pv[t >> 1][(t & 1) * 2], a1 = pv[t >> 1][(t & 1) * 2 + 1];
  const uint32_t hi = pack_bf16x2(a0, a1);
  ph[t] = hi;
  pl[t] = pack_bf16x2(a0 - bf16_lo(hi), a1 - bf16_hi(hi));
  }
  // value slices of keys past the segment may hold anything (even NaN): zero them
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
}

// Writes one wave's result for its (sequence, KV head, partition): the
// normalised output when the sequence has one partition, else the partition's
// (max, sum, unnormalised output) for the merge kernel.
template <int D>
__device__ __forceinline__ void wave_write(WaveAcc<D>& acc, const DecodeArgs& a, int slot, int qrow, int g, int G,
                                           bool single, int c16, int q4, int ncols) {
  const float L = strided_sum<16>(acc.lsum);
  if (c16 >= ncols) return;
  if (single) {
    const float inv = L > 0.f ? 1.f / L : 0.f;  // no keys (an empty range): zeros
    if (a.lse != nullptr && q4 == 0) a.lse[(size_t)qrow * a.num_heads + g * G + c16] = (acc.m + log2f(L)) * kLn2;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * a.num_heads + g * G + c16) * D + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      uint2 w;
      w.x = pack_bf16x2(acc.o[dt][0] * inv, acc.o[dt][1] * inv);
      w.y = pack_bf16x2(acc.o[dt][2] * inv, acc.o[dt][3] * inv);
      *reinterpret_cast<uint2*>(op + dt * 16) = w;
    }
  } else {
    const size_t rec = (size_t)slot * a.rec_cols + c16;
    float* op = a.part_o + rec * D + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(op + dt * 16) = acc.o[dt];
    if (q4 == 0) {
      a.part_ml[rec * 2] = acc.m;
      a.part_ml[rec * 2 + 1] = L;
    }
  }
}

// Physical block ids of a stream, uniform over the wave. From a block-table
// row in global memory: scalar loads through the constant address space (a
// vector load would make the compiler wait for every outstanding K/V load
// before using the id).
struct TableIds {
  const int* bt;
  __device__ __forceinline__ int operator()(int i) const {
    typedef __attribute__((address_space(4))) const int cint;
    return ((const cint*)bt)[i];
  }
};
// From a table in LDS (byte address `base`): LDS reads count on their own
// counter, so they do not make the K/V loads wait either.
struct LdsIds {
  uint32_t base;
  __device__ __forceinline__ int operator()(int i) const {
    typedef __attribute__((address_space(3))) const int lint;
    return __builtin_amdgcn_readfirstlane(*(const lint*)(uintptr_t)(base + 4u * (uint32_t)i));
  }
};

// The blocks [b, blk1) of one stream segment, in pairs, with the next pair's
// loads in flight while one is computed. Only the first pair (a window
// start) and the last (context or segment end) can need masks; the pairs in
// between run in a loop whose loads are unconditional, so that the compiler
// keeps one pair's loads outstanding across the other's arithmetic.
template <int CK, int D, typename Ids = TableIds>
__device__ __forceinline__ void wave_blocks(WaveAcc<D>& acc, const u32x4* qf, const uint8_t* kcache,
                                            const uint8_t* vcache, Ids id_of, int b, int blk1, int lo,
                                            int ctx, size_t head_stride, const DecodeArgs& a, int c16, int q4) {
  const int np = (blk1 - b + 1) >> 1;
  if (np <= 0) return;
  auto ids = [&](int n, size_t& p0, size_t& p1) {
    const int bb = b + 2 * n;
    p0 = (size_t)id_of(bb);
    p1 = (bb + 1 < blk1) ? (size_t)id_of(bb + 1) : p0;
  };
  auto run = [&](const PairRegs<CK, D>& r, size_t p0, size_t p1, int n) {
    const int bb = b + 2 * n;
    if (bb * 16 < lo || bb * 16 + 32 > ctx) pair_step<CK, D, true>(acc, r, qf, p0, p1, bb, lo, ctx, a, c16, q4);
    else pair_step<CK, D, false>(acc, r, qf, p0, p1, bb, lo, ctx, a, c16, q4);
  };
  auto run_interior = [&](const PairRegs<CK, D>& r, size_t p0, size_t p1, int n) {
    pair_step<CK, D, false>(acc, r, qf, p0, p1, b + 2 * n, lo, ctx, a, c16, q4);
  };
  PairRegs<CK, D> ra, rb;
  size_t a0, a1, b0 = 0, b1 = 0;
  ids(0, a0, a1);
  load_pair<CK, D>(ra, kcache, vcache, a0, a1, head_stride, c16, q4);
  if (np >= 2) {
    ids(1, b0, b1);
    load_pair<CK, D>(rb, kcache, vcache, b0, b1, head_stride, c16, q4);
  }
  run(ra, a0, a1, 0);
  int n = 1;  // rb holds pair n
  for (; n + 2 < np; n += 2) {  // pairs n and n + 1 are interior, n + 2 exists
    ids(n + 1, a0, a1);
    load_pair<CK, D>(ra, kcache, vcache, a0, a1, head_stride, c16, q4);
    run_interior(rb, b0, b1, n);
    ids(n + 2, b0, b1);
    load_pair<CK, D>(rb, kcache, vcache, b0, b1, head_stride, c16, q4);
    run_interior(ra, a0, a1, n + 1);
  }
  if (n < np) {
    if (n + 1 < np) {
      ids(n + 1, a0, a1);
      load_pair<CK, D>(ra, kcache, vcache, a0, a1, head_stride, c16, q4);
    }
    run(rb, b0, b1, n);
    if (n + 1 < np) run(ra, a0, a1, n + 1);
  }
}

// Query columns of a wave: column c16 < ncols is head g*G + c16 % G of query
// row qrow + c16 / G (one row for a sequence's own keys; the rows of several
// sequences for a shared prefix).
template <int CK, int D>
__device__ __forceinline__ void load_query(u32x4* qf, const DecodeArgs& a, int qrow, int g, int G, int c16,
                                           int q4, int ncols) {
  constexpr int E = CacheElem<CK>::bytes;
  // G is a power of two (1..16): a shift and a mask, which the register
  // allocator recomputes where it kept a division's results live across the
  // block loop (and spilled them: the shared-prefix kernel on bf16 caches
  // then ran ~6% slower than plain decode on the same bytes)
  const int lg = __builtin_ctz((unsigned)G);
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    if (c16 < ncols) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.query) +
                           ((size_t)(qrow + (c16 >> lg)) * a.num_heads + g * G + (c16 & (G - 1))) * D +
                           kstep_d0<E>(j, q4);
      qf[j] = load16(qp);
    } else {
      qf[j] = u32x4{0, 0, 0, 0};
    }
  }
}

// Blocks of sequence s's own key range [lo, ctx) (0 for rows of longer
// chunks in a mixed batch, which the prefill kernel serves); keys below
// `shared` (a shared prefix read once for its group) are not its own.
__device__ __forceinline__ int seq_blocks(const DecodeArgs& a, int s, int& qrow, int& ctx, int& lo, int shared = 0) {
  qrow = s;
  ctx = 0;
  lo = 0;
  if (a.cu_seqlens != nullptr) {
    const int q0 = a.cu_seqlens[s];
    if (a.cu_seqlens[s + 1] - q0 != 1) return 0;
    qrow = q0;
  }
  ctx = a.context_lens[s];
  lo = max(shared, a.window > 0 ? max(0, ctx - a.window) : 0);
  return max(0, ((ctx - 1) >> 4) - (lo >> 4) + 1);
}

// Exclusive prefix sums of n(i), i < count, into out[0..count] (LDS), with a
// 256-int scan scratch. Returns the total. Requires blockDim.x == 256.
template <typename F>
__device__ __forceinline__ int lds_exclusive_scan(int count, F n_of, int* out, int* scan) {
  const int tid = threadIdx.x;
  int running = 0;
  for (int base = 0; base < count; base += 256) {
    const int i = base + tid;
    const int n = i < count ? n_of(i) : 0;
    scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    if (i < count) out[i] = running + scan[tid] - n;
    running += scan[255];
    __syncthreads();
  }
  if (tid == 0) out[count] = running;
  __syncthreads();
  return running;
}

// Last index k in [0, n) with v[k] <= x (v non-decreasing, v[0] <= x).
__device__ __forceinline__ int last_le(const int* v, int n, long long x, long long scale = 1) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((long long)v[mid] * scale <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Shared prefixes: sequences [cu_groups[k], cu_groups[k+1]) read the
// physical blocks of their first `prefix` tokens in common. Fills, in LDS,
// sg[s] = group of sequence s (-1: none), effp[k] = the prefix each member
// can use (the given length, at most every member's context minus its own
// new token, in whole blocks) and cbase = exclusive prefix sums of the
// groups' column chunks (16/G members per chunk). Returns the chunk count.
//
// Groups must be disjoint ordered runs (0 <= cu_groups[k] <= cu_groups[k+1]
// <= S); if they are not, no group is used and the result is plain decode
// (the groups only change which reads are shared, never the result).
__device__ __forceinline__ int shared_prefix_setup(const DecodeArgs& a, int G, int* sg, int* cbase, int* effp,
                                                   int* scan) {
  const int S = a.num_seqs, MPC = 16 / G;
  int bad = 0;
  for (int k = threadIdx.x; k < a.num_groups; k += 256) {
    const int b = a.cu_groups[k], e = a.cu_groups[k + 1];
    bad |= (b < 0) | (e < b) | (e > S);
  }
  const int NG = __syncthreads_or(bad) ? 0 : a.num_groups;
  for (int s = threadIdx.x; s < S; s += 256) sg[s] = -1;
  if (threadIdx.x == 0) cbase[0] = 0;
  __syncthreads();
  for (int k = threadIdx.x; k < NG; k += 256) {
    const int b = min(max(a.cu_groups[k], 0), S), e = min(max(a.cu_groups[k + 1], b), S);
    int minctx = 0x7fffffff;
    for (int s = b; s < e; ++s) minctx = min(minctx, a.context_lens[s]);
    const int p = e > b ? max(0, min(a.group_prefix_len[k], minctx - 1)) & ~15 : 0;
    effp[k] = p;
    if (p > 0)  // a group without a whole shared block shares nothing
      for (int s = b; s < e; ++s) sg[s] = k;
  }
  __syncthreads();
  return lds_exclusive_scan(
      NG,
      [&](int k) {
        const int b = min(max(a.cu_groups[k], 0), S), e = min(max(a.cu_groups[k + 1], b), S);
        return effp[k] > 0 ? (e - b + MPC - 1) / MPC : 0;
      },
      cbase, scan);
}

// Offsets into the meta buffer the split kernel leaves for the merge kernel.
__host__ __device__ __forceinline__ int meta_sg(int S) { return 2 + 2 * S; }
__host__ __device__ __forceinline__ int meta_cbase(int S) { return 2 + 3 * S; }
int shared_prefix_meta_ints(int num_seqs, int num_groups) { return meta_cbase(num_seqs) + num_groups + 1; }

// Blocks each wave takes: an even share of T block-heads, at least 8 and even.
__device__ __forceinline__ int split_chunk(int total, int nwaves) {
  int c = (total + nwaves - 1) / nwaves;
  c = max(c, 8);
  return (c + 1) & ~1;
}

// Decode with an even split: the (sequence, KV head) block streams, sequence
// major, are laid end to end (T block-heads in all) and wave w takes
// [w*C, (w+1)*C) with C = ceil(T / waves). A wave walks the one to few
// stream segments in its range on its own (no workgroup barrier in the loop);
// a stream covered by one segment is finished in place, others leave one
// (max, sum, unnormalised output) summary per segment in slot wave + stream
// for the merge kernel.
//
// With shared prefixes (SHARED), the streams of the sequences cover only
// their own keys after their group's prefix, and after them come one stream
// per (column chunk of a group, KV head) over the prefix blocks: its MFMA
// columns are the query heads of up to 16/G member sequences, so a shared
// block is read once per chunk instead of once per member. Every member's
// summaries (its own stream's and its chunk's) go to the merge kernel.
template <int CK, int D, bool SHARED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_mfma_split(
    DecodeArgs a) {
  using S = MfmaDecodeShape<CK, D>;
  // LDS: [sg S][cbase NG+1][effp NG] (shared prefixes only), psum over the
  // streams, 256 scan slots
  extern __shared__ int lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, q4 = lane >> 4;
  const int H = a.num_kv_heads;
  const int G = a.num_heads / H;
  const int NSEQ = a.num_seqs;
  const int NG = SHARED ? a.num_groups : 0;
  int* sg = lds;
  int* cbase = sg + NSEQ;
  int* effp = cbase + NG + 1;
  int* psum = SHARED ? effp + NG : lds;
  int* scan = psum + (SHARED ? 2 * NSEQ + 1 : NSEQ + 1);

  if constexpr (!SHARED) {
    if (a.one_per_stream) {  // uniform: no barrier is reached on this path
      const int w = blockIdx.x * 4 + wave;
      if (w >= NSEQ * H) return;
      const int s = w / H, g = w % H;
      if (a.cu_seqlens != nullptr && a.cu_seqlens[s + 1] - a.cu_seqlens[s] != 1) return;  // a chunk row
      int qrow, ctx, lo;
      const int nb = seq_blocks(a, s, qrow, ctx, lo);
      WaveAcc<D> acc;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) acc.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc.m = -INFINITY;
      acc.lsum = 0.f;
      if (nb > 0) {
        u32x4 qf[S::DS];
        load_query<CK, D>(qf, a, qrow, g, G, c16, q4, G);
        wave_blocks<CK, D>(acc, qf, reinterpret_cast<const uint8_t*>(a.k_cache) + (size_t)g * S::TILE,
                           reinterpret_cast<const uint8_t*>(a.v_cache) + (size_t)g * S::TILE,
                           TableIds{a.block_table + (size_t)s * a.bt_stride}, lo >> 4, (lo >> 4) + nb, lo, ctx,
                           (size_t)H * S::TILE, a, c16, q4);
      }
      wave_write<D>(acc, a, 0, qrow, g, G, true, c16, q4, G);  // an empty range: zeros, lse -inf
      return;
    }
  }
  int nstreams = NSEQ;
  if constexpr (SHARED) nstreams += shared_prefix_setup(a, G, sg, cbase, effp, scan);
  const int per_head = lds_exclusive_scan(
      nstreams,
      [&](int i) {
        int qr, cx, l0;
        if (!SHARED) return seq_blocks(a, i, qr, cx, l0);
        if (i < NSEQ) return seq_blocks(a, i, qr, cx, l0, sg[i] >= 0 ? effp[sg[i]] : 0);
        return effp[last_le(cbase, NG, i - NSEQ)] >> 4;
      },
      psum, scan);
  const long long T = (long long)per_head * H;
  const int C = split_chunk((int)min<long long>(T, 0x7fffffff), a.split_waves);
  if (blockIdx.x == 0) {  // for the merge kernel
    if (tid == 0) a.meta[0] = C;
    for (int i = tid; i <= nstreams; i += 256) a.meta[1 + i] = psum[i];
    if constexpr (SHARED) {
      for (int i = tid; i < NSEQ; i += 256) a.meta[meta_sg(NSEQ) + i] = sg[i];
      for (int i = tid; i <= NG; i += 256) a.meta[meta_cbase(NSEQ) + i] = cbase[i];
    }
  }

  const int w = blockIdx.x * 4 + wave;
  const long long x_end = min<long long>((long long)(w + 1) * C, T);
  const size_t head_stride = (size_t)H * S::TILE;
  long long x = (long long)w * C;
  while (x < x_end) {
    // stream containing block-head x: last i with psum[i]*H <= x (uniform)
    const int i = __builtin_amdgcn_readfirstlane(last_le(psum, nstreams, x, H));
    const int nb = __builtin_amdgcn_readfirstlane(psum[i + 1] - psum[i]);
    const long long base = (long long)__builtin_amdgcn_readfirstlane(psum[i]) * H;
    const int g = (int)((x - base) / nb);
    const long long sstart = base + (long long)g * nb;  // this stream's first block-head
    const long long seg_end = min(x_end, sstart + nb);
    const uint8_t* kcache = reinterpret_cast<const uint8_t*>(a.k_cache) + (size_t)g * S::TILE;
    const uint8_t* vcache = reinterpret_cast<const uint8_t*>(a.v_cache) + (size_t)g * S::TILE;
    const int slot = w + i * H + g;
    u32x4 qf[S::DS];
    WaveAcc<D> acc;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) acc.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.m = -INFINITY;
    acc.lsum = 0.f;
    if (!SHARED || i < NSEQ) {
      const int s = i;
      const bool grouped = SHARED && sg[s] >= 0;
      int qrow, ctx, lo;
      seq_blocks(a, s, qrow, ctx, lo, grouped ? effp[sg[s]] : 0);
      const int blk0 = (lo >> 4) + (int)(x - sstart);
      const int blk1 = (lo >> 4) + (int)(seg_end - sstart);
      const int kend = min(ctx, blk1 * 16);
      load_query<CK, D>(qf, a, qrow, g, G, c16, q4, G);
      wave_blocks<CK, D>(acc, qf, kcache, vcache, TableIds{a.block_table + (size_t)s * a.bt_stride}, blk0, blk1,
                         lo, kend, head_stride, a, c16, q4);
      const bool single = !grouped && (sstart / C) == ((sstart + nb - 1) / C);
      wave_write<D>(acc, a, slot, qrow, g, G, single, c16, q4, G);
    } else {
      // column chunk j of group k: members m0 .. m0 + nmem - 1, prefix blocks
      // read through the first member's table
      const int c = i - NSEQ;
      const int k = last_le(cbase, NG, c);
      const int MPC = 16 / G;
      const int first = min(max(a.cu_groups[k], 0), NSEQ);
      const int end = min(max(a.cu_groups[k + 1], first), NSEQ);
      const int m0 = first + (c - cbase[k]) * MPC;
      const int nmem = min(MPC, end - m0);
      const int blk0 = (int)(x - sstart);
      const int blk1 = (int)(seg_end - sstart);
      load_query<CK, D>(qf, a, m0, g, G, c16, q4, nmem * G);
      wave_blocks<CK, D>(acc, qf, kcache, vcache, TableIds{a.block_table + (size_t)first * a.bt_stride}, blk0,
                         blk1, 0, blk1 * 16, head_stride, a, c16, q4);
      wave_write<D>(acc, a, slot, 0, g, G, false, c16, q4, nmem * G);
    }
    x = seg_end;
  }
}

// Exact merge of a (sequence, query head)'s summaries: one wave each;
// M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L. The
// summaries are the segments of the sequence's own stream and, with shared
// prefixes, those of its group chunk's stream (column of the member).
template <int D, bool SHARED>
__global__ __launch_bounds__(256) void decode_split_merge(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= a.num_seqs * a.num_heads) return;
  const int H = a.num_kv_heads, G = a.num_heads / H, NSEQ = a.num_seqs;
  const int s = idx / a.num_heads, hq = idx % a.num_heads, g = hq / G, h = hq % G;
  // rows of longer chunks in a mixed batch belong to the prefill kernel,
  // which may run concurrently: never write them
  if (a.cu_seqlens != nullptr && a.cu_seqlens[s + 1] - a.cu_seqlens[s] != 1) return;
  const int* psum = a.meta + 1;
  const int C = a.meta[0];
  // the sequence's own stream: segments w0..w1, summary slot w + stream
  const int nb = psum[s + 1] - psum[s];
  const long long sstart = (long long)psum[s] * H + (long long)g * nb;
  const int w0 = (int)(sstart / C), w1 = nb > 0 ? (int)((sstart + nb - 1) / C) : w0 - 1;
  const int n1 = w1 - w0 + 1;
  const int stream1 = s * H + g;
  // its group chunk's stream, if any
  int n2 = 0, w20 = 0, stream2 = 0, col2 = 0;
  if constexpr (SHARED) {
    const int k = a.meta[meta_sg(NSEQ) + s];
    if (k >= 0) {
      const int MPC = 16 / G;
      const int mi = s - min(max(a.cu_groups[k], 0), NSEQ);
      const int i2 = NSEQ + a.meta[meta_cbase(NSEQ) + k] + mi / MPC;
      const int nb2 = psum[i2 + 1] - psum[i2];
      if (nb2 > 0) {
        const long long st2 = (long long)psum[i2] * H + (long long)g * nb2;
        w20 = (int)(st2 / C);
        n2 = (int)((st2 + nb2 - 1) / C) - w20 + 1;
        stream2 = i2 * H + g;
        col2 = (mi % MPC) * G + h;
      }
    }
  }
  if (n2 == 0 && n1 == 1) return;  // finished in place
  int qrow = s;
  if (a.cu_seqlens != nullptr) qrow = a.cu_seqlens[s];
  const int n = n1 + n2;
  // record of summary i: (slot, column)
  auto rec = [&](int i) -> size_t {
    return i < n1 ? (size_t)(w0 + i + stream1) * a.rec_cols + h
                  : (size_t)(w20 + (i - n1) + stream2) * a.rec_cols + col2;
  };
  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, a.part_ml[rec(i) * 2]);
  M = strided_max<1>(M);
  constexpr int DL = D / 64;
  float o[DL];
#pragma unroll
  for (int k = 0; k < DL; ++k) o[k] = 0.f;
  float L = 0.f;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const float wgt = (i < n) ? __builtin_amdgcn_exp2f(a.part_ml[rec(i) * 2] - M) : 0.f;
    if (i < n) L += a.part_ml[rec(i) * 2 + 1] * wgt;
    const int cnt = min(64, n - i0);
    for (int j0 = 0; j0 < cnt; j0 += 8) {
      float v[8][DL];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = j0 + u < cnt;
        const float* row = a.part_o + (ok ? rec(i0 + j0 + u) : 0) * D;
#pragma unroll
        for (int k = 0; k < DL; ++k) v[u][k] = ok ? row[k * 64 + lane] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), (j0 + u) & 63));
#pragma unroll
        for (int k = 0; k < DL; ++k) o[k] = fmaf(wj, v[u][k], o[k]);
      }
    }
  }
  L = strided_sum<1>(L);
  // no keys at all (an empty context range): zero output, lse = -inf
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (a.lse != nullptr && lane == 0) a.lse[(size_t)qrow * a.num_heads + hq] = (M + log2f(L)) * kLn2;
#pragma unroll
  for (int k = 0; k < DL; ++k)
    reinterpret_cast<uint16_t*>(a.out)[((size_t)qrow * a.num_heads + hq) * D + k * 64 + lane] =
        f32_to_bf16(o[k] * inv);
}

template <int CK, int D, bool SHARED>
static hipError_t run_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  if (!SHARED && a.one_per_stream) {  // a wave per (sequence, KV head), finished in place
    const long long streams = (long long)a.num_seqs * a.num_kv_heads;
    hipLaunchKernelGGL((decode_mfma_split<CK, D, SHARED>), dim3((unsigned)((streams + 3) / 4)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(a.split_waves / 4));
  const size_t lds = SHARED ? (size_t)(3 * a.num_seqs + 2 * a.num_groups + 2 + 256) * sizeof(int)
                            : (size_t)(a.num_seqs + 1 + 256) * sizeof(int);
  hipLaunchKernelGGL((decode_mfma_split<CK, D, SHARED>), grid, dim3(256), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = a.num_seqs * a.num_heads;
  hipLaunchKernelGGL((decode_split_merge<D, SHARED>), dim3((waves + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <bool SHARED>
static hipError_t run_decode_mfma_kind(const DecodeArgs& a, int cache_kind, int head_size, hipStream_t st) {
  if (cache_kind == KBF16 && head_size == 128) return run_decode_mfma<KBF16, 128, SHARED>(a, st);
  if (cache_kind == KBF16 && head_size == 64) return run_decode_mfma<KBF16, 64, SHARED>(a, st);
  if (cache_kind == KFP8 && head_size == 128) return run_decode_mfma<KFP8, 128, SHARED>(a, st);
  if (cache_kind == KFP8 && head_size == 64) return run_decode_mfma<KFP8, 64, SHARED>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int cache_kind, int head_size, hipStream_t st) {
  return a.num_groups > 0 ? run_decode_mfma_kind<true>(a, cache_kind, head_size, st)
                          : run_decode_mfma_kind<false>(a, cache_kind, head_size, st);
}

// ---------------------------------------------------------------------------
// Sparse decode in one launch (many streams, short lists)
// ---------------------------------------------------------------------------
// Sparse attention reads only the blocks an indexer ranks highest ("宣稱省下
// 106 倍成本…", "背景：什麼是稀疏注意力"), one list per sequence for all of its
// heads. With at least two (sequence, KV head) streams per CU, each stream
// gets a workgroup of its own, which
//  * turns the sequence's list into its distinct blocks in ascending logical
//    order, the newest block always last (an LDS bitmap drops repeats and
//    ids outside [0, newest block); each first setter appends its block to
//    a list and every listed block goes to its rank among them), and looks
//    up their physical ids into a table in LDS;
//  * splits that table evenly over its 4 waves, which walk their parts with
//    the loop of the split kernel above (block ids read from the LDS table);
//  * merges the 4 waves' (max, sum, unnormalised output) summaries in LDS,
//    exactly as the merge kernel does, and writes the output rows.
// So the selection, the decode and the merge are one launch, with no
// workspace. The computation is that of the selection kernel followed by the
// split plan, up to where the stream is cut into segments.
template <int CK, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_sparse_fused(
    DecodeArgs a, SparseSelectArgs sa) {
  using S = MfmaDecodeShape<CK, D>;
  // LDS: [bitmap words_max][list max_selected + 1][table max_selected + 1];
  // after the walk, the same bytes hold the waves' summaries
  extern __shared__ int lds[];
  __shared__ int nlisted;
  unsigned int* bits = reinterpret_cast<unsigned int*>(lds);
  int* listed = lds + sa.words_max;
  int* tbl = listed + sa.max_selected + 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, q4 = lane >> 4;
  const int H = a.num_kv_heads, G = a.num_heads / H;
  const int s = blockIdx.x / H, g = blockIdx.x % H;
  u32x4 qf[S::DS];
  load_query<CK, D>(qf, a, s, g, G, c16, q4, G);  // in flight during the selection

  const int ctx = a.context_lens[s];
  const int nbk = min(ctx > 0 ? (ctx + 15) >> 4 : 0, sa.blocks_max);
  const int m = sparse_mark(sa, s, nbk, bits, listed, &nlisted);
  sparse_rank(listed, m, sa.block_table + (size_t)s * sa.bt_stride, tbl);
  __syncthreads();
  const int keys = sparse_keys(m, ctx, nbk);

  // this wave's part of the stream: whole pairs, the last part shorter
  const int per = (((m + 3) >> 2) + 1) & ~1;
  const int blk0 = min(m, wave * per), blk1 = min(m, blk0 + per);
  WaveAcc<D> acc;
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) acc.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc.m = -INFINITY;
  acc.lsum = 0.f;
  wave_blocks<CK, D>(acc, qf, reinterpret_cast<const uint8_t*>(a.k_cache) + (size_t)g * S::TILE,
                     reinterpret_cast<const uint8_t*>(a.v_cache) + (size_t)g * S::TILE, LdsIds{lds_addr(tbl)}, blk0,
                     blk1, 0, min(keys, blk1 * 16), (size_t)H * S::TILE, a, c16, q4);
  const float L = strided_sum<16>(acc.lsum);
  __syncthreads();  // every wave is done with the table

  // summaries: o [4][G][D], then max [4][G] and sum [4][G]
  float* mo = reinterpret_cast<float*>(lds);
  float* mm = mo + 4 * G * D;
  float* ml = mm + 4 * G;
  if (c16 < G) {
    float* op = mo + (size_t)(wave * G + c16) * D + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) *reinterpret_cast<f32x4*>(op + dt * 16) = acc.o[dt];
    if (q4 == 0) {
      mm[wave * G + c16] = acc.m;
      ml[wave * G + c16] = L;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int c = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mm[w * G + c]);
    float sum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = mm[w * G + c];
      const float wt = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);  // a wave without keys adds nothing
      sum += ml[w * G + c] * wt;
      o += mo[(size_t)(w * G + c) * D + d] * wt;
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;  // no keys at all: zeros
    const size_t row = (size_t)s * a.num_heads + g * G + c;
    reinterpret_cast<uint16_t*>(a.out)[row * D + d] = f32_to_bf16(o * inv);
    if (a.lse != nullptr && d == 0) a.lse[row] = (M + log2f(sum)) * kLn2;
  }
}

size_t decode_sparse_fused_lds_bytes(int words_max, int max_selected, int group, int head_size) {
  if (max_selected < 0 || max_selected >= kSparseRankMax || group < 1 || group > 16 || words_max < 0) return 0;
  const size_t pick = ((size_t)words_max + 2 * (size_t)(max_selected + 1)) * sizeof(int);
  const size_t merge = (size_t)4 * group * (head_size + 2) * sizeof(float);
  const size_t need = std::max(pick, merge);
  return need + 16 <= kSparseMaxLds ? need : 0;  // (+ the static list counter)
}

template <int CK, int D>
static hipError_t run_decode_sparse_fused(const DecodeArgs& a, const SparseSelectArgs& sa, size_t lds,
                                          hipStream_t st) {
  const unsigned grid = (unsigned)((long long)a.num_seqs * a.num_kv_heads);
  hipLaunchKernelGGL((decode_sparse_fused<CK, D>), dim3(grid), dim3(256), lds, st, a, sa);
  return hipGetLastError();
}

hipError_t launch_decode_sparse_fused(const DecodeArgs& a, const SparseSelectArgs& sa, int cache_kind,
                                      int head_size, hipStream_t st) {
  const size_t lds = decode_sparse_fused_lds_bytes(sa.words_max, sa.max_selected, a.num_heads / a.num_kv_heads,
                                                   head_size);
  if (lds == 0 || a.num_seqs <= 0) return hipErrorInvalidValue;
  if (cache_kind == KBF16 && head_size == 128) return run_decode_sparse_fused<KBF16, 128>(a, sa, lds, st);
  if (cache_kind == KBF16 && head_size == 64) return run_decode_sparse_fused<KBF16, 64>(a, sa, lds, st);
  if (cache_kind == KFP8 && head_size == 128) return run_decode_sparse_fused<KFP8, 128>(a, sa, lds, st);
  if (cache_kind == KFP8 && head_size == 64) return run_decode_sparse_fused<KFP8, 64>(a, sa, lds, st);
  return hipErrorInvalidValue;
}


// ---------------------------------------------------------------------------
// Decode beside a running prefill (mixed batches)
// ---------------------------------------------------------------------------
// In a step that mixes one-token rows with a long chunk ("从静态批处理到状态化
// 推理集群", "Chunked prefill：在共置引擎里治理阶段干扰") the decode rows are
// bound by HBM and the chunk by the matrix cores, so the two can share the
// chip. The prefill kernel's workgroups hold most of a CU (8 waves of at
// most 224 registers: 448 of each SIMD's 512, and ~68 KB of LDS), so a
// decode kernel beside it must fit in the rest: one wave per SIMD of at most
// 64 registers and one workgroup per CU of at most ~92 KB of LDS. This kernel keeps its
// loads in flight in LDS instead of registers: each wave streams its 4 KiB
// K and V tiles through a 20 KiB ring (5 bf16 or 10 fp8 tiles) with direct global->LDS
// copies (nontemporal: read once), and more than 80 KB of LDS per workgroup
// keeps a second one off the same CU (which would leave no room there for a
// prefill workgroup).
//
// Per 16-key block and KV head (G = 4 query heads, head size 128; groups of
// 1 and 2 repeat their heads over the 4 rows, groups of 8 add a second set
// of rows, 4..7, broadcast from block 4q + 1):
//  * scores S^T = K Q^T on four 16x16x32 bf16 MFMAs; the 16 columns are the 4
//    heads repeated, so lane 16q + i (i < 4) ends up holding head i's scores
//    of keys 4q..4q+3;
//  * O = P V on 4x4x4 (16-block) bf16 MFMAs: block b of output half h holds
//    heads 0..3 x head dims 64h + 4b..4b+3, so lane l holds the 4 heads of dim
//    64h + l (8 accumulator registers instead of the 32 a 16-column tile
//    takes); P of key quad q is broadcast from block 4q, which is exactly
//    where the score MFMA left it; P enters as bf16 hi + lo (two MFMAs).
// The split plan, summary records and merge are those of decode_mfma_split
// (wave w takes block-heads [w*C, (w+1)*C), summaries in slot w + stream).
constexpr int kSideWaves = 4;
constexpr int kSideRingBytes = kSideWaves * 20 * 1024;        // 20 KiB ring per wave
// a wave's query rows (bf16 [rows][128]): 4 rows (the group's heads
// repeated) for groups of up to 4, 8 for groups of 8
__host__ __device__ constexpr int side_q_rows(int group) { return group == 8 ? 8 : 4; }

size_t decode_side_lds_bytes(int num_seqs, int group) {
  return (size_t)kSideRingBytes + (size_t)kSideWaves * side_q_rows(group) * 256 +
         (size_t)(num_seqs + 1 + 256) * sizeof(int);
}

typedef short side_s16x4 __attribute__((ext_vector_type(4)));


// The value product of one key quad with P broadcast from block ABID (4q
// for the quad's heads 0..3, 4q + 1 for heads 4..7), P as bf16 hi + lo
// against the quad's value operand (b0, b1).
template <int ABID>
__device__ __forceinline__ f32x4 side_pv(uint32_t h0, uint32_t h1, uint32_t l0, uint32_t l1, uint32_t b0, uint32_t b1,
                                         f32x4 o) {
  const side_s16x4 B = __builtin_bit_cast(side_s16x4, (u32x2){b0, b1});
  o = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(side_s16x4, (u32x2){h0, h1}), B, o, 4, ABID, 0);
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(side_s16x4, (u32x2){l0, l1}), B, o, 4, ABID, 0);
}

// (amdgpu_num_vgpr counts half the registers on this target: 32 -> 64)
template <int CK, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_num_vgpr(32))) void decode_side(DecodeArgs a) {
  constexpr int D = 128;
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "groups of 1, 2, 4 or 8 query heads");
  constexpr int QR = side_q_rows(G);  // query rows per wave (row r: head r % G)
  constexpr bool G8 = G == 8;         // heads 4..7 in a second set of accumulators
  constexpr bool FP8 = CK == KFP8;
  constexpr uint32_t TILE = 16 * D * (FP8 ? 1 : 2);           // one (block, KV head) tile
  constexpr int CPT = (int)TILE / 1024;                        // 1 KiB copies per tile
  constexpr int NS = kSideRingBytes / kSideWaves / (int)TILE;  // tiles in a wave's ring (5 bf16, 10 fp8)
  extern __shared__ __attribute__((aligned(16))) int side_lds[];
  uint8_t* ring = reinterpret_cast<uint8_t*>(side_lds);
  uint8_t* qslots = ring + kSideRingBytes;
  int* psum = reinterpret_cast<int*>(qslots + kSideWaves * QR * 256);
  int* scan = psum + a.num_seqs + 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.num_kv_heads, NSEQ = a.num_seqs;

  const int per_head = lds_exclusive_scan(
      NSEQ, [&](int i) { int qr, cx, l0; return seq_blocks(a, i, qr, cx, l0); }, psum, scan);
  const long long T = (long long)per_head * H;
  const int C = split_chunk((int)min<long long>(T, 0x7fffffff), gridDim.x * kSideWaves);
  if (blockIdx.x == 0) {  // for the merge kernel
    if (tid == 0) a.meta[0] = C;
    for (int i = tid; i <= NSEQ; i += 256) a.meta[1 + i] = psum[i];
  }

  const uint32_t ring_lds = lds_addr(ring) + wave * NS * TILE;
  const uint32_t q_lds = lds_addr(qslots) + wave * QR * 256;
  // Per-lane global offsets of the copies; copy c lands lane l's 16 bytes at
  // byte 1024 c + 16 l of the slot, where lane l reads them:
  //  bf16 K copy c: key l%16, 16-byte chunk 4c + l/16 (the score operand of
  //   k-step c); fp8 K copy c: key l%16, bytes 64c + 16(l/16) (k-steps 2c and
  //   2c + 1, 8 bytes each: the dims kstep_d0<1> assigns);
  //  bf16 V copy 2h + c: dim row 64h + l, chunk c (keys 8c..8c+7); fp8 V copy
  //   h: dim row 64h + l (16 keys).
  const uint32_t koff = (uint32_t)((lane & 15) * (D * (FP8 ? 1 : 2)) + 16 * (lane >> 4));
  const uint32_t voff = (uint32_t)((FP8 ? 16 : 32) * lane);
  typedef __attribute__((address_space(4))) const int cint;
  typedef __attribute__((address_space(4))) const float cfloat;

  const int w = blockIdx.x * kSideWaves + wave;
  const long long x_end = min<long long>((long long)(w + 1) * C, T);
  const size_t head_stride = (size_t)H * TILE;
  long long x = (long long)w * C;
  while (x < x_end) {
    const int i = __builtin_amdgcn_readfirstlane(last_le(psum, NSEQ, x, H));
    const int nb = __builtin_amdgcn_readfirstlane(psum[i + 1] - psum[i]);
    const long long base = (long long)__builtin_amdgcn_readfirstlane(psum[i]) * H;
    const int g = (int)((x - base) / nb);
    const long long sstart = base + (long long)g * nb;
    const long long seg_end = min(x_end, sstart + nb);
    const int slot = w + i * H + g;
    int qrow, ctx, lo;
    seq_blocks(a, i, qrow, ctx, lo);
    qrow = __builtin_amdgcn_readfirstlane(qrow);  // uniform: scalar copy bases
    ctx = __builtin_amdgcn_readfirstlane(ctx);
    lo = __builtin_amdgcn_readfirstlane(lo);
    const int blk0 = (lo >> 4) + (int)(x - sstart);
    const int nblk = (int)(seg_end - x);
    const int kend = min(ctx, (blk0 + nblk) * 16);
    const cint* bt = (const cint*)(a.block_table + (size_t)i * a.bt_stride);
    const uint8_t* kcache = reinterpret_cast<const uint8_t*>(a.k_cache) + (size_t)g * TILE;
    const uint8_t* vcache = reinterpret_cast<const uint8_t*>(a.v_cache) + (size_t)g * TILE;

    // the group's G query heads to LDS, repeated over the 4 MFMA rows (row r
    // holds head r % G; groups of 8: 8 rows), then the first tiles
    wait_lgkmcnt0();
    {
      const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.query) + ((size_t)qrow * a.num_heads + g * G) * D * 2;
      if constexpr (G8) {
        copy16_to_lds<true>(qsrc, 16u * lane, q_lds);
        copy16_to_lds<true>(qsrc + 1024, 16u * lane, q_lds + 1024);
      } else {
        copy16_to_lds<true>(qsrc, 16u * (uint32_t)(lane % (16 * G)), q_lds);
      }
    }
    const int ntile = 2 * nblk;  // tile u: block blk0 + u/2, K if u is even, else V
    auto issue = [&](int u) {
      const uint8_t* src = ((u & 1) ? vcache : kcache) + (size_t)(uint32_t)bt[blk0 + (u >> 1)] * head_stride;
      const uint32_t dst = ring_lds + (uint32_t)(u % NS) * TILE;
      if ((u & 1) && !FP8) {
#pragma unroll
        for (int c = 0; c < 4; ++c) copy16_to_lds<true>(src + 2048 * (c >> 1) + 16 * (c & 1), voff, dst + 1024 * c);
      } else if (u & 1) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) copy16_to_lds<true>(src + 1024 * c, voff, dst + 1024 * c);
      } else {
#pragma unroll
        for (int c = 0; c < CPT; ++c) copy16_to_lds<true>(src + 64 * c, koff, dst + 1024 * c);
      }
    };
    for (int u = 0; u < NS - 1 && u < ntile; ++u) issue(u);
    // tile u is in LDS once at most CPT * (NS - 1) copies issued after it are
    // outstanding; tile u + NS - 1 reuses the slot of tile u - 1
    auto next = [&](int u) {
      wait_lgkmcnt0();
      if (u + NS - 1 < ntile) {
        issue(u + NS - 1);
        wait_vmcnt<CPT * (NS - 1)>();
      } else {
        wait_vmcnt<0>();
      }
    };

    // O rows 0..3 (o0: dims 0..63, o1: 64..127) and, for groups of 8, rows
    // 4..7 (o2, o3)
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f}, o2 = {0.f, 0.f, 0.f, 0.f}, o3 = {0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;
    for (int n = 0; n < nblk; ++n) {
      const int b = blk0 + n;
      // ---- scores of block b ----
      next(2 * n);
      const uint32_t ks = ring_lds + (uint32_t)((2 * n) % NS) * TILE;
      const uint32_t qs = q_lds + (uint32_t)((lane & (QR - 1)) * 256);
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
      float kscale = a.scale_log2, vscale = 1.f;
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 kw = lds_read16(ks + 1024 * h + 16 * lane);
#pragma unroll
          for (int t = 0; t < 2; ++t) {  // k-step 2h + t: dims 64h + 16(l/16) + 8t
            const u32x4 qf = lds_read16(qs + 128 * h + 32 * (lane >> 4) + 16 * t);
            st = mfma_bf16_16x16x32(fp8x8_to_bf16x8(kw[2 * t], kw[2 * t + 1]), qf, st);
          }
        }
        const uint32_t phys = (uint32_t)bt[b];  // the block's scales (scalar loads)
        kscale *= ((const cfloat*)a.k_scale)[phys];
        vscale = ((const cfloat*)a.v_scale)[phys];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 kf = lds_read16(ks + 1024 * j + 16 * lane);
          const u32x4 qf = lds_read16(qs + 64 * j + 16 * (lane >> 4));
          st = mfma_bf16_16x16x32(kf, qf, st);
        }
      }
      // lane's keys: b*16 + 4*(lane/16) + r, head row lane % QR
      const bool edge = b * 16 < lo || b * 16 + 16 > kend;
      float xs[4], lmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = st[r] * kscale;
        if (edge) {
          const int kp = b * 16 + 4 * (lane >> 4) + r;
          v = (kp >= lo && kp < kend) ? v : -INFINITY;
        }
        xs[r] = v;
        lmax = fmaxf(lmax, v);
      }
      // lazy rescaling as in pair_step: the max moves only when a block's
      // exceeds it by more than 2^8. The block's max over the four lane
      // groups of a head is taken only when some lane's own scores do (a
      // wave vote decides: the same outcome, without two cross-lane
      // exchanges through LDS on most blocks)
      if (__any(lmax > m + 8.f)) {
        const float tmax = strided_max<16>(lmax);
        const bool up = tmax > m + 8.f;
        const float alpha = up ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;
        m = up ? tmax : m;
        lsum *= alpha;
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {  // lane hh holds head row hh's factor
          const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), hh));
          o0[hh] *= ah;
          o1[hh] *= ah;
          if constexpr (G8) {
            const float bh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 4 + hh));
            o2[hh] *= bh;
            o3[hh] *= bh;
          }
        }
      }
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(xs[r] - m);
        lsum += e;
        p[r] = e * vscale;  // (fp8: the block's V scale moves onto the weights)
      }
      const uint32_t h0 = pack_bf16x2(p[0], p[1]), h1 = pack_bf16x2(p[2], p[3]);
      const uint32_t l0 = pack_bf16x2(p[0] - bf16_lo(h0), p[1] - bf16_hi(h0));
      const uint32_t l1 = pack_bf16x2(p[2] - bf16_lo(h1), p[3] - bf16_hi(h1));

      // ---- O += P V of block b ----
      next(2 * n + 1);
      const uint32_t vs = ring_lds + (uint32_t)((2 * n + 1) % NS) * TILE;
      const bool vtail = b * 16 + 16 > kend;  // keys past the context may hold anything: zero them
      // mask of the key pair (kk, kk + 1) in a packed bf16 word
      auto keep2 = [&](int kk) {
        return (kk < kend ? 0x0000ffffu : 0u) | (kk + 1 < kend ? 0xffff0000u : 0u);
      };
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // dim row 64h + lane, 16 keys
          const u32x4 vw = lds_read16(vs + 1024 * h + 16 * lane);
          uint32_t vb[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) fp8x4_to_bf16x4(vw[q], vb[2 * q], vb[2 * q + 1]);
          if (vtail) {
#pragma unroll
            for (int t = 0; t < 8; ++t) vb[t] &= keep2(b * 16 + 2 * t);
          }
          f32x4& o = h ? o1 : o0;
          o = side_pv<0>(h0, h1, l0, l1, vb[0], vb[1], o);
          o = side_pv<4>(h0, h1, l0, l1, vb[2], vb[3], o);
          o = side_pv<8>(h0, h1, l0, l1, vb[4], vb[5], o);
          o = side_pv<12>(h0, h1, l0, l1, vb[6], vb[7], o);
          if constexpr (G8) {
            f32x4& ob = h ? o3 : o2;
            ob = side_pv<1>(h0, h1, l0, l1, vb[0], vb[1], ob);
            ob = side_pv<5>(h0, h1, l0, l1, vb[2], vb[3], ob);
            ob = side_pv<9>(h0, h1, l0, l1, vb[4], vb[5], ob);
            ob = side_pv<13>(h0, h1, l0, l1, vb[6], vb[7], ob);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          u32x4 v0 = lds_read16(vs + 1024 * c + 16 * lane);        // dim lane, keys 8c..8c+7
          u32x4 v1 = lds_read16(vs + 1024 * (2 + c) + 16 * lane);  // dim 64 + lane
          if (vtail) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const uint32_t msk = keep2(b * 16 + 8 * c + 2 * t);
              v0[t] &= msk;
              v1[t] &= msk;
            }
          }
          if (c == 0) {
            o0 = side_pv<0>(h0, h1, l0, l1, v0[0], v0[1], o0);
            o1 = side_pv<0>(h0, h1, l0, l1, v1[0], v1[1], o1);
            o0 = side_pv<4>(h0, h1, l0, l1, v0[2], v0[3], o0);
            o1 = side_pv<4>(h0, h1, l0, l1, v1[2], v1[3], o1);
            if constexpr (G8) {
              o2 = side_pv<1>(h0, h1, l0, l1, v0[0], v0[1], o2);
              o3 = side_pv<1>(h0, h1, l0, l1, v1[0], v1[1], o3);
              o2 = side_pv<5>(h0, h1, l0, l1, v0[2], v0[3], o2);
              o3 = side_pv<5>(h0, h1, l0, l1, v1[2], v1[3], o3);
            }
          } else {
            o0 = side_pv<8>(h0, h1, l0, l1, v0[0], v0[1], o0);
            o1 = side_pv<8>(h0, h1, l0, l1, v1[0], v1[1], o1);
            o0 = side_pv<12>(h0, h1, l0, l1, v0[2], v0[3], o0);
            o1 = side_pv<12>(h0, h1, l0, l1, v1[2], v1[3], o1);
            if constexpr (G8) {
              o2 = side_pv<9>(h0, h1, l0, l1, v0[0], v0[1], o2);
              o3 = side_pv<9>(h0, h1, l0, l1, v1[0], v1[1], o3);
              o2 = side_pv<13>(h0, h1, l0, l1, v0[2], v0[3], o2);
              o3 = side_pv<13>(h0, h1, l0, l1, v1[2], v1[3], o3);
            }
          }
        }
      }
    }

    // ---- the segment's result: lane hh (< 4) holds head row hh's max and
    // sum; rows hh < G are the group's heads ----
    const float L = strided_sum<16>(lsum);
    const bool single = (sstart / C) == ((sstart + nb - 1) / C);
    if (single) {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * a.num_heads + g * G) * D + lane;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float Lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(L), hh));
        const float inv = Lh > 0.f ? 1.f / Lh : 0.f;
        const float va = hh < 4 ? o0[hh & 3] : o2[hh & 3], vb = hh < 4 ? o1[hh & 3] : o3[hh & 3];
        op[hh * D] = f32_to_bf16(va * inv);
        op[hh * D + 64] = f32_to_bf16(vb * inv);
      }
      if (a.lse != nullptr && lane < G)
        a.lse[(size_t)qrow * a.num_heads + g * G + lane] = (m + log2f(L)) * kLn2;
    } else {
      const size_t rec = (size_t)slot * a.rec_cols;
      float* op = a.part_o + rec * D + lane;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        op[hh * D] = hh < 4 ? o0[hh & 3] : o2[hh & 3];
        op[hh * D + 64] = hh < 4 ? o1[hh & 3] : o3[hh & 3];
      }
      if (lane < G) {
        a.part_ml[(rec + lane) * 2] = m;
        a.part_ml[(rec + lane) * 2 + 1] = L;
      }
    }
    x = seg_end;
  }
}

bool decode_side_supported(int q_kind, int cache_kind, int head_size, int group) {
  return q_kind == KBF16 && (cache_kind == KBF16 || cache_kind == KFP8) && head_size == 128 &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

template <int CK, int G>
static hipError_t run_decode_side(const DecodeArgs& a, hipStream_t st) {
  const int grid = device_cu_count();
  const size_t lds = decode_side_lds_bytes(a.num_seqs, G);
  // the dynamic-LDS limit this instantiation was raised to, per device
  static std::atomic<size_t> lds_set[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || lds_set[dev].load(std::memory_order_relaxed) < lds) {
    e = hipFuncSetAttribute((const void*)decode_side<CK, G>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) lds_set[dev].store(lds, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((decode_side<CK, G>), dim3(grid), dim3(256), lds, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = a.num_seqs * a.num_heads;
  hipLaunchKernelGGL((decode_split_merge<128, false>), dim3((waves + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

// The side kernel (one workgroup per CU) and the merge, on `st`. The
// workspace is the split plan's (a.split_waves >= the side kernel's waves).
hipError_t launch_decode_side(const DecodeArgs& a, int cache_kind, hipStream_t st) {
  if (a.split_waves < device_cu_count() * kSideWaves || a.one_per_stream) return hipErrorInvalidValue;
  const int G = a.num_heads / a.num_kv_heads;
  if (cache_kind == KBF16) {
    if (G == 8) return run_decode_side<KBF16, 8>(a, st);
    if (G == 4) return run_decode_side<KBF16, 4>(a, st);
    if (G == 2) return run_decode_side<KBF16, 2>(a, st);
    if (G == 1) return run_decode_side<KBF16, 1>(a, st);
  } else if (cache_kind == KFP8) {
    if (G == 8) return run_decode_side<KFP8, 8>(a, st);
    if (G == 4) return run_decode_side<KFP8, 4>(a, st);
    if (G == 2) return run_decode_side<KFP8, 2>(a, st);
    if (G == 1) return run_decode_side<KFP8, 1>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
