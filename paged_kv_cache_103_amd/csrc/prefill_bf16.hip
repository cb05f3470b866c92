// Chunked-prefill paged attention for bf16 and fp8 (e4m3fn) KV caches on
// gfx950 matrix cores: scores on 32x32x16 bf16 MFMA, the weighted sum of
// values on 32x32x16 fp16 MFMA, both with fp32 accumulation.
//
// What it computes: every query row of a chunk longer than one token attends
// causally to its sequence's cached keys, read through the block table; query
// row r of a chunk of q_len rows in a context of ctx tokens sits at position
// ctx - q_len + r ("大模型推理优化学习笔记", "Chunked Prefill";
// "从静态批处理到状态化推理集群", "Chunked prefill：在共置引擎里治理阶段干扰").
// Each cached K/V row serves many queries, so the work is a dense contraction
// ("大模型推理优化学习笔记", "计算密集与访存密集") and runs on MFMA.
//
// Shape of the work (one workgroup = 8 waves = 256 query columns of one KV
// head: 256/G tokens x the G query heads of the group; one workgroup per
// CU, so that the staging of each K/V step is shared by 8 waves):
//  * keys advance in steps of 32 (two 16-token blocks). A wave computes the
//    32 x 32 score tile S^T = K Q^T of its 32 columns with head_size/16 MFMAs
//    (queries are the B operand, kept in registers), then O^T += V^T P^T with
//    head_size/32 output tiles x 2 key halves;
//  * the softmax weights enter the PV product as fp16 (11 significant bits;
//    bf16's 8 move outputs dominated by a few keys by up to 2^-9 |v|), scaled
//    by 2^7 so that they stay in fp16's range (p <= 2^15) and keep 2^-31 of
//    resolution below the running maximum. The values are therefore
//    converted to fp16 once per workgroup, in LDS: exact for |v| in
//    [2^-14, 65504], and smaller magnitudes keep 2^-24 of absolute
//    resolution. A value beyond fp16's range becomes infinity there and
//    leaves inf or NaN in the accumulators of every column; a tile whose
//    accumulators end non-finite is computed again with the value product
//    taken from the cache itself: the values as bf16 (exact; fp8 widened
//    exactly, its block scale moved onto the weights) against the weights
//    split into bf16 hi + lo, two MFMAs per term. Every finite cached value
//    is in the kernel's domain; the fp32 accumulator bounds it only through
//    2^15 * sum |v| < 3.4e38;
//  * score rows are fed in a permuted key order, so that the accumulator of
//    lane l holds, for its column, exactly the 8-key runs the PV B operand
//    wants from it: probabilities never leave the lane. A column's 32 keys
//    live in lanes l and l^32, so its running max needs one lane swap;
//  * the loop is software-pipelined inside each wave: iteration i issues the
//    score MFMAs of step i+1 and the PV MFMAs of step i-1 while the vector
//    ALUs run the softmax of step i. The O^T rescale that a new running max
//    asks for (lazy: only when the max grows by more than 2^8) is applied at
//    the top of the next iteration, after step i-1's PV and before step i's;
//  * K and V reach LDS by direct global->LDS copies issued three steps
//    ahead, into rings of three (K) and five (V) 32-key slots, one barrier
//    per step. The 32 tiles of a KV head read each block through their
//    XCD's L2 (HBM fetches 1.00x the chunk's K/V); beside the decode kernel
//    of a mixed batch the copies are nontemporal instead (the step ~2%
//    faster there, at 1.33x the fetched bytes). A V slot is converted to fp16 in place two steps after its
//    copy was issued and read by the PV product two steps later (each
//    thread converts one 16-byte chunk). The copies place 16-byte chunks so
//    that the MFMA operand reads hit distinct LDS banks;
//  * masks (causal edge, sliding window, context end) are evaluated only in
//    the steps that cross an edge; values of keys past the context are
//    zeroed in the last step, because the block of a partial last block may
//    hold anything past the context;
//  * fp8 caches (one fp32 scale per block for K and one for V): the K tiles
//    stay e4m3 in LDS (half the bytes) and are widened to bf16 in registers
//    just before their MFMA (exact); the score takes the block's K scale.
//    The V tiles are copied to a ring of their own and the conversion pass
//    writes them as fp16 values times the block's V scale into the V slots
//    the bf16 path uses (a tile whose scaled values overflow fp16 is computed
//    again with the exact product above).
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "prefill_tiles.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16_f16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}
// Two floats as packed fp16, rounded to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}

template <int D>
struct PfShape {
  static constexpr int STEP = 32;            // keys per step (two blocks)
  static constexpr int DK = D / 16;          // score MFMAs per step (k = 16 over head_size)
  static constexpr int DT = D / 32;          // 32-row tiles of head_size in O^T
  static constexpr int KSLOT = STEP * D;     // bf16 elements of one K slot: [32][D]
  static constexpr int VSLOT = 2 * D * 16;   // one V slot: two [D][16] block tiles
  static constexpr int AHEAD = 3;            // steps a copy is issued ahead of its step
  static constexpr int KSLOTS = AHEAD;
  static constexpr int VSLOTS = AHEAD + 2;
  static constexpr int BLK_BYTES = 16 * D * 2;
};

// Chunk swizzles (16-byte chunk index XOR a function of the row), chosen so
// that the 16 lanes the LDS serves together read 16 distinct bank groups:
// K rows are read by 32 lanes (32 permuted keys, one chunk column each);
// V^T rows by 32 lanes (32 consecutive rows, one of two chunks).
template <int D>
__device__ __forceinline__ int k_swizzle(int key) {
  if constexpr (D == 128) return key & 15;
  else return (key >> 1) & 7;
}
__device__ __forceinline__ int v_swizzle(int d) { return (d >> 3) & 1; }
// fp8 K rows (D bytes = D/16 chunks), read 16 bytes per lane: each group
// of 16 lanes reads one chunk column of 16 keys (key bits 0..3), and the
// swizzle by the key bits the row stride leaves alone puts them on 16
// distinct bank groups.
template <int D>
__device__ __forceinline__ int k8_swizzle(int key) {
  if constexpr (D == 128) return (key >> 1) & 7;
  else return (key >> 2) & 3;
}

// Score row m of a step holds this key of the step.
__device__ __forceinline__ int step_key_of_row(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

constexpr int PF_NW = 8;             // waves per workgroup
constexpr int PF_NT = 64 * PF_NW;    // threads per workgroup

template <int D, int G, int CK>
// Register budget: at most 224 per wave (the attribute's count is doubled on
// this target, whose VGPR file holds the accumulation registers too), so
// that two waves per SIMD leave 64 of the 512 to a decode wave running beside
// them (decode_side).
__global__ __launch_bounds__(PF_NT) __attribute__((amdgpu_waves_per_eu(2, 2), amdgpu_num_vgpr(112))) void
prefill_bf16_kernel(PrefillArgs a) {
  using S = PfShape<D>;
  constexpr int NW = PF_NW, NT = PF_NT;
  constexpr int TQ = 32 * NW / G;
  constexpr bool FP8 = CK == KFP8;
  constexpr int E = FP8 ? 1 : 2;          // bytes per cached element
  constexpr int KSLOTB = 32 * D * E;      // bytes of one K slot
  constexpr int RVSLOTB = 32 * D;         // bytes of one raw fp8 V slot
  __shared__ __attribute__((aligned(16))) uint16_t kring[S::KSLOTS * KSLOTB / 2];
  __shared__ __attribute__((aligned(16))) uint16_t vring[S::VSLOTS * S::VSLOT];
  __shared__ __attribute__((aligned(16))) uint8_t rvring[FP8 ? S::KSLOTS * RVSLOTB : 16];
  __shared__ int sh_scan[NT];
  __shared__ int sh_found[3];
  __shared__ int sh_redo;  // some column's accumulators ended non-finite

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x % a.num_kv_heads;
  const PrefillTile tile = find_prefill_tile<NT>(a.cu_seqlens, a.num_seqs, TQ, blockIdx.x / a.num_kv_heads, sh_scan,
                                             sh_found);
  if (tile.seq < 0) return;
  const int s = tile.seq;

  // lengths and block ids are read-only for the kernel's lifetime: read them
  // through the constant address space, so that the uniform ones take scalar
  // loads (vector loads would share the counter of the in-flight copies)
  typedef __attribute__((address_space(4))) const int cint;
  const cint* cu = ((const cint*)(a.cu_seqlens));
  const int q0 = cu[s];
  const int qlen = cu[s + 1] - q0;
  const int ctx = ((const cint*)(a.context_lens))[s];
  const int tok0 = tile.tile * TQ;
  const int ntok = min(TQ, qlen - tok0);
  const int qpos_first = ctx - qlen + tok0;
  const int qpos_last = qpos_first + ntok - 1;
  const int W = a.window;
  const int lo_first = W > 0 ? max(0, qpos_first - W + 1) : 0;
  const int b_last = (ctx - 1) >> 4;
  const cint* bt = ((const cint*)(a.block_table)) + (size_t)s * a.bt_stride;
  const int jstart = (lo_first >> 5) << 5;
  const int nsteps = (qpos_last - jstart) / 32 + 1;

  // ---- this lane's column and its queries (B operand of S^T = K Q^T) ----
  const int h = lane >> 5, c32 = lane & 31;
  const int col = wave * 32 + c32;
  const int tok = col / G, head = col % G;
  const int qpos = qpos_first + tok;
  // scores are max-reduced before scaling, so the scale must be positive: a
  // negative scale flips the query signs instead (exact in bf16)
  const bool neg = a.scale_log2 < 0.f;
  float c = fabsf(a.scale_log2);
  c = c > 0.f ? c : 1.17549435e-38f;  // scale 0 (uniform weights) as the smallest normal
  // bf16 caches: k-step ks of the score product covers dims 16 ks + 8 h ..
  // + 7 for lane half h; fp8 caches read 16 key bytes per lane, so there
  // k-steps 2 m and 2 m + 1 cover the lane half's 16 dims 32 m + 16 h .. + 15
  // (the order of a dot product's terms is free; K and Q use the same one)
  u32x4 qf[S::DK];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.query) +
                         ((size_t)(q0 + tok0 + tok) * a.num_heads + g * G + head) * D;
    const uint32_t flip = neg ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < S::DK; ++ks) {
      const int d0 = FP8 ? 32 * (ks >> 1) + 16 * h + 8 * (ks & 1) : 16 * ks + 8 * h;
      qf[ks] = tok < ntok ? load16(qp + d0) : u32x4{0, 0, 0, 0};
      qf[ks][0] ^= flip; qf[ks][1] ^= flip; qf[ks][2] ^= flip; qf[ks][3] ^= flip;
    }
  }

  // ---- global -> LDS copies: a step's K slot and V slot are each written
  // by D/16 copies of 1 KiB (one 16-byte chunk per lane, lane i to byte
  // 16 i of the copy's region); wave w issues copies w + NW n, the first
  // D/16 of them K, the rest V. Each lane fetches the global chunk that
  // lands, swizzled, where the MFMA operand reads expect it. Blocks past the
  // context re-read the last block (masked, zeroed).
  constexpr int KCOPIES = D * E / 32;       // 1 KiB copies per K slot (and per V slot)
  constexpr int NCOPY = 2 * KCOPIES;
  constexpr int CPW = NCOPY >= NW ? NCOPY / NW : 1;  // copies per copying wave per step
  static_assert(NCOPY % NW == 0 || NCOPY < NW, "copy split");
  const bool copier = NCOPY >= NW || wave < NCOPY;  // (fp8, head size 64: half the waves copy)
  constexpr uint32_t TILE_BYTES = 16 * D * E;      // one (block, head) tile
  const uint32_t head_stride = (uint32_t)a.num_kv_heads * TILE_BYTES;
  const uint8_t* kcache = reinterpret_cast<const uint8_t*>(a.k_cache) + (size_t)g * TILE_BYTES;
  const uint8_t* vcache = reinterpret_cast<const uint8_t*>(a.v_cache) + (size_t)g * TILE_BYTES;
  const int b0 = jstart >> 4;
  constexpr int CPR = D / 8;  // chunks per K row
  uint32_t cp_off[CPW];
#pragma unroll
  for (int n = 0; n < CPW; ++n) {
    const int j = wave + NW * n;
    const int p = 64 * (j < KCOPIES ? j : j - KCOPIES) + lane;  // 16-byte position in the slot
    if constexpr (FP8) {
      if (j < KCOPIES) {  // K rows of D bytes, chunk-swizzled
        const int key = p / (D / 16);
        cp_off[n] = (key % 16) * D + 16 * ((p % (D / 16)) ^ k8_swizzle<D>(key));
      } else {            // raw V: the two blocks' [D][16] tiles as they are
        cp_off[n] = (p % D) * 16;
      }
    } else {
      if (j < KCOPIES) {
        const int key = p / CPR;
        cp_off[n] = (key % 16) * (2 * D) + 16 * ((p % CPR) ^ k_swizzle<D>(key));
      } else {
        const int d = (p / 2) % D;
        cp_off[n] = d * 32 + 16 * ((p % 2) ^ v_swizzle(d));
      }
    }
  }
  const uint32_t kring_lds = lds_addr(kring), vring_lds = lds_addr(vring);
  const uint32_t rvring_lds = FP8 ? lds_addr(reinterpret_cast<const uint16_t*>(rvring)) : 0u;
  // block ids are non-negative and a head's block stride is below 4 GiB
  auto copy_step = [&](int step, int kslot, int vslot) {
    if constexpr (CPW == 2) {
      // one K and one V copy per wave, both of block wave / (2 D / 64) of
      // the step
      const int b = min(b0 + 2 * step + (64 * wave) / (D * E), b_last);
      const uint64_t off = (uint64_t)(uint32_t)bt[b] * head_stride;
      const uint32_t kdst = kring_lds + kslot * KSLOTB + 1024 * wave;
      const uint32_t vdst = vring_lds + vslot * (2 * S::VSLOT) + 1024 * wave;
      if (a.nontemporal_kv)
        copy16x2_to_lds<true>(kcache + off, cp_off[0], kdst, vcache + off, cp_off[1], vdst);
      else
        copy16x2_to_lds<false>(kcache + off, cp_off[0], kdst, vcache + off, cp_off[1], vdst);
    } else {
      static_assert(CPW == 1, "one or two copies per wave");
      if (!copier) return;
      const bool isv = wave >= KCOPIES;
      const int jj = isv ? wave - KCOPIES : wave;
      const int b = min(b0 + 2 * step + (64 * jj) / (D * E), b_last);
      const uint64_t off = (uint64_t)(uint32_t)bt[b] * head_stride;
      // (fp8: the raw V ring turns with the K ring)
      const uint32_t vdst = FP8 ? rvring_lds + kslot * RVSLOTB : vring_lds + vslot * (2 * S::VSLOT);
      const uint32_t lds = isv ? vdst + 1024 * jj : kring_lds + kslot * KSLOTB + 1024 * jj;
      if (a.nontemporal_kv)
        copy16_to_lds<true>((isv ? vcache : kcache) + off, cp_off[0], lds);
      else
        copy16_to_lds<false>((isv ? vcache : kcache) + off, cp_off[0], lds);
    }
  };

  // ---- per-lane LDS read offsets ----
  const int key_l = step_key_of_row(c32);
  const int kswz_l = k_swizzle<D>(key_l);
  const int vswz_l = v_swizzle(c32);
  const uint16_t* vrow = vring + c32 * 16 + 8 * (h ^ vswz_l);
  // per-lane byte offsets of the K operand chunks (the slot adds a uniform
  // offset)
  constexpr int KREADS = FP8 ? S::DK / 2 : S::DK;  // 16-byte K operand reads per step
  uint32_t kaddr[KREADS];
#pragma unroll
  for (int j = 0; j < KREADS; ++j) {
    if constexpr (FP8)
      kaddr[j] = lds_addr(kring) + key_l * D + 16 * ((2 * j + h) ^ k8_swizzle<D>(key_l));
    else
      kaddr[j] = lds_addr(kring) + 2 * (key_l * D + 8 * ((2 * j + h) ^ kswz_l));
  }
  u32x4 kf[KREADS];  // fp8: raw bytes of two k-steps, widened just before their MFMAs
  auto scores_load = [&](int slot) {
    const uint32_t sb = __builtin_amdgcn_readfirstlane(slot * KSLOTB);
    typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
#pragma unroll
    for (int j = 0; j < KREADS; ++j) kf[j] = *(const lds_u32x4*)(uintptr_t)(kaddr[j] + sb);
  };
  auto scores_mfma = [&]() {
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < S::DK; ++ks) {
      if constexpr (FP8) {
        const int j = ks >> 1, w = 2 * (ks & 1);
        acc = mfma32x32x16(fp8x8_to_bf16x8(kf[j][w], kf[j][w + 1]), qf[ks], acc);
      } else {
        acc = mfma32x32x16(kf[ks], qf[ks], acc);
      }
    }
    return acc;
  };
  auto scores = [&](int slot) { scores_load(slot); return scores_mfma(); };

  f32x16 o[S::DT];
  float m, lsum, alpha;
  bool pending;                    // o waits for a rescale by alpha
  u32x4 pf[2];                     // P of the previous step (fp16, x 2^7), per key half

  auto pv = [&](int slot, const u32x4* pk, const uint32_t (*vmask)[4]) {
    const uint16_t* vp = vrow + slot * S::VSLOT;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 vf = *reinterpret_cast<const u32x4*>(vp + t * D * 16 + dt * 32 * 16);
        if (vmask) { vf[0] &= vmask[t][0]; vf[1] &= vmask[t][1]; vf[2] &= vmask[t][2]; vf[3] &= vmask[t][3]; }
        o[dt] = mfma32x32x16_f16(vf, pk[t], o[dt]);
      }
  };
  // The same product without the fp16 values, for a tile whose values do
  // not all fit fp16: the lane's 8 keys of each value row come straight from
  // the cache tile (bf16 exact; fp8 widened exactly and its block scale
  // moved onto the weights), the weights (fp16, x 2^7) split exactly into
  // bf16 hi + lo, two MFMAs per term.
  typedef __attribute__((address_space(4))) const float cfloat;
  auto pv_exact = [&](int step, const u32x4* pk, const uint32_t (*vmask)[4]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t bid = (uint32_t)bt[min(b0 + 2 * step + t, b_last)];
      const uint8_t* tile = vcache + (size_t)bid * head_stride;
      const float vs = FP8 ? ((const cfloat*)a.v_scale)[bid] : 1.f;
      u32x4 phi, plo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // (through a named scalar: hipcc's bit_cast of a vector element
        // subscript reads element 0 whatever the index)
        const uint32_t pe = pk[t][e];
        const f16x2_t w = __builtin_bit_cast(f16x2_t, pe);
        const float f0 = (float)w.x * vs, f1 = (float)w.y * vs;
        const uint32_t h0 = __float_as_uint(f0) & 0xffff0000u, h1 = __float_as_uint(f1) & 0xffff0000u;
        phi[e] = (h0 >> 16) | h1;
        plo[e] = pack_bf16x2(f0 - __uint_as_float(h0), f1 - __uint_as_float(h1));
      }
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) {
        const int row = dt * 32 + c32;
        u32x4 vf;
        if constexpr (FP8) {
          const u32x2 raw = *reinterpret_cast<const u32x2*>(tile + row * 16 + 8 * h);
          vf = fp8x8_to_bf16x8(raw[0], raw[1]);
        } else {
          vf = load16(tile + (row * 16 + 8 * h) * 2);
        }
        if (vmask) { vf[0] &= vmask[t][0]; vf[1] &= vmask[t][1]; vf[2] &= vmask[t][2]; vf[3] &= vmask[t][3]; }
        o[dt] = mfma32x32x16(vf, phi, o[dt]);
        o[dt] = mfma32x32x16(vf, plo, o[dt]);
        __builtin_amdgcn_sched_barrier(0);  // one value fragment live at a time (rare path)
      }
    }
  };
  // bf16 -> fp16 in place: thread tid owns the 16-byte chunk tid of the
  // slot (4 D chunks; threads past them idle). The chunk is read early in an
  // iteration and written back at its end.
  // (fp8: thread tid < 2 D owns raw chunk tid = 16 keys of dim tid % D of
  // block tid / D, and writes them as two fp16 chunks times the V scale)
  constexpr int VCH = FP8 ? 2 * D : 4 * D;
  static_assert(VCH <= NT, "one chunk per thread");
  const bool converts = VCH == NT || tid < VCH;
  u32x4 cvt = {0, 0, 0, 0};
  float cvt_scale = 1.f;
  auto convert_load = [&](int slot, int raw_slot, int step) {
    if constexpr (FP8) {
      if (converts) {
        cvt = reinterpret_cast<const u32x4*>(rvring + raw_slot * RVSLOTB)[tid];
        // both blocks' scales by uniform (scalar) loads, then picked per thread
        const float s0 = ((const cfloat*)a.v_scale)[bt[min(b0 + 2 * step, b_last)]];
        const float s1 = ((const cfloat*)a.v_scale)[bt[min(b0 + 2 * step + 1, b_last)]];
        cvt_scale = tid >= D ? s1 : s0;
      }
    } else {
      if (converts) cvt = reinterpret_cast<const u32x4*>(vring + slot * S::VSLOT)[tid];
    }
  };
  auto convert_store = [&](int slot) {
    if constexpr (FP8) {
      if (converts) {
        const int t = tid / D, d = tid % D;
        uint16_t* row = vring + slot * S::VSLOT + t * D * 16 + d * 16;
#pragma unroll
        for (int c = 0; c < 2; ++c) {  // keys 8c .. 8c + 7
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t src = cvt[2 * c + (e >> 1)];
            const f32x2 f = (e & 1) ? fp8x2_hi(src) : fp8x2_lo(src);
            w[e] = pack_f16x2(f.x * cvt_scale, f.y * cvt_scale);
          }
          *reinterpret_cast<u32x4*>(row + 8 * (c ^ v_swizzle(d))) = w;
        }
      }
    } else {
      if (converts) {
        u32x4 w = cvt;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_f16x2(bf16_lo(w[e]), bf16_hi(w[e]));
        reinterpret_cast<u32x4*>(vring + slot * S::VSLOT)[tid] = w;
      }
    }
  };

  // One pass over the tile's keys; EXACT takes the value product from the
  // cache (pv_exact) instead of the fp16 slots.
  auto pass = [&](auto exact_tag) {
  constexpr bool EXACT = decltype(exact_tag)::value;
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) o[dt] = f32x16{};
  m = -INFINITY;
  lsum = 0.f;
  alpha = 1.f;
  pending = false;
#pragma unroll
  for (int t = 0; t < 2; ++t) pf[t] = u32x4{0, 0, 0, 0};
  // ---- prologue: K and V of steps 0..2; V of step 0 converted; the V slot
  // of step -1 (read with P = 0 by the first iteration) cleared ----
#pragma unroll
  for (int i = 0; i < S::AHEAD; ++i) copy_step(i, i, i);
  {
    u32x4* vz = reinterpret_cast<u32x4*>(vring + (S::VSLOTS - 1) * S::VSLOT);
    for (int i = tid; i < S::VSLOT / 8; i += NT) vz[i] = u32x4{0, 0, 0, 0};
  }
  wait_vmcnt<0>();
  __syncthreads();
  convert_load(0, 0, 0);
  convert_store(0);
  f32x16 sc = scores(0), sc2;
  int krot = 0;  // step % KSLOTS of the next iteration
  int vrot = 0;  // step % VSLOTS of the next iteration

  // lane's keys in a step: key_off(v) + 8h, v = 0..15 (value v of the score
  // accumulator)
  auto iteration = [&](auto masked_tag, int st, f32x16& sc, f32x16& sn) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    wait_vmcnt<(S::AHEAD - 2) * CPW>();  // the copies of step st+1 have landed
    barrier_keep_loads();
    if (pending) {
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) o[dt] *= alpha;
    }
    constexpr int KS = S::KSLOTS, VS = S::VSLOTS;
    const int slot_ka = krot;                               // K of step st+AHEAD replaces K of step st
    const int slot_k1 = krot == KS - 1 ? 0 : krot + 1;      // K of step st+1
    krot = slot_k1;
    const int slot_vp = vrot == 0 ? VS - 1 : vrot - 1;      // V of step st-1
    const int slot_v1 = vrot == VS - 1 ? 0 : vrot + 1;      // V of step st+1
    const int slot_va = vrot >= 2 ? vrot - 2 : vrot + VS - 2;  // V of step st+AHEAD replaces V of step st-2
    vrot = slot_v1;
    copy_step(st + S::AHEAD, slot_ka, slot_va);
    convert_load(slot_v1, slot_k1, st + 1);  // converted below; read by the PV product two iterations on
    scores_load(slot_k1);
    __builtin_amdgcn_sched_barrier(0);
    sn = scores_mfma();                     // S of step st+1 (unused past the end)
    if constexpr (EXACT) {                  // (step -1 has P = 0: nothing to add)
      if (st > 0) pv_exact(st - 1, pf, nullptr);
    } else {
      pv(slot_vp, pf, nullptr);             // O^T += V^T P^T of step st-1
    }

    // ---- softmax of step st ----
    float x[16];
    float tmax = -INFINITY;
    const int kbase = jstart + 32 * st + 8 * h;
    float ksc[2] = {1.f, 1.f};  // fp8: K scales of the step's two blocks (scalar loads)
    if constexpr (FP8) {
      ksc[0] = ((const cfloat*)a.k_scale)[bt[min(b0 + 2 * st, b_last)]];
      ksc[1] = ((const cfloat*)a.k_scale)[bt[min(b0 + 2 * st + 1, b_last)]];
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float sv = FP8 ? sc[v] * ksc[v >> 3] : sc[v];
      if constexpr (MASKED) {
        const int kp = kbase + 16 * (v >> 3) + 4 * ((v >> 2) & 1) + (v & 3);
        const bool ok = kp <= qpos && kp < ctx && (W <= 0 || kp > qpos - W);
        sv = ok ? sv : -INFINITY;
      }
      x[v] = sv;
      tmax = fmaxf(tmax, sv);
    }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
    }
    // lazy rescaling: the running max moves only when the step's max exceeds
    // it by more than 2^8 (p stays below 256 otherwise); the final division
    // uses the same max
    const bool up = tmax > m + 8.f;
    alpha = up ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;  // 0 when m was -inf
    m = up ? tmax : m;
    lsum *= alpha;
    pending = __any(up);
    const float nb = (m == -INFINITY) ? 0.f : 7.f - m;  // weights carry a factor 2^7
    float p[16];
    float ps = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      p[v] = __builtin_amdgcn_exp2f(fmaf(x[v], c, nb));
      ps += p[v];
    }
    lsum += ps;
    // P^T operand of key half t: logical k = 8h + e <-> value v = 8t + e
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) pf[t][e] = pack_f16x2(p[8 * t + 2 * e], p[8 * t + 2 * e + 1]);
    convert_store(slot_v1);
  };

  // steps that need no mask: every column sees all 32 keys causally and
  // inside its window
  const int x1 = qpos_first - 31 - jstart;
  const int y2 = W > 0 ? qpos_last - W + 1 - jstart : 0;
  const int a_end = min(nsteps, y2 > 0 ? (y2 + 31) / 32 : 0);
  const int b_end = max(a_end, min(nsteps, x1 >= 0 ? x1 / 32 + 1 : 0));
  int st = 0;
  for (; st < a_end; ++st) { iteration(std::true_type{}, st, sc, sc2); sc = sc2; }
  for (; st + 2 <= b_end; st += 2) {  // two steps per trip: the score tiles swap roles
    iteration(std::false_type{}, st, sc, sc2);
    iteration(std::false_type{}, st + 1, sc2, sc);
  }
  for (; st < b_end; ++st) { iteration(std::false_type{}, st, sc, sc2); sc = sc2; }
  for (; st < nsteps; ++st) { iteration(std::true_type{}, st, sc, sc2); sc = sc2; }

  // ---- epilogue: PV of the last step, values past the context zeroed ----
  wait_vmcnt<0>();
  barrier_keep_loads();
  if (pending) {
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) o[dt] *= alpha;
  }
  {
    uint32_t vmask[2][4];
    const int kb = jstart + 32 * (nsteps - 1) + 8 * h;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kp = kb + 16 * t + 2 * e;
        vmask[t][e] = (kp < ctx ? 0x0000ffffu : 0u) | (kp + 1 < ctx ? 0xffff0000u : 0u);
      }
    if constexpr (EXACT) pv_exact(nsteps - 1, pf, vmask);
    else pv((nsteps - 1) % S::VSLOTS, pf, vmask);  // V of step nsteps-1
  }
  };  // pass

  if (tid == 0) sh_redo = 0;  // (read after the barriers of the first pass)
  pass(std::false_type{});
  {
    // a value beyond fp16's range leaves inf or NaN in the accumulators of
    // every column it reaches: then the tile is computed again, exactly
    bool bad = false;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) bad |= !(fabsf(o[dt][i]) <= 3.4028235e38f);
    if (__any(bad) && lane == 0) sh_redo = 1;
    __syncthreads();  // (also: no wave still reads the rings)
    if (sh_redo) pass(std::true_type{});
  }

  // ---- normalise and write: lane holds rows d = 32 dt + 8 i + 4 h + r of
  // its column ----
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    const float L = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const float inv = 1.f / L;
    // the lane's column again, from a fresh lane id: the compiler would
    // otherwise keep the query row offset live across the whole loop
    const int le = lane_id_here();
    const int col_e = wave * 32 + (le & 31);
    const int tok_e = col_e / G, head_e = col_e % G;
    if (tok_e < ntok) {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) +
                     ((size_t)(q0 + tok0 + tok_e) * a.num_heads + g * G + head_e) * D + 4 * (le >> 5);
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint2 w;
          w.x = pack_bf16x2(o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv);
          w.y = pack_bf16x2(o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv);
          *reinterpret_cast<uint2*>(op + dt * 32 + 8 * i) = w;
        }
    }
  }
}

template <int D, int G, int CK>
static hipError_t run_prefill_bf16(const PrefillArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)a.num_tiles * (unsigned)a.num_kv_heads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G, CK>), dim3(blocks), dim3(PF_NT), 0, st, a);
  return hipGetLastError();
}

template <int D, int CK>
static hipError_t run_prefill_bf16_g(const PrefillArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return run_prefill_bf16<D, 1, CK>(a, st);
    case 2: return run_prefill_bf16<D, 2, CK>(a, st);
    case 4: return run_prefill_bf16<D, 4, CK>(a, st);
    case 8: return run_prefill_bf16<D, 8, CK>(a, st);
    case 16: return run_prefill_bf16<D, 16, CK>(a, st);
  }
  return hipErrorInvalidValue;
}

int prefill_tokens_per_tile(int group) { return 32 * PF_NW / group; }

bool prefill_supported(int q_kind, int cache_kind, int head_size, int group) {
  if (head_size != 64 && head_size != 128) return false;
  if (!(group == 1 || group == 2 || group == 4 || group == 8 || group == 16)) return false;
  return q_kind == KBF16 && (cache_kind == KBF16 || cache_kind == KFP8);
}

size_t prefill_lds_bytes(int cache_kind, int head_size, int group) {
  const void* f = nullptr;
#define PA_PF_CASE(D, GG, CK) \
  if (head_size == D && group == GG && cache_kind == CK) f = (const void*)prefill_bf16_kernel<D, GG, CK>;
#define PA_PF_GROUPS(D, CK) PA_PF_CASE(D, 1, CK) PA_PF_CASE(D, 2, CK) PA_PF_CASE(D, 4, CK) PA_PF_CASE(D, 8, CK) PA_PF_CASE(D, 16, CK)
  PA_PF_GROUPS(64, KBF16) PA_PF_GROUPS(128, KBF16) PA_PF_GROUPS(64, KFP8) PA_PF_GROUPS(128, KFP8)
#undef PA_PF_GROUPS
#undef PA_PF_CASE
  if (f == nullptr) return 0;
  hipFuncAttributes at;
  if (hipFuncGetAttributes(&at, f) != hipSuccess) return 0;
  return at.sharedSizeBytes;
}

hipError_t launch_prefill(const PrefillArgs& a, int cache_kind, int head_size, hipStream_t stream) {
  const int G = a.num_heads / a.num_kv_heads;
  if (cache_kind == KBF16 && head_size == 64) return run_prefill_bf16_g<64, KBF16>(a, G, stream);
  if (cache_kind == KBF16 && head_size == 128) return run_prefill_bf16_g<128, KBF16>(a, G, stream);
  if (cache_kind == KFP8 && head_size == 64) return run_prefill_bf16_g<64, KFP8>(a, G, stream);
  if (cache_kind == KFP8 && head_size == 128) return run_prefill_bf16_g<128, KFP8>(a, G, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
