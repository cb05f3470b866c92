// Device helpers shared by the paged-attention kernels (gfx950 / CDNA4).
//
// Element storage: fp32 as float, bf16 as its 16 bits (uint16_t), OCP e4m3fn
// as a byte. bf16 pairs travel packed in one 32-bit register so that the
// dot2 instruction (two bf16 products accumulated in fp32) can consume them
// without unpacking.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

enum CacheKind { KF32 = 0, KBF16 = 1, KFP8 = 2 };

template <int CK> struct CacheElem;
template <> struct CacheElem<KF32> { typedef float T; static constexpr int bytes = 4; };
template <> struct CacheElem<KBF16> { typedef uint16_t T; static constexpr int bytes = 2; };
template <> struct CacheElem<KFP8> { typedef uint8_t T; static constexpr int bytes = 1; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 (the compiler emits v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// acc + a.lo*b.lo + a.hi*b.hi for packed bf16 pairs, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Two e4m3fn bytes (bytes 0,1 or 2,3 of w) -> two floats, exact.
__device__ __forceinline__ f32x2 fp8x2_lo(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}
__device__ __forceinline__ f32x2 fp8x2_hi(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
}
// Four e4m3fn bytes -> two packed bf16 pairs (exact: every e4m3 value is a bf16
// value). gfx950 converts a byte pair straight to packed bf16 (scale 1.0:
// checked equal to the fp32 route for all 65536 code pairs, NaNs included).
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& p01, uint32_t& p23) {
  p01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  p23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Eight e4m3fn bytes (two words) -> eight bf16 (four packed pairs).
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  uint32_t a, b, c, d;
  fp8x4_to_bf16x4(w0, a, b);
  fp8x4_to_bf16x4(w1, c, d);
  return u32x4{a, b, c, d};
}

// ---- cross-lane reductions -------------------------------------------------
// DPP row (16-lane) patterns: quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror. After the first two a quad holds its total; half-mirror pairs
// quad i with quad 1-i of each 8-lane half, mirror pairs the two halves.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_QP_1032 = 0xB1;
constexpr int DPP_QP_2301 = 0x4E;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// Sum over aligned groups of N lanes (N in {1,2,4,8,16,32,64}); every lane of
// the group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<DPP_QP_1032>(x);
  if constexpr (N >= 4) x += dpp<DPP_QP_2301>(x);
  if constexpr (N >= 8) x += dpp<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp<DPP_ROW_MIRROR>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Max / sum over lanes that share (lane % STRIDE) — i.e. across the 64/STRIDE
// groups of STRIDE consecutive lanes. STRIDE is a power of two.
template <int STRIDE>
__device__ __forceinline__ float strided_max(float x) {
  if constexpr (STRIDE <= 1) x = fmaxf(x, dpp<DPP_QP_1032>(x));
  if constexpr (STRIDE <= 2) x = fmaxf(x, dpp<DPP_QP_2301>(x));
  if constexpr (STRIDE <= 4) x = fmaxf(x, __shfl_xor(x, 4));
  if constexpr (STRIDE <= 8) x = fmaxf(x, __shfl_xor(x, 8));
  if constexpr (STRIDE <= 16) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (STRIDE <= 32) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
template <int STRIDE>
__device__ __forceinline__ float strided_sum(float x) {
  if constexpr (STRIDE <= 1) x += dpp<DPP_QP_1032>(x);
  if constexpr (STRIDE <= 2) x += dpp<DPP_QP_2301>(x);
  if constexpr (STRIDE <= 4) x += __shfl_xor(x, 4);
  if constexpr (STRIDE <= 8) x += __shfl_xor(x, 8);
  if constexpr (STRIDE <= 16) x += __shfl_xor(x, 16);
  if constexpr (STRIDE <= 32) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming loads for data read once per call (decode K/V): the nontemporal
// hint keeps them from displacing cached lines and measured ~12% faster on
// scattered 4 KiB tiles than ordinary loads.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 load8_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// log2(e): scores are kept premultiplied by scale*log2(e) so that exp2 is used.
constexpr float LOG2E = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- LDS staging: direct global -> LDS copies and the waits around them ----
// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding):
// at most N of this wave's vector memory operations (loads and global -> LDS
// copies, in issue order) still outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0) alone: this wave's LDS (and scalar) operations done.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Workgroup barrier that does not wait for this wave's outstanding memory
// operations (copies of later steps stay in flight across it).
__device__ __forceinline__ void barrier_keep_loads() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// A 16-byte global -> LDS copy per lane, from base + lane_offset (base
// uniform): lane i's chunk lands at byte lds_base + 16 i. Written as inline
// assembly so that the compiler does not see an LDS store: it would
// otherwise drain every outstanding copy before each LDS read of a loop.
// Completion is tracked by the vector-memory counter (wait_vmcnt); other
// waves see the data after a barrier. M0 holds the LDS base of a copy (read
// when the copy issues) and is restored afterwards; a copy must not directly
// follow a write of M0. NT: nontemporal (data read once).
template <bool NT = false>
__device__ __forceinline__ void copy16_to_lds(const void* base, uint32_t lane_offset, uint32_t lds_base) {
  uint32_t saved;
  if constexpr (NT) {
    __asm__ volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(lane_offset), "s"(base), "s"(lds_base)
        : "memory");
  } else {
    __asm__ volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(lane_offset), "s"(base), "s"(lds_base)
        : "memory");
  }
}

// Two such copies (a K and a V chunk, each from its own base) in one block.
template <bool NT = false>
__device__ __forceinline__ void copy16x2_to_lds(const void* base0, uint32_t off0, uint32_t lds0, const void* base1,
                                                uint32_t off1, uint32_t lds1) {
  uint32_t saved;
  if constexpr (NT) {
    __asm__ volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %6\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %4 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off0), "s"(base0), "v"(off1), "s"(base1), "s"(lds0), "s"(lds1)
        : "memory");
  } else {
    __asm__ volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %6\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %4\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off0), "s"(base0), "v"(off1), "s"(base1), "s"(lds0), "s"(lds1)
        : "memory");
  }
}

// The lane id, recomputed where it is used: the compiler cannot hoist a
// volatile asm, so values derived from it are rematerialised instead of
// being kept live across a loop (or spilled, and a spill reload waits for
// every copy in flight).
__device__ __forceinline__ int lane_id_here() {
  int l;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// LDS byte address of a __shared__ object (uniform), and raw LDS accesses by
// address.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  typedef __attribute__((address_space(3))) const T lds_t;
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_t*)p);
}
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
  return *(const lds_u32x4*)(uintptr_t)addr;
}
__device__ __forceinline__ void lds_write8(uint32_t addr, uint32_t lo, uint32_t hi) {
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  *(lds_u32x2*)(uintptr_t)addr = u32x2{lo, hi};
}

}  // namespace pa
