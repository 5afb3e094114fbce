// Device-side helpers shared by the gfx950 kernels of libra.
//
// Register layouts of the two matrix-core instructions used here (CDNA3/CDNA4
// MFMA, 64-lane wavefront, lane l, half h = l / 32):
//
//   v_mfma_f32_32x32x16_bf16   A: 32(M) x 16(K), lane holds 8 bf16 of row m = l%32
//                              B: 16(K) x 32(N), lane holds 8 bf16 of column n = l%32
//                              (lanes of half h hold the K-slice h; A and B must agree
//                              on which k each register element is, nothing else)
//   v_mfma_f32_32x32x2_f32     A, B: one float per lane, k = h
//   C/D (both): 16 floats per lane; element i is row (i/4)*8 + 4h + i%4, column l%32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Combine a value across the two 32-lane halves of the wavefront.  v_permlane32_swap
// with the same register as both operands returns {value of lane l%32, value of lane
// 32 + l%32} in every lane, so max / sum of the pair is the same in both halves (and the
// sum is formed in the same order in both halves, so the halves agree bitwise).
// max(a, b) for a, b below +inf (scores are finite, or -inf where masked): the median of
// (a, b, FLT_MAX), one instruction that needs no quieting of its inputs (fmaxf of values
// the compiler cannot prove quiet, such as MFMA results, costs three)
__device__ __forceinline__ float max_finite(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, 3.40282347e38f);
}

__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_finite(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats -> two bf16 (round to nearest even) packed in one dword, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a;
  __bf16 y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &u) { return __builtin_bit_cast(bf16x8, u); }

// Byte select across two dwords (v_perm_b32): selector bytes 0-3 pick from `lo`, 4-7 from `hi`.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// ---- LDS addressing and direct global->LDS loads -------------------------------
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// 32-bit LDS offset of a __shared__ object (generic -> local address space).
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  return (uint32_t)(size_t)(const lds_u8 *)p;
}
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  return *(const lds_u32x4 *)(size_t)addr;
}
__device__ __forceinline__ s16x4 lds_read_tr16_b64(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(size_t)addr);
}

// One 16-byte-per-lane direct load from global memory into LDS: lane l's bytes land at
// LDS offset lds + 16*l (lds must be wave-uniform).  Issued through inline assembly so
// the compiler's wait analysis does not see an LDS write in flight (it would otherwise
// drain every LDS read queue).  Consequences the callers honour: every reader of the
// destination waits explicitly (s_waitcnt vmcnt(0), then a barrier); loads the compiler
// does track stay correctly waited, because memory loads complete in issue order and
// uncounted extra loads only make the compiler's vmcnt(N) waits stricter.  M0 needs one
// wait state before the load reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0: no compiler-generated code here uses it
__device__ __forceinline__ void dma_b128(const void *tile_base, int lane_off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(lane_off), "s"(tile_base), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Document of token t in a packed stream: [ds, de) with cu[d] <= t < cu[d+1] (the last
// such d; cu[0] is 0).  A token past the last document, or offsets that break the rules,
// give the empty range [t+1, t+1).  At most ceil(log2(n+1)) probes, all inside cu[0..n].
__device__ __forceinline__ void doc_bounds(const int32_t *cu, int n, int t, int T, int &ds,
                                           int &de) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  ds = de = t + 1;
  if (lo >= n) return;
  const int a0 = min(max(cu[lo], 0), T), a1 = min(max(cu[lo + 1], a0), T);
  if (a0 <= t && t < a1) {
    ds = a0;
    de = a1;
  }
}

}  // namespace ra
