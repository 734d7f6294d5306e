// Device helpers for gfx950 (CDNA4): code widening, MFMA, cross-lane ops.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aqp_internal.h"

namespace aqp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
// 16 wave-uniform block-table entries, kept as one vector value (registers): an array here ends
// up in scratch memory once a select between two of its elements becomes an indexed load
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr float kLog2e = 1.4426950408889634f;

// 16x16x32 bf16 MFMA: D = A(16x32) * B(32x16) + C.
// Lane l supplies A row (l % 16), k = 8*(l/16) .. +7; B column (l % 16), same k;
// and holds C rows 4*(l/16) .. +3 of column (l % 16).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x16 bf16 MFMA: lane l supplies A row (l % 16), k = 4*(l/16) .. +3; B column (l % 16),
// same k; C as above.
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Widen four 1-byte codes (one dword) to four bf16, exactly: every E4M3, E5M2
// and INT8 value is representable in bf16.
template <int DT>
__device__ __forceinline__ void widen4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  if constexpr (DT == AQP_KV_FP8_E4M3) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
    lo = __builtin_bit_cast(uint32_t, a);
    hi = __builtin_bit_cast(uint32_t, b);
  } else if constexpr (DT == AQP_KV_FP8_E5M2) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w, 1.0f, true);
    lo = __builtin_bit_cast(uint32_t, a);
    hi = __builtin_bit_cast(uint32_t, b);
  } else {
    // int8: sign-extend each byte, convert to fp32 (exact), keep the top half
    // (an integer of magnitude <= 128 has at most 8 significant bits).
    const float f0 = (float)(((int32_t)(w << 24)) >> 24);
    const float f1 = (float)(((int32_t)(w << 16)) >> 24);
    const float f2 = (float)(((int32_t)(w << 8)) >> 24);
    const float f3 = (float)(((int32_t)w) >> 24);
    // one byte permute packs the upper halves of two floats
    lo = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1), __builtin_bit_cast(uint32_t, f0), 0x07060302u);
    hi = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f3), __builtin_bit_cast(uint32_t, f2), 0x07060302u);
  }
}

// Eight codes (two dwords) -> MFMA operand of eight bf16.
template <int DT>
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
  uint32_t r0, r1, r2, r3;
  widen4<DT>(w0, r0, r1);
  widen4<DT>(w1, r2, r3);
  uint4 u = make_uint4(r0, r1, r2, r3);
  return __builtin_bit_cast(bf16x8, u);
}

// Eight codes of one scale (per-group mode) -> bf16(value * s), rounded to nearest even once.
template <int DT>
__device__ __forceinline__ bf16x8 widen8_scaled(uint32_t w0, uint32_t w1, float s) {
  const bf16x8 e = widen8<DT>(w0, w1);
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)((float)e[i] * s);
  return r;
}

template <int DT>
__device__ __forceinline__ bf16x4 widen4v(uint32_t w) {
  uint32_t r0, r1;
  widen4<DT>(w, r0, r1);
  return __builtin_bit_cast(bf16x4, make_uint2(r0, r1));
}

// LDS transpose read of 8-bit data (gfx950 ds_read_b64_tr_b8). Within each
// group of 16 lanes, lanes 2i and 2i+1 point at bytes 0..7 and 8..15 of
// "row" i (i = 0..7); output lane j of the group receives byte (j % 8) of the
// half (j / 8) of rows 0..7, i.e. column j of the 8 x 16 byte tile.
__device__ __forceinline__ i32x2 lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
}

// Direct global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4): lane l's
// 16 bytes from `g` land at LDS byte address lds_base + 16 * l. lds_base must be wave-uniform.
// Issued by hand so that the waits below can be exact: the compiler's own tracking of these
// copies waits for every outstanding one before any LDS read, which would drain a multi-stage
// pipeline.
__device__ __forceinline__ void dma16_to_lds(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(g) : "memory");
}

// Direct global -> LDS copy of 4 bytes per lane (global_load_lds_dword): lane l's 4 bytes land at
// LDS byte address lds_base + 4 * l (lanes with exec off write nothing). lds_base wave-uniform.
__device__ __forceinline__ void dma4_to_lds(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(g) : "memory");
}

// Wait until at most n of this wave's vector memory operations are outstanding (n < 16).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
  }
}

// LDS byte address of a pointer into the dynamic shared allocation.
// Compile-time form of the wait above.
template <int N>
__device__ __forceinline__ void wait_vmcnt_c() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait for the oldest of this wave's tile copies when `ahead` later tiles (ipt copies each) may
// stay in flight; ahead < ns.
template <int IPT, int NS>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  static_assert(NS >= 2 && NS <= 3, "ring depth");
  if (NS == 3 && ahead >= 2) wait_vmcnt_c<IPT * (NS - 1)>();
  else if (ahead >= 1) wait_vmcnt_c<IPT>();
  else wait_vmcnt_c<0>();
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Read-only view in the constant address space: uniform indexes then compile to scalar loads
// (block tables, schedule items), which leave the vector memory counter to the KV traffic.
template <typename T>
using cptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ __forceinline__ cptr<T> as_const(const T* p) {
  return (cptr<T>)(p);
}

// Copy a record (a multiple of 16 bytes) out of the constant address space.
template <typename T>
__device__ __forceinline__ T load_const(cptr<T> p) {
  static_assert(sizeof(T) % 16 == 0, "records are whole 16-byte words");
  typedef int v4i __attribute__((ext_vector_type(4)));
  v4i w[sizeof(T) / 16];
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 16); ++i) w[i] = ((cptr<v4i>)p)[i];
  T r;
  __builtin_memcpy(&r, w, sizeof(T));
  return r;
}

// n / d for the constants of invariant_divisor (uniform operands keep it on the scalar unit)
__device__ __forceinline__ uint32_t div_invariant(uint32_t n, uint32_t m, int32_t shift) {
  const uint32_t t = __umulhi(n, m);
  return (t + ((n - t) >> 1)) >> shift;
}

// n / d for 0 <= n < d + 128 and 1 <= d <= 65536, from rd = 1.0f / d (rounded to float): the
// quotient of (n + 1/2) / d lies at least 1/(2d) from an integer, and the rounding of rd and of
// the product move it by less than 2^-23 of its value (< (d + 129) / d * 2^-23 < 1/(2d)), so
// truncation gives the exact integer quotient. (Used where a 16-key tile meets blocks of any
// size: n is a row offset inside the tile's first block plus a row of the tile.)
__device__ __forceinline__ int small_quot(int n, float rd) { return (int)(((float)n + 0.5f) * rd); }

// e[j] for a per-lane j in [0, 16) and 16 wave-uniform values (a select tree on j's bits).
__device__ __forceinline__ int32_t sel16(i32x16 e, int j) {
  const bool b0 = j & 1, b1 = j & 2, b2 = j & 4, b3 = j & 8;
  const int32_t a0 = b0 ? e[1] : e[0], a1 = b0 ? e[3] : e[2], a2 = b0 ? e[5] : e[4], a3 = b0 ? e[7] : e[6];
  const int32_t a4 = b0 ? e[9] : e[8], a5 = b0 ? e[11] : e[10], a6 = b0 ? e[13] : e[12], a7 = b0 ? e[15] : e[14];
  const int32_t c0 = b1 ? a1 : a0, c1 = b1 ? a3 : a2, c2 = b1 ? a5 : a4, c3 = b1 ? a7 : a6;
  const int32_t d0 = b2 ? c1 : c0, d1 = b2 ? c3 : c2;
  return b3 ? d1 : d0;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh from its definition via exp: tanh(t) = sign(t) * (1 - e^{-2|t|}) / (1 + e^{-2|t|}),
// with e^y computed as 2^(y log2 e) on the hardware exp2 and a hardware reciprocal.
__device__ __forceinline__ float tanh_via_exp2(float t) {
  const float e = fast_exp2(-2.0f * kLog2e * fabsf(t));
  const float r = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
  return copysignf(r, t);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Max / sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows of a wave), in VALU:
// v_permlane16_swap exchanges rows 0<->1 and 2<->3, v_permlane32_swap the two halves.
__device__ __forceinline__ float max_over_rows(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}
__device__ __forceinline__ float sum_over_rows(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), false, false);
  v = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), false, false);
  return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);  // finite inputs
  return (uint16_t)(u >> 16);
}

}  // namespace aqp
