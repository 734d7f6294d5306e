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
    lo = (__builtin_bit_cast(uint32_t, f0) >> 16) | (__builtin_bit_cast(uint32_t, f1) & 0xFFFF0000u);
    hi = (__builtin_bit_cast(uint32_t, f2) >> 16) | (__builtin_bit_cast(uint32_t, f3) & 0xFFFF0000u);
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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh from its definition via exp: tanh(t) = sign(t) * (1 - e^{-2|t|}) / (1 + e^{-2|t|}),
// with e^y computed as 2^(y log2 e) on the hardware exp2 and a hardware reciprocal.
__device__ __forceinline__ float tanh_via_exp2(float t) {
  const float e = fast_exp2(-2.0f * kLog2e * fabsf(t));
  const float r = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
  return copysignf(r, t);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

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
