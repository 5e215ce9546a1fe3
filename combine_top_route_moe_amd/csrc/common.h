// Device helpers shared by the gfx950 kernels of the MoE hot path.
//
// Number formats:
//   bf16  — the upper 16 bits of an IEEE binary32, rounded to nearest even
//           (integer operations, so the rounding is explicit);
//   e4m3  — OCP FP8 E4M3FN (bias 7, 3 mantissa bits, max 448, subnormal
//           step 2^-9), rounded to nearest even by the gfx950 conversion
//           instructions; callers clamp to +-448 first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// binary32 -> bf16 bits, round to nearest, ties to even.  NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// FP8 fake-quant of one value with scale s > 0, given inv_s = 1.0f / s:
//   bf16( e4m3( clamp(x / s, -448, 448) ) * s )
// with the IEEE binary32 quotient x / s and product.  The quotient is formed
// as x * inv_s where that is provably the same after E4M3 rounding: the
// product lies within 3 ulp of the quotient (two roundings of at most 2^-24
// relative against the quotient's one), and E4M3 rounding keeps 3 of the 23
// mantissa bits, so wherever the product's 20 dropped bits are more than 16
// ulp from the halfway point both round alike.  Elsewhere (near a halfway
// point, in the E4M3 subnormal range below 2^-6, or when the scale is so
// small or large that its reciprocal loses precision) the quotient itself is
// computed.  The rounding to E4M3 is the hardware conversion
// (v_cvt_pk_fp8_f32, OCP E4M3FN, round to nearest even on gfx950) and back
// (v_cvt_f32_fp8, exact); the clamp keeps it away from overflow.
__device__ __forceinline__ bool rcp_scale_ok(float s) {
  return s >= 0x1p-125f && s <= 0x1p125f;
}
__device__ __forceinline__ uint32_t qdq_e4m3_rcp(float x, float s, float inv_s, bool rcp_ok) {
  float r = x * inv_s;
  const uint32_t a = __float_as_uint(r) & 0x7fffffffu;
  const int d = (int)(a & 0xfffffu) - 0x80000;
  if (!rcp_ok || a < 0x3c800000u || (d > -16 && d < 16)) r = x / s;
  r = fminf(fmaxf(r, -448.0f), 448.0f);
  const int p = __builtin_amdgcn_cvt_pk_fp8_f32(r, r, 0, false);
  return f32_to_bf16(__builtin_amdgcn_cvt_f32_fp8(p, 0) * s);
}

__device__ __forceinline__ void raise_error(int32_t* err, int code) {
  if (err) atomicCAS(err, 0, code);
}

// 8 bf16 values <-> uint4
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ uint4 pack8(const uint32_t* h) {
  uint4 v;
  v.x = h[0] | (h[1] << 16);
  v.y = h[2] | (h[3] << 16);
  v.z = h[4] | (h[5] << 16);
  v.w = h[6] | (h[7] << 16);
  return v;
}

}  // namespace moe
