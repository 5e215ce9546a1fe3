// Device helpers shared by the gfx950 kernels of the MoE hot path.
//
// Number formats are implemented from their definitions with integer
// operations so that every rounding is explicit:
//   bf16  — the upper 16 bits of an IEEE binary32, rounded to nearest even;
//   e4m3  — OCP FP8 E4M3FN (bias 7, 3 mantissa bits, max 448, subnormal
//           step 2^-9), rounded to nearest even; callers clamp to +-448.
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

// Nearest E4M3FN value (as a float) to v, |v| <= 448, ties to even.
// Below 2^-6 the grid is uniform with step 2^-9, so scaling by 2^9 (exact)
// and rounding to an integer (round-half-even) gives the code; above it the
// 23-bit binary32 mantissa is rounded to 3 bits with the usual carry.
__device__ __forceinline__ float e4m3_round(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = u & 0x80000000u;
  uint32_t a = u & 0x7fffffffu;
  if (a < 0x3c800000u) {  // |v| < 2^-6
    float r = __builtin_rintf(__uint_as_float(a) * 512.0f) * (1.0f / 512.0f);
    return __uint_as_float(__float_as_uint(r) | sign);
  }
  a += 0x7ffffu + ((a >> 20) & 1u);
  a &= 0xfff00000u;
  return __uint_as_float(a | sign);
}

// Fake-quant of one value with scale s > 0 (IEEE division and product).
__device__ __forceinline__ uint32_t qdq_e4m3(float x, float s) {
  float r = x / s;
  r = fminf(fmaxf(r, -448.0f), 448.0f);
  float q = e4m3_round(r);
  return f32_to_bf16(q * s);
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
