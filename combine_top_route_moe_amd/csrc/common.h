// Device helpers shared by the gfx950 kernels of the MoE hot path.
//
// Number formats:
//   bf16  — the upper 16 bits of an IEEE binary32, rounded to nearest even
//           (the gfx950 conversion instruction);
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

// binary32 -> bf16 bits, round to nearest, ties to even; NaN -> a quiet NaN.
// The conversion is the gfx950 instruction (v_cvt_pk_bf16_f32), which was
// checked on the GPU against the integer form (add 0x7fff plus the kept
// lsb, keep the upper half) over all 2^32 binary32 patterns: identical for
// every non-NaN input, denormals included.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// FP8 fake-quant of bf16 values x with scale s > 0, given inv_s = 1.0f / s
// (the IEEE quotient, i.e. the correctly rounded reciprocal):
//   bf16( e4m3( clamp(x / s, -448, 448) ) * s )
// with the IEEE binary32 quotient x / s and product.  The quotient comes
// from the reciprocal by one correction step (Markstein's: q = x * inv_s,
// the residual q * s - x is exact in one FMA, and q - residual * inv_s
// rounds to the correctly rounded quotient).  That holds for every bf16 x
// while the residual cannot underflow, which rcp_scale_ok's range
// guarantees; it was checked on the host against the IEEE quotient for every
// finite bf16 x with 57 000 scales (every amax / 448 and random and
// edge-pattern scales across the range).  Before the correction q is clamped
// to +-512 so that an overflowing product stays finite (anything past 448
// saturates either way).  The quotient has the sign of x; copying that sign
// onto the clamped value keeps a zero's sign too.  The rounding to E4M3 is
// the hardware conversion (v_cvt_pk_fp8_f32, OCP E4M3FN, round to nearest
// even on gfx950) and back (v_cvt_pk_f32_fp8, exact); the clamp keeps it
// away from overflow.  Outside the range the quotient itself is computed.
__device__ __forceinline__ bool rcp_scale_ok(float s) {
  return s >= 0x1p-90f && s <= 0x1p90f;
}
// 8 values at once; out[j] holds the bf16 results of values 2j and 2j+1
// (low half first).
__device__ __forceinline__ void qdq8_rcp(const float* x, float s, float inv_s, bool rcp_ok,
                                         uint32_t* out) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  float r[8];
  if (rcp_ok) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q = __builtin_amdgcn_fmed3f(x[j] * inv_s, -512.0f, 512.0f);
      const float res = __builtin_fmaf(q, s, -x[j]);
      r[j] = __builtin_fmaf(-res, inv_s, q);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = x[j] / s;
  }
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const float r0 = __builtin_copysignf(__builtin_amdgcn_fmed3f(r[j], -448.0f, 448.0f), x[j]);
    const float r1 =
        __builtin_copysignf(__builtin_amdgcn_fmed3f(r[j + 1], -448.0f, 448.0f), x[j + 1]);
    const int p = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
    const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8(p, false);
    const f32x2_t q = {d.x * s, d.y * s};
    out[j / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(q, bf16x2_t));
  }
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
