// Fake-quantization of bf16 rows: FP8 (OCP E4M3FN) per 1x128 block or with
// one per-tensor scale, NVFP4 and MXFP4 (E2M1 elements in 16- and 32-channel
// blocks), plus max calibration.
//
// Source: "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM
// Mega-MoE", PR summary and "How it works" (dispatch and combine
// quantizers, calibrated or constant combine scale); "[Kernel] DeepEP
// dispatch-combine kernel integration", review thread on the low-latency
// dispatch (FP8 with per-block scales).  The FP4 units are named, not
// defined, by the Mega-MoE page (NVFP4 dispatch and combine units) and the
// permute-scratch page (an MXFP4 expert path); their definitions here are
// the formats' published ones (see the header).
//
// Layout: every thread owns 8 consecutive channels (one 16-byte vector), so
// 16 lanes cover one 128-channel block (2 an NVFP4 block, 4 an MXFP4 block)
// and the block amax is a butterfly over those lanes.  Loads and stores are fully coalesced 16-byte accesses.
#include "common.h"

namespace moe {

// E2M1 (FP4) rounding of r with |r| <= 6: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
// 6; a value halfway between two goes to the one with mantissa bit 0 (so the
// halfway points 0.25, 1.25, 2.5 and 5 round down, 0.75, 1.75 and 3.5 up).
// The sign is kept, also on a zero.
__device__ __forceinline__ float e2m1_round(float r) {
  const float a = fabsf(r);
  const float q = a <= 0.25f  ? 0.0f
                  : a < 0.75f ? 0.5f
                  : a <= 1.25f ? 1.0f
                  : a < 1.75f ? 1.5f
                  : a <= 2.5f ? 2.0f
                  : a < 3.5f  ? 3.0f
                  : a <= 5.0f ? 4.0f
                              : 6.0f;
  return copysignf(q, r);
}

// MODE: 0 FP8 per-tensor scale, 1 FP8 per 128-channel block, 2 NVFP4 (16-
// channel blocks, E4M3 block scale under the per-tensor scale), 3 MXFP4
// (32-channel blocks, power-of-two scale).
template <int MODE>
__global__ void __launch_bounds__(256) fake_quant_kernel(
    const uint16_t* __restrict__ in, uint16_t* out, int64_t n_rows, int H,
    const int32_t* __restrict__ row_src, const float* __restrict__ scale,
    float* __restrict__ block_scales, float* __restrict__ amax_out) {
  // lanes per block (each lane holds 8 channels); 0: no blocks
  constexpr int kGroup = MODE == 1 ? 16 : MODE == 2 ? 2 : MODE == 3 ? 4 : 0;
  const int vec_per_row = H / 8;
  const int64_t nvec = n_rows * vec_per_row;
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // Every lane of a group shares one row and one block (128 | H), and nvec
  // is a multiple of 16, so a group is either wholly in range or not.
  const bool in_range = v < nvec;
  const int64_t r = in_range ? v / vec_per_row : 0;
  const bool active = in_range && (row_src == nullptr || row_src[r] >= 0);

  uint4 raw = make_uint4(0, 0, 0, 0);
  if (in_range) raw = reinterpret_cast<const uint4*>(in)[v];
  float f[8];
  unpack8(raw, f);
  float m = 0.0f;
  if (active) {
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
  }
  if (kGroup > 1) {
#pragma unroll
    for (int off = kGroup / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kGroup));
  }

  // the block's scale: s (FP8), S = b * g (NVFP4) or X (MXFP4); bscale is
  // what block_scales receives
  float s = 0.0f, bscale = 0.0f;
  int xexp = 0;
  const float g = scale ? *scale : 0.0f;
  if (MODE == 0) {
    s = g;
  } else if (MODE == 1) {
    s = m / 448.0f;  // IEEE division
    bscale = s;
  } else if (MODE == 2) {
    float q = m / (6.0f * g);  // IEEE; 0 / 0 (an all-zero block) -> 0
    if (q != q) q = 0.0f;
    q = fminf(q, 448.0f);
    const int p = __builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false);  // E4M3, nearest even
    bscale = __builtin_amdgcn_cvt_f32_fp8(p, 0);
    s = bscale * g;
  } else {
    if (m > 0.0f) {
      int e;
      frexpf(m, &e);  // m = f 2^e, f in [0.5, 1): floor(log2 m) = e - 1
      xexp = min(max(e - 1 - 2, -127), 127);
      s = ldexpf(1.0f, xexp);
    }
    bscale = s;
  }
  if (kGroup && block_scales && in_range && !(MODE == 2 && scale == nullptr) &&
      (threadIdx.x & (kGroup - 1)) == 0)
    block_scales[v / kGroup] = active ? bscale : 0.0f;  // block = row * (H / 8G) + block

  if (amax_out) {
    float wm = m;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wm = fmaxf(wm, __shfl_xor(wm, off, kWave));
    if ((threadIdx.x & 63) == 0 && wm > 0.0f)
      atomicMax(reinterpret_cast<unsigned int*>(amax_out), __float_as_uint(wm));
  }

  if (!in_range) return;
  if ((MODE == 0 || MODE == 2) && scale == nullptr) return;  // calibration only
  uint4 res;
  if (!active) {
    if (out == in) return;
    res = raw;
  } else if (!(s > 0.0f)) {
    res = make_uint4(0, 0, 0, 0);
  } else if (MODE <= 1) {
    uint32_t w[4];
    qdq8_rcp(f, s, 1.0f / s, rcp_scale_ok(s), w);
    res = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    // NVFP4: IEEE quotient by S; MXFP4: exact scaling by 2^-xexp.  Both
    // saturate at 6 and round to E2M1; q * S is one rounding, q * X exact.
    const float inv = MODE == 3 ? ldexpf(1.0f, -xexp) : 0.0f;
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = MODE == 2 ? f[j] / s : f[j] * inv;
      h[j] = f32_to_bf16(e2m1_round(fminf(fmaxf(x, -6.0f), 6.0f)) * s);
    }
    res = pack8(h);
  }
  reinterpret_cast<uint4*>(out)[v] = res;
}

// The per-tensor scale from a calibrated amax, one IEEE division by the
// format's largest code magnitude: 448 for E4M3 (FP8), 6 * 448 = 2688 for
// the NVFP4 tensor scale (E2M1's 6 under an E4M3 block scale's 448).
__global__ void scale_from_amax_kernel(const float* __restrict__ amax, float* __restrict__ scale,
                                       float divisor) {
  if (threadIdx.x == 0) scale[0] = amax[0] / divisor;
}

int launch_scale_from_amax(const float* amax, float* scale, int mode, hipStream_t stream) {
  const float divisor = mode == MOE_FQ_NVFP4 ? 6.0f * 448.0f : 448.0f;
  hipLaunchKernelGGL(scale_from_amax_kernel, dim3(1), dim3(64), 0, stream, amax, scale, divisor);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_fake_quant(const uint16_t* in, uint16_t* out, int64_t n_rows, int H,
                      const int32_t* row_src, int mode, const float* scale, float* block_scales,
                      float* amax_out, hipStream_t stream) {
  const int64_t nvec = n_rows * (H / 8);
  if (nvec == 0) return MOE_OK;
  dim3 block(256), grid((unsigned)((nvec + 255) / 256));
#define MOE_FQ_LAUNCH(M)                                                                    \
  hipLaunchKernelGGL(fake_quant_kernel<M>, grid, block, 0, stream, in, out, n_rows, H, row_src, \
                     scale, block_scales, amax_out)
  switch (mode) {
    case MOE_FQ_PER_TENSOR: MOE_FQ_LAUNCH(0); break;
    case MOE_FQ_BLOCK: MOE_FQ_LAUNCH(1); break;
    case MOE_FQ_NVFP4: MOE_FQ_LAUNCH(2); break;
    case MOE_FQ_MXFP4: MOE_FQ_LAUNCH(3); break;
    default: return MOE_ERR_INVALID_ARG;
  }
#undef MOE_FQ_LAUNCH
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
