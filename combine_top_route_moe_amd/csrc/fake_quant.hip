// FP8 (OCP E4M3FN) fake-quantization of bf16 rows, per 1x128 block or with
// one per-tensor scale, plus max calibration.
//
// Source: "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM
// Mega-MoE", PR summary and "How it works" (dispatch and combine
// quantizers, calibrated or constant combine scale); "[Kernel] DeepEP
// dispatch-combine kernel integration", review thread on the low-latency
// dispatch (FP8 with per-block scales).
//
// Layout: every thread owns 8 consecutive channels (one 16-byte vector), so
// 16 lanes cover one 128-channel block and the block amax is a 16-lane
// butterfly.  Loads and stores are fully coalesced 16-byte accesses.
#include "common.h"

namespace moe {

template <bool BLOCK>
__global__ void __launch_bounds__(256) fake_quant_kernel(
    const uint16_t* __restrict__ in, uint16_t* out, int64_t n_rows, int H,
    const int32_t* __restrict__ row_src, const float* __restrict__ scale,
    float* __restrict__ block_scales, float* __restrict__ amax_out) {
  const int vec_per_row = H / 8;
  const int64_t nvec = n_rows * vec_per_row;
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // Every lane of a 16-lane group shares one row and one block (128 | H), and
  // nvec is a multiple of 16, so a group is either wholly in range or not.
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

  float s;
  if (BLOCK) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 16));
    s = m / 448.0f;  // IEEE division
    if (block_scales && active && (threadIdx.x & 15) == 0) {
      const int64_t b = v / 16;  // block index = row * (H / 128) + block
      block_scales[b] = s;
    }
    if (in_range && !active && block_scales && row_src && (threadIdx.x & 15) == 0)
      block_scales[v / 16] = 0.0f;
  } else {
    s = scale ? *scale : 0.0f;
  }

  if (amax_out) {
    float wm = m;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wm = fmaxf(wm, __shfl_xor(wm, off, kWave));
    if ((threadIdx.x & 63) == 0 && wm > 0.0f)
      atomicMax(reinterpret_cast<unsigned int*>(amax_out), __float_as_uint(wm));
  }

  if (!in_range) return;
  if (!BLOCK && scale == nullptr) return;  // calibration only
  uint4 res;
  if (!active) {
    if (out == in) return;
    res = raw;
  } else {
    if (s == 0.0f) {
      res = make_uint4(0, 0, 0, 0);
    } else {
      uint32_t w[4];
      qdq8_rcp(f, s, 1.0f / s, rcp_scale_ok(s), w);
      res = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  reinterpret_cast<uint4*>(out)[v] = res;
}

__global__ void scale_from_amax_kernel(const float* __restrict__ amax, float* __restrict__ scale) {
  if (threadIdx.x == 0) scale[0] = amax[0] / 448.0f;
}

int launch_scale_from_amax(const float* amax, float* scale, hipStream_t stream) {
  hipLaunchKernelGGL(scale_from_amax_kernel, dim3(1), dim3(64), 0, stream, amax, scale);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_fake_quant(const uint16_t* in, uint16_t* out, int64_t n_rows, int H,
                      const int32_t* row_src, int mode, const float* scale, float* block_scales,
                      float* amax_out, hipStream_t stream) {
  const int64_t nvec = n_rows * (H / 8);
  if (nvec == 0) return MOE_OK;
  dim3 block(256), grid((unsigned)((nvec + 255) / 256));
  if (mode == MOE_FQ_BLOCK)
    hipLaunchKernelGGL(fake_quant_kernel<true>, grid, block, 0, stream, in, out, n_rows, H,
                       row_src, scale, block_scales, amax_out);
  else
    hipLaunchKernelGGL(fake_quant_kernel<false>, grid, block, 0, stream, in, out, n_rows, H,
                       row_src, scale, block_scales, amax_out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
