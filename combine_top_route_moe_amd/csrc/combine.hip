// Ordered combine of the per-(token, slot) rows.
//
// Source: "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM
// Mega-MoE", PR summary and "How it works": the order is fixed there — the
// token's routed rows are added slot by slot, lowest slot index first, into
// a float32 sum that begins at zero; the result is rounded to bf16 once; a
// fused shared expert comes after all routed slots and is never quantized.
//
// Each thread owns 8 consecutive channels of one token (a 16-byte vector):
// it walks the token's K slots in order, gathers one vector per valid slot
// (a contiguous 16-byte load from that slot's row) and adds it with plain
// binary32 adds — the file is built with -ffp-contract=off and there is no
// multiply to fuse with — so the order of the adds is exactly the page's.
// Stores are coalesced 16-byte vectors of the output row.
#include "common.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes, native vector

// The ordered sum for one 16-byte vector (channels 8c .. 8c+7) of token t,
// rounded once to bf16.  Returns whether the token has a valid routed slot.
template <bool QDQ>
__device__ __forceinline__ bool combine_vec(const uint16_t* __restrict__ rows, int64_t num_rows,
                                            const int32_t* __restrict__ ro,
                                            const uint16_t* __restrict__ shared, int K, int H,
                                            int64_t t, int c, float s, float inv_s, bool rcp_ok,
                                            int32_t* __restrict__ dev_error, uint4& out) {
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  bool routed = false;
  // the shared expert's vector depends on nothing: load it first
  const uint4 sraw =
      shared ? reinterpret_cast<const uint4*>(shared + t * H)[c] : make_uint4(0, 0, 0, 0);
  // slots in groups of 8: the group's row gathers are all issued before its
  // adds, which then run in slot order
  for (int k0 = 0; k0 < K; k0 += 8) {
    int32_t r[8];
    uint4 raw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      r[j] = k0 + j < K ? ro[k0 + j] : -1;
      if (r[j] >= num_rows) {
        raise_error(dev_error, MOE_DEVERR_ROW_RANGE);
        r[j] = -1;
      }
    }
    // every routed row is read exactly once: non-temporal loads (measured:
    // the 1.1 GB combine of a 16k-token batch 209 -> 186 us)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 v = r[j] >= 0 ? __builtin_nontemporal_load(
                                      reinterpret_cast<const u32x4*>(rows + (int64_t)r[j] * H) + c)
                                : u32x4{0u, 0u, 0u, 0u};
      raw[j] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (r[j] < 0) continue;
      routed = true;
      float f[8];
      unpack8(raw[j], f);
      if (QDQ) {
        uint32_t w[4];
        qdq8_rcp(f, s, inv_s, rcp_ok, w);
        unpack8(make_uint4(w[0], w[1], w[2], w[3]), f);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = acc[i] + f[i];
    }
  }
  if (shared) {
    float f[8];
    unpack8(sraw, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = acc[j] + f[j];
  }
  uint32_t h[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) h[j] = f32_to_bf16(acc[j]);
  out = pack8(h);
  return routed;
}

template <bool QDQ>
__global__ void __launch_bounds__(256) combine_kernel(
    const uint16_t* __restrict__ rows, int64_t num_rows, const int32_t* __restrict__ row_of,
    const uint16_t* __restrict__ shared, int T, int K, int H,
    const float* __restrict__ qdq_scale, uint16_t* __restrict__ out,
    int32_t* __restrict__ dev_error) {
  const int vec_per_row = H / 8;
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= (int64_t)T * vec_per_row) return;
  const int64_t t = v / vec_per_row;
  const int c = (int)(v - t * vec_per_row);
  const float s = QDQ ? *qdq_scale : 1.0f;
  const float inv_s = QDQ ? 1.0f / s : 1.0f;
  const bool rcp_ok = QDQ && rcp_scale_ok(s);
  uint4 o;
  combine_vec<QDQ>(rows, num_rows, row_of + t * K, shared, K, H, t, c, s, inv_s, rcp_ok,
                   dev_error, o);
  reinterpret_cast<uint4*>(out + t * H)[c] = o;
}

// Layout check: the same sum without QDQ, compared bit for bit with the
// output a fused kernel produced.  `state` bits: 1 = checked (the call
// returns at once), 2 = this call saw a routed slot, 4 = this call saw a
// mismatch; combine_check_finish_kernel folds them into 0 or 1.
__global__ void __launch_bounds__(256) combine_check_kernel(
    const uint16_t* __restrict__ rows, int64_t num_rows, const int32_t* __restrict__ row_of,
    const uint16_t* __restrict__ shared, int T, int K, int H,
    const uint16_t* __restrict__ kernel_out, int32_t* state, int32_t* __restrict__ dev_error) {
  if (state && *state == 1) return;
  const int vec_per_row = H / 8;
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bool routed = false, bad = false;
  if (v < (int64_t)T * vec_per_row) {
    const int64_t t = v / vec_per_row;
    const int c = (int)(v - t * vec_per_row);
    uint4 o;
    routed = combine_vec<false>(rows, num_rows, row_of + t * K, shared, K, H, t, c, 1.0f, 1.0f,
                                false, dev_error, o);
    const uint4 k = reinterpret_cast<const uint4*>(kernel_out + t * H)[c];
    bad = o.x != k.x || o.y != k.y || o.z != k.z || o.w != k.w;
    if (bad) raise_error(dev_error, MOE_DEVERR_LAYOUT);
  }
  if (state) {
    const uint64_t any_routed = __ballot(routed), any_bad = __ballot(bad);
    if ((threadIdx.x & 63) == 0 && (any_routed || any_bad))
      atomicOr(state, (any_routed ? 2 : 0) | (any_bad ? 4 : 0));
  }
}

__global__ void combine_check_finish_kernel(int32_t* state) {
  if (threadIdx.x != 0) return;
  const int32_t s = *state;
  if (s == 1) return;
  *state = ((s & 2) && !(s & 4)) ? 1 : 0;
}

int launch_combine_check(const uint16_t* rows, int64_t num_rows, const int32_t* row_of,
                         const uint16_t* shared, int T, int K, int H, const uint16_t* kernel_out,
                         int32_t* state, int32_t* dev_error, hipStream_t stream) {
  const int64_t nvec = (int64_t)T * (H / 8);
  if (nvec > 0)
    hipLaunchKernelGGL(combine_check_kernel, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0,
                       stream, rows, num_rows, row_of, shared, T, K, H, kernel_out, state,
                       dev_error);
  if (state)
    hipLaunchKernelGGL(combine_check_finish_kernel, dim3(1), dim3(64), 0, stream, state);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_combine(const uint16_t* rows, int64_t num_rows, const int32_t* row_of,
                   const uint16_t* shared, int T, int K, int H, const float* qdq_scale,
                   uint16_t* out, int32_t* dev_error, hipStream_t stream) {
  const int64_t nvec = (int64_t)T * (H / 8);
  if (nvec == 0) return MOE_OK;
  dim3 block(256), grid((unsigned)((nvec + 255) / 256));
  if (qdq_scale)
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, stream, rows, num_rows, row_of,
                       shared, T, K, H, qdq_scale, out, dev_error);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, stream, rows, num_rows, row_of,
                       shared, T, K, H, qdq_scale, out, dev_error);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
