// Top-k routing: one wavefront per token row.
//
// Each lane holds the logits of experts lane, lane+64, ... in registers; the
// K winners are extracted one at a time by a wave-wide argmax with the
// (larger value, then lower index) order, so slot 0 is the largest logit
// and equal logits go to the lower expert index.  Selection compares the
// float32 logits themselves; the weights are softmax terms over the chosen
// slots (or over all experts) evaluated in double and stored as float.
// Source: "[Kernel] DeepEP dispatch-combine kernel integration", review
// threads (router ids and weights [T, K]); "Add MoE dispatch/combine fake
// quantization for vLLM's DeepGEMM Mega-MoE", review thread on the buffer
// check (padding slots carry -1).
#include "common.h"

namespace moe {

// One DPP lane movement within each row of 16 lanes (every lane active).
template <int kCtrl>
__device__ __forceinline__ int row16_dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}

// Wave-wide max (float) and min (int), the result in every lane: within each
// 16-lane row by two quad permutations and the half-row and row mirrors
// (register moves, no LDS), then the four rows' results by readlane.
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __int_as_float(row16_dpp<0xB1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(row16_dpp<0x4E>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(row16_dpp<0x141>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(row16_dpp<0x140>(__float_as_int(v))));
  const int b = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)),
                     __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)),
                     __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}
__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, row16_dpp<0xB1>(v));
  v = min(v, row16_dpp<0x4E>(v));
  v = min(v, row16_dpp<0x141>(v));
  v = min(v, row16_dpp<0x140>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Sum of x over lanes 0 .. n-1 (n <= 64, the same in every lane), read lane
// by lane in ascending order: no LDS traffic.
__device__ __forceinline__ double sum_lanes_below(double x, int n) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  double s = 0.0;
  for (int k = 0; k < n; ++k) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, k);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), k);
    s += __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
  }
  return s;
}

// A NaN logit ranks as -inf: it can never hide a real candidate from the
// argmax (every comparison with a NaN is false) and the order stays total.
__device__ __forceinline__ float rank_value(float x) { return x != x ? -__builtin_inff() : x; }

// exp(l - l_max) in double, with an l equal to l_max counting exp(0) even
// when both are infinite (inf - inf would be NaN): the limit of the softmax
// as the infinite logits grow, and for finite logits the same value.
__device__ __forceinline__ double weight_term(float l, float lmax) {
  return l == lmax ? 1.0 : exp((double)l - (double)lmax);
}

// EPL: experts per lane (E <= 64 * EPL).
template <int EPL>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits,
                                                    const uint8_t* __restrict__ row_valid,
                                                    int T, int E, int K, int renorm,
                                                    int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (t >= T) return;
  int32_t* out_idx = topk_idx + (int64_t)t * K;
  float* out_w = topk_w + (int64_t)t * K;
  if (row_valid && !row_valid[t]) {
    for (int k = lane; k < K; k += kWave) {
      out_idx[k] = -1;
      out_w[k] = 0.0f;
    }
    return;
  }

  const float* row = logits + (int64_t)t * E;
  float v[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    int e = lane + j * kWave;
    v[j] = e < E ? rank_value(row[e]) : 0.0f;
  }
  uint32_t taken = 0;  // bit j: expert lane + 64 j already chosen (or absent)
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (lane + j * kWave >= E) taken |= 1u << j;

  float sel_v = 0.0f;  // lane k keeps slot k's logit (k < 64)
  int sel_e = -1;
  float lmax = 0.0f;
  for (int k = 0; k < K; ++k) {
    // lane-local best among untaken: higher value, then lower index
    bool has = false;
    float bv = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      if (taken & (1u << j)) continue;
      int e = lane + j * kWave;
      if (!has || v[j] > bv || (v[j] == bv && e < be)) {
        has = true;
        bv = v[j];
        be = e;
      }
    }
    // wave argmax: the largest value, then the lowest index holding it (a
    // lane with no candidate offers -inf and no index, so a real expert
    // always wins); no LDS traffic — K rounds of shuffle butterflies through
    // LDS permutes took a 16k-token, 128-expert batch 35 us
    if (!has) {
      bv = -__builtin_inff();
      be = 0x7fffffff;
    }
    const float mv = wave_max_f32(bv);
    be = wave_min_i32(has && bv == mv ? be : 0x7fffffff);   // +0 and -0 tie, as in the order
    bv = mv;
    // every lane now holds the winner (bv, be)
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (k == 0) lmax = bv;
    if (lane == k) {
      sel_v = bv;
      sel_e = be;
    }
  }

  // weights: exp(l_k - l_max) / sum, in double
  double num = 0.0;
  if (lane < K) num = weight_term(sel_v, lmax);
  double den = 0.0;
  if (renorm) {
    den = sum_lanes_below(num, K);   // the K slot terms, slot order
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + j * kWave < E) den += weight_term(v[j], lmax);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, kWave);
  }
  if (lane < K) {
    out_idx[lane] = sel_e;
    out_w[lane] = (float)(num / den);
  }
}

// Rank form for E <= 64: every lane counts how many logits precede its own
// in the (larger value, then lower index) order — reading the row back from
// LDS as broadcasts — and the lanes whose rank is below K write that slot
// directly, with no serial argmax rounds.  The count costs E^2/64 compares
// per lane, so wider rows use the argmax kernel above.
template <int EPL>
__global__ void __launch_bounds__(256) route_rank_kernel(const float* __restrict__ logits,
                                                         const uint8_t* __restrict__ row_valid,
                                                         int T, int E, int K, int renorm,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  constexpr int kMaxE = EPL * kWave;
  __shared__ __attribute__((aligned(16))) float row_lds[4][kMaxE];
  __shared__ float sel_lds[4][32];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  int32_t* out_idx = topk_idx + (int64_t)t * K;
  float* out_w = topk_w + (int64_t)t * K;
  if (row_valid && !row_valid[t]) {
    for (int k = lane; k < K; k += kWave) {
      out_idx[k] = -1;
      out_w[k] = 0.0f;
    }
    return;
  }
  const float* row = logits + (int64_t)t * E;
  float v[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + j * kWave;
    v[j] = e < E ? rank_value(row[e]) : 0.0f;
    row_lds[wv][e] = v[j];
  }
  // one wave owns row_lds[wv]; its writes are visible to its own later reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  int rank[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) rank[j] = 0;
  for (int c = 0; c < E; c += 4) {
    const float4 q = *reinterpret_cast<const float4*>(&row_lds[wv][c]);
    const float qv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ej = c + u;
      if (ej >= E) break;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = lane + j * kWave;
        rank[j] += (qv[u] > v[j]) || (qv[u] == v[j] && ej < e);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + j * kWave;
    if (e < E && rank[j] < K) {
      out_idx[rank[j]] = e;
      sel_lds[wv][rank[j]] = v[j];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  // weights: exp(l_k - l_max) / sum, in double; lane k < K holds slot k
  const float lmax = sel_lds[wv][0];
  double num = 0.0;
  if (lane < K) num = weight_term(sel_lds[wv][lane], lmax);
  double den = 0.0;
  if (renorm) {
    den = sum_lanes_below(num, K);   // the K slot terms, slot order
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + j * kWave < E) den += weight_term(v[j], lmax);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, kWave);
  }
  if (lane < K) out_w[lane] = (float)(num / den);
}

int launch_route(const float* logits, const uint8_t* row_valid, int T, int E, int K, int renorm,
                 int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  const int waves = 4;
  dim3 grid((T + waves - 1) / waves), block(waves * kWave);
  int epl = (E + kWave - 1) / kWave;
  if (E % 4 == 0 && epl <= 1) {
    hipLaunchKernelGGL(route_rank_kernel<1>, grid, block, 0, stream, logits, row_valid, T, E, K,
                       renorm, topk_idx, topk_w);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
#define MOE_ROUTE_CASE(N)                                                                  \
  if (epl <= N) {                                                                          \
    hipLaunchKernelGGL(route_kernel<N>, grid, block, 0, stream, logits, row_valid, T, E, K, \
                       renorm, topk_idx, topk_w);                                          \
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;                         \
  }
  MOE_ROUTE_CASE(1)
  MOE_ROUTE_CASE(2)
  MOE_ROUTE_CASE(4)
  MOE_ROUTE_CASE(8)
  MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
