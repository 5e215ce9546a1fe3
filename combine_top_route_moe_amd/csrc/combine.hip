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
#include <algorithm>
#include <atomic>

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

// The combine with FP8 QDQ through a table.  The quantizer's arithmetic
// (qdq8_rcp: about eleven vector operations per element) made the
// large combines ALU-bound; its result depends only on the 16-bit input, and
// on the sign only through a copy of it (the quotient, the clamp, the E4M3
// and bf16 roundings and the product are all odd in x, and the clamped value
// takes x's sign explicitly), so each workgroup first evaluates the same
// function once for every magnitude pattern (32768 entries, 64 KB of LDS)
// and then looks each element up: qdq(x) = table[x & 0x7fff] | sign(x).  The
// grid is persistent (one 1024-thread workgroup per CU, each building its
// table once), and used only for combines large enough that building the
// table costs less than the arithmetic it saves.
constexpr int kLutThreads = 1024;
constexpr int kLutEntries = 1 << 15;

__device__ __forceinline__ void lut_unpack8(const uint4& v, const uint16_t* tab, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = ((uint32_t)tab[w[j] & 0x7fffu] << 16) | ((w[j] << 16) & 0x80000000u);
    const uint32_t hi = ((uint32_t)tab[(w[j] >> 16) & 0x7fffu] << 16) | (w[j] & 0x80000000u);
    f[2 * j] = __uint_as_float(lo);
    f[2 * j + 1] = __uint_as_float(hi);
  }
}

__global__ void __launch_bounds__(kLutThreads) combine_lut_kernel(
    const uint16_t* __restrict__ rows, int64_t num_rows, const int32_t* __restrict__ row_of,
    const uint16_t* __restrict__ shared, int T, int K, int H,
    const float* __restrict__ qdq_scale, uint16_t* __restrict__ out,
    int32_t* __restrict__ dev_error) {
  __shared__ uint16_t tab[kLutEntries];
  const float s = *qdq_scale;
  const float inv_s = 1.0f / s;
  const bool rcp_ok = rcp_scale_ok(s);
  // the table: thread t evaluates magnitudes 8 (t + i kLutThreads) .. +8
  for (int e0 = threadIdx.x * 8; e0 < kLutEntries; e0 += kLutThreads * 8) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = bf16_to_f32((uint32_t)(e0 + j));
    uint32_t q[4];
    qdq8_rcp(x, s, inv_s, rcp_ok, q);
    *reinterpret_cast<uint4*>(&tab[e0]) = make_uint4(q[0], q[1], q[2], q[3]);
  }
  __syncthreads();
  const int vec_per_row = H / 8;
  const int64_t nvec = (int64_t)T * vec_per_row;
  for (int64_t v = (int64_t)blockIdx.x * kLutThreads + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * kLutThreads) {
    const int64_t t = v / vec_per_row;
    const int c = (int)(v - t * vec_per_row);
    const int32_t* ro = row_of + t * K;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    const uint4 sraw =
        shared ? reinterpret_cast<const uint4*>(shared + t * H)[c] : make_uint4(0, 0, 0, 0);
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
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4 x = r[j] >= 0 ? __builtin_nontemporal_load(
                                        reinterpret_cast<const u32x4*>(rows + (int64_t)r[j] * H) + c)
                                  : u32x4{0u, 0u, 0u, 0u};
        raw[j] = make_uint4(x.x, x.y, x.z, x.w);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (r[j] < 0) continue;
        float f[8];
        lut_unpack8(raw[j], tab, f);
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
    reinterpret_cast<uint4*>(out + t * H)[c] = pack8(h);
  }
}

// CUs of the current device (cached per device).
static int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
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

// From this many 16-byte output vectors (8M elements) on, the table form:
// measured on the deepseek-shape combine (T=4096, H=7168, K=8 plus a shared
// slot), the arithmetic form takes about 130 us and the table form about
// 100 us; building the table takes a few microseconds per workgroup.
constexpr int64_t kLutMinVectors = int64_t(1) << 20;

int launch_combine(const uint16_t* rows, int64_t num_rows, const int32_t* row_of,
                   const uint16_t* shared, int T, int K, int H, const float* qdq_scale,
                   uint16_t* out, int32_t* dev_error, hipStream_t stream) {
  const int64_t nvec = (int64_t)T * (H / 8);
  if (nvec == 0) return MOE_OK;
  dim3 block(256), grid((unsigned)((nvec + 255) / 256));
  if (qdq_scale && nvec >= kLutMinVectors) {
    const int64_t slots = cu_count();
    const int64_t need = (nvec + kLutThreads - 1) / kLutThreads;
    hipLaunchKernelGGL(combine_lut_kernel, dim3((unsigned)std::min(slots, need)),
                       dim3(kLutThreads), 0, stream, rows, num_rows, row_of, shared, T, K, H,
                       qdq_scale, out, dev_error);
  } else if (qdq_scale)
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, stream, rows, num_rows, row_of,
                       shared, T, K, H, qdq_scale, out, dev_error);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, stream, rows, num_rows, row_of,
                       shared, T, K, H, qdq_scale, out, dev_error);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
