// C ABI of the MoE hot path: host-side argument checks, size queries and
// kernel launches.  Every check here looks at scalars and pointers only —
// nothing reads device memory or synchronizes — so the calls stay
// asynchronous and can be captured into a HIP graph.
#include <string.h>

#include "common.h"

namespace moe {
int launch_route(const float*, const uint8_t*, int, int, int, int, int32_t*, float*, hipStream_t);
int launch_fake_quant(const uint16_t*, uint16_t*, int64_t, int, const int32_t*, int, const float*,
                      float*, float*, hipStream_t);
int launch_scale_from_amax(const float*, float*, int, hipStream_t);
int launch_combine(const uint16_t*, int64_t, const int32_t*, const uint16_t*, int, int, int,
                   const float*, uint16_t*, int32_t*, hipStream_t);
int launch_combine_check(const uint16_t*, int64_t, const int32_t*, const uint16_t*, int, int, int,
                         const uint16_t*, int32_t*, int32_t*, hipStream_t);
size_t permute_workspace_bytes(int64_t, int);
int launch_permute(const int32_t*, const float*, const uint16_t*, int, int, int, int, int, int, int,
                   int, int64_t, int32_t*, int32_t*, uint16_t*, int32_t*, int32_t*, float*, void*,
                   int32_t*, hipStream_t);
size_t permute_noalloc_scratch_bytes();
int launch_permute_noalloc(const int32_t*, const float*, const uint16_t*, int, int, int, int, int,
                           int, int, int, int64_t, int32_t*, int32_t*, uint16_t*, int32_t*,
                           int32_t*, float*, int32_t*, hipStream_t);
size_t grouped_ffn_workspace_bytes(int64_t, int, int);
int launch_grouped_ffn(const uint16_t*, const int32_t*, const int32_t*, int, int, int,
                       const void*, const float*, const void*, const float*, const float*,
                       uint16_t*, int64_t, int, void*, int32_t*, hipStream_t);
int launch_pack_weights(const uint16_t*, const uint16_t*, int, int, int, uint16_t*, uint16_t*,
                        hipStream_t);
int launch_pack_weights_fp8(const uint16_t*, const uint16_t*, int, int, int, uint8_t*, float*,
                            uint8_t*, float*, int, hipStream_t);
int launch_quant_rows_fp8(const uint16_t*, int64_t, int, const int32_t*, uint8_t*, float*, int64_t,
                          hipStream_t);
size_t w8a8_workspace_bytes(int64_t, int, int);
int launch_grouped_ffn_w8a8(const uint8_t*, const float*, int64_t, const int32_t*, int,
                            const int32_t*, const int32_t*, int, int, int, const uint8_t*, const float*, const uint8_t*,
                            const float*, const float*, uint16_t*, int64_t, int, void*, int32_t*,
                            hipStream_t);

// Each workgroup copies runs of 4 x 256 vectors: the four loads of a thread
// are in flight together, and both sides stream past the caches
// (measured on a 1 GiB copy: 4.9 TB/s for one vector per thread and
// iteration, 5.9 TB/s for this form).
typedef uint32_t copy_vec_t __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) copy_kernel(const copy_vec_t* __restrict__ src,
                                                   copy_vec_t* __restrict__ dst, int64_t n) {
  constexpr int kUnroll = 4;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kUnroll; base < n;
       base += (int64_t)gridDim.x * 256 * kUnroll) {
    copy_vec_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      v[u] = i < n ? __builtin_nontemporal_load(src + i) : copy_vec_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}
// The read-only stream: runs of 8 x 256 vectors per workgroup, all eight
// loads of a thread in flight together, non-temporal; the xor of what a
// thread read is written only if it equals a marker, which keeps the loads.
__global__ void __launch_bounds__(256) read_kernel(const copy_vec_t* __restrict__ src,
                                                   copy_vec_t* __restrict__ sink, int64_t n) {
  constexpr int kUnroll = 8;
  copy_vec_t acc = {0u, 0u, 0u, 0u};
  for (int64_t base = (int64_t)blockIdx.x * 256 * kUnroll; base < n;
       base += (int64_t)gridDim.x * 256 * kUnroll) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      if (i < n) acc ^= __builtin_nontemporal_load(src + i);
    }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x5ca1ab1eu) sink[(blockIdx.x * 256 + threadIdx.x) & 4095] = acc;
}
}  // namespace moe

using namespace moe;

static inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or bad flag)";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape (H and I must be multiples of 128; E, G <= 1024; K <= 32)";
    case MOE_ERR_WORKSPACE: return "workspace smaller than the size query requires";
    case MOE_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case MOE_ERR_DEVICE: return "the current device is not a gfx950 (MI355X-class) GPU";
    case MOE_ERR_SCRATCH:
      return "the call needs more than moe_permute_noalloc's fixed device scratch (4 MiB); "
             "use moe_permute with a caller workspace";
    default: return "unknown status";
  }
}

int moe_device_check(int device) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return MOE_ERR_HIP;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_DEVICE;
  return MOE_OK;
}

int moe_route(const float* logits, const uint8_t* row_valid, int T, int E, int K, int flags,
              int32_t* topk_idx, float* topk_w, void* stream) {
  if (T < 0 || E < 1 || K < 1 || K > E) return MOE_ERR_INVALID_ARG;
  if (K > 32 || E > 1024) return MOE_ERR_UNSUPPORTED;
  if (flags & ~MOE_ROUTE_RENORM) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  return launch_route(logits, row_valid, T, E, K, (flags & MOE_ROUTE_RENORM) ? 1 : 0, topk_idx,
                      topk_w, as_stream(stream));
}

int64_t moe_permute_capacity(int T, int K, int num_local_experts, int flags) {
  if (T < 0 || K < 1 || num_local_experts < 1) return 0;
  const int64_t tk = (int64_t)T * K;
  if (!(flags & MOE_PERMUTE_PAD_POW2)) return tk;
  // sum_e next_pow2(c_e) <= sum_e (2 c_e - 1) over non-empty experts, and
  // each non-empty expert pads by at most next_pow2(tk) - 1 rows
  const int64_t bound = 2 * tk;
  int64_t p = 1;
  while (p < tk) p <<= 1;
  const int64_t per_expert = (int64_t)num_local_experts * p;
  return bound < per_expert ? bound : per_expert;
}

size_t moe_permute_workspace_bytes(int T, int K, int num_local_experts, int flags) {
  (void)flags;
  if (T < 0 || K < 1 || num_local_experts < 1) return 0;
  return permute_workspace_bytes((int64_t)T * K, num_local_experts);
}

// Argument checks shared by moe_permute and moe_permute_noalloc (scalars and
// pointers only).
static int check_permute_args(const int32_t* topk_idx, const float* topk_w, const uint16_t* hidden,
                              int T, int K, int H, int num_experts, int expert_begin,
                              int num_local_experts, int flags, int64_t capacity,
                              const int32_t* counts, const int32_t* cu_seqlens,
                              const uint16_t* x_perm, const int32_t* row_of,
                              const int32_t* src_of, const float* w_perm) {
  if (T < 0 || K < 1 || H < 1 || num_local_experts < 1 || capacity < 0 || expert_begin < 0)
    return MOE_ERR_INVALID_ARG;
  if ((int64_t)expert_begin + num_local_experts > (int64_t)num_experts) return MOE_ERR_INVALID_ARG;
  if (flags & ~(MOE_PERMUTE_PAD_POW2 | MOE_PERMUTE_DISPATCH_FP8)) return MOE_ERR_INVALID_ARG;
  if (H % 128 || num_local_experts > 1024 || K > 64) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * K > 0x7fffffffLL || capacity > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (!counts || !cu_seqlens) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_idx || !topk_w || !hidden || !row_of)) return MOE_ERR_INVALID_ARG;
  if (capacity > 0 && (!x_perm || !src_of || !w_perm)) return MOE_ERR_INVALID_ARG;
  if ((hidden && !aligned16(hidden)) || (x_perm && !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int moe_permute(const int32_t* topk_idx, const float* topk_w, const uint16_t* hidden, int T, int K,
                int H, int num_experts, int expert_begin, int num_local_experts, int flags,
                int64_t capacity, int32_t* counts, int32_t* cu_seqlens, uint16_t* x_perm,
                int32_t* row_of, int32_t* src_of, float* w_perm, void* workspace,
                size_t workspace_bytes, int32_t* dev_error, void* stream) {
  const int st = check_permute_args(topk_idx, topk_w, hidden, T, K, H, num_experts, expert_begin,
                                    num_local_experts, flags, capacity, counts, cu_seqlens,
                                    x_perm, row_of, src_of, w_perm);
  if (st != MOE_OK) return st;
  const size_t need = permute_workspace_bytes((int64_t)T * K, num_local_experts);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  return launch_permute(topk_idx, topk_w, hidden, T, K, H, num_experts, expert_begin,
                        num_local_experts, (flags & MOE_PERMUTE_PAD_POW2) ? 1 : 0,
                        (flags & MOE_PERMUTE_DISPATCH_FP8) ? 1 : 0, capacity, counts, cu_seqlens,
                        x_perm, row_of, src_of, w_perm, workspace, dev_error, as_stream(stream));
}

size_t moe_permute_noalloc_scratch_bytes(void) { return permute_noalloc_scratch_bytes(); }

int moe_permute_noalloc(const int32_t* topk_idx, const float* topk_w, const uint16_t* hidden,
                        int T, int K, int H, int num_experts, int expert_begin,
                        int num_local_experts, int flags, int64_t capacity, int32_t* counts,
                        int32_t* cu_seqlens, uint16_t* x_perm, int32_t* row_of, int32_t* src_of,
                        float* w_perm, int32_t* dev_error, void* stream) {
  const int st = check_permute_args(topk_idx, topk_w, hidden, T, K, H, num_experts, expert_begin,
                                    num_local_experts, flags, capacity, counts, cu_seqlens,
                                    x_perm, row_of, src_of, w_perm);
  if (st != MOE_OK) return st;
  return launch_permute_noalloc(topk_idx, topk_w, hidden, T, K, H, num_experts, expert_begin,
                                num_local_experts, (flags & MOE_PERMUTE_PAD_POW2) ? 1 : 0,
                                (flags & MOE_PERMUTE_DISPATCH_FP8) ? 1 : 0, capacity, counts,
                                cu_seqlens, x_perm, row_of, src_of, w_perm, dev_error,
                                as_stream(stream));
}

size_t moe_grouped_ffn_workspace_bytes(int64_t capacity, int num_groups, int H, int I) {
  (void)H;
  if (capacity < 0 || I < 1 || num_groups < 1) return 0;
  return grouped_ffn_workspace_bytes(capacity, num_groups, I);
}

int moe_grouped_ffn(const uint16_t* x, const int32_t* cu_seqlens, const int32_t* counts,
                    int num_groups, int H, int I, const uint16_t* w13, const uint16_t* w2,
                    const float* row_scale, uint16_t* y, int64_t capacity, int flags,
                    void* workspace, size_t workspace_bytes, int32_t* dev_error, void* stream) {
  if (num_groups < 1 || H < 1 || I < 1 || capacity < 0) return MOE_ERR_INVALID_ARG;
  if ((flags & ~(MOE_FFN_ALL | MOE_FFN_PACKED_WEIGHTS)) || !(flags & MOE_FFN_ALL))
    return MOE_ERR_INVALID_ARG;
  const int stages = flags & MOE_FFN_ALL;
  if (H % 128 || I % 128 || num_groups > 1024) return MOE_ERR_UNSUPPORTED;
  if (capacity > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (capacity == 0) return MOE_OK;   // no rows: nothing to read or write
  if (!cu_seqlens || !counts) return MOE_ERR_INVALID_ARG;
  if ((stages & MOE_FFN_GATE_UP) && (!x || !w13)) return MOE_ERR_INVALID_ARG;
  if ((stages & MOE_FFN_DOWN) && (!y || !w2)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (y && !aligned16(y)) || (w13 && !aligned16(w13)) ||
      (w2 && !aligned16(w2)))
    return MOE_ERR_INVALID_ARG;
  const size_t need = grouped_ffn_workspace_bytes(capacity, num_groups, I);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  return launch_grouped_ffn(x, cu_seqlens, counts, num_groups, H, I, w13, nullptr, w2, nullptr,
                            row_scale, y, capacity, flags, workspace, dev_error,
                            as_stream(stream));
}

int moe_grouped_ffn_fp8(const uint16_t* x, const int32_t* cu_seqlens, const int32_t* counts,
                        int num_groups, int H, int I, const uint8_t* w13q, const float* w13_scales,
                        const uint8_t* w2q, const float* w2_scales, const float* row_scale,
                        uint16_t* y, int64_t capacity, int flags, void* workspace,
                        size_t workspace_bytes, int32_t* dev_error, void* stream) {
  if (num_groups < 1 || H < 1 || I < 1 || capacity < 0) return MOE_ERR_INVALID_ARG;
  if ((flags & ~MOE_FFN_ALL) || !(flags & MOE_FFN_ALL)) return MOE_ERR_INVALID_ARG;
  if (H % 128 || I % 128 || num_groups > 1024) return MOE_ERR_UNSUPPORTED;
  if (capacity > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (capacity == 0) return MOE_OK;   // no rows: nothing to read or write
  if (!cu_seqlens || !counts) return MOE_ERR_INVALID_ARG;
  if ((flags & MOE_FFN_GATE_UP) && (!x || !w13q || !w13_scales)) return MOE_ERR_INVALID_ARG;
  if ((flags & MOE_FFN_DOWN) && (!y || !w2q || !w2_scales)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (y && !aligned16(y)) || (w13q && !aligned16(w13q)) ||
      (w2q && !aligned16(w2q)) || (w13_scales && !aligned16(w13_scales)) ||
      (w2_scales && !aligned16(w2_scales)))
    return MOE_ERR_INVALID_ARG;
  const size_t need = grouped_ffn_workspace_bytes(capacity, num_groups, I);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  // the FP8 kernels take the scale pointers as their mark: pass both (only
  // the selected stage reads its own)
  const float* s13 = w13_scales ? w13_scales : w2_scales;
  const float* s2 = w2_scales ? w2_scales : w13_scales;
  return launch_grouped_ffn(x, cu_seqlens, counts, num_groups, H, I, w13q, s13, w2q, s2,
                            row_scale, y, capacity, flags | MOE_FFN_PACKED_WEIGHTS, workspace,
                            dev_error, as_stream(stream));
}

int moe_pack_ffn_weights(const uint16_t* w13, const uint16_t* w2, int num_groups, int H, int I,
                         uint16_t* w13_packed, uint16_t* w2_packed, void* stream) {
  if (num_groups < 1 || H < 1 || I < 1) return MOE_ERR_INVALID_ARG;
  if (H % 128 || I % 128) return MOE_ERR_UNSUPPORTED;
  if (!w13 != !w13_packed || !w2 != !w2_packed) return MOE_ERR_INVALID_ARG;
  if ((w13 && (!aligned16(w13) || !aligned16(w13_packed))) ||
      (w2 && (!aligned16(w2) || !aligned16(w2_packed))))
    return MOE_ERR_INVALID_ARG;
  if ((w13 && w13 == w13_packed) || (w2 && w2 == w2_packed)) return MOE_ERR_INVALID_ARG;
  return launch_pack_weights(w13, w2, num_groups, H, I, w13_packed, w2_packed, as_stream(stream));
}

int moe_quant_rows_fp8(const uint16_t* in, int64_t n_rows, int H, const int32_t* row_src,
                       uint8_t* codes, float* scales, int64_t scale_stride, void* stream) {
  if (n_rows < 0 || H < 1 || scale_stride < n_rows) return MOE_ERR_INVALID_ARG;
  if (H % 128) return MOE_ERR_UNSUPPORTED;
  if (n_rows == 0) return MOE_OK;
  if (!in || !codes || !scales || !aligned16(in) || !aligned16(codes)) return MOE_ERR_INVALID_ARG;
  return launch_quant_rows_fp8(in, n_rows, H, row_src, codes, scales, scale_stride,
                               as_stream(stream));
}

size_t moe_grouped_ffn_w8a8_workspace_bytes(int64_t capacity, int num_groups, int H, int I) {
  (void)H;
  if (capacity < 0 || num_groups < 1 || I < 1) return 0;
  return w8a8_workspace_bytes(capacity, num_groups, I);
}

int moe_grouped_ffn_w8a8(const uint8_t* xq, const float* x_scales, int64_t scale_stride,
                         const int32_t* scale_src, int scale_div, const int32_t* cu_seqlens, const int32_t* counts, int num_groups, int H,
                         int I, const uint8_t* w13q, const float* w13_scales, const uint8_t* w2q,
                         const float* w2_scales, const float* row_scale, uint16_t* y,
                         int64_t capacity, int flags, void* workspace, size_t workspace_bytes,
                         int32_t* dev_error, void* stream) {
  if (num_groups < 1 || H < 1 || I < 1 || capacity < 0) return MOE_ERR_INVALID_ARG;
  if ((flags & ~MOE_FFN_ALL) || !(flags & MOE_FFN_ALL)) return MOE_ERR_INVALID_ARG;
  if (H % 128 || I % 128 || num_groups > 1024) return MOE_ERR_UNSUPPORTED;
  if (capacity > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  if (capacity == 0) return MOE_OK;   // no rows: nothing to read or write
  if (!cu_seqlens || !counts) return MOE_ERR_INVALID_ARG;
  if ((flags & MOE_FFN_GATE_UP) &&
      (!xq || !x_scales || !w13q || !w13_scales || scale_stride < 1 ||
       (!scale_src && scale_stride < capacity) || (scale_src && scale_div < 1)))
    return MOE_ERR_INVALID_ARG;
  if (scale_stride > 0x3fffffffLL) return MOE_ERR_UNSUPPORTED;
  if ((flags & MOE_FFN_DOWN) && (!y || !w2q || !w2_scales)) return MOE_ERR_INVALID_ARG;
  if ((xq && !aligned16(xq)) || (y && !aligned16(y)) || (w13q && !aligned16(w13q)) ||
      (w2q && !aligned16(w2q)))
    return MOE_ERR_INVALID_ARG;
  const size_t need = w8a8_workspace_bytes(capacity, num_groups, I);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  return launch_grouped_ffn_w8a8(xq, x_scales, scale_stride, scale_src, scale_div, cu_seqlens,
                                 counts, num_groups, H, I,
                                 w13q, w13_scales, w2q, w2_scales, row_scale, y, capacity, flags,
                                 workspace, dev_error, as_stream(stream));
}

int moe_pack_ffn_weights_fp8(const uint16_t* w13, const uint16_t* w2, int num_groups, int H,
                             int I, uint8_t* w13q, float* w13_scales, uint8_t* w2q,
                             float* w2_scales, int flags, void* stream) {
  if (num_groups < 1 || H < 1 || I < 1) return MOE_ERR_INVALID_ARG;
  if (flags & ~MOE_FP8_LAYOUT_K128) return MOE_ERR_INVALID_ARG;
  if (H % 128 || I % 128) return MOE_ERR_UNSUPPORTED;
  if (!w13 != !w13q || !w13 != !w13_scales || !w2 != !w2q || !w2 != !w2_scales)
    return MOE_ERR_INVALID_ARG;
  if ((w13 && (!aligned16(w13) || !aligned16(w13q) || !aligned16(w13_scales))) ||
      (w2 && (!aligned16(w2) || !aligned16(w2q) || !aligned16(w2_scales))))
    return MOE_ERR_INVALID_ARG;
  return launch_pack_weights_fp8(w13, w2, num_groups, H, I, w13q, w13_scales, w2q, w2_scales,
                                 (flags & MOE_FP8_LAYOUT_K128) ? 1 : 0, as_stream(stream));
}

int moe_fake_quant_rows(const uint16_t* in, uint16_t* out, int64_t n_rows, int H,
                        const int32_t* row_src, int mode, int block, const float* scale,
                        float* block_scales, float* amax_out, void* stream) {
  if (n_rows < 0 || H < 1) return MOE_ERR_INVALID_ARG;
  if (mode < MOE_FQ_PER_TENSOR || mode > MOE_FQ_MXFP4) return MOE_ERR_INVALID_ARG;
  if (H % 128) return MOE_ERR_UNSUPPORTED;
  if ((mode == MOE_FQ_BLOCK && block != 128) || (mode == MOE_FQ_NVFP4 && block != 16) ||
      (mode == MOE_FQ_MXFP4 && block != 32))
    return MOE_ERR_UNSUPPORTED;
  if (n_rows == 0) return MOE_OK;
  const bool writes = mode == MOE_FQ_BLOCK || mode == MOE_FQ_MXFP4 || scale;
  if (!in || (!out && writes)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(in) || (out && !aligned16(out))) return MOE_ERR_INVALID_ARG;
  return launch_fake_quant(in, out, n_rows, H, row_src, mode, scale, block_scales, amax_out,
                           as_stream(stream));
}

int moe_scale_from_amax(const float* amax, float* scale, int mode, void* stream) {
  if (!amax || !scale) return MOE_ERR_INVALID_ARG;
  if (mode != MOE_FQ_PER_TENSOR && mode != MOE_FQ_NVFP4) return MOE_ERR_INVALID_ARG;
  return launch_scale_from_amax(amax, scale, mode, as_stream(stream));
}

int moe_combine(const uint16_t* rows, int64_t num_rows, const int32_t* row_of,
                const uint16_t* shared, int T, int K, int H, const float* row_qdq_scale,
                uint16_t* out, int32_t* dev_error, void* stream) {
  if (T < 0 || K < 1 || H < 1 || num_rows < 0) return MOE_ERR_INVALID_ARG;
  if (H % 128) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!row_of || !out || (num_rows > 0 && !rows)) return MOE_ERR_INVALID_ARG;
  if ((rows && !aligned16(rows)) || !aligned16(out) || (shared && !aligned16(shared)))
    return MOE_ERR_INVALID_ARG;
  return launch_combine(rows, num_rows, row_of, shared, T, K, H, row_qdq_scale, out, dev_error,
                        as_stream(stream));
}

int moe_combine_check(const uint16_t* rows, int64_t num_rows, const int32_t* row_of,
                      const uint16_t* shared, int T, int K, int H, const uint16_t* kernel_out,
                      int32_t* state, int32_t* dev_error, void* stream) {
  if (T < 0 || K < 1 || H < 1 || num_rows < 0) return MOE_ERR_INVALID_ARG;
  if (H % 128) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!row_of || !kernel_out || (num_rows > 0 && !rows))) return MOE_ERR_INVALID_ARG;
  if ((rows && !aligned16(rows)) || (kernel_out && !aligned16(kernel_out)) ||
      (shared && !aligned16(shared)))
    return MOE_ERR_INVALID_ARG;
  return launch_combine_check(rows, num_rows, row_of, shared, T, K, H, kernel_out, state,
                              dev_error, as_stream(stream));
}

int moe_copy_bytes(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes % 16) return MOE_ERR_INVALID_ARG;
  if (bytes == 0) return MOE_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return MOE_ERR_INVALID_ARG;
  const int64_t n = (int64_t)(bytes / 16);
  int64_t blocks = (n + 1023) / 1024;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const copy_vec_t*>(src), static_cast<copy_vec_t*>(dst), n);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_read_bytes(const void* src, size_t bytes, void* sink, void* stream) {
  if (bytes % 16) return MOE_ERR_INVALID_ARG;
  if (bytes == 0) return MOE_OK;
  if (!src || !sink || !aligned16(src) || !aligned16(sink)) return MOE_ERR_INVALID_ARG;
  const int64_t n = (int64_t)(bytes / 16);
  int64_t blocks = (n + 2047) / 2048;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const copy_vec_t*>(src), static_cast<copy_vec_t*>(sink), n);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
