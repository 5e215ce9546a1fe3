/*
 * moe.h — C ABI of the MI355X (gfx950) MoE-layer hot path.
 *
 * The layer: route each token to its top-k experts, optionally fake-quantize
 * the expert inputs to FP8, permute the routed (token, slot) rows into
 * expert-contiguous segments, run every expert's SwiGLU FFN over its segment
 * as a grouped GEMM, optionally fake-quantize the per-(token, slot) rows, and
 * combine them in a fixed order.
 *
 * Conventions for every entry point
 *   - Tensor arguments are DEVICE pointers to contiguous row-major arrays on
 *     the current HIP device; bf16 tensors are passed as uint16_t bit
 *     patterns.  bf16 rows must start on 16-byte boundaries (guaranteed when
 *     the base pointer is 16-byte aligned and H is a multiple of 128).
 *   - The caller owns every buffer.  No entry point allocates, frees or
 *     synchronizes; each only enqueues kernels on `stream` (a hipStream_t;
 *     NULL is the default stream), so every call can be captured into a
 *     HIP graph.  Size queries tell the caller how much workspace to own.
 *   - Argument errors that the host can see from scalars and pointers return
 *     a negative status synchronously and enqueue nothing.
 *   - Errors that depend on device data (an out-of-range row index, a
 *     segment larger than the buffer) never trap: the offending element is
 *     skipped and, when `dev_error` is non-NULL, the first such error's
 *     MOE_DEVERR_* code is stored into *dev_error (only if it was 0).  The
 *     caller zeroes *dev_error and reads it back whenever it chooses.
 *   - Calls are stateless and re-entrant; two calls race only if they share
 *     an output or workspace buffer on concurrent streams.
 *
 * Sources (titles of the pages the operations come from):
 *   [P1] "Add MoE dispatch/combine fake quantization for vLLM's DeepGEMM
 *        Mega-MoE" (NVIDIA Model-Optimizer pull request)
 *   [P2] "[Kernel] DeepEP dispatch-combine kernel integration" (vLLM)
 *   [P3] "[Distributed][MoonEP] BF16 integration of MoonEP balanced EP
 *        backend" (vLLM)
 *   [P4] "[Bugfix][MoE] Size the permute scratch from its inputs" (vLLM)
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes (return values) ------------------------------------- */
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null required pointer, negative size, K > E */
  MOE_ERR_UNSUPPORTED = -2, /* shape outside what the kernels handle (e.g.
                               H or I not a multiple of 128, E > 1024)     */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than the size query says */
  MOE_ERR_HIP = -4,         /* a HIP runtime call or launch failed        */
  MOE_ERR_DEVICE = -5,      /* the current device is not a gfx950 GPU     */
  MOE_ERR_SCRATCH = -6      /* moe_permute_noalloc: the call needs more than
                               its fixed device scratch                   */
};

/* ---- device error word codes (first error wins) ----------------------- */
enum {
  MOE_DEVERR_ROW_RANGE = 1, /* a row index points outside its buffer       */
  MOE_DEVERR_CAPACITY = 2,  /* the segments need more rows than `capacity` */
  MOE_DEVERR_LAYOUT = 3,    /* moe_combine_check: rows do not reproduce the
                               output they were checked against          */
  MOE_DEVERR_EXPERT_RANGE = 4 /* moe_permute: a router id >= num_experts */
};

/* ---- flags -------------------------------------------------------------- */
enum { MOE_ROUTE_RENORM = 1 };        /* moe_route: renormalise over top-k */
enum { MOE_PERMUTE_PAD_POW2 = 1,      /* moe_permute: pow2 segment buckets */
       MOE_PERMUTE_DISPATCH_FP8 = 2   /* moe_permute: FP8 fake-quant of the rows (1x128) */
};
enum { MOE_FFN_GATE_UP = 1,           /* moe_grouped_ffn flags: stages ... */
       MOE_FFN_DOWN = 2,
       MOE_FFN_ALL = 3,
       MOE_FFN_PACKED_WEIGHTS = 4 };  /* ... and the weight layout          */
enum { MOE_FQ_PER_TENSOR = 0,         /* moe_fake_quant_rows modes         */
       MOE_FQ_BLOCK = 1,
       MOE_FQ_NVFP4 = 2,
       MOE_FQ_MXFP4 = 3 };
enum { MOE_FP8_LAYOUT_K128 = 1 };     /* moe_pack_ffn_weights_fp8: the FP8
                                         matrix-core GEMM's weight order     */

/* Human-readable text for a status code (static storage, never NULL). */
const char* moe_status_string(int status);

/* Check that `device` is a gfx950 GPU this library was built for.
 * Returns MOE_OK, MOE_ERR_DEVICE (another architecture) or MOE_ERR_HIP.
 * A host that cannot run the path fails here with a clear status rather
 * than inside a kernel launch ([P3], review thread on the system-support
 * probe run at backend selection). */
int moe_device_check(int device);

/* ---- route --------------------------------------------------------------
 * Per token t with row_valid[t] != 0 (all tokens when row_valid is NULL):
 * choose the K experts with the largest float32 logits — slot 0 the
 * largest, ties to the lower expert index — and give them the weights
 * exp(l_k - l_max) / sum_j exp(l_j - l_max), the sum running over the K
 * chosen experts with MOE_ROUTE_RENORM, else over all E experts (computed
 * in double, stored as float).  Padding tokens get topk_idx = -1 and
 * topk_w = 0 in every slot ([P1] review thread on the buffer check:
 * `valid = topk_idx >= 0`; [P2] review threads: router ids and weights
 * are [T, K] per token; the workloads' softmax -> top-k -> renormalise).
 *
 *   logits    [T, E] float32        row_valid  [T] uint8 or NULL
 *   topk_idx  [T, K] int32 (out)    topk_w     [T, K] float32 (out)
 * Requires 1 <= K <= min(E, 32), E <= 1024.  T = 0 enqueues nothing.
 * Non-finite logits: a NaN ranks as -inf (below every number, ties among
 * them to the lower index), so every id written lies in [0, E); in the
 * weights, a logit equal to l_max counts exp(0) = 1 even when both are
 * infinite (a row whose chosen logits are all -inf or NaN gets 1/K each,
 * with MOE_ROUTE_RENORM), and a -inf below a finite l_max counts 0. */
int moe_route(const float* logits, const uint8_t* row_valid, int T, int E, int K,
              int flags, int32_t* topk_idx, float* topk_w, void* stream);

/* ---- permute ------------------------------------------------------------
 * Group the routed (token, slot) pairs of the local experts
 * [expert_begin, expert_begin + num_local_experts) into expert-contiguous
 * segments ([P3] "Purpose": tokens arrive grouped per expert as [NvS, H]
 * plus cu_seqlens; [P4] PR summary and "Details": index metadata over the
 * expanded rows, sized from the inputs received, power-of-two receive
 * buckets, the permuted hidden states in a caller buffer).
 *
 * Slot (t, k) with flat index i = t*K + k is routed to local expert
 * e = topk_idx[i] - expert_begin when 0 <= e < num_local_experts.  A
 * negative id is a padding slot ([P1] review thread on the buffer check: a
 * slot is valid iff its id is >= 0); an id in [0, num_experts) outside the
 * local range belongs to another rank's expert; both are not routed here.
 * An id >= num_experts (the layer's total expert count) names no expert at
 * all: it is not routed either, and raises MOE_DEVERR_EXPERT_RANGE, so a
 * corrupt router output fails closed instead of silently vanishing from the
 * combine ([P1] review thread on graph capture: a device-side check that
 * records the failure without destroying the context).
 *   counts[e]      number of rows routed to e
 *   cu_seqlens[e]  first row of segment e; segment sizes are counts[e], or
 *                  next_pow2(counts[e]) (0 stays 0) with MOE_PERMUTE_PAD_POW2;
 *                  cu_seqlens[num_local_experts] = rows used
 *   rows of a segment: its routed slots in ascending flat index i, then the
 *                  pow2 padding rows
 *   row_of[i]      permuted row of slot i, or -1 when not routed here
 *   src_of[r]      flat slot index of row r, or -1 for a padding row and for
 *                  every unused row in [cu_seqlens[num_local_experts], capacity)
 *   w_perm[r]      topk_w[src_of[r]], 0 for padding and unused rows
 *   x_perm[r, :]   hidden[src_of[r] / K, :]; padding and unused rows are not
 *                  written.  With MOE_PERMUTE_DISPATCH_FP8 the row is the
 *                  dispatch quantizer's output instead ([P1] PR summary and
 *                  "How it works": the dispatch rows are fake-quantized to
 *                  FP8 before the experts' staging; [P2] review thread on the
 *                  low-latency dispatch: 1x128 blocks): bit for bit what
 *                  moe_fake_quant_rows(MOE_FQ_BLOCK, block 128) writes for
 *                  that hidden row, so quantizing `hidden` first and
 *                  permuting the result gives the same x_perm.  The block
 *                  scales are not returned.
 *
 *   topk_idx [T, K] int32   topk_w [T, K] float32   hidden [T, H] bf16
 *   (without MOE_PERMUTE_DISPATCH_FP8 rows are copied as opaque 2-byte
 *   units, so any 2H-byte row payload can be permuted this way — FP8 codes
 *   of 2H channels, for instance)
 *   counts [E_l] int32, cu_seqlens [E_l + 1] int32, row_of [T*K] int32,
 *   src_of [capacity] int32, w_perm [capacity] float32,
 *   x_perm [capacity, H] bf16 — all outputs.
 * `capacity` is the number of rows the caller allocated in x_perm, src_of
 * and w_perm; moe_permute_capacity() is always enough.  If the segments
 * need more rows, rows at or past `capacity` are not written and
 * MOE_DEVERR_CAPACITY is raised.  `workspace` holds
 * moe_permute_workspace_bytes() bytes of scratch (contents on entry are
 * ignored).  Requires H % 128 == 0, 1 <= num_local_experts <= 1024,
 * 0 <= expert_begin and expert_begin + num_local_experts <= num_experts. */
int64_t moe_permute_capacity(int T, int K, int num_local_experts, int flags);
size_t moe_permute_workspace_bytes(int T, int K, int num_local_experts, int flags);
int moe_permute(const int32_t* topk_idx, const float* topk_w, const uint16_t* hidden,
                int T, int K, int H, int num_experts, int expert_begin, int num_local_experts,
                int flags,
                int64_t capacity, int32_t* counts, int32_t* cu_seqlens, uint16_t* x_perm,
                int32_t* row_of, int32_t* src_of, float* w_perm, void* workspace,
                size_t workspace_bytes, int32_t* dev_error, void* stream);

/* moe_permute without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same operation, arguments, outputs, flags
 * and errors as moe_permute, with the chunk table and ranks kept in a
 * fixed array of moe_permute_noalloc_scratch_bytes() (4 MiB) in device
 * memory that the library owns (one copy per GPU, held until the process
 * ends; its address is looked up once per device on the first call there).
 * Nothing is allocated or freed, by this call or any library routine it
 * uses.  A call whose moe_permute_workspace_bytes() exceeds the scratch
 * returns MOE_ERR_SCRATCH and enqueues nothing (about T*K <= 900 000 slots
 * with 128 local experts).  The kernels overwrite every scratch entry they
 * read, so no state carries over between calls; but every call on one GPU
 * shares the array, so calls that may overlap on that GPU (concurrent
 * streams, or graphs replayed concurrently) race and must be serialized by
 * the caller. */
size_t moe_permute_noalloc_scratch_bytes(void);
int moe_permute_noalloc(const int32_t* topk_idx, const float* topk_w, const uint16_t* hidden,
                        int T, int K, int H, int num_experts, int expert_begin,
                        int num_local_experts, int flags, int64_t capacity, int32_t* counts,
                        int32_t* cu_seqlens, uint16_t* x_perm, int32_t* row_of, int32_t* src_of,
                        float* w_perm, int32_t* dev_error, void* stream);

/* ---- grouped SwiGLU FFN -------------------------------------------------
 * For every group g with n = counts[g] rows starting at row c = cu_seqlens[g]
 * of x ([P3] commit message adding the modular experts: gate, up and down
 * grouped matmuls over the cu_seqlens segments, route weights applied before
 * the down projection, empty segments skipped; [P2] review thread on the
 * DeepEP + DeepGEMM test: w1 holds 2n rows, gate and up):
 *   h      = x[c:c+n] @ w13[g]^T            (float32 accumulate)  [n, 2I]
 *   a      = bf16( silu(h[:, :I]) * h[:, I:] )                    [n, I]
 *   y[c:c+n] = bf16( row_scale[c:c+n] * (a @ w2[g]^T) )           [n, H]
 * row_scale NULL means 1.  Rows of a segment past counts[g] (pow2 padding)
 * are neither read nor written.  The shared expert is the case
 * num_groups = 1, counts = {T}, cu_seqlens = {0, T}, row_scale = NULL.
 *
 *   x [capacity, H] bf16;  w13 [G, 2I, H] bf16 (gate rows [0, I), up rows
 *   [I, 2I)); w2 [G, H, I] bf16; row_scale [capacity] float32 or NULL;
 *   y [capacity, H] bf16 (out); cu_seqlens [G + 1], counts [G] int32.
 * `flags` selects the stages — MOE_FFN_GATE_UP (writes `a` into the
 * workspace), MOE_FFN_DOWN (reads it) or MOE_FFN_ALL; a DOWN-only call must
 * get the workspace a GATE_UP call with the same segments filled — and, with
 * MOE_FFN_PACKED_WEIGHTS, says that w13 and w2 are in the packed layout
 * moe_pack_ffn_weights() produces.  Segments that reach past `capacity` are
 * skipped and raise MOE_DEVERR_ROW_RANGE.  Segments are meant to be
 * disjoint (the permute's output is); with packed weights, tiles whose
 * place in the workspace (counted from the counts, each clamped to
 * `capacity`) would fall past its ceil(capacity/128) + G row tiles, which
 * only overlapping segments or oversized counts produce, are skipped with
 * the same error.  capacity 0 (an empty batch)
 * returns MOE_OK after the scalar checks, touching no pointer (the FP8 and
 * FP8-path variants below behave the same).
 * Requires H % 128 == 0, I % 128 == 0, 1 <= G <= 1024. */
size_t moe_grouped_ffn_workspace_bytes(int64_t capacity, int num_groups, int H, int I);
int moe_grouped_ffn(const uint16_t* x, const int32_t* cu_seqlens, const int32_t* counts,
                    int num_groups, int H, int I, const uint16_t* w13, const uint16_t* w2,
                    const float* row_scale, uint16_t* y, int64_t capacity, int flags,
                    void* workspace, size_t workspace_bytes, int32_t* dev_error, void* stream);

/* Rearrange expert weights, once, into the layout the grouped GEMM streams
 * straight into its matrix-core registers ("fragment order", K-major).  For
 * group g, K-step ks (32 columns of the reduction dimension) and column tile
 * ct (64 weight rows), the tile's four 16 x 32 fragments f = 0..3 sit at
 * 16-byte unit ((g * (Kdim/32) + ks) * n_ct + ct) * 256 + f * 64 + l, where
 * lane l = 0..63 holds the 8 values W[row0(ct, f) + l % 16][32 ks + 8 (l / 16)
 * .. +8].  For w2 [G, H, I] (Kdim = I, n_ct = H/64) row0 = 64 ct + 16 f; for
 * w13 [G, 2I, H] (Kdim = H, n_ct = I/32) fragments 0, 1 are gate rows
 * 32 ct + 16 f and fragments 2, 3 the matching up rows I + 32 ct + 16 (f - 2).
 * Outputs have the inputs' sizes; either pair may be NULL; outputs must not
 * alias inputs.  Weights are static, so this runs at load time, not per
 * layer call.  Requires H % 128 == 0, I % 128 == 0. */
int moe_pack_ffn_weights(const uint16_t* w13, const uint16_t* w2, int num_groups, int H, int I,
                         uint16_t* w13_packed, uint16_t* w2_packed, void* stream);

/* ---- FP8 expert weights (the weight half of the FP8 grouped GEMM) -------
 * [P2] review thread on the DeepEP + DeepGEMM test (FP8 expert weights with
 * one scale per block_n x block_k tile; here 128 x 128, the size of the
 * activation blocks): each 128 x 128 tile of w13[g] [2I, H]
 * and w2[g] [H, I] gets s = fl32(amax / 448) (0 for an all-zero tile) and
 * every element the OCP E4M3FN code of clamp(fl32(w / s), +-448), rounded to
 * nearest even (code 0 where s = 0).
 *   w13q [G, 2I, H] / w2q [G, H, I] uint8 (out): one code per weight, in the
 *     packed order of moe_pack_ffn_weights with 8 codes (8 bytes) per lane
 *     where the bf16 packing holds 8 values (16 bytes): unit index
 *     ((g * (Kdim/32) + ks) * n_ct + ct) * 256 + f * 64 + l, 8 bytes each.
 *   w13_scales [G, 2I/128, H/128], w2_scales [G, H/128, I/128] float32 (out),
 *     tile (row block, column block) row-major per group.
 * With flags = MOE_FP8_LAYOUT_K128 the codes are instead in the order
 * moe_grouped_ffn_w8a8 streams: 16-byte unit
 * ((((g * (Kdim/128) + kb) * n_ct + ct) * 4 + f) * 2 + h) * 64 + l holds weight
 * row row0(ct, f) + l % 16 (rows as above), columns
 * 128 kb + 64 h + 16 (l / 16) .. +16.
 * Either group of three (w13, w13q, w13_scales) / (w2, ...) may be all NULL.
 * Pointers 16-byte aligned.  Runs once at load time.  Unknown flag bits:
 * MOE_ERR_INVALID_ARG.  Requires H % 128 == 0, I % 128 == 0. */
int moe_pack_ffn_weights_fp8(const uint16_t* w13, const uint16_t* w2, int num_groups, int H,
                             int I, uint8_t* w13q, float* w13_scales, uint8_t* w2q,
                             float* w2_scales, int flags, void* stream);

/* moe_grouped_ffn with the FP8 weights above: the same operation, segments,
 * flags (stage bits only; the weights are always the packed FP8 ones),
 * workspace and errors, where every weight the matmuls read is the
 * dequantized bf16( fl32(code * s) ) of its tile — exactly
 * moe_grouped_ffn on the FP8 fake-quantized bf16 weights.  Activations stay
 * bf16; half the weight bytes are read.  The stage(s) selected need their
 * codes and scales (others may be NULL). */
int moe_grouped_ffn_fp8(const uint16_t* x, const int32_t* cu_seqlens, const int32_t* counts,
                        int num_groups, int H, int I, const uint8_t* w13q, const float* w13_scales,
                        const uint8_t* w2q, const float* w2_scales, const float* row_scale,
                        uint16_t* y, int64_t capacity, int flags, void* workspace,
                        size_t workspace_bytes, int32_t* dev_error, void* stream);

/* ---- FP8 activations and weights on the FP8 matrix cores -----------------
 * The dispatch quantizer for real ([P2] review thread on the low-latency
 * dispatch: tokens handed over as FP8 codes with their block scales): for
 * every row r and 128-channel block kb of bf16 rows in [n_rows, H],
 * s = fl32(amax / 448) and codes e4m3(clamp(fl32(x / s), +-448)) (IEEE
 * quotient, round to nearest even) — the codes and scales whose dequant
 * bf16(q * s) is moe_fake_quant_rows(MOE_FQ_BLOCK).  Rows with
 * row_src[r] < 0 (row_src may be NULL) and all-zero blocks get codes 0 and
 * scale 0.
 *   codes [n_rows, H] uint8 (out), 16-byte aligned;
 *   scales (out) K-block-major: scales[kb * scale_stride + r], float32,
 *     scale_stride >= n_rows.
 * Requires H % 128 == 0. */
int moe_quant_rows_fp8(const uint16_t* in, int64_t n_rows, int H, const int32_t* row_src,
                       uint8_t* codes, float* scales, int64_t scale_stride, void* stream);

/* The grouped SwiGLU FFN on FP8 rows and FP8 weights ([P2] review threads on
 * the low-latency dispatch and on the DeepEP + DeepGEMM test: FP8 tokens
 * with block scales times FP8 weights with tile scales in the grouped GEMMs;
 * [P3] commit message adding the modular experts): per segment g (rows as in
 * moe_grouped_ffn),
 *   h[r, n] = sum_kb sx[r, kb] * sw13[g][n/128, kb] * sum_{k in kb} qx[r, k] qw13[g][n, k]
 *   a = bf16(silu(h[:, :I]) * h[:, I:]), quantized per 1 x 128 block like
 *       moe_quant_rows_fp8 (codes qa, scales sa; kept in the workspace)
 *   y[r] = bf16(row_scale[r] * sum_kb sa[r, kb] * sw2[g][n/128, kb] * (qa . qw2))
 * with every K-block's code products summed by the matrix cores in float32
 * and scaled into a float32 accumulator.
 *   xq [capacity, H] uint8 and x_scales (K-block-major, stride
 *     scale_stride) from moe_quant_rows_fp8.  With scale_src NULL, row r's
 *     scales are x_scales[kb * scale_stride + r] (scale_stride >= capacity);
 *     otherwise row r's are those of row scale_src[r] / scale_div
 *     (scale_div >= 1) — moe_permute's src_of and K, so that the scales of
 *     the unpermuted [T, H] rows serve the permuted codes, which moe_permute
 *     moves like any other row payload; scale_stride must then exceed every
 *     such row (>= T): a routed row whose scale_src entry is negative or
 *     names a row at or past scale_stride raises MOE_DEVERR_ROW_RANGE (and
 *     takes row 0's scales instead of reading outside x_scales);
 *   w13q / w2q and their tile scales from moe_pack_ffn_weights_fp8 with
 *     MOE_FP8_LAYOUT_K128; row_scale, y, cu_seqlens, counts, capacity as in
 *     moe_grouped_ffn.
 * flags: MOE_FFN_GATE_UP (writes qa, sa into the workspace), MOE_FFN_DOWN
 * (reads them; needs the workspace of a GATE_UP call on the same segments)
 * or MOE_FFN_ALL.  Segments past capacity, and tiles past the workspace
 * (as for moe_grouped_ffn with packed weights), are skipped with
 * MOE_DEVERR_ROW_RANGE.  Requires H % 128 == 0, I % 128 == 0, G <= 1024. */
size_t moe_grouped_ffn_w8a8_workspace_bytes(int64_t capacity, int num_groups, int H, int I);
int moe_grouped_ffn_w8a8(const uint8_t* xq, const float* x_scales, int64_t scale_stride,
                         const int32_t* scale_src, int scale_div, const int32_t* cu_seqlens, const int32_t* counts, int num_groups, int H,
                         int I, const uint8_t* w13q, const float* w13_scales, const uint8_t* w2q,
                         const float* w2_scales, const float* row_scale, uint16_t* y,
                         int64_t capacity, int flags, void* workspace, size_t workspace_bytes,
                         int32_t* dev_error, void* stream);

/* ---- FP8 and FP4 fake-quant of bf16 rows -------------------------------
 * QDQ to OCP E4M3FN and back ([P1] PR summary and "How it works": the
 * dispatch quantizer fake-quantizes the experts' input tokens, the combine
 * quantizer the router-weighted per-(token, slot) BF16 rows with a
 * calibrated (max) or constant global scale; [P2] review thread on the
 * low-latency dispatch: FP8 with block scales):
 *   x' = bf16( fl32( e4m3( clamp(fl32(x / s), -448, 448) ) * s ) )
 * with IEEE float32 division and multiplication, e4m3 and bf16 both
 * round-to-nearest-even.
 *   MOE_FQ_BLOCK:      s = fl32(amax / 448) per row and per `block`
 *                      contiguous channels; an all-zero block gives +0;
 *                      block_scales [n_rows, H/block] float32 (or NULL)
 *                      receives s.  `scale` is ignored.
 *   MOE_FQ_PER_TENSOR: s = *scale (a device scalar, s > 0).  With scale ==
 *                      NULL nothing is written to `out` (calibration only).
 * Rows with row_src != NULL and row_src[r] < 0 are skipped: copied from
 * `in` unchanged when out != in, else untouched.  When amax_out != NULL,
 * max |x| over the rows not skipped is max-accumulated into *amax_out
 * (the caller sets it to 0 once; repeated calls give the running max, the
 * calibrated amax of [P1] "Testing").  in == out (in place) is allowed.
 * Requires H % block == 0 and block == 128 in block mode. */
int moe_fake_quant_rows(const uint16_t* in, uint16_t* out, int64_t n_rows, int H,
                        const int32_t* row_src, int mode, int block, const float* scale,
                        float* block_scales, float* amax_out, void* stream);
/* The FP4 modes ([P1] names NVFP4 dispatch and combine units, [P4]'s test
 * plan an MXFP4 expert path; the pages do not define the formats, so these
 * are the published definitions).  Elements are E2M1 (magnitudes 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6), round-to-nearest with ties to the even code, saturating
 * at 6; the sign of a zero is kept.
 *   MOE_FQ_MXFP4 (block must be 32): per row and 32 channels, the OCP MX
 *     power-of-two scale X = 2^(floor(log2 amax) - 2), exponent clamped to
 *     [-127, 127]; x' = bf16( e2m1(clamp(x / X, -6, 6)) * X ) (exact); an
 *     all-zero block gives +0; block_scales [n_rows, H/32] receives X.
 *     `scale` is ignored.
 *   MOE_FQ_NVFP4 (block must be 16): g = *scale, the per-tensor scale
 *     (calibrated, e.g. amax / (6 * 448), or constant; NULL = calibration
 *     only); per row and 16 channels b = e4m3( min(fl32(amax / fl32(6 g)),
 *     448) ), S = fl32(b * g), x' = bf16( fl32( e2m1(clamp(fl32(x / S), -6,
 *     6)) * S ) ); S == 0 gives +0; block_scales [n_rows, H/16] receives b. */

/* The constant per-tensor scale from a calibrated amax, on the device, so
 * that it never leaves the GPU ([P1] "How it works": a calibrated (max) or
 * constant global combine scale; the workloads' 1/448 * max|row|):
 *   mode MOE_FQ_PER_TENSOR (FP8):  scale[0] = fl32(amax[0] / 448)
 *   mode MOE_FQ_NVFP4:             scale[0] = fl32(amax[0] / 2688), the
 *        NVFP4 tensor scale (6, the largest E2M1 magnitude, times 448, the
 *        largest E4M3 block scale)
 * one IEEE float32 division each.  Both pointers are device scalars.  Any
 * other mode: MOE_ERR_INVALID_ARG. */
int moe_scale_from_amax(const float* amax, float* scale, int mode, void* stream);

/* ---- combine ------------------------------------------------------------
 * out[t, :] = bf16( ((+0 + r_{t,k0}) + r_{t,k1}) + ... + shared[t, :] )
 * over the valid slots k0 < k1 < ... of token t (row_of[t*K + k] >= 0),
 * each r_{t,k} = rows[row_of[t*K + k], :], every add one IEEE float32
 * add in exactly this order, then one round-to-nearest-even to bf16; the
 * shared expert's row is added last and never quantized ([P1] PR summary
 * and "How it works" fix this order: the kernel re-adds each token's
 * routed rows slot by slot in increasing slot index into a float32 sum
 * that begins at zero, rounds to bf16 once at the end, and places a fused
 * shared expert after every routed slot, without quantizing it).
 * row_qdq_scale != NULL fake-quantizes each routed row with that per-tensor
 * device scalar before it is added (the same bits as moe_fake_quant_rows
 * in MOE_FQ_PER_TENSOR mode followed by this call).
 *   rows [num_rows, H] bf16; row_of [T*K] int32; shared [T, H] bf16 or
 *   NULL; out [T, H] bf16 (out).  row_of entries >= num_rows are skipped
 *   and raise MOE_DEVERR_ROW_RANGE.  A token with no valid slot and no
 *   shared row gets +0.  Requires H % 128 == 0. */
int moe_combine(const uint16_t* rows, int64_t num_rows, const int32_t* row_of,
                const uint16_t* shared, int T, int K, int H, const float* row_qdq_scale,
                uint16_t* out, int32_t* dev_error, void* stream);

/* ---- layout check for a fused kernel's combine ---------------------------
 * [P1] PR summary, "How it works" and the review thread on graph capture:
 * where one fused kernel both combines and leaves its per-(token, slot) rows
 * in a buffer, the quantizer relies on knowing that buffer's layout.  It
 * checks, on the first batch that has routed rows, that the rows re-summed in
 * the kernel's order reproduce the kernel's output bit for bit, and fails
 * closed otherwise; a graph captured before that check carries the check
 * itself, so replays perform it on the device.
 *
 * This call re-sums `rows` exactly as moe_combine does without QDQ (valid
 * slots ascending, float32 from +0, `shared` last, one bf16 rounding) and
 * compares every element with `kernel_out` [T, H] bit for bit; on any
 * difference it stores MOE_DEVERR_LAYOUT into *dev_error (first error wins).
 * rows, num_rows, row_of, shared, T, K, H mean what they mean for
 * moe_combine.  `state` (nullable, one device int32, zero before the first
 * call on a buffer): a call that finds 1 does nothing (the buffer has been
 * checked); otherwise the call leaves 1 when the batch had at least one
 * routed slot and everything matched, else 0 — so padding-only batches defer
 * the check to the next batch with routed rows.  With state NULL every call
 * checks.  No host sync; capturable (replays of a captured call keep reading
 * and updating the state word).  Requires H % 128 == 0. */
int moe_combine_check(const uint16_t* rows, int64_t num_rows, const int32_t* row_of,
                      const uint16_t* shared, int T, int K, int H, const uint16_t* kernel_out,
                      int32_t* state, int32_t* dev_error, void* stream);

/* ---- streaming copy -----------------------------------------------------
 * dst[0:bytes) = src[0:bytes) with 16-byte vector loads and stores: the
 * plain copy kernel whose measured time and HBM byte counters calibrate the
 * bandwidth and counter figures of the kernels above.  `bytes` must be a
 * multiple of 16 and both pointers 16-byte aligned. */
int moe_copy_bytes(const void* src, void* dst, size_t bytes, void* stream);

/* ---- streaming read -----------------------------------------------------
 * Reads src[0:bytes) once with 16-byte non-temporal vector loads and folds
 * it into a 32-bit checksum per thread; `sink` (at least 64 KiB, 16-byte
 * aligned, device) receives only checksums equal to 0x5ca1ab1e, so in
 * practice nothing is written.  The read-only counterpart of
 * moe_copy_bytes: its measured rate is the practical ceiling of the
 * weight-streaming kernels.  `bytes` must be a multiple of 16, `src`
 * 16-byte aligned. */
int moe_read_bytes(const void* src, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
