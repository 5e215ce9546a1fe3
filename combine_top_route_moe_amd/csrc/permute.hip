// Permute of the routed (token, slot) rows into expert-contiguous segments.
//
// Source: "[Distributed][MoonEP] BF16 integration of MoonEP balanced EP
// backend", "Purpose" (rows grouped per expert as [NvS, H] + cu_seqlens);
// "[Bugfix][MoE] Size the permute scratch from its inputs", PR summary and
// "Details" (int32 metadata over the expanded rows sized from the inputs,
// power-of-two receive buckets, permuted rows in a caller buffer).
//
// Rows inside a segment are ordered by the flat slot index i = t*K + k, so
// the result is unique and deterministic.  Three launches:
//   1. chunk_rank: one workgroup per chunk of 1024 flat slots; each of its
//      four wavefronts walks a quarter, 64 slots at a time.  Lanes holding
//      the same expert find each other with one ballot per bit of the
//      expert id; a lane's rank is the number of same-expert lanes below it
//      plus the wave's running count of that expert (in LDS) plus the
//      counts of the earlier waves.  Writes rank[i] and the chunk's
//      per-expert totals.
//   2. scan: one workgroup (each expert's chunk column split over
//      1024 / El threads) turns the chunk totals into per-expert counts,
//      segment sizes (optionally next_pow2), cu_seqlens, and the absolute
//      first row of every (chunk, expert) pair, and checks the capacity.
//   3. scatter: one workgroup per token group computes row_of / src_of /
//      w_perm for its slots and copies each token row once from HBM into
//      its K destination rows with 16-byte vector loads and stores; the
//      workgroups also mark the pow2 padding rows (workgroup b those of
//      expert b) and the unused rows up to `capacity` (src_of = -1,
//      w_perm = 0).
// When the chunk table is small (at most kFuseTable entries: a few
// thousand routed slots), launch 2 is folded into launch 3: every scatter
// workgroup scans the table itself from LDS (a few hundred integers), and
// workgroup 0 writes counts and cu_seqlens — one kernel launch less on the
// latency-bound small batches.  At most kSmallTK slots, all three are one
// launch, permute_small_kernel: every workgroup counts all the slots itself
// (two LDS histograms), which for a few thousand slots costs less than the
// launches and dependent round trips to memory it saves.
//
// With MOE_PERMUTE_DISPATCH_FP8 the copies also apply the dispatch FP8
// fake-quant ("Add MoE dispatch/combine fake quantization for vLLM's
// DeepGEMM Mega-MoE", PR summary and "How it works"; 1 x 128 blocks as in
// "[Kernel] DeepEP dispatch-combine kernel integration", review thread on
// the low-latency dispatch) to each row vector on its way.
#include <atomic>

#include "common.h"

namespace moe {

// Permuted rows are written with non-temporal stores: each wave writes whole
// 1 KB runs of a row, which the grouped GEMM reads next from other XCDs.
// Measured on the balanced, deepseek and prefill batches: the permute itself
// within 2 % either way, and the gate/up GEMM that follows 1-4 % faster than
// after ordinary stores.  (Non-temporal reads of the token rows made the
// prefill permute slower.)
typedef uint32_t row_vec_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_row_vec(uint16_t* row, int c, const uint4& v) {
  __builtin_nontemporal_store(row_vec_t{v.x, v.y, v.z, v.w}, reinterpret_cast<row_vec_t*>(row) + c);
}

// FP8 fake-quant of a 16-byte vector (8 channels) of a 1 x 128 block whose
// 16 vectors sit in 16 consecutive lanes, all of which call this together:
// the block amax across them in registers, s = amax / 448 (IEEE), an
// all-zero block gives +0, else qdq8_rcp — the block mode of the dispatch
// fake-quantizer, value for value.
// One DPP lane movement within each row of 16 lanes (every lane active).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ uint4 fq_block128_vec(const uint4& raw) {
  float f[8];
  unpack8(raw, f);
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
  // the block's 16 lanes are one DPP row: the max over it by two quad
  // permutations (lane ^ 1, lane ^ 2), the half-row mirror (lane i <-> 7 - i)
  // and the row mirror (lane i <-> 15 - i), all in registers; max is exact,
  // so the order does not matter
  m = fmaxf(m, dpp_f32<0xB1>(m));   // quad_perm [1, 0, 3, 2]
  m = fmaxf(m, dpp_f32<0x4E>(m));   // quad_perm [2, 3, 0, 1]
  m = fmaxf(m, dpp_f32<0x141>(m));  // row_half_mirror
  m = fmaxf(m, dpp_f32<0x140>(m));  // row_mirror
  const float s = m / 448.0f;  // IEEE division
  if (!(s > 0.0f)) return make_uint4(0, 0, 0, 0);
  uint32_t w[4];
  qdq8_rcp(f, s, 1.0f / s, rcp_scale_ok(s), w);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

constexpr int kChunk = 1024;
constexpr int kFuseTable = 4096;   // chunk-table entries up to which the scan is fused
constexpr int kFuseChunks = 16;    // ... and chunks (each workgroup sums its table columns)

// An id at or past the layer's expert count names no expert: it is not
// routed (the local-range test below already excludes it, since the local
// experts lie inside [0, num_experts)) and the error word records it.
__device__ __forceinline__ void check_expert_id(int id, int num_experts, int32_t* dev_error) {
  if (id >= num_experts) raise_error(dev_error, MOE_DEVERR_EXPERT_RANGE);
}

__global__ void __launch_bounds__(256) permute_chunk_rank_kernel(
    const int32_t* __restrict__ topk_idx, int64_t TK, int num_experts, int expert_begin, int El,
    int nbits, int32_t* __restrict__ table /* [nchunks][El] */,
    int32_t* __restrict__ rank /* [TK] */, int32_t* __restrict__ dev_error) {
  // wave w ranks slots [256 w, 256 w + 256) of the chunk, 64 at a time, with
  // its own running per-expert counts; afterwards each slot adds the counts
  // of the waves before it
  __shared__ int32_t cnt[4][1024];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int e = lane; e < El; e += kWave) cnt[w][e] = 0;
  const int64_t base = (int64_t)blockIdx.x * kChunk + w * (kChunk / 4);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int kSteps = kChunk / 4 / kWave;
  int my_e[kSteps], my_r[kSteps];
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int64_t i = base + step * kWave + lane;
    int e = -1;
    if (i < TK) {
      const int id = topk_idx[i];
      const int le = id - expert_begin;
      if (id >= 0 && le >= 0 && le < El) e = le;
      check_expert_id(id, num_experts, dev_error);
    }
    uint64_t peers = __ballot(e >= 0);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const int below = __popcll(peers & lt_mask);
    int before = 0;
    if (e >= 0) before = cnt[w][e];
    // every lane has read cnt[] before a leader updates it (one wave, LDS
    // operations retire in program order)
    if (e >= 0 && below == 0) cnt[w][e] = before + __popcll(peers);
    my_e[step] = e;
    my_r[step] = before + below;
  }
  __syncthreads();
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int64_t i = base + step * kWave + lane;
    if (i >= TK) continue;
    const int e = my_e[step];
    int r = -1;
    if (e >= 0) {
      r = my_r[step];
      for (int v = 0; v < w; ++v) r += cnt[v][e];
    }
    rank[i] = r;
  }
  int32_t* trow = table + (int64_t)blockIdx.x * El;
  for (int e = threadIdx.x; e < El; e += blockDim.x)
    trow[e] = cnt[0][e] + cnt[1][e] + cnt[2][e] + cnt[3][e];
}

__device__ __forceinline__ int next_pow2_dev(int n) {
  if (n <= 1) return n;
  return 1 << (32 - __clz(n - 1));
}

// One workgroup of 1024 threads.  Each expert's column of chunk counts is
// split into P = 1024 / El contiguous blocks of chunks, one thread each
// (thread p*El + e: reads stay coalesced across experts), so no thread walks
// more than ceil(nchunks / P) chunks; the partial sums meet in LDS.  Up to
// kScanRegs chunks per thread, a thread loads its whole block into registers
// at once and later overwrites it from there: one round trip to memory
// instead of one per chunk (and per chunk again for the load-then-store
// pass, whose loads and stores the compiler cannot reorder).
constexpr int kScanRegs = 32;
__global__ void __launch_bounds__(1024) permute_scan_kernel(
    int32_t* __restrict__ table, int nchunks, int El, int pad_pow2, int64_t capacity,
    int32_t* __restrict__ counts, int32_t* __restrict__ cu_seqlens,
    int32_t* __restrict__ dev_error) {
  __shared__ int32_t part[1024];   // [P][El] partial sums
  __shared__ int32_t s_start[1024];
  __shared__ int32_t s_wave[16];
  const int tid = threadIdx.x;
  const int P = max(1, 1024 / El);
  const bool act = tid < P * El;
  const int e = act ? tid % El : 0, p = act ? tid / El : 0;
  const int L = (nchunks + P - 1) / P;
  const int c0 = min(p * L, nchunks), c1 = min(c0 + L, nchunks);
  const bool in_regs = L <= kScanRegs;   // the same for every thread
  int vals[kScanRegs];
  if (act) {
    int sum = 0;
    if (in_regs) {
      // groups of 8 loads under a uniform guard, each load unconditional
      // with its index clamped into the thread's block (so all are issued
      // before the first wait); entries past the block count 0
      const int n = c1 - c0;
      const int64_t last = (int64_t)(c1 - 1) * El + e;
#pragma unroll
      for (int g = 0; g < kScanRegs / 8; ++g) {
        if (8 * g < L && n > 0) {
#pragma unroll
          for (int u = 0; u < 8; ++u)
            vals[8 * g + u] = table[min((int64_t)(c0 + 8 * g + u) * El + e, last)];
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) vals[8 * g + u] = 0;
        }
      }
#pragma unroll
      for (int j = 0; j < kScanRegs; ++j) sum += j < n ? vals[j] : 0;
    } else {
      for (int c = c0; c < c1; ++c) sum += table[(int64_t)c * El + e];
    }
    part[tid] = sum;
  }
  __syncthreads();
  int total = 0;
  if (tid < El)
    for (int q = 0; q < P; ++q) total += part[q * El + tid];
  const int size = (tid < El) ? (pad_pow2 ? next_pow2_dev(total) : total) : 0;
  // block-wide inclusive scan of size over 1024 threads (thread = expert)
  const int lane = tid & 63, wid = tid >> 6;
  int x = size;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = lane < 16 ? s_wave[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      int y = __shfl_up(w, off, kWave);
      if (lane >= off) w += y;
    }
    if (lane < 16) s_wave[lane] = w;
  }
  __syncthreads();
  const int incl = x + (wid > 0 ? s_wave[wid - 1] : 0);
  if (tid < El) {
    const int start = incl - size;
    s_start[tid] = start;
    counts[tid] = total;
    cu_seqlens[tid] = start;
    if (tid == El - 1) {
      cu_seqlens[El] = incl;
      if ((int64_t)incl > capacity) raise_error(dev_error, MOE_DEVERR_CAPACITY);
    }
  }
  __syncthreads();
  if (act) {
    // absolute first row of every (chunk, expert) pair in this thread's block
    int running = s_start[e];
    for (int q = 0; q < p; ++q) running += part[q * El + e];
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < kScanRegs; ++j) {
        if (j < c1 - c0) {
          table[(int64_t)(c0 + j) * El + e] = running;
          running += vals[j];
        }
      }
    } else {
      for (int c = c0; c < c1; ++c) {
        const int64_t k = (int64_t)c * El + e;
        const int cnt = table[k];
        table[k] = running;
        running += cnt;
      }
    }
  }
  // the pow2 padding rows are marked by the scatter kernel's workgroups
  // (one workgroup, one expert per lane, made every store instruction touch
  // 64 cache lines: 23 us of a 128-expert batch's 245 us permute)
}

// FUSED: `table` holds the chunk_rank totals and the workgroup does the
// scan's work itself from a copy of the table in LDS (see the file comment).
// COLS: `table` holds the totals too (at most kColChunks chunks, at most 256
// experts), and each workgroup reads only the table's columns: thread e sums
// expert e's chunk counts (all of them, those before the workgroup's first
// chunk, and those up to it; its slots span at most two chunks), then a
// block-wide scan of the sizes gives the starts.  The loads of a column are
// all in flight together and hit L2, so this costs each workgroup about one
// memory round trip and saves the one-workgroup scan launch.
// Otherwise `table` holds the absolute first row of every (chunk, expert)
// pair written by the scan.
// QDQ (both scatter kernels): each row vector is the dispatch FP8
// fake-quant's output (fq_block128_vec).  The 16 vectors of a 1 x 128 block
// are 16 consecutive indices of the copy loop, so 16 consecutive lanes of
// one wave, which take every branch of the loop together (H / 8 and the
// loop stride are multiples of 16).
constexpr int kColChunks = 32;
template <bool FUSED, bool COLS, bool QDQ>
__global__ void __launch_bounds__(256) permute_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const uint16_t* __restrict__ hidden, int T, int K, int H, int expert_begin, int El,
    int tok_per_block, int64_t capacity, const int32_t* __restrict__ table, int nchunks,
    int pad_pow2, const int32_t* __restrict__ rank, uint16_t* __restrict__ x_perm,
    int32_t* __restrict__ row_of, int32_t* __restrict__ src_of, float* __restrict__ w_perm,
    int32_t* __restrict__ dev_error, int32_t* __restrict__ counts,
    int32_t* __restrict__ cu_seqlens) {
  __shared__ int32_t dest[256];
  __shared__ int32_t s_tab[FUSED ? kFuseTable : 1];
  __shared__ int32_t s_start[FUSED ? 1024 : COLS ? 256 : 1];
  __shared__ int32_t s_tot[FUSED ? 1024 : COLS ? 256 : 1];
  __shared__ int32_t s_size[FUSED ? 1024 : COLS ? 256 : 1];
  __shared__ int32_t s_pre[COLS ? 2 : 1][COLS ? 256 : 1];
  __shared__ int32_t s_wave[4];
  const int tid = threadIdx.x;
  const int c0 = COLS ? (int)((int64_t)blockIdx.x * tok_per_block * K / kChunk) : 0;
  // this workgroup's slots: their rank, id and weight, loaded before the
  // start rows are worked out, so the two sets of loads overlap
  const int t0 = blockIdx.x * tok_per_block;
  const int nslots = tok_per_block * K;
  const int64_t my_i = (int64_t)t0 * K + tid;
  const bool my_slot = tid < nslots && t0 + tid / K < T;
  int my_rank = -1, my_id = -1;
  float my_w = 0.0f;
  if (my_slot) {
    my_rank = rank[my_i];
    my_id = topk_idx[my_i];
    my_w = topk_w[my_i];
  }
  int64_t used_end;   // end of the last segment
  if (FUSED) {
    const int n = nchunks * El;
    for (int j = tid; j < n; j += blockDim.x) s_tab[j] = table[j];
    __syncthreads();
    // each thread owns experts 4 tid .. 4 tid + 3 (El <= 1024): totals,
    // sizes, then a block-wide exclusive scan of the sizes
    int tot[4], sz[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * tid + j;
      tot[j] = 0;
      if (e < El)
        for (int c = 0; c < nchunks; ++c) tot[j] += s_tab[c * El + e];
      sz[j] = (e < El) ? (pad_pow2 ? next_pow2_dev(tot[j]) : tot[j]) : 0;
      local += sz[j];
    }
    const int lane = tid & 63, wid = tid >> 6;
    int x = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wid] = x;
    __syncthreads();
    int before = x - local;
    for (int q = 0; q < wid; ++q) before += s_wave[q];
    const int grand = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    int run = before;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * tid + j;
      if (e < El) {
        s_start[e] = run;
        s_tot[e] = tot[j];
        s_size[e] = sz[j];
        if (blockIdx.x == 0) {
          counts[e] = tot[j];
          cu_seqlens[e] = run;
        }
      }
      run += sz[j];
    }
    if (blockIdx.x == 0 && tid == 0) {
      cu_seqlens[El] = grand;
      if ((int64_t)grand > capacity) raise_error(dev_error, MOE_DEVERR_CAPACITY);
    }
    __syncthreads();
    // pow2 padding rows: workgroup b marks those of experts b, b + grid, ...
    if (pad_pow2)
      for (int e = blockIdx.x; e < El; e += gridDim.x)
        for (int r = s_start[e] + s_tot[e] + tid; r < s_start[e] + s_size[e] && (int64_t)r < capacity;
             r += blockDim.x) {
          src_of[r] = -1;
          w_perm[r] = 0.0f;
        }
    used_end = grand;
  } else if (COLS) {
    int tot = 0, pre0 = 0, pre1 = 0;
    if (tid < El && nchunks > 0) {
      // every load unconditional (index clamped), so all are in flight
      // before the first use; chunks past the end count 0
      int vals[kColChunks];
#pragma unroll
      for (int c = 0; c < kColChunks; ++c) vals[c] = table[min(c, nchunks - 1) * El + tid];
#pragma unroll
      for (int c = 0; c < kColChunks; ++c) {
        const int v = c < nchunks ? vals[c] : 0;
        tot += v;
        pre0 += c < c0 ? v : 0;
        pre1 += c <= c0 ? v : 0;
      }
    }
    const int sz = tid < El ? (pad_pow2 ? next_pow2_dev(tot) : tot) : 0;
    const int lane = tid & 63, wid = tid >> 6;
    int x = sz;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wid] = x;
    __syncthreads();
    int before = x - sz;
    for (int q = 0; q < wid; ++q) before += s_wave[q];
    const int grand = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    if (tid < El) {
      s_start[tid] = before;
      s_tot[tid] = tot;
      s_size[tid] = sz;
      s_pre[0][tid] = pre0;
      s_pre[1][tid] = pre1;
      if (blockIdx.x == 0) {
        counts[tid] = tot;
        cu_seqlens[tid] = before;
      }
    }
    if (blockIdx.x == 0 && tid == 0) {
      cu_seqlens[El] = grand;
      if ((int64_t)grand > capacity) raise_error(dev_error, MOE_DEVERR_CAPACITY);
    }
    __syncthreads();
    // pow2 padding rows: workgroup b marks those of experts b, b + grid, ...
    if (pad_pow2)
      for (int e = blockIdx.x; e < El; e += gridDim.x)
        for (int r = s_start[e] + s_tot[e] + tid; r < s_start[e] + s_size[e] && (int64_t)r < capacity;
             r += blockDim.x) {
          src_of[r] = -1;
          w_perm[r] = 0.0f;
        }
    used_end = grand;
  } else {
    used_end = cu_seqlens[El];
    // pow2 padding rows: workgroup b marks those of experts b, b + grid, ...
    if (pad_pow2)
      for (int e = blockIdx.x; e < El; e += gridDim.x) {
        const int r1 = cu_seqlens[e + 1];
        for (int r = cu_seqlens[e] + counts[e] + tid; r < r1 && (int64_t)r < capacity;
             r += blockDim.x) {
          src_of[r] = -1;
          w_perm[r] = 0.0f;
        }
      }
  }
  // rows past the last segment are unused: mark them as well, so that every
  // row of the caller's buffer has a defined src_of and w_perm
  for (int64_t r = used_end + (int64_t)blockIdx.x * blockDim.x + tid; r < capacity;
       r += (int64_t)gridDim.x * blockDim.x) {
    src_of[r] = -1;
    w_perm[r] = 0.0f;
  }
  if (tid < nslots) {
    int r = -1;
    if (my_slot) {
      const int64_t i = my_i;
      const int rk = my_rank;
      if (rk >= 0) {
        const int e = my_id - expert_begin;
        int64_t first;   // absolute first row of (chunk of i, e)
        if (FUSED) {
          first = s_start[e];
          for (int c = 0; c < (int)(i / kChunk); ++c) first += s_tab[c * El + e];
        } else if (COLS) {
          first = s_start[e] + s_pre[(int)(i / kChunk) > c0 ? 1 : 0][e];
        } else {
          first = table[(i / kChunk) * El + e];
        }
        const int64_t rr = first + rk;
        if (rr < capacity) {
          r = (int)rr;
          src_of[r] = (int32_t)i;
          w_perm[r] = my_w;
        } else {
          raise_error(dev_error, MOE_DEVERR_CAPACITY);
        }
      }
      row_of[i] = r;
    }
    dest[tid] = r;
  }
  __syncthreads();
  const int nvec = H / 8;
  const int total = tok_per_block * nvec;
  for (int idx = tid; idx < total; idx += blockDim.x) {
    const int tl = idx / nvec;
    const int c = idx - tl * nvec;
    const int t = t0 + tl;
    if (t >= T) break;
    bool any = false;
    for (int k = 0; k < K; ++k) any |= dest[tl * K + k] >= 0;
    if (!any) continue;
    uint4 val = reinterpret_cast<const uint4*>(hidden + (int64_t)t * H)[c];
    if (QDQ) val = fq_block128_vec(val);
    for (int k = 0; k < K; ++k) {
      const int r = dest[tl * K + k];
      if (r >= 0) store_row_vec(x_perm + (int64_t)r * H, c, val);
    }
  }
}

// The whole permute in one launch, for at most kSmallTK slots and 1024 local
// experts.  Every workgroup loads all the slot ids and its own tokens' rows
// at once (neither depends on anything else).  It needs only the per-expert
// totals and the ranks of its own slots, so it builds two histograms in LDS
// (no-return atomic adds): of all slots, and of the slots before its first
// one.  An own slot's rank is the second histogram's count for its expert
// plus the same-expert own slots before it — its position among the
// expert's slots in flat-index order, as the multi-launch path ranks them.
// It then scans the totals as the fused scatter does and copies its tokens'
// rows to their destinations: one round trip to memory instead of the three
// of rank -> table -> rows.  Workgroup 0 writes counts and cu_seqlens.
constexpr int kSmallTK = 4096;
constexpr int kSmallIds = kSmallTK / 256;          // slot ids per thread
constexpr int kSmallPre = 4;                       // row vectors per thread loaded up front

template <bool QDQ>
__global__ void __launch_bounds__(256) permute_small_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const uint16_t* __restrict__ hidden, int T, int K, int H, int num_experts, int expert_begin,
    int El,
    int tok_per_block, int pad_pow2, int64_t capacity, uint16_t* __restrict__ x_perm,
    int32_t* __restrict__ row_of, int32_t* __restrict__ src_of, float* __restrict__ w_perm,
    int32_t* __restrict__ dev_error, int32_t* __restrict__ counts,
    int32_t* __restrict__ cu_seqlens) {
  __shared__ int32_t hist[1024], hist_pre[1024];
  __shared__ int32_t s_start[1024], s_tot[1024], s_size[1024];
  __shared__ int32_t own_e[256], dest[256];
  __shared__ int32_t s_wave[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int TK = T * K;
  const int t0 = blockIdx.x * tok_per_block;
  const int i0 = t0 * K;                                   // first slot of this workgroup
  const int nslots = max(0, min(tok_per_block * K, TK - i0));
  const int nvec = H / 8;
  const int total = max(0, min(tok_per_block, T - t0)) * nvec;  // row vectors to copy
  // the local expert of a slot id, or -1 (padding, or another rank's expert)
  auto local_expert = [&](int id) {
    const int le = id - expert_begin;
    return (id >= 0 && le >= 0 && le < El) ? le : -1;
  };

  // loads that depend on nothing: the tokens' rows, every slot id, own slots
  uint4 pre[kSmallPre];
#pragma unroll
  for (int j = 0; j < kSmallPre; ++j) {
    const int idx = tid + j * 256;
    pre[j] = make_uint4(0, 0, 0, 0);
    if (idx < total) {
      const int tl = idx / nvec, c = idx - tl * nvec;
      pre[j] = reinterpret_cast<const uint4*>(hidden + (int64_t)(t0 + tl) * H)[c];
    }
  }
  int ids[kSmallIds];
#pragma unroll
  for (int q = 0; q < kSmallIds; ++q) {
    const int i = tid + q * 256;
    ids[q] = i < TK ? topk_idx[i] : -1;
  }
  const int own_id = tid < nslots ? topk_idx[i0 + tid] : -1;
  const float wt = tid < nslots ? topk_w[i0 + tid] : 0.0f;

  for (int e = tid; e < El; e += 256) {
    hist[e] = 0;
    hist_pre[e] = 0;
  }
  if (tid < 256) own_e[tid] = local_expert(own_id);
  if (tid < nslots) check_expert_id(own_id, num_experts, dev_error);   // each slot once
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kSmallIds; ++q) {
    const int i = tid + q * 256;
    const int e = local_expert(ids[q]);
    if (e >= 0) {
      atomicAdd(&hist[e], 1);
      if (i < i0) atomicAdd(&hist_pre[e], 1);
    }
  }
  __syncthreads();

  // per-expert totals and sizes (thread tid owns experts 4 tid .. 4 tid + 3),
  // then a block-wide exclusive scan of the sizes
  int tot[4], sz[4], local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    tot[j] = e < El ? hist[e] : 0;
    sz[j] = e < El ? (pad_pow2 ? next_pow2_dev(tot[j]) : tot[j]) : 0;
    local += sz[j];
  }
  int x = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[w] = x;
  __syncthreads();
  int run = x - local;
  for (int q = 0; q < w; ++q) run += s_wave[q];
  const int grand = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    if (e < El) {
      s_start[e] = run;
      s_tot[e] = tot[j];
      s_size[e] = sz[j];
      if (blockIdx.x == 0) {
        counts[e] = tot[j];
        cu_seqlens[e] = run;
      }
    }
    run += sz[j];
  }
  if (blockIdx.x == 0 && tid == 0) {
    cu_seqlens[El] = grand;
    if ((int64_t)grand > capacity) raise_error(dev_error, MOE_DEVERR_CAPACITY);
  }
  __syncthreads();
  // pow2 padding rows (workgroup b marks those of experts b, b + grid, ...)
  // and the rows past the last segment
  if (pad_pow2)
    for (int e = blockIdx.x; e < El; e += gridDim.x)
      for (int r = s_start[e] + s_tot[e] + tid; r < s_start[e] + s_size[e] && (int64_t)r < capacity;
           r += blockDim.x) {
        src_of[r] = -1;
        w_perm[r] = 0.0f;
      }
  for (int64_t r = grand + (int64_t)blockIdx.x * blockDim.x + tid; r < capacity;
       r += (int64_t)gridDim.x * blockDim.x) {
    src_of[r] = -1;
    w_perm[r] = 0.0f;
  }

  // destinations of the own slots: segment start + rank among the earlier
  // slots of the same expert (those before the workgroup's first slot, then
  // the own slots before this one)
  if (tid < tok_per_block * K) {
    int r = -1;
    if (tid < nslots) {
      const int e = own_e[tid];
      if (e >= 0) {
        int rk = hist_pre[e];
        for (int m = 0; m < tid; ++m) rk += own_e[m] == e;
        const int64_t rr = (int64_t)s_start[e] + rk;
        if (rr < capacity) {
          r = (int)rr;
          src_of[r] = i0 + tid;
          w_perm[r] = wt;
        } else {
          raise_error(dev_error, MOE_DEVERR_CAPACITY);
        }
      }
      row_of[i0 + tid] = r;
    }
    dest[tid] = r;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSmallPre; ++j) {
    const int idx = tid + j * 256;
    if (idx < total) {
      const int tl = idx / nvec, c = idx - tl * nvec;
      const uint4 v = QDQ ? fq_block128_vec(pre[j]) : pre[j];
      for (int k = 0; k < K; ++k) {
        const int r = dest[tl * K + k];
        if (r >= 0) store_row_vec(x_perm + (int64_t)r * H, c, v);
      }
    }
  }
  for (int idx = tid + kSmallPre * 256; idx < total; idx += 256) {  // rows past the preload
    const int tl = idx / nvec, c = idx - tl * nvec;
    bool any = false;
    for (int k = 0; k < K; ++k) any |= dest[tl * K + k] >= 0;
    if (!any) continue;
    uint4 val = reinterpret_cast<const uint4*>(hidden + (int64_t)(t0 + tl) * H)[c];
    if (QDQ) val = fq_block128_vec(val);
    for (int k = 0; k < K; ++k) {
      const int r = dest[tl * K + k];
      if (r >= 0) store_row_vec(x_perm + (int64_t)r * H, c, val);
    }
  }
}

size_t permute_workspace_bytes(int64_t TK, int El) {
  const int64_t nchunks = (TK + kChunk - 1) / kChunk;
  size_t table = (size_t)nchunks * El * sizeof(int32_t);
  table = (table + 255) & ~(size_t)255;
  size_t rank = (size_t)TK * sizeof(int32_t);
  return table + ((rank + 255) & ~(size_t)255);
}

int launch_permute(const int32_t* topk_idx, const float* topk_w, const uint16_t* hidden, int T,
                   int K, int H, int num_experts, int expert_begin, int El, int pad_pow2,
                   int dispatch_fp8,
                   int64_t capacity,
                   int32_t* counts, int32_t* cu_seqlens, uint16_t* x_perm, int32_t* row_of,
                   int32_t* src_of, float* w_perm, void* workspace, int32_t* dev_error,
                   hipStream_t stream) {
  const int64_t TK = (int64_t)T * K;
  const int nchunks = (int)((TK + kChunk - 1) / kChunk);
  size_t table_bytes = ((size_t)nchunks * El * sizeof(int32_t) + 255) & ~(size_t)255;
  int32_t* table = static_cast<int32_t*>(workspace);
  int32_t* rank = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + table_bytes);
  int nbits = 1;
  while ((1 << nbits) < El) ++nbits;

  const int nvec = H / 8;
  int tpb = 256 / nvec;
  if (tpb < 1) tpb = 1;
  if (tpb * K > 256) tpb = 256 / K;
  const int grid = T > 0 ? (T + tpb - 1) / tpb : 1;
  if (TK <= kSmallTK && El <= 1024) {
#define MOE_PERMUTE_SMALL(Q)                                                                   \
  hipLaunchKernelGGL(permute_small_kernel<Q>, dim3(grid), dim3(256), 0, stream, topk_idx, topk_w, \
                     hidden, T, K, H, num_experts, expert_begin, El, tpb, pad_pow2, capacity,      \
                     x_perm, row_of, src_of, w_perm, dev_error, counts, cu_seqlens)
    if (dispatch_fp8) MOE_PERMUTE_SMALL(true); else MOE_PERMUTE_SMALL(false);
#undef MOE_PERMUTE_SMALL
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  if (nchunks > 0)
    hipLaunchKernelGGL(permute_chunk_rank_kernel, dim3(nchunks), dim3(256), 0, stream, topk_idx,
                       TK, num_experts, expert_begin, El, nbits, table, rank, dev_error);
  const bool fused = (int64_t)nchunks * El <= kFuseTable && nchunks <= kFuseChunks && El <= 1024;
  // up to kColChunks chunks and 256 experts, the scatter's workgroups read
  // the table's columns themselves and the scan kernel is not launched
  const bool cols = !fused && T > 0 && nchunks <= kColChunks && El <= 256;
  if (!fused && !cols)
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, stream, table, nchunks, El,
                       pad_pow2, capacity, counts, cu_seqlens, dev_error);
#define MOE_PERMUTE_SCATTER(F, C, Q)                                                            \
  hipLaunchKernelGGL((permute_scatter_kernel<F, C, Q>), dim3(grid), dim3(256), 0, stream, topk_idx, \
                     topk_w, hidden, T, K, H, expert_begin, El, tpb, capacity, table, nchunks,     \
                     pad_pow2, rank, x_perm, row_of, src_of, w_perm, dev_error, counts, cu_seqlens)
  if (fused) {
    if (dispatch_fp8) MOE_PERMUTE_SCATTER(true, false, true); else MOE_PERMUTE_SCATTER(true, false, false);
  } else if (cols) {
    if (dispatch_fp8) MOE_PERMUTE_SCATTER(false, true, true); else MOE_PERMUTE_SCATTER(false, true, false);
  } else if (T > 0 || capacity > 0) {
    if (dispatch_fp8) MOE_PERMUTE_SCATTER(false, false, true); else MOE_PERMUTE_SCATTER(false, false, false);
  }
#undef MOE_PERMUTE_SCATTER
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---------------------------------------------------------------------------
// The permute without a caller workspace (moe_permute_noalloc): the chunk
// table and the ranks live in a fixed device array instead.  Each GPU the
// library runs on holds its own copy of `scratch` until the process ends;
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept here.  In host code the array's name is
// only a host-side stand-in, never a device address, so nothing but the
// looked-up pointer is ever handed to a kernel.  The kernels write every
// table entry and rank they later read, so nothing needs clearing between
// calls; calls that overlap on one GPU share the array and race.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxDevices];

size_t permute_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// The current device's copy of `scratch`, or nullptr with *status set.
static void* current_device_scratch(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    *status = MOE_ERR_HIP;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = MOE_ERR_UNSUPPORTED;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
    *status = MOE_ERR_HIP;
    return nullptr;
  }
  g_scratch_ptr[dev].store(q, std::memory_order_release);   // racing threads store the same
  return q;
}

int launch_permute_noalloc(const int32_t* topk_idx, const float* topk_w, const uint16_t* hidden,
                           int T, int K, int H, int num_experts, int expert_begin, int El,
                           int pad_pow2, int dispatch_fp8, int64_t capacity, int32_t* counts,
                           int32_t* cu_seqlens, uint16_t* x_perm, int32_t* row_of,
                           int32_t* src_of, float* w_perm, int32_t* dev_error,
                           hipStream_t stream) {
  if (permute_workspace_bytes((int64_t)T * K, El) > kNoAllocScratchBytes) return MOE_ERR_SCRATCH;
  int status = MOE_OK;
  void* ws = current_device_scratch(&status);
  if (!ws) return status;
  return launch_permute(topk_idx, topk_w, hidden, T, K, H, num_experts, expert_begin, El,
                        pad_pow2, dispatch_fp8, capacity, counts, cu_seqlens, x_perm, row_of,
                        src_of, w_perm, ws, dev_error, stream);
}

}  // namespace moe
