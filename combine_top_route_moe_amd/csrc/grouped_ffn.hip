// Grouped SwiGLU expert FFN over expert-contiguous segments: two grouped
// GEMMs on BF16 MFMA (v_mfma_f32_16x16x32_bf16), float32 accumulate.
//
// Source: "[Distributed][MoonEP] BF16 integration of MoonEP balanced EP
// backend", commit message adding the modular experts (gate, up and down
// grouped matmuls over the cu_seqlens segments, route weights before the
// down projection, empty segments skipped; H and I multiples of 128) and
// "Known limitations" (a tuned grouped GEMM in place of a segment loop);
// "[Kernel] DeepEP dispatch-combine kernel integration", review thread on
// the DeepEP + DeepGEMM test (w1 has 2n rows: gate and up).
//
//   gate/up:  a[r, j] = bf16( silu(x[r] . w13[e, j]) * (x[r] . w13[e, I + j]) )
//   down:     y[r, n] = bf16( row_scale[r] * (a[r] . w2[e, n]) )
//
// Both are "NT" products — every operand row is contiguous along the
// reduction dimension — which is the layout the MFMA fragments want: a lane
// reads 8 consecutive bf16 (16 bytes) of one row for both A and B.
//
// Two kernels.  With weights packed once by moe_pack_ffn_weights (the
// layer's path), the fragment-streaming kernel further down.  With row-major
// weights, grouped_gemm_kernel: a workgroup of 4 wavefronts owns a BM x BN
// output tile (BM = BN = 128); wave (wm, wn) owns a 64 x 64 quarter as 4 x 4
// MFMA 16x16 tiles.
// K advances 64 at a time through LDS (rows padded by 16 bytes to spread
// banks), with the next K-slab prefetched into registers while the MFMAs
// run on the current one.  For gate/up the 128 B-rows of a tile are 64 gate
// rows and the 64 matching up rows, arranged so that each lane's gate and
// up accumulators hold the same (row, j): SwiGLU is lane-local in the
// epilogue and the [n, 2I] intermediate never exists.
//
// Scheduling: the grid is sized from an upper bound on tiles (rows /BM + G
// m-tiles), and each workgroup decodes its tile from the device-side
// counts (no host sync): tiles are numbered expert by expert, n-tile by
// n-tile, m-tile fastest, so the m-tiles that share one weight panel run
// back to back, and runs of consecutive tile numbers are mapped to one XCD
// so that a weight panel and an activation panel are fetched once into that
// XCD's L2.
// Workgroups past the last tile exit at once.  MFMA sub-tiles lying wholly
// past the segment's last row are skipped.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "gemm_common.h"

namespace moe {

// the row-major-weight kernel's block tile
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kLdsStride = kBK + 8;  // bf16 elements per LDS row
constexpr int kThreads = 256;

template <bool GATE_UP>
__global__ void __launch_bounds__(kThreads, 2) grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ counts, int G,
    int Kdim /* reduction */, int Nw /* rows of W per group */, int Nout /* out cols */,
    const float* __restrict__ row_scale, uint16_t* __restrict__ Out, int64_t capacity,
    int32_t* __restrict__ dev_error) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLdsStride];

  const int n_tiles = GATE_UP ? Nout / (kBN / 2) : Nout / kBN;
  const int pid = xcd_remap(blockIdx.x);
  int g, mt, nt;
  if (!decode_tile(pid, counts, G, n_tiles, capacity, g, mt, nt)) return;

  const int seg0 = cu_seqlens[g];
  const int nrows = counts[g];
  if ((int64_t)seg0 + nrows > capacity || seg0 < 0) {
    if ((threadIdx.x & 63) == 0) raise_error(dev_error, MOE_DEVERR_ROW_RANGE);
    return;
  }
  const int m0 = mt * kBM;                       // first row of the tile within the segment
  const int valid = min(kBM, nrows - m0);        // rows of this tile that exist
  if (valid <= 0) return;
  const int64_t row_base = (int64_t)seg0 + m0;

  const uint16_t* Wg = W + (int64_t)g * Nw * Kdim;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wid >> 1, wn = wid & 1;

  // global -> register staging: each thread moves 4 A and 4 B 16-byte vectors
  // per K-slab (a slab row is 64 bf16 = 8 vectors)
  const u32x4_t* a_src[4];
  const u32x4_t* b_src[4];
  int lds_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = tid + j * kThreads;  // 0..1023
    const int r = v >> 3, c = v & 7;
    lds_off[j] = r * kLdsStride + c * 8;
    // rows past the segment re-read its last row: their results are never
    // stored, and an unconditional load keeps the staging in registers
    a_src[j] = reinterpret_cast<const u32x4_t*>(A + (row_base + min(r, valid - 1)) * Kdim) + c;
    int wrow;
    if (GATE_UP)
      wrow = (r < kBN / 2) ? nt * (kBN / 2) + r : Nout + nt * (kBN / 2) + (r - kBN / 2);
    else
      wrow = nt * kBN + r;
    b_src[j] = reinterpret_cast<const u32x4_t*>(Wg + (int64_t)wrow * Kdim) + c;
  }

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // which 16-row M sub-tiles of this wave hold at least one real row
  bool m_live[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) m_live[i] = wm * 64 + i * 16 < valid;
  int b_row[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (GATE_UP)
      b_row[j] = (j < 2) ? wn * 32 + j * 16 : kBN / 2 + wn * 32 + (j - 2) * 16;
    else
      b_row[j] = wn * 64 + j * 16;
  }

  u32x4_t ra[4], rb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ra[j] = a_src[j][0];
    rb[j] = b_src[j][0];
  }
  const int nk = Kdim / kBK;
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4_t*>(&As[lds_off[j]]) = ra[j];
      *reinterpret_cast<u32x4_t*>(&Bs[lds_off[j]]) = rb[j];
    }
    __syncthreads();
    if (kt + 1 < nk) {
      const int adv = (kt + 1) * (kBK / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ra[j] = a_src[j][adv];
        rb[j] = b_src[j][adv];
      }
    }
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      const int kofs = kk + 8 * (lane >> 4);
      bf16x8_t bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[(b_row[j] + (lane & 15)) * kLdsStride + kofs]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!m_live[i]) continue;
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(
            &As[(wm * 64 + i * 16 + (lane & 15)) * kLdsStride + kofs]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds D[4*(lane/16) + q][lane%16] of every 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!m_live[i]) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = wm * 64 + i * 16 + 4 * (lane >> 4) + q;
      if (r >= valid) continue;
      const int64_t orow = row_base + r;
      if (GATE_UP) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float gv = acc[i][j][q], uv = acc[i][j + 2][q];
          const int col = nt * (kBN / 2) + wn * 32 + j * 16 + (lane & 15);
          Out[orow * Nout + col] = (uint16_t)f32_to_bf16(silu_f(gv) * uv);
        }
      } else {
        const float sc = row_scale ? row_scale[orow] : 1.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = nt * kBN + wn * 64 + j * 16 + (lane & 15);
          Out[orow * Nout + col] = (uint16_t)f32_to_bf16(sc * acc[i][j][q]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Packed weights and the fragment-streaming GEMM.
//
// Packed layout ("fragment order", K-major): for every group and every
// 32-wide K-step, the column tiles of 64 weight rows follow one another, and
// each holds its four 16x32 MFMA B-fragments back to back, each as 64 lanes x
// 16 bytes in lane order: lane l holds W[row0 + l%16][k0 + 8*(l/16) .. +8].
// A w13 column tile is 32 gate rows (fragments 0, 1) and the 32 matching up
// rows (fragments 2, 3); a w2 column tile is 64 consecutive rows.  A wave
// therefore streams its weights as perfectly coalesced 1 KB loads straight
// into the registers the MFMA reads, with no LDS round trip and no barrier;
// and all the workgroups of one expert, kept in step, read one compact
// window of memory at a time (better DRAM row locality than one stream per
// column tile).
//
// The kernel: a workgroup of NW waves covers up to 128 rows of one segment
// (8 m-subtiles; the ones past the segment end are skipped) and NW column
// tiles (wave w owns tile NW*cb + w).  Weights are prefetched kPrefetch
// K-steps ahead in registers.  The activation rows are shared by all the
// waves: they go into LDS by direct-to-LDS DMA (global_load_lds_dwordx4), in
// the same fragment order so every LDS read is one contiguous, conflict-free
// 1 KB, through a ring of kStages stages of kChunkSteps K-steps, the DMA
// running kStages-1 chunks ahead so that its latency hides behind compute.
// Neither the DMA nor the chunk barrier may wait for the weight prefetches
// (lds_barrier and dma16 below say how), or the weight pipeline would drain
// at every chunk.
constexpr int kTallMin = 96;     // mean segment rows from which the tall tiles are used
constexpr int kPrefetch = 4;     // weight K-steps in flight per wave
constexpr int kChunkSteps = 2;   // activation K-steps per LDS stage
constexpr int kStages = 3;       // activation LDS ring: DMA runs kStages-1 chunks ahead
constexpr int kMsub = 8;         // 16-row m-subtiles per workgroup (128 rows)
constexpr int kFrags = 4;        // B fragments per wave (one column tile)
// Waves (= column tiles) per workgroup, NW: 8 when segments are long (the
// activation tile is then shared by more columns), 4 when they are short (more,
// smaller workgroups balance skewed segment sizes better).
//
// Tall tiles (FragShape<true>, the streamed kernel further down): for
// segments of about one to two m-tiles (129..256 rows would otherwise take
// two 128-row m-tiles, the second reading the whole weight panel again for a
// handful of rows), a workgroup covers 256 rows and each wave half a column
// tile: 16 m-subtiles x 2 fragments (w13: the 16 gate rows and the 16
// matching up rows; w2: 32 consecutive rows).  The accumulators stay at
// 16 x 2 x 4 = 128 registers, each weight byte streams into the CU once per
// segment, and a CU still runs 8 weight streams; the cost is twice the LDS
// activation reads per MFMA, which the weight-streaming workloads this is
// used for have to spare.
template <bool TALL> struct FragShape {
  static constexpr int kMs = TALL ? 16 : kMsub;        // 16-row m-subtiles per workgroup
  static constexpr int kFr = TALL ? 2 : kFrags;        // B fragments per wave
  static constexpr int kRows = 16 * kMs;               // rows per tile
  static constexpr int kSB = kMs * kChunkSteps;        // 1 KB blocks per LDS stage
};


// FP8 weights: a lane's 8 E4M3 codes (a B-fragment row piece) to the bf16
// fragment the MFMA reads, bf16(fl32(code * s)) with the tile's scale s —
// the FP8 fake-quant of the original weight, exactly.
__device__ __forceinline__ bf16x8_t dequant8(u32x2_t c, float s) {
  const f32x2_t v0 = __builtin_amdgcn_cvt_pk_f32_fp8(c.x, false) * s;
  const f32x2_t v1 = __builtin_amdgcn_cvt_pk_f32_fp8(c.x, true) * s;
  const f32x2_t v2 = __builtin_amdgcn_cvt_pk_f32_fp8(c.y, false) * s;
  const f32x2_t v3 = __builtin_amdgcn_cvt_pk_f32_fp8(c.y, true) * s;
  const u32x4_t w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(v0, bf16x2_t)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(v1, bf16x2_t)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, bf16x2_t)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(v3, bf16x2_t))};
  return __builtin_bit_cast(bf16x8_t, w);
}

// The epilogue's 16-byte output stores.  The gate/up activations, read once
// by the down GEMM, are stored non-temporally; the down projection's rows
// with ordinary stores (the combine that reads them next is faster when part
// of them is still cached: measured, non-temporal there cost it 6 %).
template <bool NT>
__device__ __forceinline__ void epi_store(u32x4_t* p, const u32x4_t& v) {
  if (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// The weight element of a B-fragment lane: 16 bytes of bf16, or 8 FP8 codes.
template <bool F8>
using WFrag = typename std::conditional<F8, u32x2_t, u32x4_t>::type;

template <bool GATE_UP, bool NT, int NW, bool F8>
__device__ __forceinline__ void frag_gemm_body(
    u32x4_t (*As)[FragShape<false>::kSB][kWave], const WFrag<F8>* __restrict__ wp, int kstride,
    const float* __restrict__ sc_g, const float* __restrict__ sc_u,
    const uint16_t* a_base, const int64_t* a_uoff, const uint32_t* a_voff, int a_chunk_stride,
    int w, int lane, int nks, int nlive,
    int valid, int ct, bool ct_ok, int64_t row_base, int64_t mt_glob, int Nout,
    const float* tile_scale, uint16_t* __restrict__ Out, int crot, bool prio, uint16_t* epi) {
  constexpr int MS = FragShape<false>::kMs, FR = FragShape<false>::kFr;
  constexpr int kDmaPerWave = FragShape<false>::kSB / NW;
  // every workgroup walks K from its own starting chunk (crot) and wraps
  // around, so the many weight streams do not all hit the same offsets —
  // and so the same HBM channels — at the same time
  const int nch = nks / kChunkSteps;
  const int krot = crot * kChunkSteps;
  // x in [0, 2n) -> x mod n, without a division in the inner loop
  auto wrap = [](int x, int n) { return x >= n ? x - n : x; };
  // LDS blocks of m-subtiles past the segment end are never read: skip them
  auto issue_chunk = [&](int chunk, int stage) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) {
      if ((w * kDmaPerWave + q) / kChunkSteps >= nlive) break;
      dma16(a_base + a_uoff[q] + (int64_t)wrap(chunk + crot, nch) * a_chunk_stride, a_voff[q],
            &As[stage][w * kDmaPerWave + q][0]);
    }
    asm volatile("" ::: "memory");
  };
  WFrag<F8> bq[kPrefetch][FR];
  // weights read exactly once stream past the caches (non-temporal)
  auto load_w = [&](int idx) -> WFrag<F8> {
    if (NT) return __builtin_nontemporal_load(&wp[idx]);
    return wp[idx];
  };
  // FP8: the tile scales of K-step kidx (128 K-columns = 4 steps per tile);
  // for w13 fragments 0, 1 are gate rows (sc_g), 2, 3 up rows (sc_u)
  float bsg[kPrefetch], bsu[kPrefetch];
  auto load_scales = [&](int s, int kidx) {
    if (F8) {
      bsg[s] = sc_g[kidx >> 2];
      bsu[s] = sc_u[kidx >> 2];
    }
  };
  auto bfrag = [&](int s, int f) -> bf16x8_t {
    if constexpr (F8)
      return dequant8(bq[s][f], f >= FR / 2 ? bsu[s] : bsg[s]);   // w13: gate, then up
    else
      return __builtin_bit_cast(bf16x8_t, bq[s][f]);
  };

  f32x4_t acc[MS][FR];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int f = 0; f < FR; ++f) acc[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nchunks = nks / kChunkSteps;
#pragma unroll
  for (int c = 0; c < kStages - 1; ++c) issue_chunk(min(c, nchunks - 1), c);
#pragma unroll
  for (int s = 0; s < kPrefetch; ++s) {
#pragma unroll
    for (int f = 0; f < FR; ++f)
      bq[s][f] = load_w(wrap(s + krot, nks) * kstride + f * kWave);
    load_scales(s, wrap(s + krot, nks));
  }
  asm volatile("" ::: "memory");

  // Loads complete in issue order, so waiting until at most n are
  // outstanding, with n no larger than the number issued after the chunk's
  // DMA, guarantees that DMA has landed.  After the DMA of chunk c (issued
  // at the start of chunk c - (kStages-1)) come at least the weight loads of
  // kStages-1 chunks (the later DMAs may be empty for this wave).  The
  // prologue's DMAs are followed by its kPrologue weight loads and the
  // refills of the chunks before c: fewer than that only for chunk 0, which
  // then waits for kPrologue.
  constexpr int kAfterDma = (kStages - 1) * kChunkSteps * FR;
  constexpr int kPrologue = kPrefetch * FR;
  static_assert(kAfterDma <= kPrologue + kChunkSteps * FR, "prologue count");
  static_assert(kPrefetch % kChunkSteps == 0, "chunk boundaries fall on prefetch slots");
  // nks is a multiple of kPrefetch = 4 (K is a multiple of 128)
  int stage = 0;  // ring slot of the current chunk
  int quarter = -1;
  for (int ks0 = 0; ks0 < nks; ks0 += kPrefetch) {
    // progress-ordered issue priority (see the kernel): 3, 2, 1, 0 over the
    // four quarters of K, so a workgroup that has fallen behind the other
    // one on its CU outranks it
    if (prio) {
      const int q = (ks0 * 4) / nks;
      if (q != quarter) {
        quarter = q;
        if (q == 0) __builtin_amdgcn_s_setprio(3);
        else if (q == 1) __builtin_amdgcn_s_setprio(2);
        else if (q == 2) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
    }
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) {
      const int ks = ks0 + s;
      if (s % kChunkSteps == 0) {
        const int chunk = ks / kChunkSteps;
        if (chunk > 0) stage = (stage + 1 == kStages) ? 0 : stage + 1;
        if (kAfterDma > kPrologue && chunk == 0)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAfterDma > kPrologue ? kPrologue : kAfterDma));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAfterDma));
        lds_barrier();
        // the slot kStages-1 ahead was last read in the previous chunk, which
        // every wave has finished; past the end this reloads a valid chunk so
        // the number of outstanding loads stays the same
        const int ahead = (stage + kStages - 1) % kStages;
        issue_chunk(min(chunk + kStages - 1, nchunks - 1), ahead);
      }
      const int sub = ks % kChunkSteps;
      bf16x8_t bfr[FR];
#pragma unroll
      for (int f = 0; f < FR; ++f) bfr[f] = bfrag(s, f);
      // the step's activation fragments are read before the MFMAs, 8
      // m-subtiles at a time (each 8 in two halves, so a segment of at most
      // 64 rows reads only the first): one LDS latency per 8 m-subtiles
      // instead of one per m-subtile
#pragma unroll
      for (int g8 = 0; g8 < MS; g8 += 8) {
        if (g8 >= nlive) break;
        u32x4_t a[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[stage][(g8 + i) * kChunkSteps + sub][lane];
        if (nlive > g8 + 4) {
#pragma unroll
          for (int i = 4; i < 8; ++i) a[i] = As[stage][(g8 + i) * kChunkSteps + sub][lane];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (g8 + i >= nlive) break;
          const bf16x8_t af = __builtin_bit_cast(bf16x8_t, a[i]);
#pragma unroll
          for (int f = 0; f < FR; ++f)
            acc[g8 + i][f] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[f], acc[g8 + i][f], 0, 0, 0);
        }
      }
      // refill this slot kPrefetch steps ahead (past the end: the last step
      // again, which keeps the outstanding-load count constant)
      const int nxt = min(ks + kPrefetch, nks - 1);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int f = 0; f < FR; ++f)
        bq[s][f] = load_w(wrap(nxt + krot, nks) * kstride + f * kWave);
      load_scales(s, wrap(nxt + krot, nks));
      asm volatile("" ::: "memory");
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA may outlive the workgroup
  if (!ct_ok) return;

  // epilogue: lane holds D[4*(lane/16) + q][lane%16] of every 16x16 tile.
  // Each 16-row subtile goes through the wave's LDS staging area (rows padded
  // so the 2-byte writes are conflict-free), and is stored back as 16-byte
  // vectors: whole 128-byte row pieces instead of 2-byte scattered stores.
  // Rows past the segment end are neither staged nor stored.
  // bf16 per staged row: the wave's output columns (gate/up: 32; down: 64) + 8
  constexpr int kEpiStride = (GATE_UP ? 8 * FR : 16 * FR) + 8;
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    if (i >= nlive) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = 4 * (lane >> 4) + q;
      const int r = i * 16 + rr;
      if (r >= valid) continue;
      if (GATE_UP) {
#pragma unroll
        for (int f = 0; f < FR / 2; ++f)
          epi[rr * kEpiStride + f * 16 + (lane & 15)] =
              (uint16_t)f32_to_bf16(silu_f(acc[i][f][q]) * acc[i][f + FR / 2][q]);
      } else {
        const float sc = tile_scale ? tile_scale[r] : 1.0f;
#pragma unroll
        for (int f = 0; f < FR; ++f)
          epi[rr * kEpiStride + f * 16 + (lane & 15)] = (uint16_t)f32_to_bf16(sc * acc[i][f][q]);
      }
    }
    // the staging area is the wave's own: its LDS operations run in order,
    // and the fences keep the compiler from moving them across each other
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (GATE_UP) {
      // a is written in the down GEMM's activation fragment order: block
      // (128-row m-tile, m-subtile, K-step ct) of 64 lanes x 8 values, where
      // lane L = row%16 + 16*(col%32 / 8) holds columns 8*(col%32 / 8) .. +8
      const int row = lane & 15;
      uint16_t* blk = Out + ((mt_glob * kMsub + i) * (int64_t)(Nout / 32) + ct) * (kWave * 8);
      if (i * 16 + row < valid) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&epi[row * kEpiStride + 8 * (lane >> 4)]);
        epi_store<true>(reinterpret_cast<u32x4_t*>(blk) + lane, v);
      }
    } else {
      // 16 rows x 64 columns = 128 pieces of 8 columns, two per lane
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int piece = lane + h * kWave, row = piece >> 3, c8 = piece & 7;
        if (i * 16 + row < valid) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&epi[row * kEpiStride + 8 * c8]);
          epi_store<false>(reinterpret_cast<u32x4_t*>(Out + (row_base + i * 16 + row) * Nout + ct * 64) + c8, v);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
}

// Two waves per SIMD: an 8-wave workgroup needs them, a 4-wave one gets two
// workgroups per CU; the register budget is 256 per lane either way.
template <bool GATE_UP, int NW, bool F8>
__global__ void __launch_bounds__(NW * kWave, 2) frag_gemm_kernel(
    const uint16_t* __restrict__ A, const void* __restrict__ Wf, const float* __restrict__ Wsc,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ counts, int G,
    int Kdim, int Nw /* weight rows per group */, int Nout, const float* __restrict__ row_scale,
    uint16_t* __restrict__ Out, int64_t capacity, int32_t* __restrict__ dev_error) {
  using Shape = FragShape<false>;
  constexpr int BMR = Shape::kRows;
  __shared__ __attribute__((aligned(16))) u32x4_t As[kStages][Shape::kSB][kWave];
  __shared__ __attribute__((aligned(16))) uint16_t Epi[NW][16 * 72];  // per-wave output staging

  const int n_ct = Nw / 64;               // column tiles per group
  const int n_wt = n_ct;                  // wave tiles per group
  const int n_cb = (n_wt + NW - 1) / NW;  // workgroups per m-tile
  const int pid = xcd_remap(blockIdx.x);
  int g, mt, cb;
  int64_t mt_before;
  if (!decode_tile(pid, counts, G, n_cb, capacity, g, mt, cb, &mt_before)) return;
  // the intermediate's m-tile must lie in the workspace (ceil(capacity/128)
  // + G m-tiles): segments that overlap, each inside [0, capacity), could
  // otherwise place later groups' m-tiles past its end
  if (mt_before + mt >= (capacity + kBM - 1) / kBM + G) {
    if ((threadIdx.x & 63) == 0) raise_error(dev_error, MOE_DEVERR_ROW_RANGE);
    return;
  }
  int mt_base = (int)mt_before;
  // the same in every lane: say so, so that addresses built from them stay scalar
  g = __builtin_amdgcn_readfirstlane(g);
  mt = __builtin_amdgcn_readfirstlane(mt);
  cb = __builtin_amdgcn_readfirstlane(cb);
  mt_base = __builtin_amdgcn_readfirstlane(mt_base);
  const int seg0 = cu_seqlens[g];
  const int nrows = counts[g];
  if ((int64_t)seg0 + nrows > capacity || seg0 < 0) {
    if ((threadIdx.x & 63) == 0) raise_error(dev_error, MOE_DEVERR_ROW_RANGE);
    return;
  }
  const int m0 = mt * BMR;
  const int valid = min(BMR, nrows - m0);
  if (valid <= 0) return;
  const int64_t row_base = (int64_t)seg0 + m0;
  const int nlive = (valid + 15) >> 4;   // m-subtiles holding real rows

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the last column block may hold fewer than NW wave tiles: the spare
  // waves stream a real tile and store nothing
  const bool ct_ok = cb * NW + w < n_wt;
  const int wt = ct_ok ? cb * NW + w : n_wt - 1;
  const int ct = wt;
  const int nks = Kdim / 32;

  // this wave's weight stream: step ks, fragment f at wp[ks * kstride + f * 64]
  // (in fragment-lane units: 16 bytes of bf16 or 8 FP8 codes)
  const int kstride = n_ct * kFrags * kWave;
  const WFrag<F8>* wp = reinterpret_cast<const WFrag<F8>*>(Wf) +
                        ((int64_t)g * nks * n_ct + ct) * (kFrags * kWave) + lane;
  // FP8: the scale rows ([G][Nw/128][Kdim/128]) of this tile's gate and up
  // rows (w13: gate rows 32 ct.., up rows Nw/2 + 32 ct..; w2: rows 64 ct..)
  const int nkb = Kdim / 128, nrb = Nw / 128;
  const float* sc_g = nullptr;
  const float* sc_u = nullptr;
  if (F8) {
    const int rb_g = GATE_UP ? (32 * ct) / 128 : (64 * ct) / 128;
    const int rb_u = GATE_UP ? (Nw / 2 + 32 * ct) / 128 : rb_g;
    sc_g = Wsc + ((int64_t)g * nrb + rb_g) * nkb;
    sc_u = Wsc + ((int64_t)g * nrb + rb_u) * nkb;
  }
  // the activation DMA: this wave fills LDS blocks kDmaPerWave*w .. of a
  // stage; block b is m-subtile b / kChunkSteps, K-step b % kChunkSteps
  constexpr int kDmaPerWave = Shape::kSB / NW;
  // gate/up reads the permuted rows (row-major); down reads the gate/up
  // output, which that kernel wrote in fragment order per 128-row m-tile.
  // Source of block q: a_base + a_uoff[q] (+ the chunk's offset) in
  // elements, uniform, plus a_voff[q] bytes per lane
  const int64_t mt_glob = (int64_t)mt_base + mt;
  const uint16_t* a_base =
      GATE_UP ? A + row_base * Kdim : A + mt_glob * kMsub * (int64_t)nks * (kWave * 8);
  int64_t a_uoff[kDmaPerWave];
  uint32_t a_voff[kDmaPerWave];
#pragma unroll
  for (int q = 0; q < kDmaPerWave; ++q) {
    const int b = w * kDmaPerWave + q;
    const int ms = b / kChunkSteps, sub = b % kChunkSteps;
    if (GATE_UP) {
      const int r = min(ms * 16 + (lane & 15), valid - 1);   // rows past the end re-read the last
      a_uoff[q] = 0;
      a_voff[q] = (uint32_t)(r * Kdim + sub * 32 + 8 * (lane >> 4)) * 2u;
    } else {
      a_uoff[q] = ((int64_t)ms * nks + sub) * (kWave * 8);
      a_voff[q] = (uint32_t)lane * 16u;
    }
  }
  const int a_chunk_stride = GATE_UP ? kChunkSteps * 32 : kChunkSteps * kWave * 8;

  // down: the tile's row scales, staged in LDS once for the epilogue
  __shared__ float rs[BMR];
  const float* tile_scale = nullptr;
  if (!GATE_UP && row_scale) {
    for (int r = threadIdx.x; r < valid; r += NW * kWave) rs[r] = row_scale[row_base + r];
    __syncthreads();
    tile_scale = rs;
  }

  // an expert whose rows fit in one tile reads each weight byte once
  const bool once = nrows <= BMR;
  // K rotation for experts read once, so that the experts in flight do not
  // all read the same K offsets (the same HBM channels) at the same time:
  // per expert with 8-wave workgroups (the expert's workgroups stay in step
  // and read one compact window), per workgroup with 4-wave ones (measured
  // faster for short segments).  Experts with several m-tiles keep every
  // workgroup in step, so that their m-tiles share the weights and their
  // column blocks share the activation tiles through L2.
  const uint32_t rkey = NW == 8 ? (uint32_t)g * 977u : (uint32_t)g * 977u + (uint32_t)cb;
  const int crot = once ? (int)((rkey * 2654435761u) >> 8) % (nks / kChunkSteps) : 0;
  // When every segment fits one m-tile, all workgroups stream the same
  // amount, and a CU holds two 4-wave ones that start together; the older
  // one's waves win the memory-issue arbitration and finish far earlier,
  // leaving the other to stream alone.  Lowering each wave's priority as it
  // passes each quarter of K keeps the two in step (measured: balanced
  // gate/up -3 %).  With longer segments the workgroups' lengths differ and
  // the same rule is slower, so it is used only when no segment exceeds an
  // m-tile (the same answer in every workgroup: all read the same counts).
  bool prio = false;
  if (NW == 4 && once) {
    bool fits = true;
    for (int e = lane; e < G; e += kWave) fits = fits && counts[e] <= BMR;
    prio = __ballot(!fits) == 0;
  }
  if (once)
    frag_gemm_body<GATE_UP, true, NW, F8>(As, wp, kstride, sc_g, sc_u, a_base, a_uoff, a_voff,
                                          a_chunk_stride, w, lane, nks, nlive, valid, ct, ct_ok,
                                          row_base, mt_glob, Nout, tile_scale, Out, crot, prio,
                                          Epi[w]);
  else
    frag_gemm_body<GATE_UP, false, NW, F8>(As, wp, kstride, sc_g, sc_u, a_base, a_uoff, a_voff,
                                           a_chunk_stride, w, lane, nks, nlive, valid, ct, ct_ok,
                                           row_base, mt_glob, Nout, tile_scale, Out, crot, false,
                                           Epi[w]);
}

// ---------------------------------------------------------------------------
// The tall tiles, streamed.  With one tile per workgroup every tile boundary
// would stall the CU's memory streams: the waves wait for all their
// loads (the weight prefetch runs kPrefetch steps past the end), decode the
// next tile from the counts in memory, store their outputs, and only then
// start the next tile's weight and activation streams, whose first bytes
// land a memory latency later.  With weight-streaming tiles of about 50 us
// that is several per cent of the time.
//
// Here a persistent workgroup walks its tiles (virtual blocks b, b + grid,
// ..., in increasing tile order) and its streams run on across each
// boundary: in a tile's last kPrefetch K-steps the weight refills fetch the
// next tile's first steps, and the DMAs of its last kStages-1 chunks fill the
// ring with the next tile's first chunks (the ring carries on slot after
// slot), so the next tile's data is in flight while this tile's epilogue
// runs.  The tile table (per group: tiles up to and including it, 128-row
// m-tiles before it, segment start, row count) is built once per workgroup
// in LDS, so a decode issues no memory load.  The down projection's row
// scales arrive by DMA with each tile's first chunk, in a double buffer.
//
// Wait accounting, per wave (loads complete in issue order; stores count in
// vmcnt too):
//  - within a tile as in the 128-row kernel: at a chunk's barrier at least
//    kAfterDma weight loads were issued after that chunk's DMA;
//  - the next tile's chunk 0 goes out with this tile's chunk L-1 (L the
//    last), followed by kAfterDma weight refills and then the epilogue's
//    stores: exactly kStreamStores of them, since every m-subtile issues one
//    buffer store whatever it holds (lanes with nothing to write aim it
//    past the buffer's range, where the hardware drops it).  So the next
//    tile's first chunk waits for vmcnt(kAfterDma + kStreamStores) and does
//    not wait for the stores just issued;
//  - its chunk 1 goes out with chunk L, followed by refills, the stores and
//    the next tile's own refills: more than kAfterDma.
// After the workgroup's last tile the refills and DMAs re-read its last step
// and chunk, as the 128-row kernel does, which keeps these counts.
constexpr int kStreamMaxG = 1024;                     // groups the LDS tile table holds
constexpr int kStreamStores = FragShape<true>::kMs;   // epilogue stores per wave and tile
constexpr uint32_t kBufferOob = 0x80000000u;          // a buffer offset past every range

// A raw buffer (stride 0) over `bytes` bytes at p, p wave-uniform: offsets
// at or past `bytes` are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_buffer(uint16_t* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, bytes, 0x00020000);
}

// One tall tile as a wave of the streamed kernel sees it: wave-uniform but
// for a_voff.
struct TallTile {
  int ok;                   // a tile is assigned
  int nlive, valid;         // m-subtiles holding rows, rows
  int ct, hsel, ct_ok;      // column tile, its half, whether this wave's half exists
  int nt, crot;             // weights read once (streamed past the caches), K rotation
  int64_t row_base, mt_glob;
  const void* wp;           // the wave's weight stream at lane 0, K-step 0
  const float* sc_g;        // FP8 weights: the tile scales of the wave's gate (or w2) rows
  const float* sc_u;        // ... and of its up rows, per 128 K
  const uint16_t* a_base;   // the activation DMA's base
  uint32_t a_voff[FragShape<true>::kSB / 8];  // gate/up: per-lane byte offsets of the DMA blocks
};

// Decode virtual block vb into t (t.ok = 0 past the last tile) from the LDS
// tile table.
template <bool GATE_UP, bool F8>
__device__ __forceinline__ void tall_decode(TallTile& t, int vb, int nvirt, const int* t_incl,
                                            const int* t_m128, const int* t_seg, const int* t_cnt,
                                            int G, int n_wt, int n_ct, int nks, int Kdim,
                                            int Nw, const uint16_t* A, const void* Wf,
                                            const float* Wsc, int w, int lane) {
  t.ok = 0;
  if (vb >= nvirt) return;
  const int pid = xcd_remap(vb);
  int g = -1;
  for (int base = 0; base < G; base += kWave) {
    const int e = base + lane;
    const uint64_t hit = __ballot(e < G && pid < t_incl[e]);
    if (hit) {
      g = base + __ffsll((unsigned long long)hit) - 1;
      break;
    }
  }
  if (g < 0) return;
  g = __builtin_amdgcn_readfirstlane(g);
  const int excl = __builtin_amdgcn_readfirstlane(g > 0 ? t_incl[g - 1] : 0);
  const int nrows = __builtin_amdgcn_readfirstlane(t_cnt[g]);
  const int seg0 = __builtin_amdgcn_readfirstlane(t_seg[g]);
  const int m128 = __builtin_amdgcn_readfirstlane(t_m128[g]);
  constexpr int BMR = FragShape<true>::kRows;
  const int mtiles = (nrows + BMR - 1) / BMR;
  const int local = pid - excl;
  const int cb = local / mtiles, mt = local - cb * mtiles;
  t.ok = 1;
  t.valid = min(BMR, nrows - mt * BMR);
  t.nlive = (t.valid + 15) >> 4;
  t.row_base = (int64_t)seg0 + mt * BMR;
  t.mt_glob = (int64_t)m128 + (int64_t)mt * (BMR / kBM);
  int wt = cb * 8 + w;
  t.ct_ok = wt < n_wt;
  if (!t.ct_ok) wt = n_wt - 1;   // a spare wave streams a real half tile and stores nothing
  t.ct = wt >> 1;
  t.hsel = wt & 1;
  t.nt = nrows <= BMR;
  // the 128-row kernel's K rotation for experts read once (per expert)
  t.crot = t.nt ? (int)((((uint32_t)g * 977u) * 2654435761u) >> 8) % (nks / kChunkSteps) : 0;
  t.wp = static_cast<const WFrag<F8>*>(Wf) + ((int64_t)g * nks * n_ct + t.ct) * (kFrags * kWave);
  if (F8) {
    // scale rows ([G][Nw/128][Kdim/128]): w13 gate rows 32 ct + 16 hsel ..,
    // up rows Nw/2 + the same; w2 rows 64 ct + 32 hsel ..; each half tile
    // lies in one 128-row scale block, that of its column tile
    const int nkb = Kdim / 128, nrb = Nw / 128;
    const int rb_g = GATE_UP ? (32 * t.ct) / 128 : (64 * t.ct) / 128;
    const int rb_u = GATE_UP ? (Nw / 2 + 32 * t.ct) / 128 : rb_g;
    t.sc_g = Wsc + ((int64_t)g * nrb + rb_g) * nkb;
    t.sc_u = Wsc + ((int64_t)g * nrb + rb_u) * nkb;
  }
  t.a_base = GATE_UP ? A + t.row_base * Kdim : A + t.mt_glob * kMsub * (int64_t)nks * (kWave * 8);
  if (GATE_UP) {
#pragma unroll
    for (int q = 0; q < FragShape<true>::kSB / 8; ++q) {
      const int b = w * (FragShape<true>::kSB / 8) + q;
      const int ms = b / kChunkSteps, sub = b % kChunkSteps;
      const int r = min(ms * 16 + (lane & 15), t.valid - 1);   // rows past the end re-read the last
      t.a_voff[q] = (uint32_t)(r * Kdim + sub * 32 + 8 * (lane >> 4)) * 2u;
    }
  }
}

template <bool GATE_UP, bool F8>
__global__ void __launch_bounds__(8 * kWave, 2) tall_stream_kernel(
    const uint16_t* __restrict__ A, const void* __restrict__ Wf, const float* __restrict__ Wsc,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ counts, int G,
    int Kdim, int Nw /* weight rows per group */, int Nout, const float* __restrict__ row_scale,
    uint16_t* __restrict__ Out, int64_t capacity, int32_t* __restrict__ dev_error, int nvirt) {
  using Shape = FragShape<true>;
  constexpr int NW = 8, MS = Shape::kMs, FR = Shape::kFr, BMR = Shape::kRows;
  constexpr int kDmaPerWave = Shape::kSB / NW;
  __shared__ __attribute__((aligned(16))) u32x4_t As[kStages][Shape::kSB][kWave];
  __shared__ __attribute__((aligned(16))) uint16_t Epi[NW][16 * 72];   // per-wave output staging
  __shared__ float rs[2][BMR];
  __shared__ int t_incl[kStreamMaxG], t_m128[kStreamMaxG], t_seg[kStreamMaxG], t_cnt[kStreamMaxG];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_ct = Nw / 64, n_wt = 2 * n_ct, n_cb = (n_wt + NW - 1) / NW;
  const int nks = Kdim / 32, nch = nks / kChunkSteps;
  const int kstride = n_ct * kFrags * kWave;

  // the tile table (the 128-row m-tile count, which places the activation
  // rows, counts every group as the 128-row kernel does)
  if (w == 0) {
    int carry = 0;
    long long carry128 = 0;
    const long long ws_mtiles = (capacity + kBM - 1) / kBM + G;
    for (int base = 0; base < G; base += kWave) {
      const int e = base + lane;
      int craw = 0, s0 = 0;
      if (e < G) {
        craw = max(counts[e], 0);
        s0 = cu_seqlens[e];
      }
      // the 128-row m-tiles before each group (the activation layout) come
      // from every group's count, clamped to the capacity and summed in 64
      // bits; a group whose segment leaves [0, capacity), or whose m-tiles
      // would end past the workspace's ceil(capacity/128) + G (overlapping
      // segments), gets no tile
      const int m128 = (int)((min((long long)craw, (long long)capacity) + kBM - 1) / kBM);
      long long incl128 = m128;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const long long y128 = __shfl_up(incl128, off, kWave);
        if (lane >= off) incl128 += y128;
      }
      incl128 += carry128;
      int c = craw;
      if (c > 0 && ((int64_t)s0 + c > capacity || s0 < 0 || incl128 > ws_mtiles)) {
        raise_error(dev_error, MOE_DEVERR_ROW_RANGE);
        c = 0;
      }
      int incl = ((c + BMR - 1) / BMR) * n_cb;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
      }
      incl += carry;
      if (e < G) {
        t_incl[e] = incl;
        t_m128[e] = (int)min(incl128 - m128, ws_mtiles);   // used only by groups with tiles
        t_seg[e] = s0;
        t_cnt[e] = c;
      }
      carry = __shfl(incl, 63, kWave);
      carry128 = __shfl(incl128, 63, kWave);
    }
  }
  __syncthreads();

  TallTile cur, nxt;
  int vb = blockIdx.x;
  tall_decode<GATE_UP, F8>(cur, vb, nvirt, t_incl, t_m128, t_seg, t_cnt, G, n_wt, n_ct,
                           nks, Kdim, Nw, A, Wf, Wsc, w, lane);
  if (!cur.ok) return;   // the whole workgroup

  const uint32_t as_lds = lds_addr(&As[0][0][0]), rs_lds = lds_addr(&rs[0][0]);
  auto wrap = [](int x, int n) { return x >= n ? x - n : x; };
  // the packed fragment of this wave's f-th B operand, the half hsel of its
  // column tile: w13 gate fragment hsel and up fragment hsel + 2; w2
  // fragments 2 hsel and 2 hsel + 1
  auto frag_of = [](const TallTile& t, int f) {
    return GATE_UP ? (f == 0 ? t.hsel : t.hsel + 2) : 2 * t.hsel + f;
  };
  // LDS blocks of m-subtiles past the segment end are never read: skip them
  auto issue_chunk = [&](const TallTile& t, int chunk, int slot) {
    const int64_t coff = (int64_t)wrap(chunk + t.crot, nch) *
                         (GATE_UP ? kChunkSteps * 32 : kChunkSteps * kWave * 8);
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) {
      const int b = w * kDmaPerWave + q;
      if (b / kChunkSteps >= t.nlive) break;
      const int64_t uoff =
          GATE_UP ? 0 : ((int64_t)(b / kChunkSteps) * nks + b % kChunkSteps) * (kWave * 8);
      const uint32_t voff = GATE_UP ? t.a_voff[q] : (uint32_t)lane * 16u;
      dma16_at(t.a_base + uoff + coff, voff, as_lds + (uint32_t)((slot * Shape::kSB + b) * kWave * 16));
    }
  };
  // down: the tile's row scales into rs[buf], rows past the end re-reading the last
  auto issue_scales = [&](const TallTile& t, int buf) {
    if (!GATE_UP && row_scale && w < BMR / kWave) {
      const int r = min(w * kWave + lane, t.valid - 1);
      dma4_at(row_scale + t.row_base, (uint32_t)r * 4u, rs_lds + (uint32_t)((buf * BMR + w * kWave) * 4));
    }
  };
  WFrag<F8> bq[kPrefetch][FR];
  float bsg[kPrefetch], bsu[kPrefetch];   // FP8: the tile scales of each slot's K-step
  // weights read once stream past the caches (non-temporal); gate/up always
  // does, without the per-tile branch (same-box A/B on the deepseek-shape
  // layer, every expert read once: gate/up 2.58 -> 2.50 ms; for down the
  // branch-free form was slower)
  auto load_step = [&](const TallTile& t, int step, int s) {
    const int kidx = wrap(step + t.crot * kChunkSteps, nks);
    const WFrag<F8>* p = static_cast<const WFrag<F8>*>(t.wp) + (int64_t)kidx * kstride + lane;
    if (F8) {   // 128 K-columns = 4 steps per scale
      bsg[s] = t.sc_g[kidx >> 2];
      bsu[s] = t.sc_u[kidx >> 2];
    }
    if (GATE_UP || t.nt) {
#pragma unroll
      for (int f = 0; f < FR; ++f) bq[s][f] = __builtin_nontemporal_load(p + frag_of(t, f) * kWave);
    } else {
#pragma unroll
      for (int f = 0; f < FR; ++f) bq[s][f] = p[frag_of(t, f) * kWave];
    }
  };

  // the first tile's prologue: scales, kStages-1 chunks, kPrefetch weight steps
  asm volatile("" ::: "memory");
  issue_scales(cur, 0);
#pragma unroll
  for (int c = 0; c < kStages - 1; ++c) issue_chunk(cur, min(c, nch - 1), c);
#pragma unroll
  for (int s = 0; s < kPrefetch; ++s) load_step(cur, s, s);
  asm volatile("" ::: "memory");

  constexpr int kAfterDma = (kStages - 1) * kChunkSteps * FR;
  static_assert(kAfterDma <= kPrefetch * FR, "prologue count");
  static_assert(kPrefetch == (kStages - 1) * kChunkSteps, "the last block's chunks are the ring's lookahead");
  static_assert(kAfterDma + kStreamStores < 64, "vmcnt range");
  int stage = kStages - 1;   // ring slot of the current chunk (the prologue filled 0 ..)
  int par = 0;               // row-scale buffer of the current tile
  bool first = true;
  f32x4_t acc[MS][FR];

  // one K-step of the current tile; `tail`: the last kPrefetch steps, whose
  // lookahead loads belong to the next tile (or, after the last, re-read)
  auto step = [&](int ks, int s, bool tail) {
    if (s % kChunkSteps == 0) {
      const int chunk = ks / kChunkSteps;
      stage = stage + 1 == kStages ? 0 : stage + 1;
      if (chunk == 0 && !first)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAfterDma + kStreamStores));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAfterDma));
      lds_barrier();
      // the slot kStages-1 ahead was last read in the previous chunk
      const int slot = stage + kStages - 1 >= kStages ? stage - 1 : stage + kStages - 1;
      const int ahead = chunk + kStages - 1;
      asm volatile("" ::: "memory");
      if (!tail) {
        issue_chunk(cur, ahead, slot);
      } else if (nxt.ok) {
        if (ahead == nch) issue_scales(nxt, par ^ 1);
        issue_chunk(nxt, ahead - nch, slot);
      } else {
        issue_chunk(cur, nch - 1, slot);
      }
      asm volatile("" ::: "memory");
    }
    const int sub = ks % kChunkSteps;
    bf16x8_t bfr[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      if constexpr (F8)   // w13: fragment 0 gate rows, 1 up rows; w2: one scale block
        bfr[f] = dequant8(bq[s][f], (GATE_UP && f == 1) ? bsu[s] : bsg[s]);
      else
        bfr[f] = __builtin_bit_cast(bf16x8_t, bq[s][f]);
    }
#pragma unroll
    for (int g8 = 0; g8 < MS; g8 += 8) {
      if (g8 >= cur.nlive) continue;
      u32x4_t a[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[stage][(g8 + i) * kChunkSteps + sub][lane];
      if (cur.nlive > g8 + 4) {
#pragma unroll
        for (int i = 4; i < 8; ++i) a[i] = As[stage][(g8 + i) * kChunkSteps + sub][lane];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (g8 + i >= cur.nlive) continue;
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, a[i]);
#pragma unroll
        for (int f = 0; f < FR; ++f)
          acc[g8 + i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[f], acc[g8 + i][f], 0, 0, 0);
      }
    }
    asm volatile("" ::: "memory");
    if (!tail)
      load_step(cur, ks + kPrefetch, s);
    else if (nxt.ok)
      load_step(nxt, ks + kPrefetch - nks, s);
    else
      load_step(cur, nks - 1, s);
    asm volatile("" ::: "memory");
  };

  constexpr int kEpiStride = (GATE_UP ? 8 * FR : 16 * FR) + 8;
  uint16_t* epi = Epi[w];
  for (;;) {
    tall_decode<GATE_UP, F8>(nxt, vb + (int)gridDim.x, nvirt, t_incl, t_m128, t_seg, t_cnt, G,
                             n_wt, n_ct, nks, Kdim, Nw, A, Wf, Wsc, w, lane);
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int f = 0; f < FR; ++f) acc[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int ks0 = 0; ks0 < nks - kPrefetch; ks0 += kPrefetch) {
#pragma unroll
      for (int s = 0; s < kPrefetch; ++s) step(ks0 + s, s, false);
    }
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) step(nks - kPrefetch + s, s, true);

    // epilogue, as in the 128-row kernel, but every m-subtile issues
    // exactly one 16-byte buffer store (see the wait accounting above)
    const bool use_scale = !GATE_UP && row_scale != nullptr;
    // gate/up: the tile's 16 m-subtile blocks of the activation layout;
    // down: the tile's rows of the output (rows past the end are out of range)
    const int nblk = Nout / 32;
    const __amdgpu_buffer_rsrc_t rsrc =
        GATE_UP ? wave_buffer(Out + cur.mt_glob * kMsub * (int64_t)nblk * (kWave * 8),
                              MS * nblk * kWave * 8 * 2)
                : wave_buffer(Out + cur.row_base * Nout, cur.valid * Nout * 2);
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      uint32_t off = kBufferOob;
      if (i < cur.nlive && cur.ct_ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = 4 * (lane >> 4) + q;
          const int r = i * 16 + rr;
          if (r >= cur.valid) continue;
          if (GATE_UP) {
            epi[rr * kEpiStride + (lane & 15)] =
                (uint16_t)f32_to_bf16(silu_f(acc[i][0][q]) * acc[i][1][q]);
          } else {
            const float sc = use_scale ? rs[par][r] : 1.0f;
#pragma unroll
            for (int f = 0; f < FR; ++f)
              epi[rr * kEpiStride + f * 16 + (lane & 15)] = (uint16_t)f32_to_bf16(sc * acc[i][f][q]);
          }
        }
        // the staging area is the wave's own: its LDS operations run in
        // order, and the fences keep the compiler from moving them across
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (GATE_UP) {
          // fragment order of the down GEMM's activations: block (m-subtile i,
          // K-step ct), lane L = row + 16 (2 hsel + c8) holding 8 columns
          const int row = lane & 15, c8 = lane >> 4;
          if (lane < 32 && i * 16 + row < cur.valid) {
            v = *reinterpret_cast<const u32x4_t*>(&epi[row * kEpiStride + 8 * c8]);
            off = (uint32_t)(((i * nblk + cur.ct) * kWave + row + 16 * (2 * cur.hsel + c8)) * 16);
          }
        } else {
          // 16 rows x 32 columns (64 ct + 32 hsel ..) = 64 pieces, one per lane
          const int row = lane >> 2, c8 = lane & 3;
          if (i * 16 + row < cur.valid) {
            v = *reinterpret_cast<const u32x4_t*>(&epi[row * kEpiStride + 8 * c8]);
            off = (uint32_t)(((i * 16 + row) * Nout + cur.ct * 64 + 32 * cur.hsel + 8 * c8) * 2);
          }
        }
      }
      // non-temporal (aux bit 1, nt): gate/up's activations are read once, by
      // the down GEMM; the down rows once, by the combine (same-box A/B on
      // the deepseek-shape layer: down 1.475 -> 1.425 ms, the combine
      // unchanged; the 128-row kernel keeps ordinary stores for its down rows)
      __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, (int)off, 0, 2);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    if (!nxt.ok) break;
    cur = nxt;
    par ^= 1;
    first = false;
    vb += gridDim.x;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA may outlive the workgroup
}

// Packing: one thread per 16-byte vector of the source (coalesced reads),
// each written to its place in the packed layout.
__global__ void __launch_bounds__(256) pack_weights_kernel(const uint16_t* __restrict__ W,
                                                           uint16_t* __restrict__ P, int G,
                                                           int N, int Kdim, int gate_up) {
  const int64_t nvec = (int64_t)G * N * Kdim / 8;
  const int nks = Kdim / 32;
  const int n_ct = N / 64;
  const int kvec = Kdim / 8;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int k8 = (int)(v % kvec);
    const int64_t gr = v / kvec;
    const int row = (int)(gr % N);
    const int64_t g = gr / N;
    int ct, f;
    if (gate_up) {
      const int half = N / 2;  // I: gate rows, then up rows
      const int r = row < half ? row : row - half;
      ct = r / 32;
      f = (row < half ? 0 : 2) + (r % 32) / 16;
    } else {
      ct = row / 64;
      f = (row % 64) / 16;
    }
    const int ks = k8 / 4;
    const int lane = (row & 15) + 16 * (k8 & 3);
    const int64_t dst = (((g * nks + ks) * n_ct + ct) * kFrags + f) * kWave + lane;
    reinterpret_cast<uint4*>(P)[dst] = reinterpret_cast<const uint4*>(W)[v];
  }
}

// FP8 weights: one workgroup per 128 x 128 tile of one group's [N, Kdim]
// matrix.  The tile's amax gives its scale s = amax / 448 (IEEE division;
// an all-zero tile gets s = 0 and codes 0); every element becomes the E4M3
// code of clamp(w / s, +-448) (round to nearest even), written in one of
// two fragment orders: k128 = 0, the order of the bf16 packing with 8 codes
// (8 bytes) per lane per 32-wide K-step (for the GEMM that dequantizes to
// bf16); k128 = 1, the order of the FP8 matrix-core GEMM, whose B fragment
// covers a whole 128-wide K-block: per K-block, column tile, fragment and
// half h, 64 lanes x 16 bytes, lane l holding row l%16, columns
// 64 h + 16 (l/16) .. +16 of the block.
__global__ void __launch_bounds__(256) pack_weights_fp8_kernel(const uint16_t* __restrict__ W,
                                                               uint8_t* __restrict__ Q,
                                                               float* __restrict__ S, int N,
                                                               int Kdim, int gate_up, int k128) {
  const int nrb = N / 128, nkb = Kdim / 128;
  const int64_t tile = blockIdx.x;
  const int kb = (int)(tile % nkb);
  const int rb = (int)((tile / nkb) % nrb);
  const int64_t g = tile / ((int64_t)nkb * nrb);
  const int c = threadIdx.x & 15;  // 16-byte vector of the tile row
  const int r0 = threadIdx.x >> 4;  // rows r0, r0 + 16, ...
  const int kvec = Kdim / 8;
  uint4 raw[8];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = (int64_t)g * N + rb * 128 + r0 + 16 * i;
    raw[i] = reinterpret_cast<const uint4*>(W)[row * kvec + kb * 16 + c];
    float f[8];
    unpack8(raw[i], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = amax / 448.0f;
  if (threadIdx.x == 0) S[((int64_t)g * nrb + rb) * nkb + kb] = s;
  const int nks = Kdim / 32, n_ct = N / 64;
  const int k8 = kb * 16 + c;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float f[8];
    unpack8(raw[i], f);
    uint32_t code[2] = {0u, 0u};
    if (s > 0.0f) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = fminf(fmaxf(f[4 * h + j] / s, -448.0f), 448.0f);
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], p, true);
        code[h] = (uint32_t)p;
      }
    }
    const int row = rb * 128 + r0 + 16 * i;
    int ct, f_;
    if (gate_up) {
      const int half = N / 2;
      const int r = row < half ? row : row - half;
      ct = r / 32;
      f_ = (row < half ? 0 : 2) + (r % 32) / 16;
    } else {
      ct = row / 64;
      f_ = (row % 64) / 16;
    }
    int64_t dst;  // in 8-byte units
    if (k128) {
      const int kk = (k8 % 16) * 8;  // column within the K-block
      const int lane = (row & 15) + 16 * ((kk % 64) / 16);
      const int64_t unit = ((((g * nkb + kb) * n_ct + ct) * kFrags + f_) * 2 + kk / 64) * kWave + lane;
      dst = unit * 2 + (kk % 16) / 8;
    } else {
      const int ks = k8 / 4;
      const int lane = (row & 15) + 16 * (k8 & 3);
      dst = (((g * nks + ks) * n_ct + ct) * kFrags + f_) * kWave + lane;
    }
    reinterpret_cast<uint2*>(Q)[dst] = make_uint2(code[0], code[1]);
  }
}

int launch_pack_weights_fp8(const uint16_t* w13, const uint16_t* w2, int G, int H, int I,
                            uint8_t* w13q, float* w13s, uint8_t* w2q, float* w2s, int k128,
                            hipStream_t stream) {
  if (w13) {
    const int64_t tiles = (int64_t)G * (2 * I / 128) * (H / 128);
    if (tiles > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(pack_weights_fp8_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, w13,
                       w13q, w13s, 2 * I, H, 1, k128);
  }
  if (w2) {
    const int64_t tiles = (int64_t)G * (H / 128) * (I / 128);
    if (tiles > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(pack_weights_fp8_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, w2,
                       w2q, w2s, H, I, 0, k128);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_pack_weights(const uint16_t* w13, const uint16_t* w2, int G, int H, int I,
                        uint16_t* w13p, uint16_t* w2p, hipStream_t stream) {
  if (w13 && w13p) {
    const int64_t nvec = (int64_t)G * 2 * I * H / 8;
    const unsigned grid = (unsigned)std::min<int64_t>((nvec + 255) / 256, 65536);
    hipLaunchKernelGGL(pack_weights_kernel, dim3(grid), dim3(256), 0, stream, w13, w13p, G, 2 * I,
                       H, 1);
  }
  if (w2 && w2p) {
    const int64_t nvec = (int64_t)G * H * I / 8;
    const unsigned grid = (unsigned)std::min<int64_t>((nvec + 255) / 256, 65536);
    hipLaunchKernelGGL(pack_weights_kernel, dim3(grid), dim3(256), 0, stream, w2, w2p, G, H, I, 0);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// The intermediate a: row-major [capacity, I] for row-major weights; with
// packed weights, fragment order per m-tile (at most ceil(capacity/128) + G
// m-tiles of 128 rows).  The workspace covers both.
size_t grouped_ffn_workspace_bytes(int64_t capacity, int G, int I) {
  const int64_t rows = std::max<int64_t>(capacity, ((capacity + kBM - 1) / kBM + G) * kBM);
  return (((size_t)rows * I * sizeof(uint16_t)) + 255) & ~(size_t)255;
}

// CUs of the current device (cached per device).
static int device_cu_count() {
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

// Grid of the streamed tall kernel for `nvirt` virtual blocks: one 8-wave
// workgroup per CU (the register budget allows no second), a multiple of 8
// so that each workgroup's virtual blocks stay on its XCD, at most nvirt.
static int64_t stream_grid(int64_t nvirt) {
  const int64_t p = ((int64_t)device_cu_count() / kNumXcd) * kNumXcd;
  return p > 0 && p < nvirt ? p : nvirt;
}

int launch_grouped_ffn(const uint16_t* x, const int32_t* cu_seqlens, const int32_t* counts, int G,
                       int H, int I, const void* w13, const float* w13s, const void* w2,
                       const float* w2s, const float* row_scale, uint16_t* y, int64_t capacity,
                       int flags, void* workspace, int32_t* dev_error, hipStream_t stream) {
  uint16_t* act = static_cast<uint16_t*>(workspace);
  const bool f8 = w13s != nullptr || w2s != nullptr;  // FP8 weights are always packed
  const bool packed = f8 || (flags & MOE_FFN_PACKED_WEIGHTS) != 0;
  const int64_t m_tiles = (capacity + kBM - 1) / kBM + G;
  const int64_t grid_unit = (int64_t)kNumXcd * kXcdChunk;
  auto grid_for = [&](int64_t n_tiles) {
    return (m_tiles * n_tiles + grid_unit - 1) / grid_unit * grid_unit;
  };
  if (capacity == 0) return MOE_OK;
  // Workgroup width (measured): gate/up uses 8 waves once the mean segment
  // fills an m-tile (each activation tile then serves 8 column tiles), else
  // 4 (smaller workgroups balance uneven segments).  The down projection
  // uses 8 only for means between one and two m-tiles; with many m-tiles per
  // expert the smaller workgroups balance better there.  With bf16 weights,
  // segments averaging kTallMin..2*kBM-1 rows (about half of them one m-tile
  // long, half two) use the 8-wave tall tiles in both stages instead, so that
  // no expert streams its weights twice (same-box A/B on the deepseek-shape
  // layer, T=4096, H=7168, 256 experts, I=2048: gate/up 2.75 -> 2.58 ms, down
  // unchanged, the layer 4.86 -> 4.71 ms), in the streamed kernel (down
  // 1.65 -> 1.48 ms more); its LDS tile table holds every group the ABI
  // accepts.  FP8 weights take the same tiles (each expert's weights read
  // once: HBM traffic 1.40 -> 1.0 x on gate/up; the same A/B: gate/up
  // unchanged at 2.38 ms, down 1.40 -> 1.37 ms: with FP8 weights the GEMM is
  // bound by its conversion and issue, not by the bytes).
  const int64_t mean_x = capacity / G;  // mean rows per group, rounded down
  const bool wide = mean_x >= kBM;
  const bool wide_down = wide && mean_x < 2 * kBM;
  const bool tall = packed && mean_x >= kTallMin && mean_x < 2 * kBM;
  const int64_t m_tiles_tall = (capacity + 2 * kBM - 1) / (2 * kBM) + G;
  auto grid_tall = [&](int64_t n_tiles) {
    return (m_tiles_tall * n_tiles + grid_unit - 1) / grid_unit * grid_unit;
  };
  if (tall && G > kStreamMaxG) return MOE_ERR_UNSUPPORTED;   // the ABI admits at most 1024
  if ((flags & MOE_FFN_GATE_UP) && tall) {
    const int64_t blocks = grid_tall((2 * (2 * I / 64) + 7) / 8);
    if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
#define MOE_TALL_GU(F8)                                                                         \
  hipLaunchKernelGGL((tall_stream_kernel<true, F8>), dim3((unsigned)stream_grid(blocks)),          \
                     dim3(8 * kWave), 0, stream, x, w13, w13s, cu_seqlens, counts, G, H, 2 * I, I, \
                     nullptr, act, capacity, dev_error, (int)blocks)
    if (f8) MOE_TALL_GU(true); else MOE_TALL_GU(false);
#undef MOE_TALL_GU
  } else if (flags & MOE_FFN_GATE_UP) {
    if (packed) {
      const int nw = wide ? 8 : 4;
      const int64_t blocks = grid_for((2 * I / 64 + nw - 1) / nw);
      if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
#define MOE_FRAG_GU(NW, F8)                                                                  \
  hipLaunchKernelGGL((frag_gemm_kernel<true, NW, F8>), dim3((unsigned)blocks), dim3(NW * kWave),        \
                     0, stream, x, w13, w13s, cu_seqlens, counts, G, H, 2 * I, I, nullptr, act,  \
                     capacity, dev_error)
      if (f8) {
        if (wide) MOE_FRAG_GU(8, true); else MOE_FRAG_GU(4, true);
      } else {
        if (wide) MOE_FRAG_GU(8, false); else MOE_FRAG_GU(4, false);
      }
#undef MOE_FRAG_GU
    } else {
      const int64_t blocks = grid_for(I / (kBN / 2));
      if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
      hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0,
                         stream, x, static_cast<const uint16_t*>(w13), cu_seqlens, counts, G, H, 2 * I, I, nullptr, act,
                         capacity, dev_error);
    }
  }
  if ((flags & MOE_FFN_DOWN) && tall) {
    const int64_t blocks = grid_tall((2 * (H / 64) + 7) / 8);
    if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
#define MOE_TALL_DN(F8)                                                                         \
  hipLaunchKernelGGL((tall_stream_kernel<false, F8>), dim3((unsigned)stream_grid(blocks)),         \
                     dim3(8 * kWave), 0, stream, act, w2, w2s, cu_seqlens, counts, G, I, H, H,    \
                     row_scale, y, capacity, dev_error, (int)blocks)
    if (f8) MOE_TALL_DN(true); else MOE_TALL_DN(false);
#undef MOE_TALL_DN
  } else if (flags & MOE_FFN_DOWN) {
    if (packed) {
      const int nw = wide_down ? 8 : 4;
      const int64_t blocks = grid_for((H / 64 + nw - 1) / nw);
      if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
#define MOE_FRAG_DN(NW, F8)                                                                   \
  hipLaunchKernelGGL((frag_gemm_kernel<false, NW, F8>), dim3((unsigned)blocks), dim3(NW * kWave),       \
                     0, stream, act, w2, w2s, cu_seqlens, counts, G, I, H, H, row_scale, y,       \
                     capacity, dev_error)
      if (f8) {
        if (wide_down) MOE_FRAG_DN(8, true); else MOE_FRAG_DN(4, true);
      } else {
        if (wide_down) MOE_FRAG_DN(8, false); else MOE_FRAG_DN(4, false);
      }
#undef MOE_FRAG_DN
    } else {
      const int64_t blocks = grid_for(H / kBN);
      if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
      hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0,
                         stream, act, static_cast<const uint16_t*>(w2), cu_seqlens, counts, G, I,
                         H, H, row_scale, y, capacity,
                         dev_error);
    }
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
