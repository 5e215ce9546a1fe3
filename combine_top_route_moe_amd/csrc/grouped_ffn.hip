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
// Tiling: a workgroup of 4 wavefronts owns a BM x BN output tile (BM = BN =
// 128); wave (wm, wn) owns a 64 x 64 quarter as 4 x 4 MFMA 16x16 tiles.
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

#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte staging

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kLdsStride = kBK + 8;  // bf16 elements per LDS row
constexpr int kThreads = 256;
constexpr int kTileVecs = kBN * kBK / 8;  // 16-byte vectors in one packed weight tile
constexpr int kNumXcd = 8;

// Workgroup ids are dealt round-robin over the 8 XCDs.  Remap them so that
// runs of kXcdChunk consecutive tile numbers land on one XCD (they share
// weight and activation panels through its L2) while successive runs go to
// successive XCDs (the work, including the empty tail, stays balanced).
// The grid is a multiple of 8 * kXcdChunk, which makes this a bijection.
constexpr int kXcdChunk = 16;
__device__ __forceinline__ int xcd_remap(int bid) {
  const int xcd = bid % kNumXcd, local = bid / kNumXcd;
  const int chunk = local / kXcdChunk, off = local % kXcdChunk;
  return (chunk * kNumXcd + xcd) * kXcdChunk + off;
}

// Decode tile number `pid` into (group, m-tile, n-tile).  Every lane of the
// calling wave returns the same answer; returns false past the last tile.
__device__ __forceinline__ bool decode_tile(int pid, const int32_t* __restrict__ counts, int G,
                                            int n_tiles, int& g, int& mt, int& nt) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int base = 0; base < G; base += kWave) {
    const int e = base + lane;
    const int c = e < G ? max(counts[e], 0) : 0;
    const int tiles = ((c + kBM - 1) / kBM) * n_tiles;
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    incl += carry;
    const int excl = incl - tiles;
    const uint64_t hit = __ballot(e < G && pid >= excl && pid < incl);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      g = base + src;
      const int local = pid - __shfl(excl, src, kWave);
      const int mtiles = (__shfl(c, src, kWave) + kBM - 1) / kBM;
      nt = local / mtiles;
      mt = local - nt * mtiles;
      return true;
    }
    carry = __shfl(incl, 63, kWave);
  }
  return false;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <bool GATE_UP, bool PACKED>
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
  if (!decode_tile(pid, counts, G, n_tiles, g, mt, nt)) return;

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
    if (PACKED) {
      // tile (nt, kt) is one contiguous [kBN][kBK] block; chunk v of it is
      // exactly what this thread stages
      b_src[j] = reinterpret_cast<const u32x4_t*>(Wg) +
                 (int64_t)nt * (Kdim / kBK) * kTileVecs + v;
    } else {
      int wrow;
      if (GATE_UP)
        wrow = (r < kBN / 2) ? nt * (kBN / 2) + r : Nout + nt * (kBN / 2) + (r - kBN / 2);
      else
        wrow = nt * kBN + r;
      b_src[j] = reinterpret_cast<const u32x4_t*>(Wg + (int64_t)wrow * Kdim) + c;
    }
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
  const int b_step = PACKED ? kTileVecs : kBK / 8;  // 16-byte vectors per K-slab
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
      const int badv = (kt + 1) * b_step;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ra[j] = a_src[j][adv];
        rb[j] = b_src[j][badv];
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

// Packed weight layout: for each group, n-tile and K-slab, the kBN x kBK
// block the GEMM stages in one step, stored contiguously (row-major inside
// the block).  For w13 an n-tile's kBN rows are its kBN/2 gate rows followed
// by the matching kBN/2 up rows.  One thread moves one 16-byte vector.
__global__ void __launch_bounds__(256) pack_weights_kernel(const uint16_t* __restrict__ W,
                                                           uint16_t* __restrict__ P, int G,
                                                           int N, int Kdim, int gate_up) {
  const int64_t nvec = (int64_t)G * N * Kdim / 8;
  const int kt_n = Kdim / kBK;
  const int nt_n = N / kBN;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int in_tile = (int)(v % kTileVecs);
    int64_t t = v / kTileVecs;
    const int kt = (int)(t % kt_n);
    t /= kt_n;
    const int nt = (int)(t % nt_n);
    const int64_t g = t / nt_n;
    const int r = in_tile >> 3, c = in_tile & 7;
    int row;
    if (gate_up) {
      const int half = N / 2;  // I
      row = (r < kBN / 2) ? nt * (kBN / 2) + r : half + nt * (kBN / 2) + (r - kBN / 2);
    } else {
      row = nt * kBN + r;
    }
    const uint4 val =
        reinterpret_cast<const uint4*>(W + (g * N + row) * (int64_t)Kdim + kt * kBK)[c];
    reinterpret_cast<uint4*>(P)[v] = val;
  }
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

size_t grouped_ffn_workspace_bytes(int64_t capacity, int I) {
  return (((size_t)capacity * I * sizeof(uint16_t)) + 255) & ~(size_t)255;
}

template <bool GATE_UP>
static void launch_gemm(bool packed, dim3 grid, hipStream_t stream, const uint16_t* A,
                        const uint16_t* W, const int32_t* cu, const int32_t* cnt, int G, int Kdim,
                        int Nw, int Nout, const float* row_scale, uint16_t* Out, int64_t capacity,
                        int32_t* dev_error) {
  if (packed)
    hipLaunchKernelGGL((grouped_gemm_kernel<GATE_UP, true>), grid, dim3(kThreads), 0, stream, A,
                       W, cu, cnt, G, Kdim, Nw, Nout, row_scale, Out, capacity, dev_error);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<GATE_UP, false>), grid, dim3(kThreads), 0, stream, A,
                       W, cu, cnt, G, Kdim, Nw, Nout, row_scale, Out, capacity, dev_error);
}

int launch_grouped_ffn(const uint16_t* x, const int32_t* cu_seqlens, const int32_t* counts, int G,
                       int H, int I, const uint16_t* w13, const uint16_t* w2,
                       const float* row_scale, uint16_t* y, int64_t capacity, int flags,
                       void* workspace, int32_t* dev_error, hipStream_t stream) {
  uint16_t* act = static_cast<uint16_t*>(workspace);
  const bool packed = (flags & MOE_FFN_PACKED_WEIGHTS) != 0;
  const int64_t m_tiles = (capacity + kBM - 1) / kBM + G;
  const int64_t grid_unit = (int64_t)kNumXcd * kXcdChunk;
  if (capacity == 0) return MOE_OK;
  if (flags & MOE_FFN_GATE_UP) {
    const int64_t blocks = (m_tiles * (I / (kBN / 2)) + grid_unit - 1) / grid_unit * grid_unit;
    if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
    launch_gemm<true>(packed, dim3((unsigned)blocks), stream, x, w13, cu_seqlens, counts, G, H,
                      2 * I, I, nullptr, act, capacity, dev_error);
  }
  if (flags & MOE_FFN_DOWN) {
    const int64_t blocks = (m_tiles * (H / kBN) + grid_unit - 1) / grid_unit * grid_unit;
    if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
    launch_gemm<false>(packed, dim3((unsigned)blocks), stream, act, w2, cu_seqlens, counts, G, I,
                       H, H, row_scale, y, capacity, dev_error);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
