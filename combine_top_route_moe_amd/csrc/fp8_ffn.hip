// The grouped SwiGLU FFN with FP8 activations and FP8 weights on the gfx950
// FP8 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x E4M3, float32
// accumulate), and the quantizer that produces its FP8 rows.
//
// Source: "[Kernel] DeepEP dispatch-combine kernel integration", review
// thread on the low-latency dispatch (the tokens travel as FP8 codes with
// their block scales and the receiving side consumes both) and review
// thread on the DeepEP + DeepGEMM test (FP8 expert weights with one scale per
// block_n x block_k tile, multiplied by DeepGEMM's FP8 grouped GEMMs);
// "[Distributed][MoonEP] BF16 integration of MoonEP balanced EP backend",
// commit message adding the modular experts (gate, up, down over the
// cu_seqlens segments, route weight before the down projection).
//
// What it computes, per segment (scales s = amax/448 per 1 x 128 block of a
// row, per 128 x 128 tile of a weight matrix):
//   h[r, n] = sum_kb sx[r, kb] * sw13[n/128, kb] * (qx[r, kb-block] . qw13[n, kb-block])
//   a       = bf16(silu(h_gate) * h_up), then quantized per 1 x 128 block: (qa, sa)
//   y[r, n] = bf16( w[r] * sum_kb sa[r, kb] * sw2[n/128, kb] * (qa[r, kb-block] . qw2[n, kb-block]) )
//
// The kernel follows the BF16 fragment-streaming GEMM (grouped_ffn.hip):
// a workgroup of NW waves covers up to 128 rows of one segment and NW
// 64-column weight tiles, each wave streaming its tile's B fragments from
// HBM straight into registers while the workgroup's activation rows come
// through an LDS ring by direct-to-LDS DMA.  The K step is one 128-wide
// K-block: one MFMA per (16-row m-subtile, 16-column fragment) gives that
// block's exact code dot products, which are then scaled by the row's block
// scale times the tile's scale and added to the float32 accumulators.
//
// Operand layout (the matrix core pairs byte p of an A lane with byte p of
// the B lane of the same lane group l/16): for a K-block, lane l holds row
// (A) or weight row (B) l%16 and the 32 codes at columns 16 (l/16) .. +16
// (bytes 0-15) and 64 + 16 (l/16) .. +16 (bytes 16-31).  Each half is one
// 1 KB block of 64 lanes x 16 bytes, so every global and LDS access is a
// contiguous 16-byte vector per lane.
#include <algorithm>

#include "gemm_common.h"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kQStages = 3;            // activation LDS ring (one K-block per stage)
constexpr int kQPrefetch = 2;          // weight K-blocks in flight per wave
constexpr int kQMsub = 8;              // 16-row m-subtiles per workgroup
constexpr int kQFrags = 4;             // 16-column B fragments per wave
constexpr int kQBlocks = kQMsub * 2;   // 1 KB activation blocks per stage

// E4M3 codes of 8 values (already divided by the scale and clamped),
// packed low byte first.
__device__ __forceinline__ uint2 e4m3x8(const float* r) {
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * h], r[4 * h + 1], 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * h + 2], r[4 * h + 3], p, true);
    w[h] = (uint32_t)p;
  }
  return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// One DPP lane movement within each row of 16 lanes (every lane active).
template <int kCtrl>
__device__ __forceinline__ float row16_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// ---------------------------------------------------------------------------
// Rows to FP8: one 16-byte vector (8 channels) per thread, 16 lanes per
// 128-channel block.  s = amax / 448 (IEEE), code = e4m3(clamp(x / s))
// (IEEE quotient, round to nearest even); rows with row_src[r] < 0 and
// all-zero blocks get codes 0 and scale 0.  Scales are stored K-block-major:
// scales[kb * sstride + r].
__global__ void __launch_bounds__(256) quant_rows_fp8_kernel(
    const uint16_t* __restrict__ in, int64_t n_rows, int H, const int32_t* __restrict__ row_src,
    uint8_t* __restrict__ codes, float* __restrict__ scales, int64_t sstride) {
  const int vec_per_row = H / 8;
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // every block of 16 lanes shares one row and one 128-channel block
  const bool in_range = v < n_rows * vec_per_row;
  const int64_t r = in_range ? v / vec_per_row : 0;
  const int c = (int)(v - r * vec_per_row);
  const bool active = in_range && (row_src == nullptr || row_src[r] >= 0);
  float f[8];
  unpack8(in_range ? reinterpret_cast<const uint4*>(in)[v] : make_uint4(0, 0, 0, 0), f);
  float m = 0.0f;
  if (active) {
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
  }
  // the block's 16 lanes are one DPP row: its max in registers by two quad
  // permutations (lane ^ 1, lane ^ 2), the half-row mirror and the row
  // mirror (max is exact, the order does not matter)
  m = fmaxf(m, row16_dpp<0xB1>(m));   // quad_perm [1, 0, 3, 2]
  m = fmaxf(m, row16_dpp<0x4E>(m));   // quad_perm [2, 3, 0, 1]
  m = fmaxf(m, row16_dpp<0x141>(m));  // row_half_mirror
  m = fmaxf(m, row16_dpp<0x140>(m));  // row_mirror
  const float s = m / 448.0f;
  if (!in_range) return;
  uint2 q = make_uint2(0, 0);
  if (s > 0.0f) {
    float rq[8];
    if (rcp_scale_ok(s)) {
      // x / s from the reciprocal by one correction step, clamped, with the
      // sign of x (the quotient steps of qdq8_rcp): the same E4M3 value as
      // the IEEE quotient clamped to +-448, zeros' signs included
      const float inv_s = 1.0f / s;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = __builtin_amdgcn_fmed3f(f[j] * inv_s, -512.0f, 512.0f);
        const float res = __builtin_fmaf(a, s, -f[j]);
        rq[j] = __builtin_copysignf(
            __builtin_amdgcn_fmed3f(__builtin_fmaf(-res, inv_s, a), -448.0f, 448.0f), f[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) rq[j] = clamp448(f[j] / s);
    }
    q = e4m3x8(rq);
  }
  reinterpret_cast<uint2*>(codes)[v] = q;
  if ((c & 15) == 0) scales[(int64_t)(c / 16) * sstride + r] = s;
}

int launch_quant_rows_fp8(const uint16_t* in, int64_t n_rows, int H, const int32_t* row_src,
                          uint8_t* codes, float* scales, int64_t sstride, hipStream_t stream) {
  const int64_t nvec = n_rows * (H / 8);
  if (nvec == 0) return MOE_OK;
  hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0,
                     stream, in, n_rows, H, row_src, codes, scales, sstride);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---------------------------------------------------------------------------
// The FP8 grouped GEMM.  A workgroup of 8 waves covers up to 128 rows of one
// segment and 4 column tiles of 64 weight rows: wave w owns column tile
// 4 cb + w % 4 and the row half w / 4 (m-subtiles 4 (w/4) .. +4), so a
// wave's accumulators are 64 x 64 (the two waves of a column tile stream the
// same weights; the second read is served by the caches).  For gate/up the
// 4 column tiles are 128 columns of a — one quantization block — so the
// block's row maxima stay inside the workgroup.
//
// GATE_UP: A = the permuted rows' codes [cap, Kdim] row-major with scales
// [Kdim/128][sstride], row r's scales in row smap[r] / sdiv of the scale
// table (smap NULL: row r itself); writes a's codes in the down GEMM's activation order
// (per m-tile, m-subtile, K-block and half: 64 lanes x 16 bytes) and a's
// scales [m-tile][Nout/128][128].  DOWN: A = those; Out = y [cap, Nout]
// bf16 with the router weight.
constexpr int kQNW = 8;                 // waves per workgroup
constexpr int kQTiles = 4;              // column tiles per workgroup
constexpr int kQSub = kQMsub / 2;       // m-subtiles per wave

// SKIP_IDLE: compiled with the early exit for idle waves below (used when
// segments average under one m-tile, where the second row half is often
// empty); the other instantiation keeps the main loop as compiled without
// that path, which measured 1-3 % faster on long segments.
template <bool GATE_UP, bool SKIP_IDLE>
__global__ void __launch_bounds__(kQNW * kWave, 2) w8a8_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ Ascale, int64_t sstride,
    const int32_t* __restrict__ smap, int sdiv,
    const uint8_t* __restrict__ Wq, const float* __restrict__ Wsc,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ counts, int G, int Kdim,
    int Nw, int Nout, const float* __restrict__ row_scale, uint8_t* __restrict__ OutQ,
    float* __restrict__ OutS, uint16_t* __restrict__ Out, int64_t capacity,
    int32_t* __restrict__ dev_error) {
  __shared__ __attribute__((aligned(16))) u32x4_t Aq[kQStages][kQBlocks][kWave];
  __shared__ __attribute__((aligned(16))) float Sa[kQStages][kBM];
  __shared__ float rs[kBM];
  __shared__ float red[GATE_UP ? kQTiles : 1][kBM];

  const int n_ct = Nw / 64;
  const int n_cb = (n_ct + kQTiles - 1) / kQTiles;
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
  const int m0 = mt * kBM;
  const int valid = min(kBM, nrows - m0);
  if (valid <= 0) return;
  const int64_t row_base = (int64_t)seg0 + m0;
  const int nlive = (valid + 15) >> 4;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = w % kQTiles, i0 = (w / kQTiles) * kQSub;
  const int my_live = min(max(nlive - i0, 0), kQSub);   // live m-subtiles of this wave
  const bool ct_ok = cb * kQTiles + cw < n_ct;
  const int ct = ct_ok ? cb * kQTiles + cw : n_ct - 1;
  const int nkb = Kdim / 128;
  const int64_t mt_glob = (int64_t)mt_base + mt;

  // weights: K-block kb, fragment f, half h at wq[kb * kstride + (2 f + h) * 64]
  const int kstride = n_ct * kQFrags * 2 * kWave;
  const u32x4_t* wq = reinterpret_cast<const u32x4_t*>(Wq) +
                      ((int64_t)g * nkb * n_ct + ct) * (kQFrags * 2 * kWave) + lane;
  // tile scales [G][Nw/128][Kdim/128] of this tile's gate and up rows
  const int nrb = Nw / 128;
  const int rb_g = GATE_UP ? (32 * ct) / 128 : (64 * ct) / 128;
  const int rb_u = GATE_UP ? (Nw / 2 + 32 * ct) / 128 : rb_g;
  const float* sc_g = Wsc + ((int64_t)g * nrb + rb_g) * nkb;
  const float* sc_u = Wsc + ((int64_t)g * nrb + rb_u) * nkb;

  // activation DMA: wave w fills the two halves of m-subtile w (if live)
  const uint8_t* a_base =
      GATE_UP ? A + row_base * Kdim : A + mt_glob * kQMsub * (int64_t)nkb * 2 * (kWave * 16);
  int64_t a_uoff[2];
  uint32_t a_voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (GATE_UP) {
      const int r = min(w * 16 + (lane & 15), valid - 1);  // rows past the end re-read the last
      a_uoff[h] = 0;
      a_voff[h] = (uint32_t)(r * Kdim + 64 * h + 16 * (lane >> 4));
    } else {
      a_uoff[h] = ((int64_t)w * nkb * 2 + h) * (kWave * 16);
      a_voff[h] = (uint32_t)lane * 16u;
    }
  }
  const int a_kstride = GATE_UP ? 128 : 2 * kWave * 16;
  // the K-block's 128 row scales: two 4-byte DMAs (rows lane, 64 + lane)
  // by wave 0, gathered through smap for gate/up
  const float* s_base = GATE_UP ? Ascale : Ascale + mt_glob * nkb * kBM;
  const int64_t s_kstride = GATE_UP ? sstride : kBM;
  // gate/up: row r's scales sit in column smap[row] / sdiv of Ascale (or the
  // row's own column); a gathered column outside [0, sstride) — a corrupt
  // map entry — is replaced by column 0 and raises the error, so the DMA
  // never leaves the array
  auto scale_row = [&](int r) -> uint32_t {
    if (!GATE_UP) return (uint32_t)r;
    const int64_t pr = row_base + min(r, valid - 1);
    if (!smap) return (uint32_t)pr;
    const int src = smap[pr];
    if (src < 0 || src / sdiv >= sstride) {
      raise_error(dev_error, MOE_DEVERR_ROW_RANGE);
      return 0u;
    }
    return (uint32_t)(src / sdiv);
  };
  const uint32_t s_voff0 = scale_row(lane) * 4u;
  const uint32_t s_voff1 = scale_row(64 + lane) * 4u;

  const float* tile_scale = nullptr;
  if (!GATE_UP && row_scale) {
    for (int r = threadIdx.x; r < valid; r += kQNW * kWave) rs[r] = row_scale[row_base + r];
    __syncthreads();
    tile_scale = rs;
  }

  // experts read once start at a hashed K-block (spreads the HBM channels)
  const bool once = nrows <= kBM;
  const int krot = once ? (int)((((uint32_t)g * 977u) * 2654435761u) >> 8) % nkb : 0;
  auto wrap = [](int x, int n) { return x >= n ? x - n : x; };

  auto issue_chunk = [&](int kb, int stage) {
    const int src = wrap(kb + krot, nkb);
    asm volatile("" ::: "memory");
    if (w < nlive) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        dma16(a_base + a_uoff[h] + (int64_t)src * a_kstride, a_voff[h], &Aq[stage][2 * w + h][0]);
    }
    if (w == 0) {
      dma4(s_base + (int64_t)src * s_kstride, s_voff0, &Sa[stage][0]);
      dma4(s_base + (int64_t)src * s_kstride, s_voff1, &Sa[stage][64]);
    }
    asm volatile("" ::: "memory");
  };

  i32x8_t bq[kQPrefetch][kQFrags];
  float bsg[kQPrefetch], bsu[kQPrefetch];
  auto fill = [&](int slot, int kb) {
    const int src = wrap(kb + krot, nkb);
#pragma unroll
    for (int f = 0; f < kQFrags; ++f) {
      const u32x4_t* p = wq + (int64_t)src * kstride + 2 * f * kWave;
      const u32x4_t lo = p[0], hi = p[kWave];
      bq[slot][f] = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    bsg[slot] = sc_g[src];
    bsu[slot] = sc_u[src];
  };

  f32x4_t acc[kQSub][kQFrags];
#pragma unroll
  for (int i = 0; i < kQSub; ++i)
#pragma unroll
    for (int f = 0; f < kQFrags; ++f) acc[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < kQStages - 1; ++c) issue_chunk(min(c, nkb - 1), c);
  // A wave of the second row half whose m-tile has at most 64 rows has no
  // live subtile: it streams no weights, only keeps the workgroup's barriers
  // (one per K-block, plus the gate/up epilogue's) and, for gate/up, zeroes
  // its half's row scales; it issues no DMA (wave 0 is never idle).
  // Measured on segments averaging 64 rows: gate/up -1 to -10 %, down -4 to
  // -8 % (the idle waves no longer duplicate their column tile's weights).
  if (SKIP_IDLE && my_live == 0) {
    for (int kb = 0; kb < nkb; ++kb) lds_barrier();
    if (GATE_UP) {
      __syncthreads();
      float* srow = OutS + (mt_glob * (Nout / 128) + cb) * kBM;
      if (cw == 0)
        for (int r = i0 * 16 + lane; r < (i0 + kQSub) * 16; r += kWave) srow[r] = 0.0f;
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < kQPrefetch; ++s) fill(s, min(s, nkb - 1));
  asm volatile("" ::: "memory");

  // The DMA of K-block kb was issued (at the start of block kb - 2, or in
  // the prologue) before at least kAfterDma weight loads of this wave: two
  // blocks' refills, or the prologue's fills.  Loads complete in order.
  constexpr int kAfterDma = (kQStages - 1) * kQFrags * 2;
  static_assert(kAfterDma <= kQPrefetch * kQFrags * 2, "prologue count");
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  int stage = 0;
  for (int kb0 = 0; kb0 < nkb; kb0 += kQPrefetch) {
#pragma unroll
    for (int s = 0; s < kQPrefetch; ++s) {
      const int kb = kb0 + s;
      // past the last K-block (odd counts) only the refill below runs: every
      // path issues the same loads, so the compiler's waits for the weight
      // slots stay as loose as the prefetch allows (a path without them
      // would make it wait for every load at each step)
      if (kb < nkb) {
      if (kb > 0) stage = (stage + 1 == kQStages) ? 0 : stage + 1;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAfterDma));
      lds_barrier();
      issue_chunk(min(kb + kQStages - 1, nkb - 1), (stage + kQStages - 1) % kQStages);
      // one m-subtile: its K-block's code products, scaled into acc
      auto subtile = [&](int ii, const i32x8_t& af, const f32x4_t& sa) {
        f32x4_t t[kQFrags];
#pragma unroll
        for (int f = 0; f < kQFrags; ++f)
          t[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bq[s][f], zero, 0, 0, 0, 127, 0,
                                                                  127);
        const f32x4_t cg = sa * bsg[s];
        const f32x4_t cu = GATE_UP ? sa * bsu[s] : cg;
#pragma unroll
        for (int f = 0; f < kQFrags; ++f) {
          const f32x4_t c = f >= 2 ? cu : cg;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[ii][f][q] = __builtin_fmaf(t[f][q], c[q], acc[ii][f][q]);
        }
      };
      auto a_frag = [&](int i) {
        return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(Aq[stage][2 * i][lane],
                                                                   Aq[stage][2 * i + 1][lane], 0,
                                                                   1, 2, 3, 4, 5, 6, 7));
      };
      auto s_frag = [&](int i) {
        return *reinterpret_cast<const f32x4_t*>(&Sa[stage][i * 16 + 4 * (lane >> 4)]);
      };
      if (my_live == kQSub) {
        // all subtiles live (the common case): straight-line code, every
        // LDS read first, so the scheduler can overlap one subtile's
        // scaling with the next subtile's MFMAs
        i32x8_t af[kQSub];
        f32x4_t sa[kQSub];
#pragma unroll
        for (int ii = 0; ii < kQSub; ++ii) {
          af[ii] = a_frag(i0 + ii);
          sa[ii] = s_frag(i0 + ii);
        }
#pragma unroll
        for (int ii = 0; ii < kQSub; ++ii) subtile(ii, af[ii], sa[ii]);
      } else {
#pragma unroll
        for (int ii = 0; ii < kQSub; ++ii) {
          if (ii >= my_live) break;
          subtile(ii, a_frag(i0 + ii), s_frag(i0 + ii));
        }
      }
      }
      // refill this slot kQPrefetch blocks ahead (past the end: the last again)
      asm volatile("" ::: "memory");
      fill(s, min(kb + kQPrefetch, nkb - 1));
      asm volatile("" ::: "memory");
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA may outlive the workgroup

  // epilogue: lane holds D[4*(lane/16) + q][lane%16] of every 16x16 tile
  if (GATE_UP) {
    // a = bf16(silu(gate) * up); the workgroup's 4 column tiles are one
    // 1 x 128 block of a, whose row maxima meet in LDS
    float av[kQSub][2][4];
#pragma unroll
    for (int ii = 0; ii < kQSub; ++ii) {
      if (ii >= my_live) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float m = 0.0f;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const float v = silu_f(acc[ii][f][q]) * acc[ii][f + 2][q];
          av[ii][f][q] = __uint_as_float(f32_to_bf16(v) << 16);
          m = fmaxf(m, fabsf(av[ii][f][q]));
        }
        // the row's 16 lanes are one DPP row (my_live is the same for the
        // whole wave, so all of them are here): its max in registers
        m = fmaxf(m, row16_dpp<0xB1>(m));
        m = fmaxf(m, row16_dpp<0x4E>(m));
        m = fmaxf(m, row16_dpp<0x141>(m));
        m = fmaxf(m, row16_dpp<0x140>(m));
        if ((lane & 15) == 0) red[cw][(i0 + ii) * 16 + 4 * (lane >> 4) + q] = m;
      }
    }
    __syncthreads();
    const int nkb_out = Nout / 128;     // cb is this block's index
    float* srow = OutS + (mt_glob * nkb_out + cb) * kBM;
#pragma unroll
    for (int ii = 0; ii < kQSub; ++ii) {
      if (ii >= my_live) break;
      const int i = i0 + ii;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = i * 16 + 4 * (lane >> 4) + q;
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < kQTiles; ++j) amax = fmaxf(amax, red[j][r]);
        const float sc = amax / 448.0f;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int kk = cw * 32 + f * 16 + (lane & 15);   // column within the block
          const float qv = sc > 0.0f ? clamp448(av[ii][f][q] / sc) : 0.0f;
          const int p = __builtin_amdgcn_cvt_pk_fp8_f32(qv, 0.0f, 0, false);
          const int64_t unit = (((mt_glob * kQMsub + i) * nkb_out + cb) * 2 + kk / 64) * kWave +
                               (r & 15) + 16 * ((kk % 64) / 16);
          OutQ[unit * 16 + (kk % 16)] = (uint8_t)(p & 0xff);
        }
        if (cw == 0 && (lane & 15) == 0) srow[r] = r < valid ? sc : 0.0f;
      }
    }
    // scales of the rows of this half that no live subtile covers
    if (cw == 0)
      for (int r = (i0 + my_live) * 16 + lane; r < (i0 + kQSub) * 16; r += kWave) srow[r] = 0.0f;
  } else {
    if (!ct_ok) return;
#pragma unroll
    for (int ii = 0; ii < kQSub; ++ii) {
      if (ii >= my_live) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = (i0 + ii) * 16 + 4 * (lane >> 4) + q;
        if (r >= valid) continue;
        const float sc = tile_scale ? tile_scale[r] : 1.0f;
        const int64_t orow = row_base + r;
#pragma unroll
        for (int f = 0; f < kQFrags; ++f) {
          const int col = ct * 64 + f * 16 + (lane & 15);
          Out[orow * Nout + col] = (uint16_t)f32_to_bf16(sc * acc[ii][f][q]);
        }
      }
    }
  }
}

// Workspace: a's codes (one byte per element, per m-tile of 128 rows, at
// most ceil(capacity/128) + G m-tiles) and a's scales.
size_t w8a8_workspace_bytes(int64_t capacity, int G, int I) {
  const int64_t m_tiles = (capacity + kBM - 1) / kBM + G;
  const size_t codes = (((size_t)m_tiles * kBM * I) + 255) & ~(size_t)255;
  const size_t scales = (size_t)m_tiles * (I / 128) * kBM * sizeof(float);
  return codes + ((scales + 255) & ~(size_t)255);
}

int launch_grouped_ffn_w8a8(const uint8_t* xq, const float* xs, int64_t sstride,
                            const int32_t* smap, int sdiv, const int32_t* cu_seqlens, const int32_t* counts, int G, int H, int I,
                            const uint8_t* w13q, const float* w13s, const uint8_t* w2q,
                            const float* w2s, const float* row_scale, uint16_t* y,
                            int64_t capacity, int flags, void* workspace, int32_t* dev_error,
                            hipStream_t stream) {
  if (capacity == 0) return MOE_OK;
  const int64_t m_tiles = (capacity + kBM - 1) / kBM + G;
  uint8_t* aq = static_cast<uint8_t*>(workspace);
  float* as = reinterpret_cast<float*>(aq + ((((size_t)m_tiles * kBM * I) + 255) & ~(size_t)255));
  const int64_t grid_unit = (int64_t)kNumXcd * kXcdChunk;
  auto grid_for = [&](int64_t n_tiles) {
    return (m_tiles * n_tiles + grid_unit - 1) / grid_unit * grid_unit;
  };
  // segments averaging under one m-tile: the instantiation whose idle
  // second-half waves leave early
  const bool short_segs = capacity / G < kBM;
  if (flags & MOE_FFN_GATE_UP) {
    const int64_t blocks = grid_for((2 * I / 64 + kQTiles - 1) / kQTiles);
    if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
#define MOE_W8A8_GU(SKIP)                                                                        \
  hipLaunchKernelGGL((w8a8_gemm_kernel<true, SKIP>), dim3((unsigned)blocks), dim3(kQNW * kWave), 0, \
                     stream, xq, xs, sstride, smap, sdiv, w13q, w13s, cu_seqlens, counts, G, H,    \
                     2 * I, I, nullptr, aq, as, nullptr, capacity, dev_error)
    if (short_segs) MOE_W8A8_GU(true); else MOE_W8A8_GU(false);
#undef MOE_W8A8_GU
  }
  if (flags & MOE_FFN_DOWN) {
    const int64_t blocks = grid_for((H / 64 + kQTiles - 1) / kQTiles);
    if (blocks > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
#define MOE_W8A8_DN(SKIP)                                                                         \
  hipLaunchKernelGGL((w8a8_gemm_kernel<false, SKIP>), dim3((unsigned)blocks), dim3(kQNW * kWave), 0, \
                     stream, aq, as, (int64_t)0, (const int32_t*)nullptr, 1, w2q, w2s, cu_seqlens,  \
                     counts, G, I, H, H, row_scale, nullptr, nullptr, y, capacity, dev_error)
    if (short_segs) MOE_W8A8_DN(true); else MOE_W8A8_DN(false);
#undef MOE_W8A8_DN
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
