// Shared pieces of the fragment-streaming grouped GEMMs (BF16 and FP8):
// vector types, the tile scheduler (device-side tile decode from the segment
// counts, XCD-aware workgroup order), the activation ring's barrier and
// direct-to-LDS DMA, and the SwiGLU activation.
#pragma once

#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte staging
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));  // 8 FP8 codes
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;     // rows per m-tile
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

// Decode tile number `pid` into (group, m-tile, n-tile).  Every lane of
// the calling wave returns the same answer; returns false past the last
// tile.  mt_base (if asked for) is the number of m-tiles of the groups
// before g.  Counts are clamped to [0, capacity] and summed in 64 bits, so
// that corrupt counts give wrong tiles (which the kernels' range checks
// reject) rather than wrapped sums.
__device__ __forceinline__ bool decode_tile(int pid, const int32_t* __restrict__ counts, int G,
                                            int n_tiles, int64_t capacity, int& g, int& mt,
                                            int& nt, int64_t* mt_base = nullptr) {
  const int lane = threadIdx.x & 63;
  long long carry = 0;
  for (int base = 0; base < G; base += kWave) {
    const int e = base + lane;
    const int c = e < G ? (int)min((int64_t)max(counts[e], 0), capacity) : 0;
    const long long tiles = (((long long)c + kBM - 1) / kBM) * n_tiles;
    long long incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    incl += carry;
    const long long excl = incl - tiles;
    const uint64_t hit = __ballot(e < G && pid >= excl && pid < incl);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      g = base + src;
      const long long ex = __shfl(excl, src, kWave);
      const int local = (int)(pid - ex);
      const int mtiles = (int)(((long long)__shfl(c, src, kWave) + kBM - 1) / kBM);
      nt = local / mtiles;
      mt = local - nt * mtiles;
      if (mt_base) *mt_base = ex / n_tiles;                   // m-tiles before g
      return true;
    }
    carry = __shfl(incl, 63, kWave);
  }
  return false;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (and for nothing else)
__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  return (n & 0xf) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xf << 8);
}

// Workgroup barrier for the activation ring, without the memory fence that
// __syncthreads() carries: with direct-to-LDS loads in flight that fence
// becomes a wait for every outstanding load, weight prefetches included, and
// drains the weight pipeline at every chunk.  The ordering it would give is
// established explicitly instead: each wave first waits (vmcnt) until its own
// DMA for the chunk has landed in LDS, so after the barrier the whole chunk
// is there; and the slot the next DMA overwrites was last read for MFMAs the
// waves had already issued, so those LDS reads were complete.  The empty asm
// statements keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The activation DMA (global_load_lds_dwordx4: 64 lanes x 16 bytes from
// global memory to LDS at M0), issued as inline assembly.  When the
// compiler's wait-count insertion sees a direct-to-LDS load, it cannot tell
// which ring slot it writes, so it makes the next LDS read (and any reuse of
// the load's address registers) wait until no vector-memory operation is
// outstanding, weight prefetches included, which drains the weight pipeline
// at every chunk.  It does not model this statement; the DMA of a chunk is
// waited for explicitly (vmcnt at the chunk barrier), and the compiler's own
// waits for the weight loads, which do not count these DMAs, are only
// stricter than needed, never looser.  The LDS reads stay ordinary loads, so
// their waits and register hazards remain the compiler's; they cannot move
// across lds_barrier(), whose empty asm statements clobber memory.
// The source address is a wave-uniform base (SGPRs) plus a 32-bit per-lane
// byte offset, which keeps the per-lane state of the DMA small.
// (dma16_at takes the LDS byte address itself.)
__device__ __forceinline__ void dma16_at(const void* sbase, uint32_t voff, uint32_t lds) {
  // one wait state between the SALU write of M0 and the DMA that reads it
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "m0");
}
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, const void* l) {
  dma16_at(sbase, voff, (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)l);
}

// The same for 4 bytes per lane (global_load_lds_dword: 64 lanes x 4 bytes
// to LDS at M0 + 4 * lane), for small per-row tables such as row scales.
__device__ __forceinline__ void dma4_at(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "m0");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, const void* l) {
  dma4_at(sbase, voff, (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)l);
}

// The LDS byte address of a __shared__ object (its generic address cast back
// once, outside any loop, so that no per-use null check is generated).
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace moe
