// LDS tile layout and access helpers shared by the attention kernels
// (forward and backward).  HIP, gfx950 only.
#pragma once

#include "common.h"
#include "geometry.h"

namespace bda {

__device__ __forceinline__ bool in_span(const Span& s, int j) {
  return (unsigned)(j - s.lo) < (unsigned)(s.hi - s.lo);
}

// LDS tiles are row-major (one key per row, d fastest, no padding) with the
// 16-byte chunks of every row XOR-permuted by swz<D>(row).  gfx950's LDS has
// 64 four-byte banks (256 bytes per clock); the permutation puts the 16 rows
// of a wavefront's K operand read (16 lanes per clock at 16 bytes) and the
// 4 rows x 4 chunks of a transpose read (32 lanes per clock at 8 bytes) on
// 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  if (D == 64) {
    const int x = (r >> 1) & 7;   // two 128-byte rows share a bank line
    return ((x & 1) << 2) | ((x >> 1) & 3);
  }
  return r & 3;
}

template <int D>
__device__ __forceinline__ int chunk_off(int r, int c) {  // element offset of chunk c of row r
  constexpr int CPR = D / 8;
  return r * D + 8 * (c ^ (swz<D>(r) & (CPR - 1)));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from global memory straight into LDS: lane i of the
// wavefront writes lds_run + 16*i (lds_run must be the same for every lane).
// Written as inline assembly so that the compiler does not pair every later
// LDS read with a wait for all such loads: the kernel waits for them itself
// (s_waitcnt vmcnt) before the barrier that publishes a stage.  M0 is set in
// the same statement and used by nothing else in these kernels.
__device__ __forceinline__ void lds_dma16(const uint16_t* g, const uint16_t* lds_run) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_run);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(base) : "memory");
}
// The same with the non-temporal hint, for data read once (streamed caches).
__device__ __forceinline__ void lds_dma16_nt(const uint16_t* g, const uint16_t* lds_run) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_run);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(base) : "memory");
}

// The same with the run starting at LDS byte address m0 (uniform).
__device__ __forceinline__ void lds_dma16s(const uint16_t* g, unsigned m0) {
  m0 = __builtin_amdgcn_readfirstlane(m0);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory");
}
// 4 bytes per lane: lane i writes LDS byte address m0 + 4*i.
__device__ __forceinline__ void lds_dma4s(const float* g, unsigned m0) {
  m0 = __builtin_amdgcn_readfirstlane(m0);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0) : "memory");
}

// ds_read_b64_tr_b16: within each 16-lane group, lane j receives element
// (j & 3) of the 4-element row read by lane 4*e + (j >> 2), for e = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

}  // namespace bda
