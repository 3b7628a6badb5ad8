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

// M0 is a reserved register to the compiler, which warns when an asm
// statement names it as clobbered; the clobber is still recorded as a def of
// M0, which is what keeps any M0 value of the compiler's from being assumed
// to survive these statements.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// 16 bytes per lane from global memory straight into LDS: lane i of the
// wavefront writes lds_run + 16*i (lds_run must be the same for every lane).
// Written as inline assembly so that the compiler does not pair every later
// LDS read with a wait for all such loads: the kernel waits for them itself
// (s_waitcnt vmcnt) before the barrier that publishes a stage.  M0 is set in
// the same statement and named as clobbered, so the compiler keeps nothing
// of its own there across these loads.
__device__ __forceinline__ void lds_dma16(const uint16_t* g, const uint16_t* lds_run) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_run);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(base) : "memory", "m0");
}
// The same with the non-temporal hint, for data read once (streamed caches).
__device__ __forceinline__ void lds_dma16_nt(const uint16_t* g, const uint16_t* lds_run) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_run);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(base) : "memory", "m0");
}

// The same with the run starting at LDS byte address m0 (uniform).
__device__ __forceinline__ void lds_dma16s(const uint16_t* g, unsigned m0) {
  m0 = __builtin_amdgcn_readfirstlane(m0);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
// 4 bytes per lane: lane i writes LDS byte address m0 + 4*i.
__device__ __forceinline__ void lds_dma4s(const float* g, unsigned m0) {
  m0 = __builtin_amdgcn_readfirstlane(m0);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}

// 16 bytes per lane from base + off (base uniform, in SGPRs; off a 32-bit
// lane offset) into LDS: lane i writes LDS byte address m0 + 16 i (m0
// uniform).  The scalar base keeps the per-lane address arithmetic out of
// the vector unit.
__device__ __forceinline__ void lds_dma16_sa(const void* base, unsigned off, unsigned m0) {
  m0 = __builtin_amdgcn_readfirstlane(m0);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}
// The same with the non-temporal hint.
__device__ __forceinline__ void lds_dma16_sa_nt(const void* base, unsigned off, unsigned m0) {
  m0 = __builtin_amdgcn_readfirstlane(m0);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}

#pragma clang diagnostic pop

// N 16-byte loads at p + 32 k bytes (k = 0 .. N-1) into x[k], followed in the
// same statement by a wait for every vector-memory load of the wavefront
// issued up to that point (these and any issued before them), so the
// outputs are written when the statement ends.
template <int N>
__device__ __forceinline__ void load_x16_stride32_wait(const void* p, u32x4 (&x)[N]) {
  static_assert(N == 2 || N == 4 || N == 8, "2, 4 or 8 loads");
  if constexpr (N == 8) {
    asm volatile(
        "global_load_dwordx4 %0, %8, off\n\t"
        "global_load_dwordx4 %1, %8, off offset:32\n\t"
        "global_load_dwordx4 %2, %8, off offset:64\n\t"
        "global_load_dwordx4 %3, %8, off offset:96\n\t"
        "global_load_dwordx4 %4, %8, off offset:128\n\t"
        "global_load_dwordx4 %5, %8, off offset:160\n\t"
        "global_load_dwordx4 %6, %8, off offset:192\n\t"
        "global_load_dwordx4 %7, %8, off offset:224\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]),
          "=&v"(x[7])
        : "v"(p)
        : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "global_load_dwordx4 %0, %4, off\n\t"
        "global_load_dwordx4 %1, %4, off offset:32\n\t"
        "global_load_dwordx4 %2, %4, off offset:64\n\t"
        "global_load_dwordx4 %3, %4, off offset:96\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
        : "v"(p)
        : "memory");
  } else {
    asm volatile(
        "global_load_dwordx4 %0, %2, off\n\t"
        "global_load_dwordx4 %1, %2, off offset:32\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1])
        : "v"(p)
        : "memory");
  }
}

// ds_read_b64_tr_b16: within each 16-lane group, lane j receives element
// (j & 3) of the 4-element row read by lane 4*e + (j >> 2), for e = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// The same at LDS byte address a (an integer, so that an offset added to a
// base register folds into the instruction's immediate).
__device__ __forceinline__ s16x4 lds_read_tr_at(unsigned a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(size_t)a);
}
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ unsigned lds_addr(const void* p) { return (unsigned)(uintptr_t)p; }

}  // namespace bda
