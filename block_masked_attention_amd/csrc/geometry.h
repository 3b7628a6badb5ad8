// Key-interval geometry of the three attention forms and the tile classifier.
//
// Every query row of every form sees the union of at most two contiguous key
// intervals of the key tensor:
//   HYBRID, x_t row at position p of block j = p / b:
//       A = x_t keys of its own block     [j*b, min(L, j*b + b))
//       C = x_0 keys of the blocks before [L, L + j*b)
//     (block-diagonal and offset block-causal parts of the hybrid mask,
//      "Block Diffusion Attention" section of the Nemotron-Labs-Diffusion-8B
//      3x analysis page; the noisy block's conditioning on earlier clean
//      blocks is the BDLM objective of the LLaDA2.0-Uni summary)
//   HYBRID, x_0 row at position p of block j:
//       A = x_0 keys of blocks up to j    [L, L + min(L, (j+1)*b))   (block-causal)
//   DECODE: A = [0, L)        (bidirectional active block over its cache)
//   CAUSAL row i of n:  A = [0, L - n + i + 1)   (bottom-right aligned)
// So a (query-rows x key-range) tile is FULL, EMPTY or PARTIAL from these
// intervals alone; no dense mask is ever built.
#pragma once

#ifdef __HIPCC__
#include <hip/hip_runtime.h>
#define BDA_HD __host__ __device__ __forceinline__
#else
#define BDA_HD inline
#endif

namespace bda {

enum Mode { kHybrid = 0, kDecode = 1, kCausal = 2 };
enum TileClass { kFull = 0, kEmpty = 1, kPartial = 2 };

struct Span {
  int lo, hi;  // [lo, hi); empty when hi <= lo
};

BDA_HD int imin(int a, int b) { return a < b ? a : b; }
BDA_HD int imax(int a, int b) { return a > b ? a : b; }

// Allowed key intervals of query row `row` (row numbering of the query
// tensor: HYBRID 0..2L-1, DECODE/CAUSAL 0..n-1).
BDA_HD void row_spans(int mode, int L, int n, int b, int row, Span& A, Span& C) {
  C.lo = 0;
  C.hi = 0;
  if (mode == kHybrid) {
    const bool noisy = row < L;
    const int p = noisy ? row : row - L;
    const int j0 = (p / b) * b;                 // first position of the block
    const int j1 = imin(L, j0 + b);             // one past its last position
    if (noisy) {
      A.lo = j0;
      A.hi = j1;
      C.lo = L;
      C.hi = L + j0;
    } else {
      A.lo = L;
      A.hi = L + j1;
    }
  } else if (mode == kDecode) {
    A.lo = 0;
    A.hi = L;
  } else {
    A.lo = 0;
    A.hi = L - n + row + 1;
  }
}

// Number of keys of [k0, k1) inside span s.
BDA_HD int inside(const Span& s, int k0, int k1) { return imax(0, imin(s.hi, k1) - imax(s.lo, k0)); }

// Class of one row against keys [k0, k1).  The two spans are disjoint but may
// touch (the last x_t block ends at L where the x_0 span starts), so count.
BDA_HD int row_class(const Span& A, const Span& C, int k0, int k1) {
  const int c = inside(A, k0, k1) + inside(C, k0, k1);
  if (c == k1 - k0) return kFull;
  return c ? kPartial : kEmpty;
}

// Tile classifier over rows [q0, q1) x keys [k0, k1) (host side; the kernels
// evaluate row_class per lane and reduce across the wavefront instead).
inline int classify_tile(int mode, int L, int n, int b, int q0, int q1, int k0, int k1) {
  if (q0 >= q1 || k0 >= k1) return kEmpty;
  bool any_full = false, any_empty = false, any_partial = false;
  for (int r = q0; r < q1; ++r) {
    Span A, C;
    row_spans(mode, L, n, b, r, A, C);
    const int c = row_class(A, C, k0, k1);
    any_full |= c == kFull;
    any_empty |= c == kEmpty;
    any_partial |= c == kPartial;
  }
  if (any_partial || (any_full && any_empty)) return kPartial;
  return any_full ? kFull : kEmpty;
}

}  // namespace bda
