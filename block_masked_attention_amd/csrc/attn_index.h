// Work decomposition and index arithmetic of the attention forward kernels:
// the work items and the key ranges and tiles each one walks, the order in
// which the persistent walk takes items, the query slots of a wavefront, the
// element offsets of every global access and the LDS tile layout.  The
// kernels call these functions, and so does the host-side replay that checks
// every index they form against the tensors' bounds, so both run the same
// arithmetic.  Mask definitions: geometry.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "geometry.h"

namespace bda {

constexpr int kBN = 64;   // keys per staged tile (two 32-key MFMA subtiles)

// The three walks of the forward kernel (see attn.hip).
enum { kWalkRegs = 0, kWalkPersistent = 1, kWalkSplit = 2 };

// The scalar arguments the index arithmetic reads.
struct AttnIndex {
  int B, Hq, Hkv, G, mode, L, n, blk, Sq, Sk;
  int rows_per_wg, n_qtiles, n_splits, split_keys, pairs_per_xcd;
  int n_items;      // work items (batch x kv head x query tile x key split)
};

// Geometry of one work item: its (batch, kv head) pair, query tile and key
// split, and the key ranges its rows need.  F is walked by the pipelined
// loop (every row of the item may see every key of it); R1 and R2 are the
// remaining keys the rows need, walked tile by tile with per-wavefront
// classification.
struct Geom {
  Span F, R1, R2;
  int nf, n1, nt;
  int pair, qt, split;
  int L;            // keys of the item's batch row (DECODE/CAUSAL; HYBRID: L per half)
};

// Work item idx.  The canonical order (index -> batch, kv head, query tile,
// key split) hands out the heaviest query tiles first.  With pairs_per_xcd >
// 0, index i runs on XCD i % 8 (workgroups are dealt to the 8 XCDs
// round-robin) and every query tile of a (batch, kv head) maps to one XCD, so
// its K/V stays in that XCD's L2.  kv_len (DECODE/CAUSAL, may be null): keys
// of each batch row, clamped to [n, L].
BDA_HD void attn_geom(const AttnIndex& a, int walk, const int32_t* kv_len, int idx, Geom& gm) {
  const int P = a.B * a.Hkv;
  if (a.pairs_per_xcd > 0) {
    const int xcd = idx & 7, i = idx >> 3;
    gm.pair = xcd * a.pairs_per_xcd + i % a.pairs_per_xcd;
    gm.qt = a.n_qtiles - 1 - i / a.pairs_per_xcd;
    gm.split = 0;
  } else {
    gm.split = idx % a.n_splits;
    const int rest = idx / a.n_splits;
    gm.pair = rest % P;
    gm.qt = a.n_qtiles - 1 - rest / P;
  }
  Span F{0, 0}, R1{0, 0}, R2{0, 0};
  gm.L = a.L;
  if (a.mode == kHybrid) {
    const int p0 = gm.qt * a.rows_per_wg;
    const int p1 = imin(a.L, p0 + a.rows_per_wg);
    const int e = imin(a.L, ((p1 - 1) / a.blk + 1) * a.blk);
    const int s_min = (p0 / a.blk) * a.blk;   // clean prefix every row of the item sees
    F = Span{a.L, a.L + (s_min / kBN) * kBN};
    R1 = Span{F.hi, a.L + e};                 // rest of the clean prefix / own clean blocks
    R2 = Span{s_min, e};                      // noisy blocks of these rows
  } else {
    int Lb = a.L;
    if (kv_len != nullptr) {
      Lb = imin(a.L, imax(a.n, kv_len[gm.pair / a.Hkv]));
      gm.L = Lb;
    }
    const int r0 = gm.qt * a.rows_per_wg;
    const int r1 = imin(a.n, r0 + a.rows_per_wg);
    const int lo = gm.split * a.split_keys;
    const int hi = imin(a.mode == kDecode ? Lb : Lb - a.n + r1, lo + a.split_keys);
    const int full_hi = imin(hi, a.mode == kDecode ? Lb : Lb - a.n + r0 + 1);
    const int nfull = full_hi > lo ? (full_hi - lo) / kBN : 0;
    F = Span{lo, lo + nfull * kBN};
    R1 = Span{F.hi, imax(F.hi, hi)};
  }
  // The persistent walk needs a boundary tile at the end of every item (its
  // ring wait relies on it); an item of full tiles only gives up its last.
  if (walk == kWalkPersistent && R1.hi <= R1.lo && R2.hi <= R2.lo && F.hi > F.lo) {
    F.hi -= kBN;
    R1 = Span{F.hi, F.hi + kBN};
  }
  gm.F = F;
  gm.R1 = R1;
  gm.R2 = R2;
  gm.nf = (F.hi - F.lo) / kBN;
  gm.n1 = R1.hi > R1.lo ? (R1.hi - R1.lo + kBN - 1) / kBN : 0;
  const int n2 = R2.hi > R2.lo ? (R2.hi - R2.lo + kBN - 1) / kBN : 0;
  gm.nt = gm.nf + gm.n1 + n2;
}

// First and one-past-last key of tile j of an item (j clamped to the last tile).
BDA_HD void attn_tile(const Geom& gm, int j, int& t0, int& t1) {
  j = imin(j, gm.nt - 1);
  if (j < gm.nf) {
    t0 = gm.F.lo + j * kBN;
    t1 = t0 + kBN;
  } else if (j < gm.nf + gm.n1) {
    t0 = gm.R1.lo + (j - gm.nf) * kBN;
    t1 = imin(gm.R1.hi, t0 + kBN);
  } else {
    t0 = gm.R2.lo + (j - gm.nf - gm.n1) * kBN;
    t1 = imin(gm.R2.hi, t0 + kBN);
  }
}

// Item of round r of persistent workgroup wg in a grid of gr, or -1 when it
// has none left: rounds are taken in snake order (within the workgroup's XCD
// when pairs_per_xcd > 0), so every workgroup gets a similar mix of heavy and
// light query tiles.
BDA_HD int attn_item_of(const AttnIndex& a, int gr, int wg, int r) {
  if (a.pairs_per_xcd > 0) {
    const int NL = gr >> 3, wl = wg >> 3;
    const int i = r * NL + ((r & 1) ? NL - 1 - wl : wl);
    return i < (a.n_items >> 3) ? i * 8 + (wg & 7) : -1;
  }
  const int i = r * gr + ((r & 1) ? gr - 1 - wg : wg);
  return i < a.n_items ? i : -1;
}

// Query slot s of an item's query tile qt and kv head g: in HYBRID, s counts
// within one half (half 0: the noisy rows x_t, 1: the clean rows x_0); the
// G heads of a row are adjacent slots.  Sets the query row (row of the query
// tensor) and head; returns whether the slot holds a row.
BDA_HD bool attn_slot(const AttnIndex& a, int half, int s, int qt, int g, int& qrow, int& head) {
  const int rloc = s / a.G;
  head = g * a.G + (s - rloc * a.G);
  if (a.mode == kHybrid) {
    const int pos = qt * a.rows_per_wg + rloc;
    qrow = half * a.L + pos;
    return rloc < a.rows_per_wg && pos < a.L;
  }
  const int r = qt * a.rows_per_wg + rloc;
  qrow = r;
  return rloc < a.rows_per_wg && r < a.n;
}

// Offsets of the global accesses, in 64 bits: rows (q / out / lse, k / v,
// split partials) and the elements of a row's first entry at head dim D.
BDA_HD size_t attn_q_row(const AttnIndex& a, int b, int head, int qrow) {
  return (size_t)(b * a.Hq + head) * a.Sq + qrow;
}
BDA_HD size_t attn_kv_row(const AttnIndex& a, int pair, int key) {
  return (size_t)pair * a.Sk + key;
}
BDA_HD size_t attn_part_row(const AttnIndex& a, int split, int b, int head, int qrow) {
  return (size_t)split * ((size_t)a.B * a.Hq * a.n) + (size_t)(b * a.Hq + head) * a.n + qrow;
}
template <int D>
BDA_HD size_t attn_q_elem(const AttnIndex& a, int b, int head, int qrow) {
  return attn_q_row(a, b, head, qrow) * D;
}
template <int D>
BDA_HD size_t attn_kv_elem(const AttnIndex& a, int pair, int key) {
  return attn_kv_row(a, pair, key) * D;
}
template <int D>
BDA_HD size_t attn_part_elem(const AttnIndex& a, int split, int b, int head, int qrow) {
  return attn_part_row(a, split, b, head, qrow) * D;
}

// LDS layout of a staged K (or V) tile of 64 keys x D (16-byte chunks, CPR =
// D / 8 per key).  Keys are taken in groups of 8: group g = key / 8 starts at
// byte g * 16 D, and within it chunk c of key r sits at byte (c / 8) * 1024 +
// 16 * ((8 (c % 8) + ((r % 8) ^ 4 ((c / 2) % 2))) ^ 8 (g % 2)).  Why this
// form:
//  * one DMA load (64 lanes x 16 bytes, 1 KB) fills 8 keys x 8 chunks (D >=
//    64) or 16 keys x 4 chunks (D = 32): every 8 lanes read one whole 128-byte
//    line of a key row, so a streamed cache line is fetched by one load;
//  * the K operand read of one k-step (16 keys x one chunk per 16 lanes) and
//    the V transpose read (4 keys x 4 chunks per 16 lanes, 32 lanes per
//    clock) each touch 16 distinct 16-byte bank groups of the 64-bank LDS;
//  * every operand address is a lane constant plus a compile-time offset: the
//    k-step moves by 512 bytes per pair of k-steps plus a parity (two K base
//    registers), the 32-column tiles of V^T by 512 bytes, the key subtiles by
//    whole key groups (two V base registers: a key and the key 8 further).
template <int D>
BDA_HD constexpr int fwd_off(int r, int c) {   // byte offset of chunk c of key r
  return (r >> 3) * (16 * D) + (c >> 3) * 1024 +
         16 * ((8 * (c & 7) + ((r & 7) ^ (4 * ((c >> 1) & 1)))) ^ (8 * ((r >> 3) & 1)));
}
// Inverse of fwd_off: the key and chunk whose 16 bytes sit at byte b (a
// multiple of 16) of a tile.
template <int D>
BDA_HD void fwd_at(int b, int& r, int& c) {
  const int g = b / (16 * D), rem = b % (16 * D);
  const int s = ((rem % 1024) >> 4) ^ (8 * (g & 1));
  c = 8 * (rem >> 10) + (s >> 3);
  r = 8 * g + ((s & 7) ^ (4 * (((s >> 3) >> 1) & 1)));
}

}  // namespace bda
