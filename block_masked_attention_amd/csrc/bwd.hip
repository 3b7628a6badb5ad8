// Backward of the hybrid-mask attention (the training form) for gfx950.
//
// The forward is the block-diffusion attention over [x_t ; x_0] ("Block
// Diffusion Attention", sec. 1 of the Nemotron-Labs-Diffusion-8B-Base 3x
// analysis page; the BDLM objective of the LLaDA2.0-Uni summary trains
// through it).  With P = softmax(scale Q K^T) over the allowed keys and the
// per-row log-sum-exp from the forward, for loss = sum(dO * O):
//   dV = P^T dO,   dP = dO V^T,   dS = P (dP - D),  D_i = sum_c dO_ic O_ic,
//   dQ = scale dS K,   dK = scale dS^T Q.
// Two launches:
//   dq     query-stationary, like the forward (it also forms D per query row
//          from O and the dO it holds): per key tile S^T = K Q^T,
//          dP^T = V dO^T, dS^T, then dQ^T += K^T dS^T (K^T by the LDS
//          transpose read, dS^T straight from the accumulator registers).
//   dkdv   key-stationary: a workgroup keeps 128 keys of one (batch, kv
//          head) in LDS and streams the blocks of 32 query slots (rows x
//          heads of the group) that see them, from the end of the sequence
//          down; two groups of 4 wavefronts (32
//          keys each) take alternate blocks: S = Q K^T, dP = dO V^T
//          (lane = key), dV += P^T dO and dK += dS^T Q (dO and Q by the LDS
//          transpose read); the groups' partial dK, dV add at the end.
// P is rebuilt exactly from the log-sum-exp (no running max); masked pairs
// get P = 0.  fp32 accumulation, bf16 MFMA operands, bf16 gradients.
#include <limits.h>

#include <type_traits>

#include "attn_index.h"
#include "common.h"
#include "geometry.h"
#include "internal.h"
#include "tiles.h"

namespace bda {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;     // [B*Hq*S] natural log
  float* delta;         // [B*Hq*S] workspace
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int B, Hq, Hkv, G, L, blk, S;
  int rows_per_wg, n_qtiles;   // dq: query tile size (per half) and count
  int nkh;                     // dkdv: 128-key tiles per half
  int pairs_per_xcd;
  float sl2, scale;
};

constexpr float kLn2Inv = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// dQ.  One workgroup per (batch, kv head, query tile) as in the forward's
// training form: NW wavefronts x 32 query slots, half of them on x_t rows
// and half on the same positions of x_0.  K/V tiles come through a 4-stage
// DMA ring; the kernel also forms D = rowsum(dO O) of its rows for dK/dV.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(const BwdArgs a) {
  constexpr int KSTEPS = D / 16, DT = D / 32, CPR = D / 8;
  constexpr int BN = 64, TCH = BN * CPR, NT = NW * 64, TE = BN * D;
  constexpr int NSQ = 4;                       // K/V tile stages, filled three tiles ahead
  __shared__ __attribute__((aligned(16))) uint16_t smem[NSQ * 2 * TE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, ql = lane & 31, hb = lane >> 5;
  const int P = a.B * a.Hkv;
  int pair, qt;
  {
    const int bid = blockIdx.x;
    if (a.pairs_per_xcd > 0) {
      const int xcd = bid & 7, i = bid >> 3;
      pair = xcd * a.pairs_per_xcd + i % a.pairs_per_xcd;
      qt = a.n_qtiles - 1 - i / a.pairs_per_xcd;
    } else {
      pair = bid % P;
      qt = a.n_qtiles - 1 - bid / P;
    }
  }
  const int b = pair / a.Hkv, g = pair - b * a.Hkv;
  const int per_half = NW / 2, half = w / per_half;
  const int s = (w - half * per_half) * 32 + ql;
  const int rloc = s / a.G;
  const int pos = qt * a.rows_per_wg + rloc;
  const bool valid = rloc < a.rows_per_wg && pos < a.L;
  const int qrow = half * a.L + pos;
  const int head = g * a.G + (s - rloc * a.G);
  const size_t rowi = (size_t)(b * a.Hq + head) * a.S + qrow;

  // key ranges of the tile (as in the forward)
  const int p0 = qt * a.rows_per_wg;
  const int p1 = imin(a.L, p0 + a.rows_per_wg);
  const int e = imin(a.L, ((p1 - 1) / a.blk + 1) * a.blk);
  const int s_min = (p0 / a.blk) * a.blk;
  const Span F{a.L, a.L + (s_min / BN) * BN};
  const Span R1{F.hi, a.L + e};
  const Span R2{s_min, e};
  const int nf = (F.hi - F.lo) / BN;
  const int n1 = R1.hi > R1.lo ? (R1.hi - R1.lo + BN - 1) / BN : 0;
  const int n2 = R2.hi > R2.lo ? (R2.hi - R2.lo + BN - 1) / BN : 0;
  const int nt = nf + n1 + n2;
  auto tile = [&](int j, int& t0, int& t1) {
    j = imin(j, nt - 1);
    if (j < nf) {
      t0 = F.lo + j * BN;
      t1 = t0 + BN;
    } else if (j < nf + n1) {
      t0 = R1.lo + (j - nf) * BN;
      t1 = imin(R1.hi, t0 + BN);
    } else {
      t0 = R2.lo + (j - nf - n1) * BN;
      t1 = imin(R2.hi, t0 + BN);
    }
  };

  bf16x8 qreg[KSTEPS], dreg[KSTEPS];
  {
    const uint16_t* qp = a.q + rowi * D + 8 * hb;
    const uint16_t* dp = a.dout + rowi * D + 8 * hb;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x4 x = valid ? *(const u32x4*)(qp + 16 * ks) : u32x4{0, 0, 0, 0};
      const u32x4 y = valid ? *(const u32x4*)(dp + 16 * ks) : u32x4{0, 0, 0, 0};
      qreg[ks] = __builtin_bit_cast(bf16x8, x);
      dreg[ks] = __builtin_bit_cast(bf16x8, y);
    }
  }
  const float lse2 = valid ? a.lse[rowi] * kLn2Inv : INFINITY;
  // D of the slot's row, sum over d of dO O in fp32: lane (ql, hb) holds
  // d = 16 ks + 8 hb + 0..7 of dO, and the two half-wavefronts add.  The
  // dK/dV kernel, launched after this one, reads it from the workspace.
  float dl;
  {
    const uint16_t* op = a.o + rowi * D + 8 * hb;
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x4 x = valid ? *(const u32x4*)(op + 16 * ks) : u32x4{0, 0, 0, 0};
      const u32x4 y = __builtin_bit_cast(u32x4, dreg[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) part += bf16_lo(x[e]) * bf16_lo(y[e]) + bf16_hi(x[e]) * bf16_hi(y[e]);
    }
    dl = half_sum(part);
    if (valid && hb == 0) a.delta[rowi] = dl;
  }
  Span A{0, 0}, C{0, 0};
  if (valid) row_spans(kHybrid, a.L, 2 * a.L, a.blk, qrow, A, C);

  const size_t kvoff = (size_t)pair * a.S * D;
  const uint16_t* kbase = a.k + kvoff;
  const uint16_t* vbase = a.v + kvoff;

  // The K and V tiles of a stage use the forward's LDS layout (fwd_off in
  // attn_index.h), so every operand address is a lane constant plus a
  // compile-time offset.  S^T / dP^T operand (key 32 sub + ql, chunk
  // 2 ks + hb): kl[ks % 2] + 256 (ks - ks % 2) + 64 D sub bytes.  K^T operand
  // of dQ^T (transpose read): lane (gi = lane / 16, j = lane % 16) reads 4
  // values at column 32 dt + 16 (gi % 2) + 4 (j % 4) of key 32 sub + 16 kk +
  // 4 hb + j / 4 (lo) and of the key 8 further (hi), at kt_lo (kt_hi) +
  // 512 dt + 32 D (2 sub + kk).
  const int kl0 = fwd_off<D>(ql, hb), kl1 = fwd_off<D>(ql, 2 + hb);
  int kt_lo, kt_hi;
  {
    const int j = lane & 15, gi = lane >> 4;
    const int r = 4 * hb + (j >> 2), c = 2 * (gi & 1) + ((j & 3) >> 1);
    kt_lo = fwd_off<D>(r, c) + 8 * (j & 1);
    kt_hi = fwd_off<D>(r + 8, c) + 8 * (j & 1);
  }

  // Tile j straight from global memory into stage st (no registers): lane i
  // of a wavefront's load fills bytes 1024 run + 16 i of the tile, so it
  // loads the key and chunk fwd_at names there, from the tile's first key
  // row (a uniform base in SGPRs) plus a 32-bit lane offset; in a short
  // tile, keys past t1 - 1 repeat key t1 - 1 (finite data the masks never
  // let through).
  constexpr int DJ = TCH >= NT ? TCH / NT : 1;   // loads per wavefront per matrix
  constexpr bool ALL_RUNS = TCH / 64 >= NW * DJ;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  int d_row[DJ];
  unsigned d_off[DJ];
#pragma unroll
  for (int q = 0; q < DJ; ++q) {
    int r, c;
    fwd_at<D>(1024 * (w * DJ + q) + 16 * lane, r, c);
    d_row[q] = r;
    d_off[q] = (unsigned)(r * 2 * D + c * 16);
  }
  auto issue = [&](int j, uint16_t* st) {
    int t0, t1;
    tile(j, t0, t1);
    const uint16_t* kb = kbase + (size_t)t0 * D;
    const uint16_t* vb = vbase + (size_t)t0 * D;
    const int last = t1 - t0 - 1;
    const unsigned mk = lds_addr(st), mv = lds_addr(st + TE);
#pragma unroll
    for (int q = 0; q < DJ; ++q) {
      const int run = wu * DJ + q;
      if (ALL_RUNS || run * 64 < TCH) {
        const unsigned off = d_off[q] - (unsigned)((d_row[q] - imin(d_row[q], last)) * 2 * D);
        lds_dma16_sa(kb, off, mk + run * 1024);
        lds_dma16_sa(vb, off, mv + run * 1024);
      }
    }
  };
  // Tile j visible to every wavefront, given that tiles 0 .. issued-1 have
  // been issued: the (up to two) tiles issued after j stay in flight.
  auto settle_for = [&](int j, int issued) {
    const int newer = imin(NSQ - 2, imax(0, issued - 1 - j));
    constexpr int T = 2 * DJ;
    asm volatile("" ::: "memory");
    if (newer >= 2)
      __builtin_amdgcn_s_waitcnt(((2 * T) & 15) | (7 << 4) | (((2 * T) >> 4) << 14));
    else if (newer == 1)
      __builtin_amdgcn_s_waitcnt((T & 15) | (7 << 4) | ((T >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt(7 << 4);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  // S^T and dP^T of one 32-key subtile
  auto sdp_sub = [&](const uint16_t* st, int sub, f32x16& sv, f32x16& dp) {
    const char* kr = (const char*)st + sub * 64 * D;
    const char* vr = kr + 2 * TE;
    sv = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int o = 256 * (ks & ~1) + ((ks & 1) ? kl1 : kl0);
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kr + o), qreg[ks], sv, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vr + o), dreg[ks], dp, 0, 0, 0);
    }
  };
  // dS^T of the subtile (keys [e0, e1); every pair allowed when full), then
  // dQ^T += K^T dS^T
  auto grad_sub = [&](const uint16_t* st, int sub, int e0, int e1, bool full, const f32x16& sv,
                      const f32x16& dp) {
    bf16x8 dsb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 pk;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float d2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 8 * kk + 2 * e2 + h;
          const int jj = e0 + 8 * (i >> 2) + 4 * hb + (i & 3);
          // bitwise, not short-circuit: a select per element, no branches
          const bool ok = full | ((jj < e1) & (in_span(A, jj) | in_span(C, jj)));
          const float p = exp2_fast(ok ? fmaf(sv[i], a.sl2, -lse2) : -INFINITY);   // masked: exp2(-inf) = 0
          d2[h] = p * (dp[i] - dl);
        }
        pk[e2] = pack_bf16x2(d2[0], d2[1]);
      }
      dsb[kk] = __builtin_bit_cast(bf16x8, pk);
    }
    unsigned b_lo = lds_addr(st) + kt_lo, b_hi = lds_addr(st) + kt_hi;
    asm volatile("" : "+v"(b_lo), "+v"(b_hi));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const unsigned kt = (2 * sub + kk) * 32 * D + dt * 512;
        const s16x4 lo = lds_read_tr_at(b_lo + kt);
        const s16x4 hi = lds_read_tr_at(b_hi + kt);
        const bf16x8 kop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, dsb[kk], acc[dt], 0, 0, 0);
      }
    }
  };
  // a boundary subtile: classified per wavefront, skipped when no lane sees it
  auto subtile = [&](const uint16_t* st, int j, int sub) {
    int t0, t1;
    tile(j, t0, t1);
    const int e0 = t0 + 32 * sub, e1 = imin(t1, e0 + 32);
    if (e0 >= e1) return;
    const int c = inside(A, e0, e1) + inside(C, e0, e1);
    const bool full = __all(!valid || (e1 - e0 == 32 && c == 32));
    if (__all(!valid || c == 0)) return;
    f32x16 sv, dp;
    sdp_sub(st, sub, sv, dp);
    grad_sub(st, sub, e0, e1, full, sv, dp);
  };

  if (nt > 0) {
    // Tile j lives in stage j % NSQ; tile j + 3 goes into the stage of tile
    // j - 1, which every wavefront finished before the last barrier.
    auto stq = [&](int j) { return smem + (j % NSQ) * 2 * TE; };
    int issued = 0;
    for (; issued < NSQ - 1 && issued < nt; ++issued) issue(issued, stq(issued));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);               // Q, dO and the first tiles
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Two loops, not one with a branch per tile: with both paths in one
    // loop body the compiler kept the dQ accumulators in two register sets
    // and copied all 64 of them twice per tile.
#pragma unroll 1
    for (int j = 0; j < nf; ++j) {
      // clean-prefix tile every row sees: no classification, no branches
      if (issued < nt) issue(issued, stq(issued)), ++issued;
      const uint16_t* cur = stq(j);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        f32x16 sv, dp;
        sdp_sub(cur, sub, sv, dp);
        grad_sub(cur, sub, 0, 0, true, sv, dp);
      }
      settle_for(j + 1, issued);
    }
#pragma unroll 1
    for (int j = nf; j < nt; ++j) {
      if (issued < nt) issue(issued, stq(issued)), ++issued;
      const uint16_t* cur = stq(j);
      subtile(cur, j, 0);
      subtile(cur, j, 1);
      settle_for(j + 1, issued);
    }
  }

  // dq = scale * dQ^T; lane (ql, hb) holds d = 32*dt + 8*(i/4) + 4*hb + (i%4).
  // Through LDS (the ring, idle after the last step's barrier), so that each
  // store writes whole rows rather than 16 bytes of 32 rows: the wavefront's
  // 32 rows go into its 32 x D region in the accumulator layout, 16-byte
  // chunks XOR-swizzled by the row, and come back 16 bytes per lane.
  static_assert(NW * 32 * 2 * D <= NSQ * 2 * TE * 2, "dq staging exceeds the ring");
  char* reg = reinterpret_cast<char*>(smem) + w * (32 * 2 * D);
  if (valid) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[dt][4 * i4] * a.scale, acc[dt][4 * i4 + 1] * a.scale);
        pk[1] = pack_bf16x2(acc[dt][4 * i4 + 2] * a.scale, acc[dt][4 * i4 + 3] * a.scale);
        const int c = 4 * dt + i4;   // 16-byte chunk of the row
        *(u32x2*)(reg + ql * (2 * D) + ((c ^ (ql & (CPR - 1))) << 4) + 8 * hb) = pk;
      }
  }
  const long long ri = valid ? (long long)rowi : -1;   // lane (ql, either half): row of slot ql
  constexpr int RPI = 64 / CPR;                       // rows per store instruction
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int r = k * RPI + lane / CPR, c = lane % CPR;
    const u32x4 x = *(const u32x4*)(reg + r * (2 * D) + ((c ^ (r & (CPR - 1))) << 4));
    const long long rr = __shfl(ri, r);
    if (rr >= 0) *(u32x4*)(a.dq + (size_t)rr * D + 8 * c) = x;
  }
}

// ---------------------------------------------------------------------------
// dK, dV with two wavefronts per SIMD.  One workgroup of 8 wavefronts per
// (batch, kv head, 128-key tile of one half); wavefronts w and w + 4 own keys
// 32(w%4) .. 32(w%4)+31 of the tile and form two groups: at step s group g
// computes query block 2s + g.  K and V stay in LDS and are read per block
// (a wavefront keeps only its dK, dV accumulators), four single-block stages
// hold the two blocks being computed and the two loading for the next step.
// At the end group 1 adds its dK, dV partials into group 0's through LDS.
template <int D>
__global__ __launch_bounds__(512, 2) void bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int KSTEPS = D / 16, DT = D / 32, CPR = D / 8;
  constexpr int TK = 128, NT = 512;
  constexpr int KE = TK * D;                   // elements of the K (or V) tile
  constexpr int QE = 32 * D;                   // elements of a Q (or dO) block
  constexpr int QCH = 32 * CPR;                // chunks of a Q block
  constexpr int NS = 4;                        // single-block stages
  // [K tile | V tile | NS x (Q block | dO block)]; reused for the merge and
  // the transposed write of dK, dV at the end
  constexpr int LDS_ELEMS = 2 * KE + NS * 2 * QE;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
  uint16_t* const kv = lds;
  uint16_t* const qd = lds + 2 * KE;
  __shared__ __attribute__((aligned(16))) float sl[NS][2][32];  // lse (natural log), delta per slot
  // Per slot, the mask as one integer t: clean-key tiles let a slot see key
  // block kb iff kb <= t (t = the row's block for an x_0 row, one less for
  // an x_t row); noisy-key tiles iff kb == t (t = the row's block for an
  // x_t row).  t = -1: no such row, or a row that sees nothing of the tile.
  __shared__ __attribute__((aligned(16))) int sthr[NS][32];
  static_assert(4 * 2 * DT * 16 * 64 * 4 <= LDS_ELEMS * 2, "merge buffer exceeds LDS");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, ql = lane & 31, hb = lane >> 5;
  const int kg = w >> 2, wk = w & 3;           // query-block group, key group
  int pair, j;
  {
    const int bid = blockIdx.x;
    if (a.pairs_per_xcd > 0) {
      const int xcd = bid & 7, i = bid >> 3;
      pair = xcd * a.pairs_per_xcd + i % a.pairs_per_xcd;
      j = i / a.pairs_per_xcd;
    } else {
      const int P = a.B * a.Hkv;
      pair = bid % P;
      j = bid / P;
    }
  }
  const bool clean = j < a.nkh;
  const int kp0 = (clean ? j : j - a.nkh) * TK;
  const int kp1 = imin(a.L, kp0 + TK);
  const int kbase_row = (clean ? a.L : 0) + kp0;
  const int b = pair / a.Hkv, g = pair - b * a.Hkv;
  const size_t kvoff = (size_t)pair * a.S * D;

  // the tile's K and V into LDS (rows past the half's end repeat its last key)
#pragma unroll
  for (int u = 0; u < (TK * CPR) / NT; ++u) {
    const int ch = tid + u * NT;
    const int r = ch / CPR, c = ch % CPR;
    const size_t off = kvoff + (size_t)(kbase_row + imin(r, kp1 - kp0 - 1)) * D + 8 * c;
    const int lo = chunk_off<D>(r, c);
    *(u32x4*)(kv + lo) = *(const u32x4*)(a.k + off);
    *(u32x4*)(kv + KE + lo) = *(const u32x4*)(a.v + off);
  }

  // query rows that see the tile: up to two position ranges, [ra0, ra1) of
  // half ha and [rb0, rb1) of x_t; heaviest tiles first (clean tiles from
  // the start of the sequence, then the noisy tiles, which only their own
  // blocks' rows see)
  const int jb = kp0 / a.blk;
  int ra0, ra1, rb0, rb1, ha;
  if (clean) {
    ha = 1;
    ra0 = jb * a.blk;
    ra1 = a.L;
    rb0 = imin(a.L, (jb + 1) * a.blk);
    rb1 = a.L;
  } else {
    ha = 0;
    ra0 = jb * a.blk;
    ra1 = imin(a.L, ((kp1 - 1) / a.blk + 1) * a.blk);
    rb0 = rb1 = 0;
  }
  const int rpb = 32 / a.G;
  const int na = ra1 > ra0 ? (ra1 - ra0 + rpb - 1) / rpb : 0;
  const int nb = rb1 > rb0 ? (rb1 - rb0 + rpb - 1) / rpb : 0;
  const int nblk = na + nb;

  constexpr int QRUNS = QCH / 64;                         // 64-chunk runs of a Q block
  constexpr int QJ = (QRUNS + 3) / 4;                     // runs per wavefront of a group per matrix
  // Blocks are taken from the end of the sequence down, the two ranges
  // interleaved (both end at the same position for a clean tile), so the
  // workgroups of one (batch, kv head) that run together read the same Q and
  // dO rows at about the same time and share them in L2.
  auto block_row0 = [&](int t, int& half, int& r0, int& r1) {
    const int m = imin(na, nb);
    bool in_a;
    int kb;
    if (t < 2 * m) {
      in_a = (t & 1) == 0;
      kb = (in_a ? na : nb) - 1 - (t >> 1);
    } else {
      in_a = na > nb;
      kb = (in_a ? na : nb) - 1 - (t - m);
    }
    if (in_a) {
      half = ha;
      r0 = ra0 + kb * rpb;
      r1 = ra1;
    } else {
      half = 0;
      r0 = rb0 + kb * rpb;
      r1 = rb1;
    }
  };
  const unsigned lds_qd = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)qd);
  const unsigned lds_sl = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)&sl[0][0][0]);
  // Block t of query slots straight from global memory into LDS stage st,
  // issued by the 4 wavefronts of one group: Q and dO rows (each lane loads
  // the 16-byte chunk the permuted layout puts at its lane slot), then the
  // slots' lse and delta (one dword per lane of lanes 0..15 of every
  // wavefront of the group: dwords 16wk .. 16wk+15 of lse[32] ++ delta[32]),
  // then the slots' thresholds.  Slots without a row load row 0 of the block
  // (finite data the thresholds never let through).
  auto issue = [&](int t, int st) {
    int half, r0, r1;
    block_row0(t, half, r0, r1);
#pragma unroll
    for (int q = 0; q < QJ; ++q) {
      const int run = imin(wk + 4 * q, QRUNS - 1);
      const int pos = run * 64 + lane;
      const int sl_ = pos / CPR, c = (pos % CPR) ^ (swz<D>(sl_) & (CPR - 1));
      const int rl = sl_ / a.G;
      const bool ok = rl < rpb && r0 + rl < r1;
      const int head = g * a.G + (ok ? sl_ - rl * a.G : 0);
      const size_t off = ((size_t)(b * a.Hq + head) * a.S + half * a.L + (ok ? r0 + rl : r0)) * D + 8 * c;
      const unsigned dst = lds_qd + (unsigned)(st * 2 * QE + run * 512) * 2;
      lds_dma16s(a.q + off, dst);
      lds_dma16s(a.dout + off, dst + QE * 2);
    }
    {
      const int x = 16 * wk + (lane & 15);
      const int slot = x & 31;
      const int rl = slot / a.G;
      const bool ok = rl < rpb && r0 + rl < r1;
      const int head = g * a.G + (ok ? slot - rl * a.G : 0);
      const size_t ri = (size_t)(b * a.Hq + head) * a.S + half * a.L + (ok ? r0 + rl : r0);
      const float* src = (x < 32 ? a.lse : a.delta) + ri;
      if (lane < 16) lds_dma4s(src, lds_sl + (unsigned)(st * 64 + 16 * wk) * 4);
    }
    if ((tid & 255) < 32) {
      const int s_ = tid & 255, rl = s_ / a.G, pos = r0 + rl;
      int t_ = -1;
      if (rl < rpb && pos < r1) {
        const int rb = pos / a.blk;
        t_ = clean ? (half == 1 ? rb : rb - 1) : (half == 0 ? rb : -1);
      }
      sthr[st][s_] = t_;
    }
  };
  // every load of this wavefront (DMA included) and every LDS access done,
  // then the workgroup barrier
  auto drain = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int key = kp0 + 32 * wk + ql;
  const bool key_ok = key < kp1;
  const int kblk = key_ok ? key / a.blk : INT_MAX / 2;
  const int wk0 = kp0 + 32 * wk, wk1 = imin(kp1, wk0 + 32);
  const int wb0 = wk0 / a.blk, wb1 = wk1 > wk0 ? (wk1 - 1) / a.blk : -1;
  const int kr_off = (32 * wk + ql) * D;
  const int k_swz = swz<D>(32 * wk + ql) & (CPR - 1);
  const int q_swz = swz<D>(ql) & (CPR - 1);
  int t_lo[DT], t_hi[DT];
  {
    const int jx = lane & 15, gi = lane >> 4;
    const int r = 4 * hb + (jx >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dcol = 32 * dt + 16 * (gi & 1) + 4 * (jx & 3);
      t_lo[dt] = chunk_off<D>(r, dcol >> 3) + (dcol & 7);
      t_hi[dt] = chunk_off<D>(r + 8, dcol >> 3) + (dcol & 7);
    }
  }

  f32x16 dka[DT], dva[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dka[dt] = dva[dt] = f32x16{};

  const bool full_wave = wk1 - wk0 == 32;
  auto seen_all = [&](int st) -> bool {
    const int my_t = sthr[st][ql];
    const bool lane_ok = clean ? my_t >= wb1 : (wb0 == wb1 && my_t == wb0);
    return full_wave && __all(lane_ok);
  };
  // the query block in stage st: S, dP (K and V operands from LDS), then P,
  // dS and the dV, dK updates
  auto block = [&](int st) {
    const uint16_t* qb = qd + st * 2 * QE;
    const uint16_t* db = qb + QE;
    const bool all_seen = __builtin_amdgcn_readfirstlane((int)seen_all(st)) != 0;   // uniform
    f32x16 sv{}, dp{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int ko = kr_off + 8 * ((2 * ks + hb) ^ k_swz);
      const int qo = ql * D + 8 * ((2 * ks + hb) ^ q_swz);
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(qb + qo), *(const bf16x8*)(kv + ko), sv, 0, 0,
                                                  0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(db + qo), *(const bf16x8*)(kv + KE + ko), dp, 0,
                                                  0, 0);
    }
    // lane = key (column), value i = slot 8*(i/4) + 4*hb + (i%4).  The
    // slots' lse, delta and threshold are read as 4-vectors, half a block at
    // a time, so the reads are unconditional and masked pairs take
    // exp2(-inf) = 0 by a select (per-element reads were sunk into a branch
    // and a full LDS wait per element).  A block every slot of the wavefront
    // sees whole takes one uniform branch to the same arithmetic without the
    // per-pair tests and selects.
    bf16x8 pb[2], sb[2];
    auto p_ds = [&](auto full_c) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        f32x4 lv[2], dvv[2];
        i32x4 tv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int o = 8 * (2 * kk + u) + 4 * hb;
          lv[u] = *(const f32x4*)(&sl[st][0][o]) * kLn2Inv;
          dvv[u] = *(const f32x4*)(&sl[st][1][o]);
          if (!FULL) tv[u] = *(const i32x4*)(&sthr[st][o]);
        }
        u32x4 pk, dk4;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float pv[2], dv2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int i = 8 * kk + 2 * e2 + h;
            const int u = (2 * e2 + h) >> 2, x = i & 3;
            float p;
            if constexpr (FULL) {
              p = exp2_fast(fmaf(sv[i], a.sl2, -lv[u][x]));
            } else {
              const int t = tv[u][x];
              const bool ok = (clean & (kblk <= t)) | (!clean & (kblk == t));
              p = exp2_fast(ok ? fmaf(sv[i], a.sl2, -lv[u][x]) : -INFINITY);
            }
            pv[h] = p;
            dv2[h] = p * (dp[i] - dvv[u][x]);
          }
          pk[e2] = pack_bf16x2(pv[0], pv[1]);
          dk4[e2] = pack_bf16x2(dv2[0], dv2[1]);
        }
        pb[kk] = __builtin_bit_cast(bf16x8, pk);
        sb[kk] = __builtin_bit_cast(bf16x8, dk4);
      }
    };
    if (all_seen)
      p_ds(std::true_type{});
    else
      p_ds(std::false_type{});
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const s16x4 dlo = lds_read_tr(db + 16 * kk * D + t_lo[dt]);
        const s16x4 dhi = lds_read_tr(db + 16 * kk * D + t_hi[dt]);
        const s16x4 qlo = lds_read_tr(qb + 16 * kk * D + t_lo[dt]);
        const s16x4 qhi = lds_read_tr(qb + 16 * kk * D + t_hi[dt]);
        const bf16x8 dop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 qop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
        dva[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pb[kk], dop, dva[dt], 0, 0, 0);
        dka[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sb[kk], qop, dka[dt], 0, 0, 0);
      }
    }
  };

  // Block t lives in stage t % NS.  Step s: group g issues block 2s + 2 + g
  // into the stage of block 2s - 2 + g (finished before the last barrier),
  // computes block 2s + g, then every load lands before the barrier.
  if (kg < nblk) issue(kg, kg);
  drain();   // also publishes the K, V tile
  const int nsteps = (nblk + 1) / 2;
#pragma unroll 1
  for (int s = 0; s < nsteps; ++s) {
    const int tn = 2 * s + 2 + kg, tc = 2 * s + kg;
    if (tn < nblk) issue(tn, tn % NS);
    if (tc < nblk) block(tc % NS);
    drain();
  }

  // group 1 adds its partials into group 0's through LDS
  float* xf = reinterpret_cast<float*>(lds);
  auto xi = [&](int which, int dt, int i) { return (((wk * 2 + which) * DT + dt) * 16 + i) * 64 + lane; };
  if (kg == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        xf[xi(0, dt, i)] = dka[dt][i];
        xf[xi(1, dt, i)] = dva[dt][i];
      }
  }
  __syncthreads();
  if (kg == 0) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dka[dt][i] += xf[xi(0, dt, i)];
        dva[dt][i] += xf[xi(1, dt, i)];
      }
  }
  __syncthreads();
  // write dK (scaled) and dV through LDS into 16-byte rows (group 0)
  uint16_t* tk = lds + wk * 2 * 32 * D;
  uint16_t* tv = tk + 32 * D;
  if (kg == 0) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kr = 8 * (i >> 2) + 4 * hb + (i & 3);
        tk[kr * D + 32 * dt + ql] = __builtin_bit_cast(uint16_t, (__bf16)(dka[dt][i] * a.scale));
        tv[kr * D + 32 * dt + ql] = __builtin_bit_cast(uint16_t, (__bf16)dva[dt][i]);
      }
  }
  __syncthreads();
  if (kg == 0) {
    for (int ch = lane; ch < 32 * CPR; ch += 64) {
      const int kr = ch / CPR, c = ch % CPR;
      const int kpos = kp0 + 32 * wk + kr;
      if (kpos < kp1) {
        const size_t off = kvoff + (size_t)((clean ? a.L : 0) + kpos) * D + 8 * c;
        *(u32x4*)(a.dk + off) = *(const u32x4*)(tk + kr * D + 8 * c);
        *(u32x4*)(a.dv + off) = *(const u32x4*)(tv + kr * D + 8 * c);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side

int bwd_make_plan(int B, int Hq, int Hkv, int L, int d, int block, BwdPlan* p, const char** why) {
  BwdPlan x{};
  x.B = B;
  x.Hq = Hq;
  x.Hkv = Hkv;
  x.G = Hq / Hkv;
  x.L = L;
  x.blk = block;
  x.d = d;
  x.nw = L >= 256 ? 8 : 4;
  if (x.G > (x.nw / 2) * 32 || x.G > 32) {
    *why = "Hq/Hkv larger than 32 is not supported by the backward";
    return 2;
  }
  x.rows_per_wg = ((x.nw / 2) * 32) / x.G;
  x.n_qtiles = (L + x.rows_per_wg - 1) / x.rows_per_wg;
  x.nkh = (L + 127) / 128;
  const long long pairs = (long long)B * Hkv;
  x.pairs_per_xcd = pairs % 8 == 0 ? (int)(pairs / 8) : 0;
  x.grid_dq = pairs * x.n_qtiles;
  x.grid_kv = pairs * 2 * x.nkh;
  if (x.grid_dq > 0x7fffffffLL || x.grid_kv > 0x7fffffffLL) {
    *why = "grid too large";
    return 2;
  }
  x.ws_bytes = (size_t)B * Hq * 2 * (size_t)L * 4;
  *p = x;
  return 0;
}

template <int D>
static hipError_t bwd_launch_d(const BwdPlan& p, const BwdArgs& a, hipStream_t st) {
  hipError_t e;
  if (p.nw == 8)
    hipLaunchKernelGGL((bwd_dq_kernel<D, 8>), dim3((unsigned)p.grid_dq), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, 4>), dim3((unsigned)p.grid_dq), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)p.grid_kv), dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t bwd_launch(const BwdPlan& p, const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv, void* ws,
                      hipStream_t st) {
  BwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)o;
  a.dout = (const uint16_t*)dout;
  a.lse = lse;
  a.delta = (float*)ws;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.L = p.L;
  a.blk = p.blk;
  a.S = 2 * p.L;
  a.rows_per_wg = p.rows_per_wg;
  a.n_qtiles = p.n_qtiles;
  a.nkh = p.nkh;
  a.pairs_per_xcd = p.pairs_per_xcd;
  a.scale = 1.f / sqrtf((float)p.d);
  a.sl2 = 1.4426950408889634f * a.scale;
  (void)hipGetLastError();
  switch (p.d) {
    case 32: return bwd_launch_d<32>(p, a, st);
    case 64: return bwd_launch_d<64>(p, a, st);
    default: return bwd_launch_d<128>(p, a, st);
  }
}

}  // namespace bda
