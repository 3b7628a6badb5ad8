// Block-diffusion attention forward for gfx950: one kernel family serves the
// hybrid training form over [x_t ; x_0], the decode form (bidirectional
// active block over a clean cache) and the causal verify/prefill form.
//
// Mask definitions: "Block Diffusion Attention" (sec. 1) and "Linear
// Speculative Decoding" (sec. 2) of the Nemotron-Labs-Diffusion-8B-Base 3x
// analysis page; the BDLM conditioning of the LLaDA2.0-Uni summary
// ("training objective"); the decode form from the DiffusionGemma pipeline
// page (intro).  The key sets are turned into two intervals per query row
// (geometry.h), so the kernel never materialises a mask.
//
// Per workgroup: NW wavefronts, each owning 32 query "slots" (a slot is one
// (query row, query head) of the kv head being served; the G = Hq/Hkv heads
// of a row are adjacent slots, so one staged K/V tile feeds all of them).
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K tile (LDS), B = Q (registers)
//   online softmax in the log2 domain on the S^T accumulator (lane = query)
//   O^T += V^T P^T  same MFMA, A = V^T read with the LDS transpose read
//                  (ds_read_b64_tr_b16) from the row-major V tile, B = P
//                  straight from the S^T accumulator registers: the two
//                  4-key transpose reads of a lane pick exactly the keys its
//                  eight P values belong to, so nothing is shuffled.
#include <atomic>

#include "common.h"
#include "geometry.h"
#include "internal.h"
#include "tiles.h"

namespace bda {

constexpr int kBN = 64;   // keys per staged tile (two 32-key MFMA subtiles)

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* part_o;    // [split][B*Hq*n][D] unnormalised partial outputs
  float* part_ml;   // [split][B*Hq*n][2] (running max in log2 units, row sum)
  int B, Hq, Hkv, G, mode, L, n, blk, Sq, Sk;
  int rows_per_wg, n_qtiles, n_splits, split_keys, pairs_per_xcd;
  int n_items;      // work items (batch x kv head x query tile x key split)
  float sl2;        // log2(e) / sqrt(D)
  const int32_t* kv_len;   // optional [B] (DECODE/CAUSAL): keys of each batch row, clamped to [n, L]
  float* lse;       // optional [B*Hq*Sq]: natural-log log-sum-exp of each row's scores
};

// Geometry of one work item: its (batch, kv head) pair, query tile and key
// split, and the key ranges its rows need (see the kernel).
struct Geom {
  Span F, R1, R2;
  int nf, n1, nt;
  int pair, qt, split;
  int L;            // keys of the item's batch row (DECODE/CAUSAL; HYBRID: L per half)
};


// One workgroup = NW wavefronts; a wavefront owns QPW query slots, handled as
// QPW/32 MFMA column blocks that share every K and V operand read from LDS
// (64 slots per wavefront halve the LDS traffic per FLOP of 32).
// STAGES = 4: the persistent DMA-fed pipelined walk (one 8-wave workgroup
// per CU at d = 128) for long query ranges (training form, prefill).
// STAGES = 5: the split-key DMA ring for short query blocks over long caches
// (decode, verify): one 8-wave workgroup per item, two groups of 4 over the
// same query slots, each computing one 32-key half of every tile.
// STAGES = 2: a register-staged double-buffered walk with 4-wave workgroups
// for short training-form sequences (L < 256).
template <int D, int NW, int QPW, int STAGES, bool VARLEN, bool LSE>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int NQB = QPW / 32;               // 32-query column blocks per wavefront
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;              // MFMA k-steps of Q K^T
  constexpr int DT = D / 32;                  // 32-row tiles of O^T
  constexpr int CPR = D / 8;                  // 16-byte chunks per key row
  constexpr int TCH = kBN * CPR;              // chunks of one K (or V) tile
  constexpr int CU = (TCH + NT - 1) / NT;     // chunks per thread per tile
  constexpr int TE = kBN * D;                 // elements of one K (or V) tile
  constexpr int STAGE = 2 * TE;
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGES * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int ql = lane & 31;
  const int hb = lane >> 5;
  // STAGES = 5 (DECODE/CAUSAL): the wavefronts form two groups over the same
  // query slots; group kg computes the 32-key half kg of every staged tile.
  constexpr bool KS = STAGES == 5;
  constexpr int NWQ = KS ? NW / 2 : NW;       // wavefronts per group of query slots
  const int kg = KS ? w / NWQ : 0;
  const int wq = KS ? w - kg * NWQ : w;

  // ---- work items.  The canonical order (index -> batch, kv head, query
  // tile, key split) hands out the heaviest query tiles first.  With
  // pairs_per_xcd > 0, index i runs on XCD i % 8 (workgroups are dealt to the
  // 8 XCDs round-robin) and every query tile of a (batch, kv head) maps to
  // one XCD, so its K/V stays in that XCD's L2.
  const int P = a.B * a.Hkv;
  // key ranges of an item: F is walked by the pipelined loop (every row of
  // the item may see every key of it); R1 and R2 are the remaining keys the
  // rows need, walked tile by tile with per-wavefront classification.
  auto geom = [&](int idx, Geom& gm) {
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
    if constexpr (VARLEN) gm.L = a.L;
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
      if constexpr (VARLEN) {
        Lb = imin(a.L, imax(a.n, a.kv_len[gm.pair / a.Hkv]));
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
    if (STAGES == 4 && R1.hi <= R1.lo && R2.hi <= R2.lo && F.hi > F.lo) {
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
  };
  // first and last key of tile j of an item (j clamped to the last tile)
  auto tile_in = [&](const Geom& gm, int j, int& t0, int& t1) {
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
  };

  // ---- the item being computed
  Geom cur{};
  int b = 0, g = 0;
  const uint16_t* kbase = a.k;
  const uint16_t* vbase = a.v;
  int qrow[NQB], head[NQB];
  bool valid[NQB];
  bf16x8 qreg[NQB][KSTEPS];
  // Switch to item idx: its geometry, my query slots (one per column block)
  // and their Q operands (lane (ql, hb) holds d = 16*ks + 8*hb + 0..7).
  auto begin_item = [&](int idx) {
    geom(idx, cur);
    b = cur.pair / a.Hkv;
    g = cur.pair - b * a.Hkv;
    const size_t kvoff = (size_t)cur.pair * a.Sk * D;
    kbase = a.k + kvoff;
    vbase = a.v + kvoff;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      if (a.mode == kHybrid) {
        const int per_half = NW / 2;
        const int half = w / per_half;
        const int s = ((w - half * per_half) * NQB + qb) * 32 + ql;
        const int rloc = s / a.G;
        const int pos = cur.qt * a.rows_per_wg + rloc;
        valid[qb] = rloc < a.rows_per_wg && pos < a.L;
        qrow[qb] = half * a.L + pos;
        head[qb] = g * a.G + (s - rloc * a.G);
      } else {
        const int s = (wq * NQB + qb) * 32 + ql;
        const int rloc = s / a.G;
        const int r = cur.qt * a.rows_per_wg + rloc;
        valid[qb] = rloc < a.rows_per_wg && r < a.n;
        qrow[qb] = r;
        head[qb] = g * a.G + (s - rloc * a.G);
      }
      const uint16_t* qp = a.q + ((size_t)(b * a.Hq + head[qb]) * a.Sq + qrow[qb]) * D + 8 * hb;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4 x = valid[qb] ? *(const u32x4*)(qp + 16 * ks) : u32x4{0, 0, 0, 0};
        qreg[qb][ks] = __builtin_bit_cast(bf16x8, x);
      }
    }
  };

  // lane-constant LDS offsets (elements, within a stage)
  const int k_row = ql * D;
  const int k_swz = swz<D>(ql) & (CPR - 1);   // rows 32*sub + ql share it
  int v_lo[DT], v_hi[DT];                       // keys 4*hb + j/4 and 8 further
  {
    const int j = lane & 15, gi = lane >> 4;
    const int r = 4 * hb + (j >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dcol = 32 * dt + 16 * (gi & 1) + 4 * (j & 3);
      v_lo[dt] = chunk_off<D>(r, dcol >> 3) + (dcol & 7);
      v_hi[dt] = chunk_off<D>(r + 8, dcol >> 3) + (dcol & 7);
    }
  }

  u32x4 kreg[CU], vreg[CU];
  // global -> registers for the tile starting at key t0 (rows past t1 repeat
  // row t1-1: finite data that the masks below never let through)
  auto gload = [&](int t0, int t1) {
#pragma unroll
    for (int j = 0; j < CU; ++j) {
      const int ch = tid + j * NT;
      if (TCH % NT == 0 || ch < TCH) {
        const int r = ch / CPR, c = ch % CPR;
        const size_t off = (size_t)imin(t0 + r, t1 - 1) * D + 8 * c;
        kreg[j] = *(const u32x4*)(kbase + off);
        vreg[j] = *(const u32x4*)(vbase + off);
      }
    }
  };
  auto lstore = [&](uint16_t* st) {
#pragma unroll
    for (int j = 0; j < CU; ++j) {
      const int ch = tid + j * NT;
      if (TCH % NT == 0 || ch < TCH) {
        const int off = chunk_off<D>(ch / CPR, ch % CPR);
        *(u32x4*)(st + off) = kreg[j];
        *(u32x4*)(st + TE + off) = vreg[j];
      }
    }
  };
  // S^T = K Q^T for one 32-key subtile of a stage, all column blocks
  auto qk_sub = [&](const uint16_t* st, int sub, f32x16 (&s)[NQB]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) s[qb] = f32x16{};
    const uint16_t* kr = st + 32 * sub * D + k_row;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const bf16x8 kop = *(const bf16x8*)(kr + 8 * ((2 * ks + hb) ^ k_swz));
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[qb][ks], s[qb], 0, 0, 0);
    }
  };
  f32x16 o[NQB][DT];
  // O^T += V^T P^T for one 32-key subtile (two 16-key MFMA k-steps)
  auto pv_sub = [&](const uint16_t* st, int sub, const bf16x8 (&pb)[NQB][2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint16_t* vt = st + TE + 16 * (2 * sub + kk) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const s16x4 lo = lds_read_tr(vt + v_lo[dt]);
        const s16x4 hi = lds_read_tr(vt + v_hi[dt]);
        const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          o[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[qb][kk], o[qb][dt], 0, 0, 0);
      }
    }
  };

  const float sl2 = a.sl2;
  const float thr = 8.f / sl2;   // keep the running max until scores exceed it by 2^8 in weight
  float m_run[NQB], l_run[NQB];
  auto reset_acc = [&]() {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      m_run[qb] = -INFINITY;
      l_run[qb] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[qb][dt] = f32x16{};
    }
  };

  // Online softmax of one 32-key subtile (lane = query of each column block,
  // 16 of the 32 keys).  The running max only moves when a score exceeds it
  // by more than thr, so the rescale of O is rare; the result is the same
  // softmax.  Returns through alpha the factor O must be scaled by.
  auto softmax_sub = [&](const f32x16 (&s)[NQB], bf16x8 (&pb)[NQB][2], float (&alpha)[NQB]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mt = s[qb][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[qb][i]);
      mt = half_max(mt);
      const bool grow = mt > m_run[qb] + thr;
      const float m_use = grow ? mt : m_run[qb];
      alpha[qb] = grow ? exp2_fast((m_run[qb] - m_use) * sl2) : 1.f;
      const float nb = m_use == -INFINITY ? 0.f : -m_use * sl2;
      float ls = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = exp2_fast(fmaf(s[qb][8 * kk + 2 * e], sl2, nb));
          const float p1 = exp2_fast(fmaf(s[qb][8 * kk + 2 * e + 1], sl2, nb));
          ls += p0 + p1;
          pk[e] = pack_bf16x2(p0, p1);
        }
        pb[qb][kk] = __builtin_bit_cast(bf16x8, pk);
      }
      l_run[qb] = l_run[qb] * alpha[qb] + ls;
      m_run[qb] = m_use;
    }
  };
  // Softmax of a subtile whose keys every row sees (the pipelined walk),
  // against the running max as it stands.  The weights are summed from their
  // bf16 values (the values P V uses).  If some lane's sum reaches 2^8 (a
  // weight may then exceed 2^8, or the max is still unset) the running max
  // moves to the subtile's max, O and l are scaled by alpha <= 1 and the
  // subtile is redone with every weight <= 1.  Usually no max is taken.
  auto softmax_fast = [&](const f32x16 (&s)[NQB], bf16x8 (&pb)[NQB][2]) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
    float ls[NQB];
    auto expo = [&](int qb, float nb) {
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = exp2_fast(fmaf(s[qb][8 * kk + 2 * e], sl2, nb));
          const float p1 = exp2_fast(fmaf(s[qb][8 * kk + 2 * e + 1], sl2, nb));
          // Summed from this temporary: reading the pair back out of pk[e]
          // for the dot product is miscompiled by this toolchain.
          const unsigned pw = pack_bf16x2(p0, p1);
          pk[e] = pw;
          if (e & 1) l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw), one2, l1, false);
          else l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw), one2, l0, false);
        }
        pb[qb][kk] = __builtin_bit_cast(bf16x8, pk);
      }
      ls[qb] = l0 + l1;
    };
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      expo(qb, -m_run[qb] * sl2);
      bad |= !(ls[qb] < 256.f);
    }
    if (__builtin_expect(__any(bad), 0)) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float mt = s[qb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[qb][i]);
        const float m_use = fmaxf(m_run[qb], half_max(mt));
        const float alpha = exp2_fast((m_run[qb] - m_use) * sl2);   // 0 while the max is unset
        expo(qb, -m_use * sl2);
        m_run[qb] = m_use;
        l_run[qb] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[qb][dt] *= alpha;
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) l_run[qb] += ls[qb];
  };
  // Keep the softmax of a subtile where it is written, so its exponentials
  // overlap the score MFMAs issued before it instead of being sunk into the
  // block of the P V MFMAs that consume them.
  auto pin = [&](bf16x8 (&pb)[NQB][2]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) asm volatile("" : "+v"(pb[qb][0]), "+v"(pb[qb][1]));
  };
  auto rescale = [&](const float (&alpha)[NQB]) {
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) any |= alpha[qb] != 1.f;
    if (__any(any)) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[qb][dt] *= alpha[qb];
    }
  };

  auto tile = [&](int j, int& t0, int& t1) { tile_in(cur, j, t0, t1); };
  auto fetch = [&](int j) {
    int t0, t1;
    tile(j, t0, t1);
    gload(t0, t1);
  };
  // Tile j straight from global memory into an LDS stage (no registers):
  // each lane of a wavefront's load lands 16 bytes at its lane slot of a
  // contiguous 1 KB run, so the lane picks the global chunk that the
  // permuted layout puts there.
  constexpr int DJ = TCH >= NT ? TCH / NT : 1;   // DMA loads per wavefront per matrix
  auto dma_keys = [&](int pair, int t0, int t1, uint16_t* st) {
    const uint16_t* kb = a.k + (size_t)pair * a.Sk * D;
    const uint16_t* vb = a.v + (size_t)pair * a.Sk * D;
#pragma unroll
    for (int q = 0; q < DJ; ++q) {
      const int run = w * DJ + q;                 // 64-chunk run of the tile
      if (run * 64 < TCH) {
        const int pos = run * 64 + lane;
        const int r = pos / CPR, pc = pos % CPR;
        const int c = pc ^ (swz<D>(r) & (CPR - 1));
        const size_t off = (size_t)imin(t0 + r, t1 - 1) * D + 8 * c;
        const uint16_t* dst = st + run * 64 * 8;
        if constexpr (KS) {   // each key is read once per item
          lds_dma16_nt(kb + off, dst);
          lds_dma16_nt(vb + off, dst + TE);
        } else {
          lds_dma16(kb + off, dst);
          lds_dma16(vb + off, dst + TE);
        }
      }
    }
  };
  auto dma = [&](const Geom& gm, int j, uint16_t* st) {
    int t0, t1;
    tile_in(gm, j, t0, t1);
    dma_keys(gm.pair, t0, t1, st);
  };
  // All but the newest tile's DMA loads (and every LDS access) have landed;
  // then the workgroup barrier (without the fence of __syncthreads, which
  // would also wait for the newest loads).
  // Every outstanding load (DMA included) has landed, then the barrier.
  // __syncthreads() would not wait for the DMA loads: the compiler does not
  // know about them.
  auto drain = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto settle = [&]() {
    constexpr int N = 2 * DJ;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // boundary tile j held in stage st: per-wavefront FULL / EMPTY / PARTIAL
  auto slow_tile = [&](const uint16_t* st, int j) {
    int t0, t1;
    tile(j, t0, t1);
    Span A[NQB], C[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      A[qb] = Span{0, 0};
      C[qb] = Span{0, 0};
      if (valid[qb]) row_spans(a.mode, VARLEN ? cur.L : a.L, a.n, a.blk, qrow[qb], A[qb], C[qb]);
    }
#pragma unroll 1
    for (int sub = KS ? kg : 0; sub < (KS ? kg + 1 : 2); ++sub) {
      const int e0 = t0 + 32 * sub, e1 = imin(t1, e0 + 32);
      if (e0 >= e1) break;
      bool full = true, empty = true;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int c = inside(A[qb], e0, e1) + inside(C[qb], e0, e1);
        full &= !valid[qb] || (e1 - e0 == 32 && c == 32);
        empty &= !valid[qb] || c == 0;
      }
      if (__all(empty)) continue;
      f32x16 s[NQB];
      qk_sub(st, sub, s);
      if (!__all(full)) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int jj = e0 + 8 * (i >> 2) + 4 * hb + (i & 3);
            const bool ok = (jj < e1) & (in_span(A[qb], jj) | in_span(C[qb], jj));   // a select, no branches
            s[qb][i] = ok ? s[qb][i] : -INFINITY;
          }
        }
      }
      bf16x8 pb[NQB][2];
      float alpha[NQB];
      softmax_sub(s, pb, alpha);
      rescale(alpha);
      pv_sub(st, sub, pb);
    }
  };

  // ---- epilogue of the current item: lane (ql, hb) holds
  // d = 32*dt + 8*(i/4) + 4*hb + (i%4)
  auto finish = [&]() {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float l_tot = half_sum(l_run[qb]);
      if (!valid[qb]) continue;
      if (a.n_splits == 1) {
        const float inv = 1.f / l_tot;
        if (LSE && hb == 0)
          a.lse[(size_t)(b * a.Hq + head[qb]) * a.Sq + qrow[qb]] = (m_run[qb] * sl2 + __log2f(l_tot)) * 0.6931471805599453f;
        uint16_t* op = a.out + ((size_t)(b * a.Hq + head[qb]) * a.Sq + qrow[qb]) * D + 4 * hb;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            u32x2 pk;
            pk[0] = pack_bf16x2(o[qb][dt][4 * i4] * inv, o[qb][dt][4 * i4 + 1] * inv);
            pk[1] = pack_bf16x2(o[qb][dt][4 * i4 + 2] * inv, o[qb][dt][4 * i4 + 3] * inv);
            *(u32x2*)(op + 32 * dt + 8 * i4) = pk;
          }
        }
      } else {
        const size_t rows = (size_t)a.B * a.Hq * a.n;
        const size_t row = (size_t)(b * a.Hq + head[qb]) * a.n + qrow[qb];
        float* po = a.part_o + ((size_t)cur.split * rows + row) * D + 4 * hb;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 x{o[qb][dt][4 * i4], o[qb][dt][4 * i4 + 1], o[qb][dt][4 * i4 + 2], o[qb][dt][4 * i4 + 3]};
            *(f32x4*)(po + 32 * dt + 8 * i4) = x;
          }
        }
        if (hb == 0) {
          float* pm = a.part_ml + ((size_t)cur.split * rows + row) * 2;
          pm[0] = m_run[qb] == -INFINITY ? -INFINITY : m_run[qb] * sl2;
          pm[1] = l_tot;
        }
      }
    }
  };

  if constexpr (STAGES == 2) {
    // One item per workgroup, double-buffered: tile i+1 is stored and tile
    // i+2 fetched after tile i.
    begin_item(blockIdx.x);
    reset_acc();
    const int nf = cur.nf, nt = cur.nt;
    if (nt > 0) {
      fetch(0);
      lstore(smem);
      fetch(1);
      __syncthreads();
      int st = 0;
#pragma unroll 1
      for (int i = 0; i < nf; ++i) {
        const uint16_t* cu = smem + st * STAGE;
        f32x16 sa[NQB], sb[NQB];
        bf16x8 pb[NQB][2];
        qk_sub(cu, 0, sa);
        qk_sub(cu, 1, sb);
        softmax_fast(sa, pb);
        pv_sub(cu, 0, pb);
        softmax_fast(sb, pb);
        pv_sub(cu, 1, pb);
        lstore(smem + (st ^ 1) * STAGE);
        fetch(i + 2);
        __syncthreads();
        st ^= 1;
      }
#pragma unroll 1
      for (int i = nf; i < nt; ++i) {
        slow_tile(smem + st * STAGE, i);
        lstore(smem + (st ^ 1) * STAGE);
        fetch(i + 2);
        __syncthreads();
        st ^= 1;
      }
    }
    finish();
  } else if constexpr (KS) {
    // ---- DECODE/CAUSAL, one item per workgroup.  A 5-stage DMA ring keeps
    // up to four 64-key tiles in flight; wavefront group kg computes the
    // 32-key half kg of every tile for all the item's query slots, and the
    // two groups merge their (max, sum, O) through LDS at the end.
    begin_item(blockIdx.x);
    reset_acc();
    const int nf = cur.nf, nt = cur.nt;
    auto stq = [&](int j) { return smem + (j % STAGES) * STAGE; };
    // Tile j visible to every wavefront, given that tiles 0 .. issued-1 have
    // been issued: the (up to three) tiles issued after j stay in flight.
    auto settle_for = [&](int j, int issued) {
      const int newer = imin(STAGES - 2, imax(0, issued - 1 - j));
      constexpr int T = 2 * DJ;                // DMA loads of one tile per wavefront
      asm volatile("" ::: "memory");
      if (newer >= 3)
        __builtin_amdgcn_s_waitcnt(((3 * T) & 15) | (7 << 4) | (((3 * T) >> 4) << 14));
      else if (newer == 2)
        __builtin_amdgcn_s_waitcnt(((2 * T) & 15) | (7 << 4) | (((2 * T) >> 4) << 14));
      else if (newer == 1)
        __builtin_amdgcn_s_waitcnt((T & 15) | (7 << 4) | ((T >> 4) << 14));
      else
        __builtin_amdgcn_s_waitcnt(7 << 4);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    int issued = 0;
    for (; issued < STAGES - 1 && issued < nt; ++issued) dma(cur, issued, stq(issued));
    drain();   // the Q operands and the first tiles
    // Tile i + 4 goes into the stage of tile i - 1, which every wavefront
    // finished before the last barrier.
#pragma unroll 1
    for (int i = 0; i < nf; ++i) {
      if (issued < nt) dma(cur, issued, stq(issued)), ++issued;
      f32x16 sc[NQB];
      bf16x8 pb[NQB][2];
      qk_sub(stq(i), kg, sc);
      softmax_fast(sc, pb);
      pv_sub(stq(i), kg, pb);
      settle_for(i + 1, issued);
    }
#pragma unroll 1
    for (int i = nf; i < nt; ++i) {
      if (issued < nt) dma(cur, issued, stq(issued)), ++issued;
      slow_tile(stq(i), i);
      settle_for(i + 1, issued);
    }
    drain();
    // group 1 hands its state to group 0 through the (drained) ring
    float* xf = reinterpret_cast<float*>(smem);
    constexpr int NE = DT * 16 + 2;
    auto xi = [&](int qb, int e) { return ((wq * NQB + qb) * NE + e) * 64 + lane; };
    static_assert(NWQ * NQB * NE * 64 * 4 <= STAGES * STAGE * 2, "merge buffer exceeds the ring");
    if (kg == 1) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) xf[xi(qb, dt * 16 + i)] = o[qb][dt][i];
        xf[xi(qb, DT * 16)] = m_run[qb];
        xf[xi(qb, DT * 16 + 1)] = l_run[qb];
      }
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float mb = xf[xi(qb, DT * 16)], lb = xf[xi(qb, DT * 16 + 1)];
        const float M = fmaxf(m_run[qb], mb);
        const float fa = m_run[qb] == -INFINITY ? 0.f : exp2_fast((m_run[qb] - M) * sl2);
        const float fb = mb == -INFINITY ? 0.f : exp2_fast((mb - M) * sl2);
        l_run[qb] = l_run[qb] * fa + lb * fb;
        m_run[qb] = M;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[qb][dt][i] = o[qb][dt][i] * fa + xf[xi(qb, dt * 16 + i)] * fb;
      }
      finish();
    }
  } else {
    // ---- persistent DMA-fed walk.  The workgroup takes items round by
    // round, in snake order (within its XCD when pairs_per_xcd > 0), so
    // every workgroup gets a similar mix of heavy and light query tiles.
    // One DMA stream runs over the tiles of all its items: stage s % 4 holds
    // stream tile s, filled three tiles ahead, so the first tiles of the
    // next item load while the current one finishes.
    const int GR = gridDim.x, wg = blockIdx.x;
    auto item_of = [&](int r) -> int {
      if (a.pairs_per_xcd > 0) {
        const int NL = GR >> 3, wl = wg >> 3;
        const int i = r * NL + ((r & 1) ? NL - 1 - wl : wl);
        return i < (a.n_items >> 3) ? i * 8 + (wg & 7) : -1;
      }
      const int i = r * GR + ((r & 1) ? GR - 1 - wg : wg);
      return i < a.n_items ? i : -1;
    };
    // prefetch cursor: tile c_j of item round c_r (geometry cg)
    Geom cg{};
    int c_r = -1, c_j = 0;
    bool c_live = true;
    auto c_next_item = [&]() {
      for (;;) {
        const int idx = item_of(++c_r);
        if (idx < 0) {
          c_live = false;
          return;
        }
        geom(idx, cg);
        c_j = 0;
        if (cg.nt > 0) return;
      }
    };
    c_next_item();
    // Returns whether a tile was issued.  The wait at the end of a tile step
    // leaves only the newest tile in flight, so the tile the next step reads
    // must not be the newest: every item ends with a boundary tile (see the
    // geometry), fast steps are always followed by at least one more issued
    // tile, and a boundary step that finds the stream exhausted waits for
    // every load before it reads its tile.
    auto c_issue = [&](uint16_t* st) -> bool {
      if (!c_live) return false;
      dma(cg, c_j, st);
      if (++c_j == cg.nt) c_next_item();
      return true;
    };
    int sp = 0;   // stream position of the current item's first tile
    auto stg = [&](int i) { return smem + ((sp + i) & 3) * STAGE; };
    c_issue(stg(0));
    c_issue(stg(1));
    c_issue(stg(2));
    drain();
#pragma unroll 1
    for (int r = 0;; ++r) {
      const int idx = item_of(r);
      if (idx < 0) break;
      begin_item(idx);
      // The Q operands land here, once per item.  Left to the compiler, the
      // wait for them sits at their first use inside the tile loop, where
      // vmcnt(0) would also wait for the DMA loads just issued three tiles
      // ahead (the counter retires in order and counts those loads too).
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0xF << 8));   // vmcnt(0) only
      reset_acc();
      const int nf = cur.nf, nt = cur.nt;
      if (nt > 0) {
        // Per fast tile: the MFMAs of the next subtile's scores are issued
        // with the softmax of the current one; the scores of subtile 0 of
        // the stream tile after the last fast one are computed and dropped,
        // so the fast body has no branch besides the rare rescale.
        f32x16 sa[NQB], sb[NQB];
        if (nf > 0) qk_sub(stg(0), 0, sa);
#pragma unroll 1
        for (int i = 0; i < nf; ++i) {
          const uint16_t* cu = stg(i);
          c_issue(stg(i + 3));
          bf16x8 pb[NQB][2];
          qk_sub(cu, 1, sb);
          softmax_fast(sa, pb);
          pin(pb);
          pv_sub(cu, 0, pb);
          qk_sub(stg(i + 1), 0, sa);
          softmax_fast(sb, pb);
          pin(pb);
          pv_sub(cu, 1, pb);
          settle();
        }
#pragma unroll 1
        for (int i = nf; i < nt; ++i) {
          if (!c_issue(stg(i + 3))) drain();
          slow_tile(stg(i), i);
          settle();
        }
        sp += nt;
      }
      finish();
    }
    drain();   // the last loads and stores land before exit
  }
}

// Fixed-order log-sum-exp merge of the key splits of DECODE/CAUSAL calls.
template <int D, int SB>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           uint16_t* __restrict__ out, float* __restrict__ lse,
                                                           long long rows, int n_splits) {
  constexpr int TPR = D / 4;  // threads per row, 4 elements each
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = t / TPR;
  const int c = (int)(t - row * TPR) * 4;
  if (row >= rows) return;
  // Splits in batches of SB (the host picks the smallest power of two that
  // covers the splits, at most 32) whose loads all go out before any
  // arithmetic; within a batch the weights are taken against the batch's
  // maximum, and the running sums are rescaled when a batch raises it.
  // Split 0 always holds keys, so M is finite after the first batch.
  float M = -INFINITY, l = 0.f;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_splits; s0 += SB) {
    f32x2 ml[SB];
    f32x4 x[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const size_t sr = (size_t)imin(s0 + j, n_splits - 1) * rows + row;
      ml[j] = *(const f32x2*)(part_ml + sr * 2);
      x[j] = *(const f32x4*)(part_o + sr * D + c);
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < SB; ++j)
      if (s0 + j < n_splits) Mb = fmaxf(Mb, ml[j][0]);
    if (Mb == -INFINITY) continue;
    if (M != -INFINITY && Mb != M) {
      const float a = exp2_fast(M - Mb);
      l *= a;
      acc *= a;
    }
    M = Mb;
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      if (s0 + j >= n_splits || ml[j][0] == -INFINITY) continue;
      const float wgt = exp2_fast(ml[j][0] - M);
      l += wgt * ml[j][1];
      acc += wgt * x[j];
    }
  }
  const float inv = 1.f / l;
  if (lse != nullptr && c == 0) lse[row] = (M + __log2f(l)) * 0.6931471805599453f;
  u32x2 pk;
  pk[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(u32x2*)(out + row * D + c) = pk;
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

int attn_make_plan(int B, int Hq, int Hkv, int L, int d, int block, int mode, AttnPlan* p,
                   const char** why) {
  AttnPlan x{};
  x.mode = mode;
  x.B = B;
  x.Hq = Hq;
  x.Hkv = Hkv;
  x.G = Hq / Hkv;
  x.L = L;
  x.blk = block;
  x.d = d;
  x.n_splits = 1;
  if (mode == kHybrid) {
    x.n = 2 * L;
    x.Sq = x.Sk = 2 * L;
    x.nw = L >= 256 ? 8 : 4;
    x.stages = L >= 256 ? 4 : 2;
    x.qpw = 32;
    const int slots_half = (x.nw / 2) * x.qpw;
    if (x.G > slots_half) {
      *why = "Hq/Hkv larger than the query slots of half a workgroup";
      return 2;
    }
    x.rows_per_wg = slots_half / x.G;
    x.n_qtiles = (L + x.rows_per_wg - 1) / x.rows_per_wg;
  } else {
    x.n = block;
    x.Sq = block;
    x.Sk = L;
    // short query blocks over long caches (decode, verify): the split-key
    // ring (one 8-wavefront workgroup per item, two groups of 4 over the
    // same slots); long query ranges (prefill): the persistent walk
    x.nw = 8;
    x.stages = block >= 128 ? 4 : 5;
    x.qpw = 32;
    const int slots = (x.stages == 5 ? x.nw / 2 : x.nw) * x.qpw;
    if (x.G > slots) {
      *why = "Hq/Hkv larger than the query slots of a workgroup";
      return 2;
    }
    x.rows_per_wg = slots / x.G;
    x.n_qtiles = (block + x.rows_per_wg - 1) / x.rows_per_wg;
    // Split the keys when (batch x kv head x query tile) alone cannot give
    // every CU a workgroup (one resident split-key workgroup per CU at
    // d = 128, 256 CUs); each split keeps at least 4 key tiles.
    const long long items = (long long)B * Hkv * x.n_qtiles;
    const long long target = x.stages == 5 ? 256 : 512;
    int splits = (int)((target + items - 1) / items);
    const int max_splits = (L + 4 * kBN - 1) / (4 * kBN);
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    int sk = (L + splits - 1) / splits;
    sk = (sk + kBN - 1) / kBN * kBN;
    x.split_keys = sk;
    x.n_splits = (L + sk - 1) / sk;
  }
  if (x.n_splits == 1) x.split_keys = x.Sk;
  const long long pairs = (long long)B * Hkv;
  x.pairs_per_xcd = (x.n_splits == 1 && pairs % 8 == 0) ? (int)(pairs / 8) : 0;
  x.grid = pairs * x.n_qtiles * x.n_splits;
  if (x.grid > 0x7fffffffLL) {
    *why = "grid too large";
    return 2;
  }
  x.ws_bytes = 0;
  if (x.n_splits > 1)
    x.ws_bytes = (size_t)x.n_splits * (size_t)B * Hq * x.n * ((size_t)d * 4 + 8);
  *p = x;
  return 0;
}

template <int D, int NW, int QPW, int STAGES>
static hipError_t launch_main(const AttnArgs& a, long long grid, hipStream_t st) {
  // per-row key counts and the log-sum-exp output are compiled in only where
  // asked for (the API never asks for both at once)
  if (a.kv_len != nullptr)
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, QPW, STAGES, true, false>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       st, a);
  else if (a.lse != nullptr)
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, QPW, STAGES, false, true>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, QPW, STAGES, false, false>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       st, a);
  return hipGetLastError();
}

// Compute units of the current device (the persistent grid size), queried
// once per device; concurrent first calls store the same value.
static int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D>
static hipError_t launch_d(const AttnPlan& p, AttnArgs a, hipStream_t st) {
  hipError_t e;
  if (p.stages == 4) {
    // persistent: as many workgroups as fit at once (by LDS: one per compute
    // unit at d = 128, two below) walk their shares of the items
    const long long slots = (long long)device_cus() * (D == 128 ? 1 : 2);
    long long grid = p.grid < slots ? p.grid : slots;
    if (a.pairs_per_xcd > 0 && grid % 8 != 0) a.pairs_per_xcd = 0;
    e = launch_main<D, 8, 32, 4>(a, grid, st);
  } else if (p.stages == 5) {
    e = launch_main<D, 8, 32, 5>(a, p.grid, st);
  } else {
    e = launch_main<D, 4, 32, 2>(a, p.grid, st);
  }
  if (e != hipSuccess || p.n_splits == 1) return e;
  const long long rows = (long long)p.B * p.Hq * p.n;
  const long long threads = rows * (D / 4);
  const long long blocks = (threads + 255) / 256;
  const int n = p.n_splits;
  if (n <= 2)
    hipLaunchKernelGGL((attn_combine_kernel<D, 2>), dim3((unsigned)blocks), dim3(256), 0, st, a.part_o, a.part_ml,
                       a.out, a.lse, rows, n);
  else if (n <= 4)
    hipLaunchKernelGGL((attn_combine_kernel<D, 4>), dim3((unsigned)blocks), dim3(256), 0, st, a.part_o, a.part_ml,
                       a.out, a.lse, rows, n);
  else if (n <= 8)
    hipLaunchKernelGGL((attn_combine_kernel<D, 8>), dim3((unsigned)blocks), dim3(256), 0, st, a.part_o, a.part_ml,
                       a.out, a.lse, rows, n);
  else if (n <= 16)
    hipLaunchKernelGGL((attn_combine_kernel<D, 16>), dim3((unsigned)blocks), dim3(256), 0, st, a.part_o, a.part_ml,
                       a.out, a.lse, rows, n);
  else
    hipLaunchKernelGGL((attn_combine_kernel<D, 32>), dim3((unsigned)blocks), dim3(256), 0, st, a.part_o, a.part_ml,
                       a.out, a.lse, rows, n);
  return hipGetLastError();
}

hipError_t attn_launch(const AttnPlan& p, const void* q, const void* k, const void* v, void* out,
                       float* lse, const int32_t* kv_len, void* ws, hipStream_t st) {
  AttnArgs a{};
  a.lse = lse;
  a.kv_len = kv_len;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.out = (uint16_t*)out;
  if (p.n_splits > 1) {
    const size_t rows = (size_t)p.B * p.Hq * p.n;
    a.part_o = (float*)ws;
    a.part_ml = (float*)((char*)ws + (size_t)p.n_splits * rows * p.d * 4);
  }
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.mode = p.mode;
  a.L = p.L;
  a.n = p.n;
  a.blk = p.blk;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.rows_per_wg = p.rows_per_wg;
  a.n_qtiles = p.n_qtiles;
  a.n_splits = p.n_splits;
  a.split_keys = p.split_keys;
  a.pairs_per_xcd = p.pairs_per_xcd;
  a.n_items = (int)p.grid;
  a.sl2 = 1.4426950408889634f / sqrtf((float)p.d);
  (void)hipGetLastError();
  switch (p.d) {
    case 32: return launch_d<32>(p, a, st);
    case 64: return launch_d<64>(p, a, st);
    default: return launch_d<128>(p, a, st);
  }
}

}  // namespace bda
