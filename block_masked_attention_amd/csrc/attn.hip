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
#include <type_traits>

#include "common.h"
#include "attn_index.h"
#include "geometry.h"
#include "internal.h"
#include "tiles.h"

namespace bda {

struct AttnArgs : AttnIndex {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* part_o;    // [split][B*Hq*n][D] unnormalised partial outputs
  float* part_ml;   // [split][B*Hq*n][2] (running max in log2 units, row sum)
  float sl2;        // log2(e) / sqrt(D)
  const int32_t* kv_len;   // optional [B] (DECODE/CAUSAL): keys of each batch row, clamped to [n, L]
  float* lse;       // optional [B*Hq*Sq]: natural-log log-sum-exp of each row's scores
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
  constexpr int KT = 2 * TE;                  // bytes of one K (or V) tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGES * STAGE];
  // persistent walk: where wavefronts 4..7 stage an item's O (waves 0..3 use
  // the ring stage of the item's last tile)
  __shared__ __attribute__((aligned(16))) uint16_t oext[STAGES == 4 ? 4 * 32 * D : 8];
  // K tiles of the ring stages first, then the V tiles (all K operand reads
  // stay below 64 KB of the LDS base, within the reads' immediate offset)
  char* const sm = reinterpret_cast<char*>(smem);
  auto kst = [&](int stage) { return sm + stage * KT; };
  auto vst = [&](int stage) { return sm + (STAGES + stage) * KT; };

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

  // ---- work items and their key ranges (attn_index.h)
  constexpr int WALK = STAGES == 4 ? kWalkPersistent : (STAGES == 5 ? kWalkSplit : kWalkRegs);
  auto geom = [&](int idx, Geom& gm) { attn_geom(a, WALK, VARLEN ? a.kv_len : nullptr, idx, gm); };
  auto tile_in = [&](const Geom& gm, int j, int& t0, int& t1) { attn_tile(gm, j, t0, t1); };

  // ---- the item being computed
  Geom cur{};
  int b = 0, g = 0;
  const uint16_t* kbase = a.k;
  const uint16_t* vbase = a.v;
  int qrow[NQB], head[NQB];
  bool valid[NQB];
  bf16x8 qreg[NQB][KSTEPS];
  // The Q operands of the current item's slots (lane (ql, hb) holds d =
  // 16*ks + 8*hb + 0..7); the compiler places the wait for them.
  auto load_q = [&]() {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const uint16_t* qp = a.q + attn_q_elem<D>(a, b, head[qb], qrow[qb]) + 8 * hb;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4 x = valid[qb] ? *(const u32x4*)(qp + 16 * ks) : u32x4{0, 0, 0, 0};
        qreg[qb][ks] = __builtin_bit_cast(bf16x8, x);
      }
    }
  };
  // Switch to item idx: its geometry, my query slots (one per column block)
  // and, with with_q, their Q operands.
  auto begin_item = [&](int idx, bool with_q = true) {
    geom(idx, cur);
    b = cur.pair / a.Hkv;
    g = cur.pair - b * a.Hkv;
    const size_t kvoff = attn_kv_elem<D>(a, cur.pair, 0);
    kbase = a.k + kvoff;
    vbase = a.v + kvoff;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      if (a.mode == kHybrid) {   // waves [0, NW/2) hold the noisy rows, the rest the clean ones
        const int per_half = NW / 2;
        const int half = w / per_half;
        valid[qb] = attn_slot(a, half, ((w - half * per_half) * NQB + qb) * 32 + ql, cur.qt, g, qrow[qb], head[qb]);
      } else {
        valid[qb] = attn_slot(a, 0, (wq * NQB + qb) * 32 + ql, cur.qt, g, qrow[qb], head[qb]);
      }
    }
    if (with_q) load_q();
  };
  // The Q operands of the current item's slots, loaded and waited for in
  // one statement (the wait also covers every load issued before it).  A
  // slot without a row reads the first row of Q and keeps zeros.
  auto load_q_wait = [&]() {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const uint16_t* qp = a.q + (valid[qb] ? attn_q_elem<D>(a, b, head[qb], qrow[qb]) + 8 * hb : 0);
      u32x4 x[KSTEPS];
      load_x16_stride32_wait<KSTEPS>(qp, x);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        qreg[qb][ks] = __builtin_bit_cast(bf16x8, valid[qb] ? x[ks] : u32x4{0, 0, 0, 0});
    }
  };

  // Lane-constant LDS byte offsets of the operand reads (fwd_off).  K: key
  // 32 sub + ql, chunk 2 ks + hb, at kl[ks % 2] + 256 (ks - ks % 2) + 64 D
  // sub.  V^T: lane (gi = lane / 16, j = lane % 16) reads 4 values at column
  // 32 dt + 16 (gi % 2) + 4 (j % 4) of key 32 sub + 16 kk + 4 hb + j / 4
  // (lo) and of the key 8 further (hi), at vl (vh) + 512 dt + 32 D (2 sub +
  // kk).
  const int kl0 = fwd_off<D>(ql, hb), kl1 = fwd_off<D>(ql, 2 + hb);
  int vl, vh;
  {
    const int j = lane & 15, gi = lane >> 4;
    const int r = 4 * hb + (j >> 2), c = 2 * (gi & 1) + ((j & 3) >> 1);
    vl = fwd_off<D>(r, c) + 8 * (j & 1);
    vh = fwd_off<D>(r + 8, c) + 8 * (j & 1);
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
  auto lstore = [&](int stage) {
#pragma unroll
    for (int j = 0; j < CU; ++j) {
      const int ch = tid + j * NT;
      if (TCH % NT == 0 || ch < TCH) {
        const int off = fwd_off<D>(ch / CPR, ch % CPR);
        *(u32x4*)(kst(stage) + off) = kreg[j];
        *(u32x4*)(vst(stage) + off) = vreg[j];
      }
    }
  };
  // S^T = K Q^T for one 32-key subtile of a stage, all column blocks
  auto qk_sub = [&](int stage, int sub, f32x16 (&s)[NQB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) s[qb] = f32x16{};
    const char* kr = kst(stage) + sub * 64 * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const bf16x8 kop = *(const bf16x8*)(kr + 256 * (ks & ~1) + ((ks & 1) ? kl1 : kl0));
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[qb][ks], s[qb], 0, 0, 0);
    }
  };
  f32x16 o[NQB][DT];
  // O^T += V^T P^T for one 32-key subtile (two 16-key MFMA k-steps)
  auto pv_sub = [&](int stage, int sub, const bf16x8 (&pb)[NQB][2]) __attribute__((always_inline)) {
    // the two lane bases of this stage, formed once; every read of the
    // subtile is one of them plus an immediate offset
    unsigned b_lo = lds_addr(vst(stage)) + vl, b_hi = lds_addr(vst(stage)) + vh;
    asm volatile("" : "+v"(b_lo), "+v"(b_hi));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const unsigned vt = (2 * sub + kk) * 32 * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const s16x4 lo = lds_read_tr_at(b_lo + vt + dt * 512);
        const s16x4 hi = lds_read_tr_at(b_hi + vt + dt * 512);
        const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          o[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[qb][kk], o[qb][dt], 0, 0, 0);
      }
    }
  };

  // The same two products with their LDS operand reads split off, so the
  // fast walk can issue the reads of a subtile well before its MFMAs (and
  // the V reads ahead of the softmax they do not depend on).
  auto k_load = [&](int stage, int sub, bf16x8 (&kop)[KSTEPS]) __attribute__((always_inline)) {
    const char* kr = kst(stage) + sub * 64 * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      kop[ks] = *(const bf16x8*)(kr + 256 * (ks & ~1) + ((ks & 1) ? kl1 : kl0));
  };
  auto qk_mma = [&](const bf16x8 (&kop)[KSTEPS], f32x16 (&s)[NQB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qreg[qb][ks], s[qb], 0, 0, 0);
  };
  auto v_load = [&](int stage, int sub, bf16x8 (&vop)[2][DT]) __attribute__((always_inline)) {
    unsigned b_lo = lds_addr(vst(stage)) + vl, b_hi = lds_addr(vst(stage)) + vh;
    asm volatile("" : "+v"(b_lo), "+v"(b_hi));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const unsigned vt = (2 * sub + kk) * 32 * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const s16x4 lo = lds_read_tr_at(b_lo + vt + dt * 512);
        const s16x4 hi = lds_read_tr_at(b_hi + vt + dt * 512);
        vop[kk][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  auto pv_mma = [&](const bf16x8 (&vop)[2][DT], const bf16x8 (&pb)[NQB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          o[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[kk][dt], pb[qb][kk], o[qb][dt], 0, 0, 0);
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
  // expo_fast is the branch-free part, fix_fast the check, the rare redo and
  // the update of l.
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  auto expo = [&](const f32x16 (&s)[NQB], bf16x8 (&pb)[NQB][2], float (&ls)[NQB], int qb, float nb)
      __attribute__((always_inline)) {
    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
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
  auto expo_fast = [&](const f32x16 (&s)[NQB], bf16x8 (&pb)[NQB][2], float (&ls)[NQB])
      __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) expo(s, pb, ls, qb, -m_run[qb] * sl2);
  };
  auto fix_fast = [&](const f32x16 (&s)[NQB], bf16x8 (&pb)[NQB][2], float (&ls)[NQB])
      __attribute__((always_inline)) {
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) bad |= !(ls[qb] < 256.f);
    if (__builtin_expect(__any(bad), 0)) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float mt = s[qb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[qb][i]);
        const float m_use = fmaxf(m_run[qb], half_max(mt));
        const float alpha = exp2_fast((m_run[qb] - m_use) * sl2);   // 0 while the max is unset
        expo(s, pb, ls, qb, -m_use * sl2);
        m_run[qb] = m_use;
        l_run[qb] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[qb][dt] *= alpha;
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) l_run[qb] += ls[qb];
  };
  auto softmax_fast = [&](const f32x16 (&s)[NQB], bf16x8 (&pb)[NQB][2]) __attribute__((always_inline)) {
    float ls[NQB];
    expo_fast(s, pb, ls);
    fix_fast(s, pb, ls);
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
  // Tile [t0, t1) of pair straight from global memory into an LDS stage (no
  // registers).  Wavefront w loads the 1 KB runs w*DJ + q of the K and of the
  // V tile; lane i of a run fills bytes 1024 run + 16 i of the stage, so it
  // loads the key and chunk that fwd_at names there.  The source is the
  // tile's first key row (a uniform base, in SGPRs) plus a 32-bit lane
  // offset; in a short tile, keys past t1 - 1 repeat key t1 - 1 (finite data
  // that the masks never let through).
  constexpr int DJ = TCH >= NT ? TCH / NT : 1;   // DMA loads per wavefront per matrix
  constexpr bool ALL_RUNS = TCH / 64 >= NW * DJ;   // every wavefront loads DJ runs (D >= 64)
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
  // n = keys of the tile (1..64) starting at kb / vb
  auto dma_at = [&](const uint16_t* kb, const uint16_t* vb, int n, int stage) __attribute__((always_inline)) {
    const unsigned mk = (unsigned)(uintptr_t)kst(stage), mv = (unsigned)(uintptr_t)vst(stage);
    if (n == kBN) {
#pragma unroll
      for (int q = 0; q < DJ; ++q) {
        const int run = wu * DJ + q;
        if (ALL_RUNS || run * 64 < TCH) {
          if constexpr (KS) {   // each key is read once per item
            lds_dma16_sa_nt(kb, d_off[q], mk + run * 1024);
            lds_dma16_sa_nt(vb, d_off[q], mv + run * 1024);
          } else {
            lds_dma16_sa(kb, d_off[q], mk + run * 1024);
            lds_dma16_sa(vb, d_off[q], mv + run * 1024);
          }
        }
      }
    } else {
      const int last = n - 1;
#pragma unroll
      for (int q = 0; q < DJ; ++q) {
        const int run = wu * DJ + q;
        if (ALL_RUNS || run * 64 < TCH) {
          const unsigned off = d_off[q] - (unsigned)((d_row[q] - imin(d_row[q], last)) * 2 * D);
          if constexpr (KS) {
            lds_dma16_sa_nt(kb, off, mk + run * 1024);
            lds_dma16_sa_nt(vb, off, mv + run * 1024);
          } else {
            lds_dma16_sa(kb, off, mk + run * 1024);
            lds_dma16_sa(vb, off, mv + run * 1024);
          }
        }
      }
    }
  };
  auto dma_keys = [&](int pair, int t0, int t1, int stage) __attribute__((always_inline)) {
    const size_t row0 = attn_kv_elem<D>(a, pair, t0);
    dma_at(a.k + row0, a.v + row0, t1 - t0, stage);
  };
  auto dma = [&](const Geom& gm, int j, int stage) __attribute__((always_inline)) {
    int t0, t1;
    tile_in(gm, j, t0, t1);
    dma_keys(gm.pair, t0, t1, stage);
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
  auto slow_tile = [&](int st, int j) {
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
  // d = 32*dt + 8*(i/4) + 4*hb + (i%4).  The persistent walk (one output,
  // no key split) sends O through oreg, its wavefront's 32 x D region of
  // LDS: written in the accumulator layout with the 16-byte chunks of a row
  // XOR-swizzled by the row, read back 16 bytes per lane so that each store
  // writes whole rows (D / 8 lanes per row) instead of 16 bytes of 32 rows.
  char* oreg = nullptr;
  // finish() writes the 32-column tiles [fin_lo, fin_hi) of O and, if
  // fin_rows, the per-row statistics (log-sum-exp, split max and sum): the
  // split-key walk's two wavefront groups each write half of every row.
  int fin_lo = 0, fin_hi = DT;
  bool fin_rows = true;
  auto finish = [&]() {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float l_tot = half_sum(l_run[qb]);
      if (!valid[qb]) continue;
      if (a.n_splits == 1) {
        const float inv = 1.f / l_tot;
        if (LSE && fin_rows && hb == 0)
          a.lse[attn_q_row(a, b, head[qb], qrow[qb])] = (m_run[qb] * sl2 + __log2f(l_tot)) * 0.6931471805599453f;
        uint16_t* op = a.out + attn_q_elem<D>(a, b, head[qb], qrow[qb]) + 4 * hb;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          if (dt < fin_lo || dt >= fin_hi) continue;
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            u32x2 pk;
            pk[0] = pack_bf16x2(o[qb][dt][4 * i4] * inv, o[qb][dt][4 * i4 + 1] * inv);
            pk[1] = pack_bf16x2(o[qb][dt][4 * i4 + 2] * inv, o[qb][dt][4 * i4 + 3] * inv);
            if constexpr (WALK == kWalkPersistent) {
              const int c = 4 * dt + i4;   // 16-byte chunk of the row
              *(u32x2*)(oreg + ql * (2 * D) + ((c ^ (ql & (CPR - 1))) << 4) + 8 * hb) = pk;
            } else {
              *(u32x2*)(op + 32 * dt + 8 * i4) = pk;
            }
          }
        }
      } else {
        const size_t prow = attn_part_row(a, cur.split, b, head[qb], qrow[qb]);
        float* po = a.part_o + attn_part_elem<D>(a, cur.split, b, head[qb], qrow[qb]) + 4 * hb;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          if (dt < fin_lo || dt >= fin_hi) continue;
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 x{o[qb][dt][4 * i4], o[qb][dt][4 * i4 + 1], o[qb][dt][4 * i4 + 2], o[qb][dt][4 * i4 + 3]};
            *(f32x4*)(po + 32 * dt + 8 * i4) = x;
          }
        }
        if (fin_rows && hb == 0) {
          float* pm = a.part_ml + prow * 2;
          pm[0] = m_run[qb] == -INFINITY ? -INFINITY : m_run[qb] * sl2;
          pm[1] = l_tot;
        }
      }
    }
    if constexpr (WALK == kWalkPersistent) {
      static_assert(NQB == 1 && NW == 8, "O staging: 8 wavefronts of 32 slots");
      if (a.n_splits == 1) {
        // lane (ql, either half) knows the output row of slot ql (-1: none)
        const long long rowi = valid[0] ? (long long)attn_q_row(a, b, head[0], qrow[0]) : -1;
        constexpr int RPI = 64 / CPR;   // rows per store instruction
#pragma unroll
        for (int k = 0; k < 32 / RPI; ++k) {
          const int r = k * RPI + lane / CPR, c = lane % CPR;
          const u32x4 x = *(const u32x4*)(oreg + r * (2 * D) + ((c ^ (r & (CPR - 1))) << 4));
          const long long rr = __shfl(rowi, r);
          // non-temporal: O is written once and not read here, and kept out
          // of L2 it leaves room there for the K/V tiles of this XCD's
          // (batch, kv head) pairs, which every later item re-reads
          if (rr >= 0) __builtin_nontemporal_store(x, (u32x4*)(a.out + (size_t)rr * D + 8 * c));
        }
        // every wavefront has read its O back before the next item's first
        // tile copy goes into the ring stage
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0) only
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
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
      lstore(0);
      fetch(1);
      __syncthreads();
      int st = 0;
#pragma unroll 1
      for (int i = 0; i < nf; ++i) {
        const int cu = st;
        f32x16 sa[NQB], sb[NQB];
        bf16x8 pb[NQB][2];
        qk_sub(cu, 0, sa);
        qk_sub(cu, 1, sb);
        softmax_fast(sa, pb);
        pv_sub(cu, 0, pb);
        softmax_fast(sb, pb);
        pv_sub(cu, 1, pb);
        lstore(st ^ 1);
        fetch(i + 2);
        __syncthreads();
        st ^= 1;
      }
#pragma unroll 1
      for (int i = nf; i < nt; ++i) {
        slow_tile(st, i);
        lstore(st ^ 1);
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
    begin_item(blockIdx.x, false);
    reset_acc();
    const int nf = cur.nf, nt = cur.nt;
    auto stq = [&](int j) { return j % STAGES; };
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
    // A short walk (a key split of a few tiles) sends tile 0's copy first
    // and the Q operands after it, in a statement that waits for both; tiles
    // 1 .. 3 follow, so tile 0's arithmetic starts while they load.  (Q
    // loaded the ordinary way would be waited for at its first use, and the
    // compiler, which does not count the copies, would wait there for every
    // load: vmcnt(0).)  A long walk keeps four tiles in flight from the start
    // and waits for all of them with Q: the stream, not the first tile's
    // arithmetic, is what bounds it.
    int issued = 0;
    if (nt <= 8) {
      if (nt > 0) dma(cur, 0, stq(0)), issued = 1;
      load_q_wait();
      for (; issued < STAGES - 1 && issued < nt; ++issued) dma(cur, issued, stq(issued));
      // every wavefront's share of tile 0 has landed
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      load_q();
      for (; issued < STAGES - 1 && issued < nt; ++issued) dma(cur, issued, stq(issued));
      drain();   // the Q operands and the first tiles
    }
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
    // The two groups hold (max, sum, O) of the same slots over different
    // keys.  Each hands the other the 32-column tiles of O that the other
    // keeps, with its max and sum, through the (drained) ring; each then
    // merges and writes half of every row (group kg: tiles [kg DT/2, (kg+1)
    // DT/2)).  Both form the row's max and sum from the same two operands,
    // so both normalise by the same value.  D = 32 (one tile): group 1 hands
    // everything to group 0.
    float* xf = reinterpret_cast<float*>(smem);
    constexpr int HD = DT >= 2 ? DT / 2 : DT;      // tiles a group keeps
    constexpr int NE = HD * 16 + 2;
    auto xi = [&](int g, int qb, int e) { return (((g * NWQ + wq) * NQB + qb) * NE + e) * 64 + lane; };
    static_assert(2 * NWQ * NQB * NE * 64 * 4 <= STAGES * STAGE * 2, "merge buffer exceeds the ring");
    // Tiles [t0, t0 + HD) of O go out (wave-uniform branches keep every
    // register index a constant).
    auto give_tiles = [&](int qb, int t0) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < HD; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) xf[xi(kg, qb, j * 16 + i)] = o[qb][t0 + j][i];
    };
    if (DT >= 2 || kg == 1) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        if (DT < 2 || kg == 1) give_tiles(qb, 0);
        else give_tiles(qb, DT - HD);
        xf[xi(kg, qb, HD * 16)] = m_run[qb];
        xf[xi(kg, qb, HD * 16 + 1)] = l_run[qb];
      }
    }
    __syncthreads();
    if (DT >= 2 || kg == 0) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int other = 1 - kg;
        const float mb = xf[xi(other, qb, HD * 16)], lb = xf[xi(other, qb, HD * 16 + 1)];
        const float M = fmaxf(m_run[qb], mb);
        const float fa = m_run[qb] == -INFINITY ? 0.f : exp2_fast((m_run[qb] - M) * sl2);
        const float fb = mb == -INFINITY ? 0.f : exp2_fast((mb - M) * sl2);
        l_run[qb] = l_run[qb] * fa + lb * fb;
        m_run[qb] = M;
        auto take_tiles = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
          for (int j = 0; j < HD; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[qb][t0 + j][i] = o[qb][t0 + j][i] * fa + xf[xi(other, qb, j * 16 + i)] * fb;
        };
        if (kg == 0) take_tiles(0);
        else take_tiles(DT - HD);
      }
      if constexpr (DT >= 2) {
        fin_lo = kg * HD;
        fin_hi = fin_lo + HD;
        fin_rows = kg == 0;
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
    auto item_of = [&](int r) -> int { return attn_item_of(a, GR, wg, r); };
    // Prefetch cursor: the next tile of the DMA stream, [c_t0, min(c_t0 + 64,
    // c_hi)) of key range c_reg (0: F, 1: R1, 2: R2) of item round c_r
    // (geometry cg), kept as a running key position so that a tile costs a
    // few scalar adds; c_kv is the byte offset of key c_t0 in the K (and V)
    // tensor.
    Geom cg{};
    int c_r = -1, c_reg = 0, c_t0 = 0, c_hi = 0;
    size_t c_kv = 0;
    bool c_live = true;
    // Moves to the first non-empty range at or after c_reg; false past R2.
    auto c_set = [&](const Span& sr) __attribute__((always_inline)) {
      c_t0 = sr.lo;
      c_hi = sr.hi;
      c_kv = attn_kv_elem<D>(a, cg.pair, c_t0) * 2;
    };
    auto c_range = [&]() __attribute__((always_inline)) -> bool {
      if (c_reg == 0) {
        if (cg.F.hi > cg.F.lo) return c_set(cg.F), true;
        c_reg = 1;
      }
      if (c_reg == 1) {
        if (cg.R1.hi > cg.R1.lo) return c_set(cg.R1), true;
        c_reg = 2;
      }
      if (c_reg == 2) {
        if (cg.R2.hi > cg.R2.lo) return c_set(cg.R2), true;
        c_reg = 3;
      }
      return false;
    };
    // Past the last item the cursor rests on a stand-in tile: key 0 of the
    // first (batch, kv head), one key, re-issued by every later step.
    auto c_next_item = [&]() __attribute__((always_inline)) {
      for (;;) {
        const int idx = item_of(++c_r);
        if (idx < 0) {
          c_live = false;
          c_t0 = 0;
          c_hi = 1;
          c_kv = 0;
          --c_r;
          return;
        }
        geom(idx, cg);
        c_reg = 0;
        if (cg.nt > 0 && c_range()) return;
      }
    };
    c_next_item();
    // Issues the next tile of the stream and returns whether there was one.
    // The wait at the end of a tile step leaves only the newest issue in
    // flight, and a fast step i reads tiles i and i + 1, so an issue must
    // follow tile i + 1: once the stream is exhausted a fast step issues the
    // stand-in into the stage the previous step freed, which no step reads.
    // Every item ends with a boundary tile (see the geometry), and a
    // boundary step that finds the stream exhausted issues nothing and
    // waits for every load before it reads its tile.
    auto c_issue = [&](int st, bool stand_in) __attribute__((always_inline)) -> bool {
      const bool live = c_live;
      const int t1 = imin(c_hi, c_t0 + kBN);
      if (stand_in || live) dma_at(a.k + c_kv / 2, a.v + c_kv / 2, t1 - c_t0, st);
      c_t0 += kBN;
      c_kv += (size_t)kBN * 2 * D;
      if (__builtin_expect(c_t0 >= c_hi, 0)) {
        ++c_reg;
        if (!c_range()) c_next_item();
      }
      return live;
    };
    int sp = 0;   // stream position of the current item's first tile
    auto stg = [&](int i) { return (sp + i) & 3; };
    c_issue(stg(0), false);
    c_issue(stg(1), false);
    c_issue(stg(2), false);
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
        // One half step, in a fixed instruction order: the K reads of the
        // next subtile; then per k-step its score MFMA (into sn), one pair of
        // exponentials of the current subtile's softmax (sc) and two of the
        // current subtile's V reads (independent of its softmax); then the
        // softmax check and the P V MFMAs.  The scheduling fences keep that
        // order, so every wavefront issues exponentials while its own score
        // MFMAs run.
        auto half_step = [&](int kstage, int ksub, int vstage, int vsub, f32x16 (&sn)[NQB],
                             const f32x16 (&sc)[NQB]) __attribute__((always_inline)) {
          constexpr int PP = 8 * NQB / KSTEPS;     // exponential pairs per k-step
          constexpr int VR = 2 * DT;              // V^T operands of a subtile
          bf16x8 kop[KSTEPS], vop[2][DT], pb[NQB][2];
          u32x4 pk[NQB][2];
          float l0[NQB], l1[NQB], nb[NQB], ls[NQB];
          k_load(kstage, ksub, kop);
          unsigned b_lo = lds_addr(vst(vstage)) + vl, b_hi = lds_addr(vst(vstage)) + vh;
          asm volatile("" : "+v"(b_lo), "+v"(b_hi));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            nb[qb] = -m_run[qb] * sl2;
            l0[qb] = 0.f;
            l1[qb] = 0.f;
            sn[qb] = f32x16{};
          }
          typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
          const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
              sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qreg[qb][ks], sn[qb], 0, 0, 0);
#pragma unroll
            for (int t = ks * PP; t < (ks + 1) * PP; ++t) {
              const int qb = t / 8, kk = (t % 8) / 4, e = t % 4;
              const float p0 = exp2_fast(fmaf(sc[qb][8 * kk + 2 * e], sl2, nb[qb]));
              const float p1 = exp2_fast(fmaf(sc[qb][8 * kk + 2 * e + 1], sl2, nb[qb]));
              // summed from this temporary (see softmax_fast)
              const unsigned pw = pack_bf16x2(p0, p1);
              pk[qb][kk][e] = pw;
              if (e & 1) l1[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw), one2, l1[qb], false);
              else l0[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw), one2, l0[qb], false);
            }
#pragma unroll
            for (int v = ks * VR / KSTEPS; v < (ks + 1) * VR / KSTEPS; ++v) {
              const int kk = v / DT, dt = v % DT;
              const unsigned vt = (2 * vsub + kk) * 32 * D + dt * 512;
              const s16x4 lo = lds_read_tr_at(b_lo + vt);
              const s16x4 hi = lds_read_tr_at(b_hi + vt);
              vop[kk][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            pb[qb][0] = __builtin_bit_cast(bf16x8, pk[qb][0]);
            pb[qb][1] = __builtin_bit_cast(bf16x8, pk[qb][1]);
            ls[qb] = l0[qb] + l1[qb];
          }
          fix_fast(sc, pb, ls);
          pv_mma(vop, pb);
        };
#pragma unroll 1
        for (int i = 0; i < nf; ++i) {
          const int cu = stg(i);
          c_issue(stg(i + 3), true);
          half_step(cu, 1, cu, 0, sb, sa);
          half_step(stg(i + 1), 0, cu, 1, sa, sb);
          settle();
        }
#pragma unroll 1
        for (int i = nf; i < nt; ++i) {
          if (!c_issue(stg(i + 3), false)) drain();
          slow_tile(stg(i), i);
          settle();
        }
        sp += nt;
      }
      {
        // the ring stage of the item's last tile is free until the next
        // item's first step copies into it
        const int ls = (sp - 1) & 3;
        oreg = w < 4 ? (w < 2 ? kst(ls) : vst(ls)) + (w & 1) * (KT / 2)
                     : reinterpret_cast<char*>(oext) + (w - 4) * (KT / 2);
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

long long attn_persistent_grid(const AttnPlan& p, int cus, int* pairs_per_xcd) {
  // as many workgroups as fit at once (by LDS: one per compute unit at d =
  // 128, two below) walk their shares of the items
  const long long slots = (long long)cus * (p.d == 128 ? 1 : 2);
  const long long grid = p.grid < slots ? p.grid : slots;
  *pairs_per_xcd = (p.pairs_per_xcd > 0 && grid % 8 == 0) ? p.pairs_per_xcd : 0;
  return grid;
}

void attn_fill_index(const AttnPlan& p, AttnIndex* a) {
  a->B = p.B;
  a->Hq = p.Hq;
  a->Hkv = p.Hkv;
  a->G = p.G;
  a->mode = p.mode;
  a->L = p.L;
  a->n = p.n;
  a->blk = p.blk;
  a->Sq = p.Sq;
  a->Sk = p.Sk;
  a->rows_per_wg = p.rows_per_wg;
  a->n_qtiles = p.n_qtiles;
  a->n_splits = p.n_splits;
  a->split_keys = p.split_keys;
  a->pairs_per_xcd = p.pairs_per_xcd;
  a->n_items = (int)p.grid;
}

template <int D>
static hipError_t launch_d(const AttnPlan& p, AttnArgs a, hipStream_t st) {
  hipError_t e;
  if (p.stages == 4) {
    const long long grid = attn_persistent_grid(p, device_cus(), &a.pairs_per_xcd);
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
  attn_fill_index(p, &a);
  a.sl2 = 1.4426950408889634f / sqrtf((float)p.d);
  (void)hipGetLastError();
  switch (p.d) {
    case 32: return launch_d<32>(p, a, st);
    case 64: return launch_d<64>(p, a, st);
    default: return launch_d<128>(p, a, st);
  }
}

}  // namespace bda
