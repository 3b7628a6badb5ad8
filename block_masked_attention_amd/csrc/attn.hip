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
//   O^T += V^T P^T  same MFMA, A = V^T tile (LDS), B = P straight from the
//                  S^T accumulator registers (no shuffle)
// V is staged transposed, with the keys of every 16-key group permuted
// (bits 2 and 3 of the key index swapped) so that each lane's eight P values
// and its eight V^T values name the same keys.
#include "common.h"
#include "geometry.h"
#include "internal.h"

namespace bda {

constexpr int kBN = 64;   // keys per staged tile (two 32-key MFMA subtiles)

template <int D>
struct Lds {
  static constexpr int KP = D + 8;      // K tile row pitch (elements), +16 B pad
  static constexpr int VP = kBN + 8;    // V^T tile row pitch (elements)
  static constexpr int KE = kBN * KP;
  static constexpr int VE = D * VP;
  static constexpr int STAGE = KE + VE;
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* part_o;    // [split][B*Hq*n][D] unnormalised partial outputs
  float* part_ml;   // [split][B*Hq*n][2] (running max in log2 units, row sum)
  int B, Hq, Hkv, G, mode, L, n, blk, Sq, Sk;
  int rows_per_wg, n_qtiles, n_splits, split_keys, pairs_per_xcd;
  float sl2;        // log2(e) / sqrt(D)
};

__device__ __forceinline__ bool in_span(const Span& s, int j) {
  return (unsigned)(j - s.lo) < (unsigned)(s.hi - s.lo);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;              // MFMA k-steps of Q K^T
  constexpr int DT = D / 32;                  // 32-row tiles of O^T
  constexpr int KCH = kBN * D / 8;            // 16-byte chunks of a K tile
  constexpr int KU = (KCH + NT - 1) / NT;
  constexpr int VUN = (D / 2) * (kBN / 8);    // (d pair, 8-key octet) units of a V tile
  constexpr int VU = (VUN + NT - 1) / NT;
  using S = Lds<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * S::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int ql = lane & 31;
  const int hb = lane >> 5;

  // ---- which (batch, kv head, query tile, key split) this workgroup serves
  const int P = a.B * a.Hkv;
  int pair, qt, split = 0;
  {
    const int bid = blockIdx.x;
    if (a.pairs_per_xcd > 0) {
      // Workgroups are dealt to the 8 XCDs round-robin: keep every query tile
      // of a (batch, kv head) on one XCD so its K/V stays in that L2, and
      // hand out the heaviest (latest) query tiles first.
      const int xcd = bid & 7, i = bid >> 3;
      pair = xcd * a.pairs_per_xcd + i % a.pairs_per_xcd;
      qt = a.n_qtiles - 1 - i / a.pairs_per_xcd;
    } else {
      split = bid % a.n_splits;
      const int rest = bid / a.n_splits;
      pair = rest % P;
      qt = a.n_qtiles - 1 - rest / P;
    }
  }
  const int b = pair / a.Hkv;
  const int g = pair - b * a.Hkv;

  // ---- my query slot
  int qrow = 0, head = 0, rloc = 0;
  bool valid;
  if (a.mode == kHybrid) {
    const int per_half = NW / 2;
    const int half = w / per_half;
    const int s = (w - half * per_half) * 32 + ql;
    rloc = s / a.G;
    const int hh = s - rloc * a.G;
    const int pos = qt * a.rows_per_wg + rloc;
    valid = rloc < a.rows_per_wg && pos < a.L;
    qrow = half * a.L + pos;
    head = g * a.G + hh;
  } else {
    const int s = w * 32 + ql;
    rloc = s / a.G;
    const int hh = s - rloc * a.G;
    const int r = qt * a.rows_per_wg + rloc;
    valid = rloc < a.rows_per_wg && r < a.n;
    qrow = r;
    head = g * a.G + hh;
  }
  Span A{0, 0}, C{0, 0};
  if (valid) row_spans(a.mode, a.L, a.n, a.blk, qrow, A, C);

  // ---- key ranges this workgroup walks (hull of its rows' spans)
  Span U1{0, 0}, U2{0, 0};
  if (a.mode == kHybrid) {
    const int p0 = qt * a.rows_per_wg;
    const int p1 = imin(a.L, p0 + a.rows_per_wg);
    const int e = imin(a.L, ((p1 - 1) / a.blk + 1) * a.blk);
    U1 = Span{(p0 / a.blk) * a.blk, e};     // x_t blocks of these rows
    U2 = Span{a.L, a.L + e};                // x_0 prefix they need
  } else {
    const int r1 = imin(a.n, (qt + 1) * a.rows_per_wg);
    const int hi = a.mode == kDecode ? a.L : a.L - a.n + r1;
    U1 = Span{imax(0, split * a.split_keys), imin(hi, (split + 1) * a.split_keys)};
  }
  const int n1 = U1.hi > U1.lo ? (U1.hi - U1.lo + kBN - 1) / kBN : 0;
  const int n2 = U2.hi > U2.lo ? (U2.hi - U2.lo + kBN - 1) / kBN : 0;
  const int nt = n1 + n2;

  // ---- Q operand in registers: lane (ql, hb) holds d = 16*ks + 8*hb + 0..7
  bf16x8 qreg[KSTEPS];
  {
    const uint16_t* qp = a.q + ((size_t)(b * a.Hq + head) * a.Sq + qrow) * D + 8 * hb;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 x = valid ? *(const u32x4*)(qp + 16 * ks) : u32x4{0, 0, 0, 0};
      qreg[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const size_t kvoff = (size_t)(b * a.Hkv + g) * a.Sk * D;
  const uint16_t* kbase = a.k + kvoff;
  const uint16_t* vbase = a.v + kvoff;

  u32x4 kreg[KU];
  unsigned vreg[VU][8];

  auto tile_range = [&](int i, int& t0, int& t1) {
    if (i < n1) {
      t0 = U1.lo + i * kBN;
      t1 = imin(U1.hi, t0 + kBN);
    } else {
      t0 = U2.lo + (i - n1) * kBN;
      t1 = imin(U2.hi, t0 + kBN);
    }
  };
  // Global -> registers.  Key rows at or past t1 are zero-filled so that no
  // stale LDS bits (possibly NaN) meet a zero softmax weight.
  auto gload = [&](int t0, int t1) {
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int c = tid + j * NT;
      const int row = c / (D / 8), col = c % (D / 8);
      const bool ok = c < KCH && t0 + row < t1;
      kreg[j] = ok ? *(const u32x4*)(kbase + (size_t)(t0 + row) * D + col * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = tid + j * NT;
      const int dp = u % (D / 2), oct = u / (D / 2);
      const int k0 = 16 * (oct >> 1) + 4 * (oct & 1);   // keys k0..k0+3, k0+8..k0+11
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = t0 + k0 + (e & 3) + 8 * (e >> 2);
        const bool ok = u < VUN && key < t1;
        vreg[j][e] = ok ? *(const unsigned*)(vbase + (size_t)key * D + 2 * dp) : 0u;
      }
    }
  };
  // Registers -> LDS stage: K row-major (padded), V transposed (d-major) with
  // the 8 keys of an octet landing on 8 consecutive permuted positions.
  auto lstore = [&](uint16_t* st) {
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int c = tid + j * NT;
      if (c < KCH) {
        const int row = c / (D / 8), col = c % (D / 8);
        *(u32x4*)(st + row * S::KP + col * 8) = kreg[j];
      }
    }
    uint16_t* vt = st + S::KE;
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = tid + j * NT;
      if (u < VUN) {
        const int dp = u % (D / 2), oct = u / (D / 2);
        u32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned x0 = vreg[j][2 * e], x1 = vreg[j][2 * e + 1];
          lo[e] = (x0 & 0xffffu) | (x1 << 16);
          hi[e] = (x0 >> 16) | (x1 & 0xffff0000u);
        }
        *(u32x4*)(vt + (2 * dp) * S::VP + 8 * oct) = lo;
        *(u32x4*)(vt + (2 * dp + 1) * S::VP + 8 * oct) = hi;
      }
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.sl2;

  if (nt > 0) {
    int t0, t1;
    tile_range(0, t0, t1);
    gload(t0, t1);
    lstore(smem);
  }
  __syncthreads();

  for (int it = 0; it < nt; ++it) {
    int t0, t1;
    tile_range(it, t0, t1);
    if (it + 1 < nt) {
      int u0, u1;
      tile_range(it + 1, u0, u1);
      gload(u0, u1);
    }
    const uint16_t* Ks = smem + (it & 1) * S::STAGE;
    const uint16_t* Vt = Ks + S::KE;

    // classify the two 32-key subtiles for this wavefront
    int cls[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int e0 = t0 + 32 * sub, e1 = imin(t1, e0 + 32);
      if (e0 >= e1) {
        cls[sub] = kEmpty;
      } else {
        const int c = inside(A, e0, e1) + inside(C, e0, e1);
        const bool full = !valid || (e1 - e0 == 32 && c == 32);
        const bool empty = !valid || c == 0;
        cls[sub] = __all(empty) ? kEmpty : (__all(full) ? kFull : kPartial);
      }
    }

    if (cls[0] != kEmpty || cls[1] != kEmpty) {
      f32x16 s[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        s[sub] = f32x16{};
        if (cls[sub] == kEmpty) continue;
        const uint16_t* kr = Ks + (32 * sub + ql) * S::KP + 8 * hb;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const bf16x8 kop = *(const bf16x8*)(kr + 16 * ks);
          s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[ks], s[sub], 0, 0, 0);
        }
        if (cls[sub] == kPartial) {
          const int e1 = imin(t1, t0 + 32 * sub + 32);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = t0 + 32 * sub + 8 * (i >> 2) + 4 * hb + (i & 3);
            const bool ok = j < e1 && (in_span(A, j) || in_span(C, j));
            s[sub][i] = ok ? s[sub][i] : -INFINITY;
          }
        }
      }
      // online softmax (each lane: one query, 16 of the 32 keys per subtile)
      float mt = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (cls[sub] == kEmpty) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[sub][i]);
      }
      mt = half_max(mt);
      const float m_new = fmaxf(m_run, mt);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f((m_run - m_use) * sl2);
      const float nb = -m_use * sl2;
      float ls = 0.f;
      bf16x8 pb[2][2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (cls[sub] == kEmpty) continue;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = exp2f(fmaf(s[sub][8 * kk + 2 * e], sl2, nb));
            const float p1 = exp2f(fmaf(s[sub][8 * kk + 2 * e + 1], sl2, nb));
            ls += p0 + p1;
            pk[e] = pack_bf16x2(p0, p1);
          }
          pb[sub][kk] = __builtin_bit_cast(bf16x8, pk);
        }
      }
      l_run = l_run * alpha + ls;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      }
      m_run = m_new;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (cls[sub] == kEmpty) continue;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const uint16_t* vr = Vt + ql * S::VP + 16 * (2 * sub + kk) + 8 * hb;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 vop = *(const bf16x8*)(vr + 32 * dt * S::VP);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[sub][kk], o[dt], 0, 0, 0);
          }
        }
      }
    }

    if (it + 1 < nt) lstore(smem + ((it + 1) & 1) * S::STAGE);
    __syncthreads();
  }

  // ---- epilogue: lane (ql, hb) holds d = 32*dt + 8*(i/4) + 4*hb + (i%4)
  const float l_tot = half_sum(l_run);
  if (!valid) return;
  if (a.n_splits == 1) {
    const float inv = 1.f / l_tot;
    uint16_t* op = a.out + ((size_t)(b * a.Hq + head) * a.Sq + qrow) * D + 4 * hb;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 pk;
        pk[0] = pack_bf16x2(o[dt][4 * i4] * inv, o[dt][4 * i4 + 1] * inv);
        pk[1] = pack_bf16x2(o[dt][4 * i4 + 2] * inv, o[dt][4 * i4 + 3] * inv);
        *(u32x2*)(op + 32 * dt + 8 * i4) = pk;
      }
    }
  } else {
    const size_t rows = (size_t)a.B * a.Hq * a.n;
    const size_t row = (size_t)(b * a.Hq + head) * a.n + qrow;
    float* po = a.part_o + ((size_t)split * rows + row) * D + 4 * hb;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 x{o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]};
        *(f32x4*)(po + 32 * dt + 8 * i4) = x;
      }
    }
    if (hb == 0) {
      float* pm = a.part_ml + ((size_t)split * rows + row) * 2;
      pm[0] = m_run == -INFINITY ? -INFINITY : m_run * sl2;
      pm[1] = l_tot;
    }
  }
}

// Fixed-order log-sum-exp merge of the key splits of DECODE/CAUSAL calls.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           uint16_t* __restrict__ out, long long rows,
                                                           int n_splits) {
  constexpr int TPR = D / 4;  // threads per row, 4 elements each
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = t / TPR;
  const int c = (int)(t - row * TPR) * 4;
  if (row >= rows) return;
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, part_ml[((size_t)s * rows + row) * 2]);
  float l = 0.f;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < n_splits; ++s) {
    const float ms = part_ml[((size_t)s * rows + row) * 2];
    if (ms == -INFINITY) continue;
    const float wgt = exp2f(ms - M);
    l += wgt * part_ml[((size_t)s * rows + row) * 2 + 1];
    const f32x4 x = *(const f32x4*)(part_o + ((size_t)s * rows + row) * D + c);
    acc += wgt * x;
  }
  const float inv = 1.f / l;
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
    const int slots_half = (x.nw / 2) * 32;
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
    x.nw = block >= 128 ? 8 : 4;
    const int slots = x.nw * 32;
    if (x.G > slots) {
      *why = "Hq/Hkv larger than the query slots of a workgroup";
      return 2;
    }
    x.rows_per_wg = slots / x.G;
    x.n_qtiles = (block + x.rows_per_wg - 1) / x.rows_per_wg;
    // Split the keys when (batch x kv head x query tile) alone cannot keep
    // every CU streaming; each split keeps at least 4 key tiles.
    const long long items = (long long)B * Hkv * x.n_qtiles;
    const long long target = 2048;
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

template <int D, int NW>
static hipError_t launch_main(const AttnArgs& a, long long grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const AttnPlan& p, const AttnArgs& a, hipStream_t st) {
  hipError_t e = p.nw == 8 ? launch_main<D, 8>(a, p.grid, st) : launch_main<D, 4>(a, p.grid, st);
  if (e != hipSuccess || p.n_splits == 1) return e;
  const long long rows = (long long)p.B * p.Hq * p.n;
  const long long threads = rows * (D / 4);
  const long long blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, st, a.part_o,
                     a.part_ml, a.out, rows, p.n_splits);
  return hipGetLastError();
}

hipError_t attn_launch(const AttnPlan& p, const void* q, const void* k, const void* v, void* out,
                       void* ws, hipStream_t st) {
  AttnArgs a{};
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
  a.sl2 = 1.4426950408889634f / sqrtf((float)p.d);
  (void)hipGetLastError();
  switch (p.d) {
    case 32: return launch_d<32>(p, a, st);
    case 64: return launch_d<64>(p, a, st);
    default: return launch_d<128>(p, a, st);
  }
}

}  // namespace bda
