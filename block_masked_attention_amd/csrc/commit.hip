// Confidence commit and speculative verify for gfx950.
//
// Confidence of a masked canvas position = its largest softmax probability
// (SPRINT section of the LLaDA2.0-Uni summary); every position above the
// threshold commits, with at least a per-step minimum number of commits
// (same section, and the block-refinement scheduler of the DiffusionGemma
// pipeline page, "Schedulers").  Verify takes each row's argmax and the
// longest prefix that agrees with the drafts (linear speculative decoding,
// sec. 2 of the Nemotron-Labs-Diffusion-8B-Base 3x analysis page).
//
// Pass 1 (stream): one workgroup per (row, vocabulary chunk) streams the
// logits once with 16-byte non-temporal loads into registers, takes the
// chunk's maximum m (wavefront and workgroup reductions), then Z = sum
// exp(l - m) against it; only the threads holding m look for its lowest
// index a.  A ragged chunk instead keeps a running (m, a, Z) per lane,
// rescaled when m grows.  Partials merge with the associative rule
// m = max(m1, m2);  Z = Z1 e^(m1-m) + Z2 e^(m2-m);  a = lowest index among
// the maxima, in a fixed order, so results do not depend on timing.
// Pass 2 (finalize): one workgroup per group merges the chunk partials of
// its rows in a fixed tree, takes p = 1/Z, applies the threshold and the
// minimum-count fallback, and writes tokens / masked.
//
// Row statistics (entropy for adaptive stopping and entropy-bound commits,
// "Adaptive stopping" and "Schedulers" of the DiffusionGemma pipeline page)
// add T = sum exp(l - m) (l - m) to the same stream; the merge rule is
// T = sum_i e^(m_i-m) (T_i + (m_i - m) Z_i), and the entropy in nats is
// H = log Z - T / Z.
#include <limits.h>

#include <atomic>

#include "common.h"
#include "internal.h"

namespace bda {

constexpr int kCommitThreads = 256;
constexpr int kChunk = 16384;            // vocabulary entries per streaming workgroup
constexpr float kLog2e = 1.4426950408889634f;

// What the stream accumulates: the argmax only, also Z, or also Z and T.
enum { kArgmax = 0, kWithZ = 1, kWithZT = 2 };

struct Partial {
  float m, z;
  int a;
  float t;
};

struct Stat {
  float m, z;
  int a;
  float t;
};

__device__ __forceinline__ Stat merge(Stat x, Stat y, int kind, float c = kLog2e) {
  Stat r;
  r.m = fmaxf(x.m, y.m);
  r.a = x.m > y.m ? x.a : (y.m > x.m ? y.a : min(x.a, y.a));
  r.z = 0.f;
  r.t = 0.f;
  if (kind != kArgmax && r.m != -INFINITY) {
    // a side whose maximum is -inf holds no value and contributes nothing
    const float dx = x.m - r.m, dy = y.m - r.m;
    const float ax = x.m == -INFINITY ? 0.f : exp2_fast(dx * c);
    const float ay = y.m == -INFINITY ? 0.f : exp2_fast(dy * c);
    r.z = x.z * ax + y.z * ay;
    if (kind == kWithZT)
      r.t = (x.m == -INFINITY ? 0.f : ax * (x.t + dx * x.z)) + (y.m == -INFINITY ? 0.f : ay * (y.t + dy * y.z));
  }
  return r;
}

// Largest of two finite values (v_maximum3_f32: no quieting of the inputs,
// which fmaxf adds for values built from raw bits).
__device__ __forceinline__ float vmax(float x, float y) { return __builtin_elementwise_maximum(x, y); }

// All-lane reductions of a wavefront without LDS: DPP within rows of 16
// (lanes i^1, i^2, the mirror within 8, the mirror within 16), then the row
// swap and the half swap.  Every step combines a lane with its partner in an
// order both lanes share, so every lane ends with the same value.
template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}
template <typename T, typename F>
__device__ __forceinline__ T wave_all(T x, F op) {
  auto as_i = [](T v) { return __builtin_bit_cast(int, v); };
  auto as_t = [](int v) { return __builtin_bit_cast(T, v); };
  x = op(x, as_t(dpp<0xB1>(as_i(x))));
  x = op(x, as_t(dpp<0x4E>(as_i(x))));
  x = op(x, as_t(dpp<0x141>(as_i(x))));
  x = op(x, as_t(dpp<0x140>(as_i(x))));
  auto r = __builtin_amdgcn_permlane16_swap((unsigned)as_i(x), (unsigned)as_i(x), false, false);
  x = op(as_t((int)r[0]), as_t((int)r[1]));
  auto h = __builtin_amdgcn_permlane32_swap((unsigned)as_i(x), (unsigned)as_i(x), false, false);
  return op(as_t((int)h[0]), as_t((int)h[1]));
}

template <bool BF16>
__device__ __forceinline__ float load_one(const void* row, int j) {
  if (BF16) return __uint_as_float((unsigned)((const uint16_t*)row)[j] << 16);
  return ((const float*)row)[j];
}

// Fold 8 values (indices base..base+7, increasing) into a lane's state.
template <int KIND>
__device__ __forceinline__ void fold8(Stat& s, const float (&x)[8], int base, float c) {
  float lm = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) lm = fmaxf(lm, x[e]);
  if (lm > s.m) {
    int idx = 7;
#pragma unroll
    for (int e = 6; e >= 0; --e) idx = x[e] == lm ? e : idx;
    if (KIND != kArgmax) {
      if (s.m == -INFINITY) {
        s.z = 0.f;
        s.t = 0.f;
      } else {
        const float d = s.m - lm, a = exp2_fast(d * c);
        if (KIND == kWithZT) s.t = a * (s.t + d * s.z);
        s.z *= a;
      }
    }
    s.m = lm;
    s.a = base + idx;
  }
  if (KIND != kArgmax && s.m != -INFINITY) {
    const float nb = -s.m * c;
    float acc = 0.f, acct = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = exp2_fast(fmaf(x[e], c, nb));
      acc += p;
      if (KIND == kWithZT) acct = fmaf(p, x[e] == -INFINITY ? 0.f : x[e] - s.m, acct);   // -inf: padding
    }
    s.z += acc;
    if (KIND == kWithZT) s.t += acct;
  }
}

template <bool BF16, int KIND>
__global__ __launch_bounds__(kCommitThreads) void stream_kernel(const void* __restrict__ logits,
                                                                const uint8_t* __restrict__ masked,
                                                                Partial* __restrict__ part, int V,
                                                                int n_chunks, int vec_ok, float xs) {
  constexpr int VPT = kChunk / (8 * kCommitThreads);   // 8-value vectors per thread
  const int bid = blockIdx.x;
  const int t = bid / n_chunks;
  const int c = bid - t * n_chunks;
  if (masked != nullptr && masked[t] == 0) return;
  const int tid = threadIdx.x;
  const size_t esz = BF16 ? 2 : 4;
  const char* row = (const char*)logits + (size_t)t * V * esz;
  const int c0 = c * kChunk;
  const int c1 = min(V, c0 + kChunk);

  Stat s{-INFINITY, 0.f, INT_MAX, 0.f};
  if (vec_ok && c1 - c0 == kChunk) {
    // Whole chunk: every load of the thread is issued before any arithmetic
    // (vector v covers values c0 + 8*(v*256 + tid) + 0..7, so a wavefront
    // reads 1 KB contiguous per load and a thread's indices increase with v).
    float x[VPT][8];
    if (BF16) {
      u32x4 w[VPT];
#pragma unroll
      for (int v = 0; v < VPT; ++v)
        w[v] = __builtin_nontemporal_load((const u32x4*)(row + (size_t)(c0 + 8 * (v * kCommitThreads + tid)) * 2));
#pragma unroll
      for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[v][2 * e] = bf16_lo(w[v][e]);
          x[v][2 * e + 1] = bf16_hi(w[v][e]);
        }
    } else {
      f32x4 w[VPT][2];
#pragma unroll
      for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          w[v][h] = __builtin_nontemporal_load(
              (const f32x4*)(row + (size_t)(c0 + 8 * (v * kCommitThreads + tid)) * 4 + 16 * h));
#pragma unroll
      for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[v][e] = w[v][e >> 2][e & 3];
    }
    // pass 1: the chunk's largest value M, known to every thread
    const int lane = tid & 63, wv = tid >> 6;
    float vm[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      vm[v] = x[v][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) vm[v] = vmax(vm[v], x[v][e]);
    }
    float tm = vm[0];
#pragma unroll
    for (int v = 1; v < VPT; ++v) tm = vmax(tm, vm[v]);
    __shared__ float wmax[kCommitThreads / 64];
    __shared__ int wa[kCommitThreads / 64];
    __shared__ float wz[kCommitThreads / 64], wt[kCommitThreads / 64];
    const float wm = wave_all(tm, vmax);
    if (lane == 0) wmax[wv] = wm;
    __syncthreads();
    float M = wmax[0];
#pragma unroll
    for (int w = 1; w < kCommitThreads / 64; ++w) M = vmax(M, wmax[w]);
    // lowest index holding M: only the threads that hold it search
    int a = INT_MAX;
    if (tm == M) {
#pragma unroll
      for (int v = VPT - 1; v >= 0; --v)
        if (vm[v] == M) {
          int idx = 7;
#pragma unroll
          for (int e = 6; e >= 0; --e) idx = x[v][e] == M ? e : idx;
          a = c0 + 8 * (v * kCommitThreads + tid) + idx;
        }
    }
    // pass 2: Z (and T) against M; every thread's sums share it, so they add
    float z = 0.f, tt = 0.f;
    // A chunk whose values are all -inf (banned tokens) holds no mass: Z = T
    // = 0, and its maximum -inf loses every merge.
    if (KIND != kArgmax && M != -INFINITY) {
      const float nb = -M * xs;
      float acc[4] = {0.f, 0.f, 0.f, 0.f}, acct[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // (l - M) xs.  For T it is clamped at -160: exp2 of anything below
          // -149 is 0 in fp32 either way, and a -inf logit then adds 0 * -160
          // instead of 0 * -inf = NaN.
          float u = fmaf(x[v][e], xs, nb);
          if (KIND == kWithZT) u = fmaxf(u, -160.f);
          const float p = exp2_fast(u);
          acc[e & 3] += p;
          if (KIND == kWithZT) acct[e & 3] = fmaf(p, u, acct[e & 3]);
        }
      z = wave_all((acc[0] + acc[1]) + (acc[2] + acc[3]), [](float u, float w) { return u + w; });
      if (KIND == kWithZT)   // T = sum p (l - M) = (sum p u) / xs
        tt = wave_all((acct[0] + acct[1]) + (acct[2] + acct[3]), [](float u, float w) { return u + w; }) / xs;
    }
    a = wave_all(a, [](int u, int w) { return min(u, w); });
    if (lane == 0) {
      wa[wv] = a;
      wz[wv] = z;
      wt[wv] = tt;
    }
    __syncthreads();
    if (tid == 0) {
      Partial p{M, wz[0], wa[0], wt[0]};
#pragma unroll
      for (int w = 1; w < kCommitThreads / 64; ++w) {
        p.a = min(p.a, wa[w]);
        p.z += wz[w];
        p.t += wt[w];
      }
      part[(size_t)t * n_chunks + c] = p;
    }
    return;
  } else if (vec_ok) {
    // 8 consecutive values per step: one 16-byte load (bf16) or two (fp32).
    for (int base = c0 + 8 * tid; base < c1; base += 8 * kCommitThreads) {
      float x[8];
      if (base + 8 <= c1) {
        if (BF16) {
          const u32x4 w = __builtin_nontemporal_load((const u32x4*)(row + (size_t)base * 2));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_lo(w[e]);
            x[2 * e + 1] = bf16_hi(w[e]);
          }
        } else {
          const f32x4 w0 = __builtin_nontemporal_load((const f32x4*)(row + (size_t)base * 4));
          const f32x4 w1 = __builtin_nontemporal_load((const f32x4*)(row + (size_t)base * 4 + 16));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = w0[e];
            x[4 + e] = w1[e];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = base + e < c1 ? load_one<BF16>(row, base + e) : -INFINITY;
      }
      fold8<KIND>(s, x, base, xs);
    }
  } else {
    for (int base = c0 + 8 * tid; base < c1; base += 8 * kCommitThreads) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = base + e < c1 ? load_one<BF16>(row, base + e) : -INFINITY;
      fold8<KIND>(s, x, base, xs);
    }
  }
  // -INFINITY padding never wins a strict comparison, and contributes 0 to Z
  // once a finite maximum exists.

#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Stat o;
    o.m = __shfl_xor(s.m, off);
    o.z = __shfl_xor(s.z, off);
    o.a = __shfl_xor(s.a, off);
    o.t = __shfl_xor(s.t, off);
    s = merge(s, o, KIND, xs);
  }
  __shared__ Stat wst[kCommitThreads / 64];
  if ((tid & 63) == 0) wst[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    Stat r = wst[0];
#pragma unroll
    for (int w = 1; w < kCommitThreads / 64; ++w) r = merge(r, wst[w], KIND, xs);
    Partial p;
    p.m = r.m;
    p.z = r.z;
    p.a = r.a;
    p.t = r.t;
    part[(size_t)t * n_chunks + c] = p;
  }
}

// Rows of a finalize workgroup are merged by groups of CH lanes (CH = the
// power of two >= the chunk count, at most 64): lane ci of a row loads the
// partials of chunks ci, ci + CH, ... at once, then the lanes merge in a
// fixed tree, every lane of the row ending with the row's Stat.  live must be
// the same in all CH lanes of a row.
__device__ __forceinline__ int lanes_per_row(int n_chunks) {
  int ch = 1;
  while (ch < n_chunks && ch < 64) ch <<= 1;
  return ch;
}
__device__ __forceinline__ Stat row_stat_lanes(const Partial* part, size_t t, bool live, int ci, int CH,
                                              int n_chunks, int kind, float c = kLog2e) {
  Stat s{-INFINITY, 0.f, INT_MAX, 0.f};
  if (live)
    for (int k = ci; k < n_chunks; k += CH) {
      const Partial q = part[t * n_chunks + k];
      s = merge(s, Stat{q.m, q.z, q.a, q.t}, kind, c);
    }
  for (int off = 1; off < CH; off <<= 1) {
    Stat o;
    o.m = __shfl_xor(s.m, off);
    o.z = __shfl_xor(s.z, off);
    o.a = __shfl_xor(s.a, off);
    o.t = __shfl_xor(s.t, off);
    s = merge(s, o, kind, c);
  }
  return s;
}

__device__ __forceinline__ int block_sum(int x, int* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kCommitThreads / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

__device__ __forceinline__ float block_sum_f(float x, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kCommitThreads / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

// Row statistics written beside a commit (STATS = true); any may be NULL.
struct StatsOut {
  float* conf;
  int64_t* argmax;
  float* entropy;
  float* mean_entropy;
};

// One workgroup per group g.  Row results (p, argmax, flag) live in LDS
// when R <= kFinRows, else in the workspace scratch rowp/rowa/rowf [G*R].
// Each row's mask byte and chunk partials are loaded together (partials of
// unmasked rows are stale and ignored), so the critical path holds one
// round trip to memory.  STATS: the partials are those of every row (with
// T), and each row's confidence, argmax and entropy and the group's mean
// entropy are written as the row statistics kernel below writes them (same
// expressions, same summation order).
constexpr int kFinRows = 2048;

template <bool IN_LDS, bool STATS>
__global__ __launch_bounds__(kCommitThreads) void commit_finalize_kernel(
    const Partial* __restrict__ part, int n_chunks, int64_t* __restrict__ tokens,
    uint8_t* __restrict__ masked, float threshold, int k_min, int R, float* __restrict__ rowp,
    int* __restrict__ rowa, uint8_t* __restrict__ rowf, const StatsOut so) {
  __shared__ int red[2][kCommitThreads / 64];
  __shared__ float redf[kCommitThreads / 64];
  __shared__ int redi[kCommitThreads / 64];
  __shared__ float lp[IN_LDS ? kFinRows : 1];
  __shared__ int la[IN_LDS ? kFinRows : 1];
  __shared__ uint8_t lf[IN_LDS ? kFinRows : 1];
  const int g = blockIdx.x, tid = threadIdx.x;
  const size_t base = (size_t)g * R;
  float* rp = IN_LDS ? lp : rowp + base;
  int* ra = IN_LDS ? la : rowa + base;
  uint8_t* rf = IN_LDS ? lf : rowf + base;
  int nmask = 0, npass = 0;
  float hsum = 0.f;
  int cnt = 0;
  const int CH = lanes_per_row(n_chunks), ci = tid % CH;
  for (int r0 = 0; r0 < R; r0 += kCommitThreads / CH) {
    const int r = r0 + tid / CH;
    const bool in = r < R;
    const uint8_t mk = in && ci == 0 ? masked[base + r] : 0;
    const Stat s = row_stat_lanes(part, base + r, in, ci, CH, n_chunks, STATS ? kWithZT : kWithZ);
    if (in && ci == 0) {
      const float p = 1.f / s.z;
      const uint8_t f = mk ? (p > threshold ? 2 : 1) : 0;
      rp[r] = p;
      ra[r] = s.a;
      rf[r] = f;
      nmask += f != 0;
      npass += f == 2;
      if constexpr (STATS) {
        const float h = logf(s.z) - s.t / s.z;
        if (so.conf) so.conf[base + r] = 1.f / s.z;
        if (so.argmax) so.argmax[base + r] = s.a;
        if (so.entropy) so.entropy[base + r] = h;
        hsum += h;
        cnt += 1;
      }
    }
  }
  if constexpr (STATS) {
    hsum = block_sum_f(hsum, redf);
    cnt = block_sum(cnt, redi);
    if (tid == 0 && so.mean_entropy) so.mean_entropy[g] = cnt > 0 ? hsum / (float)cnt : 0.f;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    nmask += __shfl_xor(nmask, off);
    npass += __shfl_xor(npass, off);
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = nmask;
    red[1][tid >> 6] = npass;
  }
  __syncthreads();   // also publishes rp, ra, rf
  nmask = 0;
  npass = 0;
#pragma unroll
  for (int w = 0; w < kCommitThreads / 64; ++w) {
    nmask += red[0][w];
    npass += red[1][w];
  }
  const int need = min(k_min, nmask) - npass;
  for (int r = tid; r < R; r += kCommitThreads) {
    const uint8_t f = rf[r];
    bool take = f == 2;
    if (f == 1 && need > 0) {
      // rank among masked rows below the threshold: larger p first, then lower row
      const float p = rp[r];
      int rank = 0;
      for (int o = 0; o < R && rank < need; ++o) {
        if (rf[o] != 1) continue;
        const float po = rp[o];
        rank += (po > p) || (po == p && o < r);
      }
      take = rank < need;
    }
    if (take) {
      tokens[base + r] = ra[r];
      masked[base + r] = 0;
    }
  }
}

// One workgroup per sequence: argmax per row, then the first disagreement.
__global__ __launch_bounds__(kCommitThreads) void verify_finalize_kernel(
    const Partial* __restrict__ part, int n_chunks, const int64_t* __restrict__ drafts,
    int64_t* __restrict__ argmax_out, int32_t* __restrict__ accept, int R, int32_t* __restrict__ kv_len,
    int kv_cap) {
  __shared__ int red[kCommitThreads / 64];
  const int b = blockIdx.x;
  int first = R;
  const int CH = lanes_per_row(n_chunks), ci = threadIdx.x % CH;
  for (int r0 = 0; r0 < R; r0 += kCommitThreads / CH) {
    const int r = r0 + (int)threadIdx.x / CH;
    const size_t t = (size_t)b * R + r;
    const int64_t dr = r < R && ci == 0 ? drafts[t] : 0;
    const Stat s = row_stat_lanes(part, t, r < R, ci, CH, n_chunks, kArgmax);
    if (r < R && ci == 0) {
      argmax_out[t] = s.a;
      if ((int64_t)s.a != dr) first = min(first, r);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) first = min(first, __shfl_xor(first, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = first;
  __syncthreads();
  if (threadIdx.x == 0) {
    int m = red[0];
    for (int w = 1; w < kCommitThreads / 64; ++w) m = min(m, red[w]);
    accept[b] = m;
    if (kv_len != nullptr) kv_len[b] = min(kv_len[b] + m, kv_cap);   // keep the accepted drafts' rows
  }
}

// One workgroup per group: per selected row the confidence 1/Z, the argmax
// and the entropy log Z - T/Z (nats); the group's mean entropy over its
// selected rows (0 when none is selected).
__global__ __launch_bounds__(kCommitThreads) void stats_finalize_kernel(
    const Partial* __restrict__ part, int n_chunks, const uint8_t* __restrict__ masked, int R,
    float* __restrict__ conf, int64_t* __restrict__ argmax_out, float* __restrict__ entropy,
    float* __restrict__ mean_entropy) {
  __shared__ float redf[kCommitThreads / 64];
  __shared__ int redi[kCommitThreads / 64];
  const int g = blockIdx.x;
  float hsum = 0.f;
  int cnt = 0;
  const int CH = lanes_per_row(n_chunks), ci = threadIdx.x % CH;
  for (int r0 = 0; r0 < R; r0 += kCommitThreads / CH) {
    const int r = r0 + (int)threadIdx.x / CH;
    const size_t t = (size_t)g * R + r;
    const bool live = r < R && ci == 0 && (masked == nullptr || masked[t] != 0);
    const Stat s = row_stat_lanes(part, t, r < R, ci, CH, n_chunks, kWithZT);   // stale for unselected rows
    if (!live) continue;
    const float h = logf(s.z) - s.t / s.z;
    if (conf) conf[t] = 1.f / s.z;
    if (argmax_out) argmax_out[t] = s.a;
    if (entropy) entropy[t] = h;
    hsum += h;
    cnt += 1;
  }
  hsum = block_sum_f(hsum, redf);
  cnt = block_sum(cnt, redi);
  if (threadIdx.x == 0 && mean_entropy) mean_entropy[g] = cnt > 0 ? hsum / (float)cnt : 0.f;
}

// Entropy-bound commit (the EntropyBoundScheduler of the DiffusionGemma
// pipeline page, "Schedulers"), one workgroup per group of R <= kEntMaxR
// rows: every masked row's entropy H (nats, of softmax(l / T)) and argmax go
// to LDS; each masked row's rank among them by (H ascending, row ascending)
// is counted; the ranked entropies are summed in rank order and the first n
// ranks are committed, n = max(min(k_min, #masked), the longest prefix whose
// sum stays <= bound).  inv_t = 1 / T (the streamed T sums are in logit
// units).
constexpr int kEntMaxR = 4096;

__global__ __launch_bounds__(kCommitThreads) void commit_entropy_finalize_kernel(
    const Partial* __restrict__ part, int n_chunks, int64_t* __restrict__ tokens, uint8_t* __restrict__ masked,
    float bound, int k_min, int R, float c, float inv_t) {
  __shared__ float sh[kEntMaxR];
  __shared__ float sorted_h[kEntMaxR];
  __shared__ int sa[kEntMaxR];
  __shared__ int red[kCommitThreads / 64];
  __shared__ int take_n;
  const int g = blockIdx.x, tid = threadIdx.x;
  const size_t base = (size_t)g * R;
  int nm = 0;
  const int CH = lanes_per_row(n_chunks), ci = tid % CH;
  for (int r0 = 0; r0 < R; r0 += kCommitThreads / CH) {
    const int r = r0 + tid / CH;
    const bool live = r < R && ci == 0 && masked[base + r];
    const Stat st = row_stat_lanes(part, base + r, r < R, ci, CH, n_chunks, kWithZT, c);   // stale for unmasked rows
    if (r >= R || ci != 0) continue;
    float h = INFINITY;                          // unmasked: never ranked
    int a = -1;
    if (live) {
      h = logf(st.z) - (st.t * inv_t) / st.z;
      a = st.a;
      nm += 1;
    }
    sh[r] = h;
    sa[r] = a;
  }
  if (R <= 64) {
    // One wavefront ranks the group in registers: lane r holds row r; ranks
    // by (H, row) from lane reads, then the rows in rank order and their
    // entropies summed in that order, as below.
    __syncthreads();                             // publishes sh, sa
    if (tid >= 64) return;
    const bool in = tid < R;
    const float h = in ? sh[tid] : INFINITY;
    const int av = in ? sa[tid] : -1;
    const bool live = av >= 0;
    int rank = 0;
    for (int o = 0; o < R; ++o) {
      const float ho = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), o));
      rank += (ho < h) || (ho == h && o < tid);
    }
    int inv = 0;                                 // lane k: the row of rank k
    for (int o = 0; o < R; ++o) {
      const int ro = __builtin_amdgcn_readlane(rank, o);
      const int lo = __builtin_amdgcn_readlane(live ? 1 : 0, o);
      if (lo && ro == tid) inv = o;
    }
    const int nmask = __popcll(__ballot(live));
    float acc = 0.f;
    int n = 0;
    for (int k = 0; k < nmask; ++k) {
      const int src = __builtin_amdgcn_readlane(inv, k);
      acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), src));
      if (acc <= bound) n = k + 1;
      else break;
    }
    if (live && rank < max(n, min(k_min, nmask))) {
      tokens[base + tid] = av;
      masked[base + tid] = 0;
    }
    return;
  }
  const int nmask = block_sum(nm, red);          // (its barriers also publish sh, sa)
  for (int r = tid; r < R; r += kCommitThreads) {
    if (sa[r] < 0) continue;
    const float h = sh[r];
    int rank = 0;
    for (int o = 0; o < R; ++o) {
      const float ho = sh[o];
      rank += (ho < h) || (ho == h && o < r);
    }
    sorted_h[rank] = h;
  }
  __syncthreads();
  if (tid == 0) {
    float acc = 0.f;
    int n = 0;
    for (int j = 0; j < nmask; ++j) {
      acc += sorted_h[j];
      if (acc <= bound) n = j + 1;
      else break;
    }
    take_n = max(n, min(k_min, nmask));
  }
  __syncthreads();
  const int n = take_n;
  for (int r = tid; r < R; r += kCommitThreads) {
    if (sa[r] < 0) continue;
    const float h = sh[r];
    int rank = 0;
    for (int o = 0; o < R && rank < n; ++o) {
      const float ho = sh[o];
      rank += (ho < h) || (ho == h && o < r);
    }
    if (rank < n) {
      tokens[base + r] = sa[r];
      masked[base + r] = 0;
    }
  }
}

// Adaptive stopping (the DiffusionGemma pipeline page, "Adaptive stopping"),
// one workgroup for all G examples, a wavefront per example at a time: an
// example already frozen keeps its state; otherwise stable[g] counts the
// consecutive steps whose argmax equals the previous step's (any change
// resets it to 0), prev takes this step's argmax, and the example freezes
// once stable[g] >= stability and mean_entropy[g] < conf_thr.  n_frozen
// (optional) receives the number of frozen examples after the step.
__global__ __launch_bounds__(1024) void adaptive_stop_kernel(const int64_t* __restrict__ argmax,
                                                             int64_t* __restrict__ prev, int32_t* __restrict__ stable,
                                                             uint8_t* __restrict__ frozen,
                                                             const float* __restrict__ mean_entropy, int G, int R,
                                                             int stability, float conf_thr,
                                                             int32_t* __restrict__ n_frozen) {
  __shared__ int cnt[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int nf = 0;
  for (int g = w; g < G; g += 16) {
    int fz = frozen[g];
    if (!fz) {
      bool changed = false;
      for (int r = lane; r < R; r += 64) {
        const size_t t = (size_t)g * R + r;
        const int64_t a = argmax[t];
        changed |= a != prev[t];
        prev[t] = a;
      }
      changed = __any(changed);
      if (lane == 0) {
        const int s = changed ? 0 : stable[g] + 1;
        stable[g] = s;
        if (s >= stability && mean_entropy[g] < conf_thr) {
          frozen[g] = 1;
          fz = 1;
        }
      }
      fz = __shfl(fz, 0);
    }
    nf += fz;
  }
  if (lane == 0) cnt[w] = nf;
  __syncthreads();
  if (threadIdx.x == 0 && n_frozen) {
    int s = 0;
    for (int i = 0; i < 16; ++i) s += cnt[i];
    *n_frozen = s;
  }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

int commit_make_plan(int G, int R, int V, int dtype, CommitPlan* p) {
  CommitPlan x{};
  x.G = G;
  x.R = R;
  x.V = V;
  x.dtype = dtype;
  x.chunk = kChunk;
  x.n_chunks = (V + kChunk - 1) / kChunk;
  const size_t rows = (size_t)G * R;
  x.ws_bytes = rows * x.n_chunks * sizeof(Partial) + rows * (4 + 4 + 1) + 256;
  *p = x;
  return 0;
}

static void carve(const CommitPlan& p, void* ws, Partial** part, float** rowp, int** rowa,
                  uint8_t** rowf) {
  const size_t rows = (size_t)p.G * p.R;
  char* c = (char*)ws;
  *part = (Partial*)c;
  c += rows * p.n_chunks * sizeof(Partial);
  *rowp = (float*)c;
  c += rows * 4;
  *rowa = (int*)c;
  c += rows * 4;
  *rowf = (uint8_t*)c;
}

static bool vec_ok(const void* logits, int V, int dtype) {
  const int per16 = dtype == 0 ? 8 : 4;
  return ((uintptr_t)logits % 16) == 0 && V % per16 == 0;
}

template <int KIND>
static hipError_t launch_stream(const CommitPlan& p, const void* logits, const uint8_t* masked,
                                Partial* part, hipStream_t st, float c = kLog2e) {
  const long long grid = (long long)p.G * p.R * p.n_chunks;
  const int vo = vec_ok(logits, p.V, p.dtype);
  if (p.dtype == 0)
    hipLaunchKernelGGL((stream_kernel<true, KIND>), dim3((unsigned)grid), dim3(kCommitThreads), 0,
                       st, logits, masked, part, p.V, p.n_chunks, vo, c);
  else
    hipLaunchKernelGGL((stream_kernel<false, KIND>), dim3((unsigned)grid), dim3(kCommitThreads), 0,
                       st, logits, masked, part, p.V, p.n_chunks, vo, c);
  return hipGetLastError();
}

hipError_t commit_launch(const CommitPlan& p, const void* logits, int64_t* tokens, uint8_t* masked,
                         float threshold, int k_min, void* ws, hipStream_t st) {
  if ((long long)p.G * p.R == 0) return hipSuccess;
  Partial* part;
  float* rowp;
  int* rowa;
  uint8_t* rowf;
  carve(p, ws, &part, &rowp, &rowa, &rowf);
  (void)hipGetLastError();
  hipError_t e = launch_stream<kWithZ>(p, logits, masked, part, st);
  if (e != hipSuccess) return e;
  if (p.R <= kFinRows)
    hipLaunchKernelGGL((commit_finalize_kernel<true, false>), dim3(p.G), dim3(kCommitThreads), 0, st, part,
                       p.n_chunks, tokens, masked, threshold, k_min, p.R, rowp, rowa, rowf, StatsOut{});
  else
    hipLaunchKernelGGL((commit_finalize_kernel<false, false>), dim3(p.G), dim3(kCommitThreads), 0, st, part,
                       p.n_chunks, tokens, masked, threshold, k_min, p.R, rowp, rowa, rowf, StatsOut{});
  return hipGetLastError();
}

hipError_t stats_commit_launch(const CommitPlan& p, const void* logits, int64_t* tokens, uint8_t* masked,
                               float threshold, int k_min, float* conf, int64_t* argmax_out, float* entropy,
                               float* mean_entropy, void* ws, hipStream_t st) {
  if (p.G == 0) return hipSuccess;
  Partial* part;
  float* rowp;
  int* rowa;
  uint8_t* rowf;
  carve(p, ws, &part, &rowp, &rowa, &rowf);
  (void)hipGetLastError();
  if (p.R > 0) {
    // every row is streamed: the statistics cover all rows, the commit the masked ones
    hipError_t e = launch_stream<kWithZT>(p, logits, nullptr, part, st);
    if (e != hipSuccess) return e;
  }
  const StatsOut so{conf, argmax_out, entropy, mean_entropy};
  if (p.R <= kFinRows)
    hipLaunchKernelGGL((commit_finalize_kernel<true, true>), dim3(p.G), dim3(kCommitThreads), 0, st, part,
                       p.n_chunks, tokens, masked, threshold, k_min, p.R, rowp, rowa, rowf, so);
  else
    hipLaunchKernelGGL((commit_finalize_kernel<false, true>), dim3(p.G), dim3(kCommitThreads), 0, st, part,
                       p.n_chunks, tokens, masked, threshold, k_min, p.R, rowp, rowa, rowf, so);
  return hipGetLastError();
}

hipError_t verify_launch(const CommitPlan& p, const void* logits, const int64_t* drafts,
                         int64_t* argmax_out, int32_t* accept, int32_t* kv_len, int kv_cap, void* ws,
                         hipStream_t st) {
  if (p.G == 0) return hipSuccess;
  Partial* part;
  float* rowp;
  int* rowa;
  uint8_t* rowf;
  carve(p, ws, &part, &rowp, &rowa, &rowf);
  (void)hipGetLastError();
  if (p.R > 0) {
    hipError_t e = launch_stream<kArgmax>(p, logits, nullptr, part, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(verify_finalize_kernel, dim3(p.G), dim3(kCommitThreads), 0, st, part,
                     p.n_chunks, drafts, argmax_out, accept, p.R, kv_len, kv_cap);
  return hipGetLastError();
}

hipError_t stats_launch(const CommitPlan& p, const void* logits, const uint8_t* masked, float* conf,
                        int64_t* argmax_out, float* entropy, float* mean_entropy, void* ws,
                        hipStream_t st) {
  if (p.G == 0) return hipSuccess;
  Partial* part;
  float* rowp;
  int* rowa;
  uint8_t* rowf;
  carve(p, ws, &part, &rowp, &rowa, &rowf);
  (void)hipGetLastError();
  if (p.R > 0) {
    hipError_t e = launch_stream<kWithZT>(p, logits, masked, part, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(stats_finalize_kernel, dim3(p.G), dim3(kCommitThreads), 0, st, part, p.n_chunks,
                     masked, p.R, conf, argmax_out, entropy, mean_entropy);
  return hipGetLastError();
}

}  // namespace bda

namespace bda {

hipError_t commit_entropy_launch(const CommitPlan& p, const void* logits, int64_t* tokens, uint8_t* masked,
                                 float bound, float temperature, int k_min, void* ws, hipStream_t st) {
  if ((long long)p.G * p.R == 0) return hipSuccess;
  Partial* part;
  float* rowp;
  int* rowa;
  uint8_t* rowf;
  carve(p, ws, &part, &rowp, &rowa, &rowf);
  (void)hipGetLastError();
  const float c = kLog2e / temperature;
  hipError_t e = launch_stream<kWithZT>(p, logits, masked, part, st, c);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_entropy_finalize_kernel, dim3(p.G), dim3(kCommitThreads), 0, st, part, p.n_chunks,
                     tokens, masked, bound, k_min, p.R, c, 1.f / temperature);
  return hipGetLastError();
}

int commit_entropy_max_rows() { return kEntMaxR; }

// ---- the commit for callers that cannot allocate: its partials and row
// scratch live in this file-scope array, one copy per GPU, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in): each device's address is taken once with
// hipGetSymbolAddress, with that device current, and kept per device.
static __device__ __align__(256) unsigned char scratch[kCommitNoAllocBytes];

static std::atomic<void*> g_scratch_ptr[kMaxDevices];

hipError_t commit_noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // concurrent first calls on one device store the same address
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t adaptive_stop_launch(const int64_t* argmax, int64_t* prev, int32_t* stable, uint8_t* frozen,
                                const float* mean_entropy, int G, int R, int stability, float conf_thr,
                                int32_t* n_frozen, hipStream_t st) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(adaptive_stop_kernel, dim3(1), dim3(1024), 0, st, argmax, prev, stable, frozen, mean_entropy, G,
                     R, stability, conf_thr, n_frozen);
  return hipGetLastError();
}

}  // namespace bda
