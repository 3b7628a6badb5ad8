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
// logits once with 16-byte non-temporal loads and keeps, per lane, the
// running maximum m, the lowest index a reaching it and Z = sum exp(l - m)
// (rescaled when m grows).  Lanes and wavefronts merge with the associative
// rule  m = max(m1, m2);  Z = Z1 e^(m1-m) + Z2 e^(m2-m);  a = lowest index
// among the maxima, in a fixed order, so results do not depend on timing.
// Pass 2 (finalize): one workgroup per group merges the chunk partials of
// its rows in chunk order, takes p = 1/Z, applies the threshold and the
// minimum-count fallback, and writes tokens / masked.
//
// Row statistics (entropy for adaptive stopping and entropy-bound commits,
// "Adaptive stopping" and "Schedulers" of the DiffusionGemma pipeline page)
// add T = sum exp(l - m) (l - m) to the same stream; the merge rule is
// T = sum_i e^(m_i-m) (T_i + (m_i - m) Z_i), and the entropy in nats is
// H = log Z - T / Z.
#include <limits.h>

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

__device__ __forceinline__ Stat merge(Stat x, Stat y, int kind) {
  Stat r;
  r.m = fmaxf(x.m, y.m);
  r.a = x.m > y.m ? x.a : (y.m > x.m ? y.a : min(x.a, y.a));
  r.z = 0.f;
  r.t = 0.f;
  if (kind != kArgmax && r.m != -INFINITY) {
    // a side whose maximum is -inf holds no value and contributes nothing
    const float dx = x.m - r.m, dy = y.m - r.m;
    const float ax = x.m == -INFINITY ? 0.f : exp2_fast(dx * kLog2e);
    const float ay = y.m == -INFINITY ? 0.f : exp2_fast(dy * kLog2e);
    r.z = x.z * ax + y.z * ay;
    if (kind == kWithZT)
      r.t = (x.m == -INFINITY ? 0.f : ax * (x.t + dx * x.z)) + (y.m == -INFINITY ? 0.f : ay * (y.t + dy * y.z));
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ float load_one(const void* row, int j) {
  if (BF16) return __uint_as_float((unsigned)((const uint16_t*)row)[j] << 16);
  return ((const float*)row)[j];
}

// Fold 8 values (indices base..base+7, increasing) into a lane's state.
template <int KIND>
__device__ __forceinline__ void fold8(Stat& s, const float (&x)[8], int base) {
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
        const float d = s.m - lm, a = exp2_fast(d * kLog2e);
        if (KIND == kWithZT) s.t = a * (s.t + d * s.z);
        s.z *= a;
      }
    }
    s.m = lm;
    s.a = base + idx;
  }
  if (KIND != kArgmax && s.m != -INFINITY) {
    const float nb = -s.m * kLog2e;
    float acc = 0.f, acct = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = exp2_fast(fmaf(x[e], kLog2e, nb));
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
                                                                int n_chunks, int vec_ok) {
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
    // pass 1: largest value and its lowest index
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      float lm = x[v][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) lm = fmaxf(lm, x[v][e]);
      if (lm > s.m) {
        int idx = 7;
#pragma unroll
        for (int e = 6; e >= 0; --e) idx = x[v][e] == lm ? e : idx;
        s.m = lm;
        s.a = c0 + 8 * (v * kCommitThreads + tid) + idx;
      }
    }
    // pass 2: Z (and T) against that maximum
    if (KIND != kArgmax) {
      const float nb = -s.m * kLog2e;
      float acc[4] = {0.f, 0.f, 0.f, 0.f}, acct[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2_fast(fmaf(x[v][e], kLog2e, nb));
          acc[e & 3] += p;
          if (KIND == kWithZT) acct[e & 3] = fmaf(p, x[v][e] - s.m, acct[e & 3]);
        }
      s.z = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      s.t = (acct[0] + acct[1]) + (acct[2] + acct[3]);
    }
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
      fold8<KIND>(s, x, base);
    }
  } else {
    for (int base = c0 + 8 * tid; base < c1; base += 8 * kCommitThreads) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = base + e < c1 ? load_one<BF16>(row, base + e) : -INFINITY;
      fold8<KIND>(s, x, base);
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
    s = merge(s, o, KIND);
  }
  __shared__ Stat wst[kCommitThreads / 64];
  if ((tid & 63) == 0) wst[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    Stat r = wst[0];
#pragma unroll
    for (int w = 1; w < kCommitThreads / 64; ++w) r = merge(r, wst[w], KIND);
    Partial p;
    p.m = r.m;
    p.z = r.z;
    p.a = r.a;
    p.t = r.t;
    part[(size_t)t * n_chunks + c] = p;
  }
}

__device__ __forceinline__ Stat row_stat(const Partial* part, size_t t, int n_chunks, int kind) {
  const Partial& q0 = part[t * n_chunks];
  Stat s{q0.m, q0.z, q0.a, q0.t};
  for (int c = 1; c < n_chunks; ++c) {
    const Partial& q = part[t * n_chunks + c];
    s = merge(s, Stat{q.m, q.z, q.a, q.t}, kind);
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

// One workgroup per group g.  rowp/rowa/rowf are workspace scratch [G*R].
__global__ __launch_bounds__(kCommitThreads) void commit_finalize_kernel(
    const Partial* __restrict__ part, int n_chunks, int64_t* __restrict__ tokens,
    uint8_t* __restrict__ masked, float threshold, int k_min, int R, float* __restrict__ rowp,
    int* __restrict__ rowa, uint8_t* __restrict__ rowf) {
  __shared__ int red[kCommitThreads / 64];
  const int g = blockIdx.x;
  const size_t base = (size_t)g * R;
  int nmask = 0, npass = 0;
  for (int r = threadIdx.x; r < R; r += kCommitThreads) {
    const size_t t = base + r;
    uint8_t f = 0;
    if (masked[t]) {
      const Stat s = row_stat(part, t, n_chunks, kWithZ);
      const float p = 1.f / s.z;
      rowp[t] = p;
      rowa[t] = s.a;
      f = p > threshold ? 2 : 1;
      nmask += 1;
      npass += f == 2;
    }
    rowf[t] = f;
  }
  nmask = block_sum(nmask, red);
  npass = block_sum(npass, red);
  const int need = min(k_min, nmask) - npass;
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += kCommitThreads) {
    const size_t t = base + r;
    const uint8_t f = rowf[t];
    bool take = f == 2;
    if (f == 1 && need > 0) {
      // rank among masked rows below the threshold: larger p first, then lower row
      const float p = rowp[t];
      int rank = 0;
      for (int o = 0; o < R && rank < need; ++o) {
        if (rowf[base + o] != 1) continue;
        const float po = rowp[base + o];
        rank += (po > p) || (po == p && o < r);
      }
      take = rank < need;
    }
    if (take) {
      tokens[t] = rowa[t];
      masked[t] = 0;
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
  for (int r = threadIdx.x; r < R; r += kCommitThreads) {
    const size_t t = (size_t)b * R + r;
    const Stat s = row_stat(part, t, n_chunks, kArgmax);
    argmax_out[t] = s.a;
    if ((int64_t)s.a != drafts[t]) first = min(first, r);
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
  for (int r = threadIdx.x; r < R; r += kCommitThreads) {
    const size_t t = (size_t)g * R + r;
    if (masked != nullptr && masked[t] == 0) continue;
    const Stat s = row_stat(part, t, n_chunks, kWithZT);
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
                                Partial* part, hipStream_t st) {
  const long long grid = (long long)p.G * p.R * p.n_chunks;
  const int vo = vec_ok(logits, p.V, p.dtype);
  if (p.dtype == 0)
    hipLaunchKernelGGL((stream_kernel<true, KIND>), dim3((unsigned)grid), dim3(kCommitThreads), 0,
                       st, logits, masked, part, p.V, p.n_chunks, vo);
  else
    hipLaunchKernelGGL((stream_kernel<false, KIND>), dim3((unsigned)grid), dim3(kCommitThreads), 0,
                       st, logits, masked, part, p.V, p.n_chunks, vo);
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
  hipLaunchKernelGGL(commit_finalize_kernel, dim3(p.G), dim3(kCommitThreads), 0, st, part,
                     p.n_chunks, tokens, masked, threshold, k_min, p.R, rowp, rowa, rowf);
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
