// SPRINT sparse prefix retention for gfx950 (SPRINT section of the
// LLaDA2.0-Uni summary): once at the start of a block, every prefix position
// i gets the score
//   s_i = alpha * n_i / mean_j(n_j) + (1 - alpha) * c_i,
// with n_i the L2 norm of position i's keys (all kv heads) and c_i its top-1
// confidence; image positions keep their best floor(r_img * count + 0.5)
// scores, text positions their best floor(r_text * count + 0.5) (ties: lower
// position first), and the kept rows of K and V are compacted in position
// order, so every later step attends to the shorter cache.
// Three launches: key norms; ranking (each
// position's rank among the batch's sort keys, counted against all of them,
// which spreads the selection over the whole chip); and compaction with the
// gather of the kept rows.
#include "common.h"
#include "internal.h"

namespace bda {

// Key norms.  Grid (ceil(L / P), B) with P = 256 / (D / 8) positions per
// workgroup; thread t owns 16-byte chunk t % (D / 8) of position t / (D / 8)
// and reads it for every head (each head's P rows are one contiguous run),
// then the chunks of a position are summed across lanes.
template <int D>
__global__ __launch_bounds__(256) void sprint_norm_kernel(const uint16_t* __restrict__ k, float* __restrict__ nrm,
                                                          int Hkv, int L) {
  constexpr int CPR = D / 8, P = 256 / CPR;
  const int b = blockIdx.y, tid = threadIdx.x, c = tid % CPR;
  const int i = blockIdx.x * P + tid / CPR;
  const int ic = min(i, L - 1);
  const uint16_t* base = k + ((size_t)b * Hkv * L + ic) * D + 8 * c;
  float acc = 0.f;
#pragma unroll 8
  for (int h = 0; h < Hkv; ++h) {
    const u32x4 x = *(const u32x4*)(base + (size_t)h * L * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf16_lo(x[e]), hi = bf16_hi(x[e]);
      acc = fmaf(lo, lo, acc);
      acc = fmaf(hi, hi, acc);
    }
  }
#pragma unroll
  for (int off = CPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (c == 0 && i < L) nrm[(size_t)b * L + i] = sqrtf(acc);
}

// order-preserving map of a float to an unsigned (ascending)
__device__ __forceinline__ unsigned f2ord(float f) {
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kRankPos = 32;     // positions ranked per workgroup
constexpr int kRankWaves = 8;    // wavefronts per ranking workgroup (16 key slices)
constexpr int kGatherPos = 16;   // positions compacted per workgroup

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Scores and kept flags.  Grid (ceil(L / 32), B), 512 threads.  Every
// workgroup rebuilds the sort keys of its batch's L positions in LDS (the mean
// norm is reduced in one fixed order, so all workgroups hold identical keys)
// and ranks its 32 positions against them: rank = number of smaller keys.
// Keys order text (modality 0) before image, then score descending, then
// position, so a position's rank within its modality is its rank minus the
// text count for image positions; it is kept iff that is below the modality's
// keep count.  flags[b, i] (i < round_up(L, 32)) = kept, 0 past L.
__global__ __launch_bounds__(kRankWaves * 64) void sprint_rank_kernel(const float* __restrict__ nrm, const float* __restrict__ conf,
                                                          const uint8_t* __restrict__ modality, float alpha,
                                                          float r_img, float r_text, int L, int Lk,
                                                          uint8_t* __restrict__ flags, float* __restrict__ scores) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  unsigned long long* keys = (unsigned long long*)dyn;                 // Lk = round_up(L, 256)
  uint8_t* mods = (uint8_t*)(keys + Lk);                               // L
  constexpr int NT = kRankWaves * 64;
  __shared__ float red[kRankWaves];
  __shared__ int redi[kRankWaves];
  __shared__ int part[kRankWaves][kRankPos];
  const int b = blockIdx.y, c0 = blockIdx.x * kRankPos, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* nb = nrm + (size_t)b * L;
  const float* cb = conf + (size_t)b * L;

  // Pass 1: norms, confidences and modalities into LDS (each key slot holds
  // the position's norm and confidence until pass 2), and the sums for the
  // mean norm and the text count: thread t adds positions t, t+512, ... in
  // order, then a wavefront tree, then the wavefronts in order.
  float sum = 0.f;
  int nt = 0;
  for (int i0 = tid; i0 < Lk; i0 += NT * 8) {
    float xn[8], xc[8];
    uint8_t xm[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {                                       // every load issued before any use
      const int ic = min(i0 + NT * u, L - 1);
      xn[u] = nb[ic];
      xc[u] = cb[ic];
      xm[u] = modality[ic];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + NT * u;
      if (i < L) {
        sum += xn[u];
        nt += xm[u] == 0;
        keys[i] = ((unsigned long long)__float_as_uint(xc[u]) << 32) | __float_as_uint(xn[u]);
        mods[i] = xm[u];
      } else if (i < Lk) {
        keys[i] = ~0ull;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sum += __shfl_xor(sum, off);
    nt += __shfl_xor(nt, off);
  }
  if (lane == 0) {
    red[w] = sum;
    redi[w] = nt;
  }
  __syncthreads();
  float tot = 0.f;
  int n_text = 0;
#pragma unroll
  for (int q = 0; q < kRankWaves; ++q) {
    tot += red[q];
    n_text += redi[q];
  }
  const float inv_mean = 1.f / (tot / (float)L);
  const int keep_text = (int)floor((double)r_text * (double)n_text + 0.5);
  const int keep_img = (int)floor((double)r_img * (double)(L - n_text) + 0.5);

  // Pass 2: the sort keys, in place
  for (int i = tid; i < L; i += NT) {
    const unsigned long long nc = keys[i];
    const float s = alpha * (__uint_as_float((unsigned)nc) * inv_mean) + (1.f - alpha) * __uint_as_float((unsigned)(nc >> 32));
    const unsigned long long seg = mods[i] ? 1ull : 0ull;
    keys[i] = (seg << 63) | ((unsigned long long)(~f2ord(s)) << 31) | (unsigned long long)i;
    if (scores && i >= c0 && i < c0 + kRankPos) scores[(size_t)b * L + i] = s;
  }
  __syncthreads();

  // lane l of wavefront w ranks position c0 + (l & 31) against key pairs
  // 2*(s + 16m), 2*(s + 16m) + 1, s = 2w + (l >> 5): the two half-wavefronts
  // read neighbouring 16-byte pairs, every other lane shares an address.
  // Lk is a multiple of 256, so every slice holds a multiple of 8 pairs.
  const int p = lane & 31, sl = 2 * w + (lane >> 5);
  const int ip = min(c0 + p, L - 1);
  const unsigned long long mine = keys[ip];
  int cnt = 0;
  const u32x4* kp = (const u32x4*)keys;
  constexpr int NS = 2 * kRankWaves;                                   // slices
  for (int q0 = sl; q0 < Lk / 2; q0 += 8 * NS) {
    u32x4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = kp[q0 + NS * u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const unsigned long long k0 = ((unsigned long long)x[u][1] << 32) | x[u][0];
      const unsigned long long k1 = ((unsigned long long)x[u][3] << 32) | x[u][2];
      cnt += (k0 < mine) + (k1 < mine);
    }
  }
  cnt += __shfl_xor(cnt, 32);
  if (lane < 32) part[w][lane] = cnt;
  __syncthreads();
  if (tid < kRankPos) {
    const int i = c0 + tid;
    int rank = 0;
#pragma unroll
    for (int q = 0; q < kRankWaves; ++q) rank += part[q][tid];
    bool kept = false;
    if (i < L) {
      const bool text = (mine >> 63) == 0;
      kept = text ? rank < keep_text : rank - n_text < keep_img;
    }
    flags[(size_t)b * round_up(L, kRankPos) + i] = kept;
  }
}

// Compaction and gather.  Grid (ceil(L / 16), B), 256 threads.  Workgroup x
// owns positions and output slots [16x, 16x + 16).  It scans the batch's
// flags (thread t holds flags 16t .. 16t+15) to find the slot of each kept
// position of its range, writes kept[b, slot] = position and copies the
// position's K and V rows (all heads) to row `slot` of k_out / v_out when
// slot < cap, and writes -1 to the entries of its slot range at or past K.
template <int D>
__global__ __launch_bounds__(256) void sprint_gather_kernel(const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const uint8_t* __restrict__ flags,
                                                            uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out,
                                                            int32_t* __restrict__ kept, int32_t* __restrict__ kept_count,
                                                            int Hkv, int L, int cap) {
  constexpr int CPR = D / 8;                                            // 16-byte chunks per row
  __shared__ int wsum[4];
  __shared__ int slot[kGatherPos];
  const int b = blockIdx.y, x = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int Lf = round_up(L, kRankPos), n16 = Lf / 16;
  const uint8_t* fb = flags + (size_t)b * Lf;
  // block-wide exclusive scan of the flag counts of 16-position groups
  int run = 0, before = 0, c = 0;
  for (int g0 = 0; g0 < n16; g0 += 256) {
    const int g = g0 + tid;
    c = 0;
    u32x4 f = {0u, 0u, 0u, 0u};
    if (g < n16) f = *(const u32x4*)(fb + 16 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) c += __builtin_popcount(f[e]);         // flags are 0 or 1 bytes
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = run;
    for (int q = 0; q < w; ++q) base += wsum[q];
    if (g == x) {
      before = base + incl - c;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool t = (f[e >> 2] >> (8 * (e & 3))) & 1u;
        slot[e] = t ? before : -1;
        before += t;
      }
    }
    run += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  const int K = run;
  if (tid == 0 && b == 0 && x == 0 && kept_count) *kept_count = K;
  if (tid < kGatherPos) {
    const int i = 16 * x + tid, sl = slot[tid];
    if (sl >= 0) kept[(size_t)b * L + sl] = i;
    if (i < L && i >= K) kept[(size_t)b * L + i] = -1;
  }
  if (cap == 0) return;
  // copy: 16 positions x Hkv heads x CPR chunks, k and v
  const int work = kGatherPos * Hkv * CPR;
  for (int t = tid; t < work; t += 256) {
    const int ch = t % CPR, r = t / CPR, h = r % Hkv, e = r / Hkv;
    const int sl = slot[e];
    if (sl < 0 || sl >= cap) continue;
    const int i = 16 * x + e;
    const size_t so = (((size_t)b * Hkv + h) * L + i) * D + 8 * ch;
    const size_t dso = (((size_t)b * Hkv + h) * cap + sl) * D + 8 * ch;
    *(u32x4*)(k_out + dso) = *(const u32x4*)(k + so);
    *(u32x4*)(v_out + dso) = *(const u32x4*)(v + so);
  }
}

int sprint_keep(int n, float r) { return (int)floor((double)r * (double)n + 0.5); }

size_t sprint_lds_bytes(int L) { return (size_t)round_up(L, 256) * 8 + (size_t)L; }

size_t sprint_ws_bytes(int B, int L) { return (size_t)B * L * 4 + (size_t)B * round_up(L, kRankPos) + 256; }

hipError_t sprint_launch(const void* k, const void* v, const float* conf, const uint8_t* modality, float alpha,
                         float r_img, float r_text, void* k_out, void* v_out, int cap, int32_t* kept,
                         int32_t* kept_count, float* scores, int B, int Hkv, int L, int d, void* ws,
                         hipStream_t st) {
  float* nrm = (float*)ws;
  (void)hipGetLastError();
  switch (d) {
    case 32: hipLaunchKernelGGL((sprint_norm_kernel<32>), dim3((L + 63) / 64, B), dim3(256), 0, st, (const uint16_t*)k, nrm, Hkv, L); break;
    case 64: hipLaunchKernelGGL((sprint_norm_kernel<64>), dim3((L + 31) / 32, B), dim3(256), 0, st, (const uint16_t*)k, nrm, Hkv, L); break;
    default: hipLaunchKernelGGL((sprint_norm_kernel<128>), dim3((L + 15) / 16, B), dim3(256), 0, st, (const uint16_t*)k, nrm, Hkv, L); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint8_t* flags = (uint8_t*)ws + ((size_t)B * L * 4 + 255) / 256 * 256;
  const size_t lds = sprint_lds_bytes(L);
  e = hipFuncSetAttribute((const void*)sprint_rank_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sprint_rank_kernel, dim3((L + kRankPos - 1) / kRankPos, B), dim3(kRankWaves * 64), lds, st, nrm,
                     conf, modality, alpha, r_img, r_text, L, round_up(L, 256), flags, scores);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gg((L + kGatherPos - 1) / kGatherPos, B);
  switch (d) {
    case 32: hipLaunchKernelGGL((sprint_gather_kernel<32>), gg, dim3(256), 0, st, (const uint16_t*)k, (const uint16_t*)v, flags, (uint16_t*)k_out, (uint16_t*)v_out, kept, kept_count, Hkv, L, cap); break;
    case 64: hipLaunchKernelGGL((sprint_gather_kernel<64>), gg, dim3(256), 0, st, (const uint16_t*)k, (const uint16_t*)v, flags, (uint16_t*)k_out, (uint16_t*)v_out, kept, kept_count, Hkv, L, cap); break;
    default: hipLaunchKernelGGL((sprint_gather_kernel<128>), gg, dim3(256), 0, st, (const uint16_t*)k, (const uint16_t*)v, flags, (uint16_t*)k_out, (uint16_t*)v_out, kept, kept_count, Hkv, L, cap); break;
  }
  return hipGetLastError();
}

}  // namespace bda
