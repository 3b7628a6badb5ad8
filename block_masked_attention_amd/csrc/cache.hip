// KV-cache append for per-row cache lengths (linear speculative decoding,
// [NLD-3x] sec. 2 and its KV-cache strategy: the cache of every sequence
// grows by the accepted drafts and is cut back past them).  Row b of the
// cache holds kv_len[b] valid keys, the last n of them the current block's;
// the block's fresh K/V rows are written there, so the lengths can stay on
// the device between steps.
#include "common.h"
#include "internal.h"

namespace bda {

// k_cache[b, h, L_b - n + j] = k_new[b, h, j] (same for v), L_b = kv_len[b]
// clamped to [n, L_cap].  One thread per 16-byte chunk.
template <int D>
__global__ __launch_bounds__(256) void kv_append_kernel(uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
                                                        const uint16_t* __restrict__ kn,
                                                        const uint16_t* __restrict__ vn,
                                                        const int32_t* __restrict__ kv_len, int Hkv, int L_cap,
                                                        int n, long long total) {
  constexpr int CPR = D / 8;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;         // over B*Hkv*n*CPR
  if (t >= total) return;
  const int c = (int)(t % CPR);
  const long long r = t / CPR;                                          // (b, h, j)
  const int j = (int)(r % n);
  const long long bh = r / n;
  const int b = (int)(bh / Hkv);
  const int Lb = min(L_cap, max(n, kv_len[b]));
  const size_t dst = ((size_t)bh * L_cap + (Lb - n + j)) * D + 8 * c;
  const size_t src = (size_t)r * D + 8 * c;
  *(u32x4*)(kc + dst) = *(const u32x4*)(kn + src);
  *(u32x4*)(vc + dst) = *(const u32x4*)(vn + src);
}

hipError_t kv_append_launch(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* kv_len, int B, int Hkv, int L_cap, int n, int d, hipStream_t st) {
  (void)hipGetLastError();
  const long long total = (long long)B * Hkv * n * (d / 8);
  const unsigned g = (unsigned)((total + 255) / 256);
  if (d == 32)
    hipLaunchKernelGGL((kv_append_kernel<32>), dim3(g), dim3(256), 0, st, (uint16_t*)k_cache, (uint16_t*)v_cache,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, kv_len, Hkv, L_cap, n, total);
  else if (d == 64)
    hipLaunchKernelGGL((kv_append_kernel<64>), dim3(g), dim3(256), 0, st, (uint16_t*)k_cache, (uint16_t*)v_cache,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, kv_len, Hkv, L_cap, n, total);
  else
    hipLaunchKernelGGL((kv_append_kernel<128>), dim3(g), dim3(256), 0, st, (uint16_t*)k_cache, (uint16_t*)v_cache,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, kv_len, Hkv, L_cap, n, total);
  return hipGetLastError();
}

}  // namespace bda
