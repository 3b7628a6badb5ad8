// Host driver for the sanitizer build of libbda's host code (test
// infrastructure).  The library's sources are compiled for the host only
// (no device code) with AddressSanitizer and UndefinedBehaviorSanitizer, and
// this program drives every path that runs before a launch: argument
// validation of every entry point with bad arguments, the workspace-size
// queries over a sweep of shapes (the plans behind them), the tile
// classifier and the SPRINT keep counts.  Nothing here touches a device.
// Prints "ok" and returns 0 when every call returned as expected.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bda.h"

static int failures = 0;
#define EXPECT(cond)                                                          \
  do {                                                                        \
    if (!(cond)) {                                                            \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond);     \
      ++failures;                                                             \
    }                                                                         \
  } while (0)

// Distinct, 16-byte aligned, far-apart stand-ins for device addresses: every
// call below fails validation before any HIP call, so none is dereferenced.
static void* fake(int i) { return (void*)((uintptr_t)i << 36); }

int main() {
  // error strings and version
  for (int c = 0; c < 6; ++c) EXPECT(bda_strerror(c) != nullptr && strlen(bda_strerror(c)) > 0);
  EXPECT(strlen(bda_version()) > 0);

  // attention: bad arguments of every kind, for all three modes
  void *q = fake(1), *k = fake(2), *v = fake(3), *o = fake(4), *ws = fake(5);
  for (int mode = 0; mode < 3; ++mode) {
    EXPECT(bda_attn_fwd(nullptr, k, v, o, 1, 4, 2, 64, 128, 8, mode, nullptr, 0, nullptr) == BDA_EINVAL);
    EXPECT(bda_attn_fwd(q, k, v, o, 1, 3, 2, 64, 128, 8, mode, nullptr, 0, nullptr) == BDA_EINVAL);
    EXPECT(bda_attn_fwd(q, k, v, o, 1, 4, 2, 64, 96, 8, mode, nullptr, 0, nullptr) == BDA_EUNSUPPORTED);
    EXPECT(bda_attn_fwd(q, k, v, o, 1, 4, 2, 64, 128, 0, mode, nullptr, 0, nullptr) == BDA_EINVAL);
    EXPECT(bda_attn_fwd(q, k, v, o, 1, 4, 2, 64, 128, 65, mode, nullptr, 0, nullptr) == BDA_EINVAL);
    EXPECT(bda_attn_fwd(q, k, v, o, 0, 4, 2, 64, 128, 8, mode, nullptr, 0, nullptr) == BDA_EINVAL);
    EXPECT(bda_attn_fwd((char*)q + 8, k, v, o, 1, 4, 2, 64, 128, 8, mode, nullptr, 0, nullptr) == BDA_EINVAL);
    EXPECT(bda_attn_fwd(q, k, v, (char*)q + 64, 1, 4, 2, 64, 128, 8, mode, nullptr, 0, nullptr) == BDA_EINVAL);
    EXPECT(bda_attn_fwd_lse(q, k, v, o, nullptr, 1, 4, 2, 64, 128, 8, mode, nullptr, 0, nullptr) == BDA_EINVAL);
    EXPECT(bda_attn_fwd_lse(q, k, v, o, (float*)((char*)o + 4), 1, 4, 2, 64, 128, 8, mode, nullptr, 0,
                            nullptr) == BDA_EINVAL);
  }
  EXPECT(bda_attn_fwd(q, k, v, o, 1, 4, 2, 64, 128, 8, 3, nullptr, 0, nullptr) == BDA_EINVAL);
  // a split-key call without its workspace, and with too little
  EXPECT(bda_attn_workspace_bytes(16, 32, 8, 8220, 128, 28, BDA_MODE_CAUSAL) > 0);
  EXPECT(bda_attn_fwd(q, k, v, o, 16, 32, 8, 8220, 128, 28, BDA_MODE_CAUSAL, nullptr, 0, nullptr) == BDA_EWORKSPACE);
  EXPECT(bda_attn_fwd(q, k, v, o, 16, 32, 8, 8220, 128, 28, BDA_MODE_CAUSAL, ws, 16, nullptr) == BDA_EWORKSPACE);
  EXPECT(bda_attn_fwd_varlen(q, k, v, o, nullptr, 2, 4, 2, 64, 128, 8, BDA_MODE_DECODE, nullptr, 0, nullptr) ==
         BDA_EINVAL);
  EXPECT(bda_attn_fwd_varlen(q, k, v, o, (const int32_t*)ws, 2, 4, 2, 64, 128, 8, BDA_MODE_HYBRID, nullptr, 0,
                             nullptr) == BDA_EUNSUPPORTED);
  EXPECT(bda_kv_append(k, v, q, o, nullptr, 2, 2, 64, 8, 128, nullptr) == BDA_EINVAL);
  EXPECT(bda_kv_append(k, v, q, o, (const int32_t*)ws, 2, 2, 4, 8, 128, nullptr) == BDA_EINVAL);
  EXPECT(bda_kv_append(k, v, q, o, (const int32_t*)ws, 2, 2, 64, 8, 96, nullptr) == BDA_EUNSUPPORTED);
  // backward: modes other than the training form, bad shapes
  EXPECT(bda_attn_bwd(q, k, v, o, q, (const float*)ws, q, k, v, 1, 2, 1, 16, 32, 8, BDA_MODE_DECODE, ws, 1 << 16,
                      nullptr) != BDA_OK);
  EXPECT(bda_attn_bwd(nullptr, k, v, o, q, (const float*)ws, q, k, v, 1, 2, 1, 16, 32, 8, BDA_MODE_HYBRID, ws,
                      1 << 16, nullptr) != BDA_OK);

  // workspace sizes (the plans behind them) over a sweep of shapes
  const int dims[3] = {32, 64, 128};
  for (int mode = 0; mode < 3; ++mode)
    for (int di = 0; di < 3; ++di)
      for (int L = 1; L <= 600; L += 37)
        for (int b = 1; b <= L; b += 1 + L / 5) {
          const size_t a = bda_attn_workspace_bytes(3, 8, 2, L, dims[di], b, mode);
          EXPECT(a == 0 || mode != BDA_MODE_HYBRID);
          if (mode == BDA_MODE_HYBRID) (void)bda_attn_bwd_workspace_bytes(3, 8, 2, L, dims[di], b, mode);
        }
  EXPECT(bda_attn_workspace_bytes(4, 32, 8, 2048, 128, 32, BDA_MODE_HYBRID) == 0);
  EXPECT(bda_attn_workspace_bytes(1, 4, 2, 64, 96, 8, 0) == 0);
  for (int V = 1; V < 300000; V = V * 3 + 1) {
    EXPECT(bda_commit_workspace_bytes(32, 28, V) > 0);
    EXPECT(bda_verify_workspace_bytes(16, 28, V) > 0);
    EXPECT(bda_row_stats_workspace_bytes(32, 28, V) > 0);
    EXPECT(bda_commit_entropy_workspace_bytes(32, 28, V) > 0);
  }
  EXPECT(bda_commit_workspace_bytes(-1, 28, 10) == 0);

  // commit family: bad arguments
  int64_t* tok = (int64_t*)fake(6);
  uint8_t* msk = (uint8_t*)fake(7);
  EXPECT(bda_commit(q, 7, tok, msk, 0.9f, 1, 2, 4, 100, ws, 1 << 20, nullptr) == BDA_EINVAL);
  EXPECT(bda_commit(q, BDA_BF16, tok, msk, 0.9f, -1, 2, 4, 100, ws, 1 << 20, nullptr) == BDA_EINVAL);
  EXPECT(bda_commit(q, BDA_BF16, tok, msk, 0.9f, 1, 2, 4, 0, ws, 1 << 20, nullptr) == BDA_EINVAL);
  EXPECT(bda_commit(q, BDA_BF16, nullptr, msk, 0.9f, 1, 2, 4, 100, ws, 1 << 20, nullptr) == BDA_EINVAL);
  EXPECT(bda_commit(q, BDA_BF16, tok, msk, 0.9f, 1, 2, 4, 100, nullptr, 0, nullptr) == BDA_EWORKSPACE);
  EXPECT(bda_commit(q, BDA_BF16, (int64_t*)q, msk, 0.9f, 1, 2, 4, 100, ws, 1 << 20, nullptr) == BDA_EINVAL);
  EXPECT(bda_commit(q, BDA_BF16, tok, msk, 0.9f, 1, 0, 4, 100, nullptr, 0, nullptr) == BDA_OK);   // nothing to do
  EXPECT(bda_commit_noalloc(q, BDA_BF16, tok, msk, 0.9f, 1, 64, 128, 131072, nullptr) == BDA_EWORKSPACE);
  EXPECT(bda_commit_noalloc(q, BDA_BF16, tok, msk, 0.9f, -1, 2, 4, 100, nullptr) == BDA_EINVAL);
  EXPECT(bda_commit_entropy(q, BDA_BF16, tok, msk, 3.f, 0.f, 1, 2, 4, 100, ws, 1 << 20, nullptr) == BDA_EINVAL);
  EXPECT(bda_commit_entropy(q, BDA_BF16, tok, msk, 3.f, 1.f, 1, 2, 5000, 100, ws, 1 << 30, nullptr) ==
         BDA_EUNSUPPORTED);
  EXPECT(bda_verify(q, BDA_BF16, (const int64_t*)k, tok, nullptr, 2, 4, 100, ws, 1 << 20, nullptr) == BDA_EINVAL);
  EXPECT(bda_verify(q, BDA_BF16, (const int64_t*)k, tok, (int32_t*)msk, 2, 4, 100, nullptr, 0, nullptr) ==
         BDA_EWORKSPACE);
  EXPECT(bda_verify_crop(q, BDA_BF16, (const int64_t*)k, tok, (int32_t*)msk, nullptr, 10, 2, 4, 100, ws, 1 << 20,
                         nullptr) == BDA_EINVAL);
  EXPECT(bda_row_stats(q, 5, nullptr, nullptr, nullptr, nullptr, nullptr, 2, 4, 100, ws, 1 << 20, nullptr) ==
         BDA_EINVAL);
  EXPECT(bda_row_stats_commit(q, 5, tok, msk, 0.9f, 1, nullptr, nullptr, nullptr, nullptr, 2, 4, 100, ws, 1 << 20,
                              nullptr) == BDA_EINVAL);
  EXPECT(bda_row_stats_commit(q, BDA_BF16, tok, msk, 0.9f, 1, nullptr, nullptr, nullptr, nullptr, 2, 4, 100, nullptr,
                              0, nullptr) == BDA_EWORKSPACE);
  EXPECT(bda_row_stats_commit(q, BDA_BF16, tok, msk, 0.9f, 1, (float*)q, nullptr, nullptr, nullptr, 2, 4, 100, ws,
                              1 << 20, nullptr) == BDA_EINVAL);   // conf overlaps the logits
  EXPECT(bda_row_stats_commit_workspace_bytes(2, 4, 100) == bda_commit_workspace_bytes(2, 4, 100));
  EXPECT(bda_adaptive_stop(tok, tok, (int32_t*)msk, msk, (const float*)ws, 2, 4, -1, 0.005f, nullptr, nullptr) ==
         BDA_EINVAL);
  EXPECT(bda_adaptive_stop(tok, tok, (int32_t*)msk, msk, (const float*)ws, 2, 4, 1, 0.005f, nullptr, nullptr) ==
         BDA_EINVAL);   // prev_argmax aliases argmax

  // SPRINT: sizes and keep counts
  for (int L = 1; L < 20000; L = L * 2 + 3) EXPECT(bda_sprint_workspace_bytes(2, L) > 0);
  EXPECT(bda_sprint_kept_count(3080, 1016, 0.8f, 1.0f) == 2464 + 1016);
  EXPECT(bda_sprint_kept_count(0, 0, 0.5f, 0.5f) == 0);
  EXPECT(bda_sprint_prune(nullptr, v, (const float*)ws, msk, 0.5f, 0.8f, 1.f, k, o, 64, nullptr, nullptr, nullptr,
                          2, 2, 64, 128, ws, 1 << 20, nullptr) != BDA_OK);

  // tile classifier: every mode over a sweep of small tiles
  for (int mode = 0; mode < 3; ++mode)
    for (int L = 1; L <= 24; ++L)
      for (int b = 1; b <= L; ++b) {
        const int rows = mode == 0 ? 2 * L : b, keys = mode == 0 ? 2 * L : L;
        for (int q0 = 0; q0 < rows; q0 += 3)
          for (int k0 = 0; k0 < keys; k0 += 5) {
            const int c = bda_classify_tile(mode, L, b, q0, q0 + 4 < rows ? q0 + 4 : rows, k0,
                                            k0 + 7 < keys ? k0 + 7 : keys);
            EXPECT(c >= 0 && c <= 2);
          }
      }
  EXPECT(bda_classify_tile(7, 8, 2, 0, 1, 0, 1) < 0);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
