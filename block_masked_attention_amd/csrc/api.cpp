// C ABI of libbda: argument validation, error reporting, dispatch to the
// kernel launchers.  Validation always runs on the host before any launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/bda.h"
#include "geometry.h"
#include "internal.h"

namespace {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return BDA_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const char* x = (const char*)a;
  const char* y = (const char*)b;
  return x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_attn(int B, int Hq, int Hkv, int L, int d, int block, int mode) {
  if (mode < BDA_MODE_HYBRID || mode > BDA_MODE_CAUSAL) return fail(BDA_EINVAL, "mode %d is not one of 0,1,2", mode);
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1) return fail(BDA_EINVAL, "B, Hq, Hkv and L must be >= 1");
  if (Hq % Hkv) return fail(BDA_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (d != 32 && d != 64 && d != 128) return fail(BDA_EUNSUPPORTED, "head dim %d not in {32, 64, 128}", d);
  if (block < 1 || block > L) return fail(BDA_EINVAL, "block %d must be in [1, L=%d]", block, L);
  if (L > (1 << 28)) return fail(BDA_EUNSUPPORTED, "L %d above 2^28", L);
  return BDA_OK;
}

}  // namespace

extern "C" {

const char* bda_strerror(int code) {
  switch (code) {
    case BDA_OK: return "ok";
    case BDA_EINVAL: return "invalid argument";
    case BDA_EUNSUPPORTED: return "unsupported configuration";
    case BDA_EWORKSPACE: return "workspace missing or too small";
    case BDA_EHIP: return "HIP runtime error";
    default: return "unknown error code";
  }
}

const char* bda_last_error(void) { return g_err; }

const char* bda_version(void) { return "bda 0.1 (gfx950)"; }

size_t bda_attn_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int block, int mode) {
  if (check_attn(B, Hq, Hkv, L, d, block, mode)) return 0;
  bda::AttnPlan p;
  const char* why = "";
  if (bda::attn_make_plan(B, Hq, Hkv, L, d, block, mode, &p, &why)) return 0;
  return p.ws_bytes;
}

static int attn_fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse,
                         const int32_t* kv_len, int B, int Hq, int Hkv, int L, int d, int block, int mode,
                         void* workspace, size_t ws_bytes, void* stream) {
  if (int e = check_attn(B, Hq, Hkv, L, d, block, mode)) return e;
  if (!q || !k || !v || !out) return fail(BDA_EINVAL, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(BDA_EINVAL, "q, k, v and out must be 16-byte aligned");
  const size_t Sq = mode == BDA_MODE_HYBRID ? 2 * (size_t)L : (size_t)block;
  const size_t Sk = mode == BDA_MODE_HYBRID ? 2 * (size_t)L : (size_t)L;
  const size_t qbytes = (size_t)B * Hq * Sq * d * 2;
  const size_t kbytes = (size_t)B * Hkv * Sk * d * 2;
  if (overlap(out, qbytes, q, qbytes) || overlap(out, qbytes, k, kbytes) || overlap(out, qbytes, v, kbytes))
    return fail(BDA_EINVAL, "out overlaps q, k or v");
  const size_t lbytes = (size_t)B * Hq * Sq * 4;
  if (lse && (!aligned16(lse) || overlap(lse, lbytes, q, qbytes) || overlap(lse, lbytes, k, kbytes) ||
              overlap(lse, lbytes, v, kbytes) || overlap(lse, lbytes, out, qbytes)))
    return fail(BDA_EINVAL, "lse must be 16-byte aligned and must not overlap q, k, v or out");
  if (kv_len && lse) return fail(BDA_EUNSUPPORTED, "per-row key counts with the log-sum-exp output");
  if (kv_len && (((uintptr_t)kv_len & 3) || overlap(kv_len, (size_t)B * 4, out, qbytes) ||
                 (lse && overlap(kv_len, (size_t)B * 4, lse, lbytes))))
    return fail(BDA_EINVAL, "kv_len must be 4-byte aligned and must not overlap out or lse");
  bda::AttnPlan p;
  const char* why = "";
  if (int e = bda::attn_make_plan(B, Hq, Hkv, L, d, block, mode, &p, &why))
    return fail(e == 2 ? BDA_EUNSUPPORTED : BDA_EINVAL, "%s", why);
  if (p.ws_bytes) {
    if (!workspace || ws_bytes < p.ws_bytes)
      return fail(BDA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                  workspace ? ws_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(BDA_EINVAL, "workspace must be 16-byte aligned");
    if (overlap(workspace, p.ws_bytes, out, qbytes) || overlap(workspace, p.ws_bytes, q, qbytes) ||
        overlap(workspace, p.ws_bytes, k, kbytes) || overlap(workspace, p.ws_bytes, v, kbytes) ||
        (lse && overlap(workspace, p.ws_bytes, lse, lbytes)))
      return fail(BDA_EINVAL, "workspace overlaps a tensor argument");
  }
  if (kv_len && p.ws_bytes && overlap(workspace, p.ws_bytes, kv_len, (size_t)B * 4))
    return fail(BDA_EINVAL, "workspace overlaps kv_len");
  hipError_t e = bda::attn_launch(p, q, k, v, out, lse, kv_len, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int bda_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv,
                 int L, int d, int block, int mode, void* workspace, size_t ws_bytes, void* stream) {
  return attn_fwd_impl(q, k, v, out, nullptr, nullptr, B, Hq, Hkv, L, d, block, mode, workspace, ws_bytes,
                       stream);
}

int bda_attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, const int32_t* kv_len, int B,
                        int Hq, int Hkv, int L_cap, int d, int block, int mode, void* workspace,
                        size_t ws_bytes, void* stream) {
  if (mode != BDA_MODE_DECODE && mode != BDA_MODE_CAUSAL)
    return fail(BDA_EUNSUPPORTED, "per-row key counts apply to the DECODE and CAUSAL forms only");
  if (!kv_len) return fail(BDA_EINVAL, "kv_len must be non-NULL");
  return attn_fwd_impl(q, k, v, out, nullptr, kv_len, B, Hq, Hkv, L_cap, d, block, mode, workspace, ws_bytes,
                       stream);
}

int bda_attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                     int Hkv, int L, int d, int block, int mode, void* workspace, size_t ws_bytes,
                     void* stream) {
  if (!lse) return fail(BDA_EINVAL, "lse must be non-NULL");
  return attn_fwd_impl(q, k, v, out, lse, nullptr, B, Hq, Hkv, L, d, block, mode, workspace, ws_bytes, stream);
}

static int check_logits(const void* logits, int dtype, int G, int R, int V, const char* gname) {
  if (dtype != BDA_BF16 && dtype != BDA_F32) return fail(BDA_EINVAL, "dtype %d is not BDA_BF16 or BDA_F32", dtype);
  if (G < 0 || R < 0) return fail(BDA_EINVAL, "%s and R must be >= 0", gname);
  if (V < 1) return fail(BDA_EINVAL, "V must be >= 1");
  if ((size_t)G * R > (size_t)0x7fffffff / 64) return fail(BDA_EUNSUPPORTED, "too many rows");
  if ((size_t)G * R > 0 && !logits) return fail(BDA_EINVAL, "logits must be non-NULL");
  return BDA_OK;
}

size_t bda_commit_workspace_bytes(int G, int R, int V) {
  if (G < 0 || R < 0 || V < 1) return 0;
  bda::CommitPlan p;
  bda::commit_make_plan(G, R, V, 0, &p);
  return p.ws_bytes;
}

int bda_commit(const void* logits, int dtype, int64_t* tokens, uint8_t* masked, float threshold,
               int k_min, int G, int R, int V, void* workspace, size_t ws_bytes, void* stream) {
  if (int e = check_logits(logits, dtype, G, R, V, "G")) return e;
  if (k_min < 0) return fail(BDA_EINVAL, "k_min must be >= 0");
  if (isnan(threshold)) return fail(BDA_EINVAL, "threshold is NaN");
  const size_t rows = (size_t)G * R;
  if (rows == 0) return ok();
  if (!tokens || !masked) return fail(BDA_EINVAL, "tokens and masked must be non-NULL");
  const size_t lbytes = rows * V * (dtype == BDA_BF16 ? 2 : 4);
  if (overlap(tokens, rows * 8, logits, lbytes) || overlap(masked, rows, logits, lbytes) ||
      overlap(tokens, rows * 8, masked, rows))
    return fail(BDA_EINVAL, "tokens, masked and logits must not overlap");
  bda::CommitPlan p;
  bda::commit_make_plan(G, R, V, dtype, &p);
  if (!workspace || ws_bytes < p.ws_bytes)
    return fail(BDA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                workspace ? ws_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(BDA_EINVAL, "workspace must be 16-byte aligned");
  if (overlap(workspace, p.ws_bytes, logits, lbytes) || overlap(workspace, p.ws_bytes, tokens, rows * 8) ||
      overlap(workspace, p.ws_bytes, masked, rows))
    return fail(BDA_EINVAL, "workspace overlaps a tensor argument");
  hipError_t e = bda::commit_launch(p, logits, tokens, masked, threshold, k_min, workspace,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

static_assert(BDA_COMMIT_NOALLOC_MAX_BYTES == bda::kCommitNoAllocBytes, "static scratch size mismatch");

int bda_commit_noalloc(const void* logits, int dtype, int64_t* tokens, uint8_t* masked, float threshold,
                       int k_min, int G, int R, int V, void* stream) {
  if (int e = check_logits(logits, dtype, G, R, V, "G")) return e;
  if (k_min < 0) return fail(BDA_EINVAL, "k_min must be >= 0");
  if (isnan(threshold)) return fail(BDA_EINVAL, "threshold is NaN");
  const size_t rows = (size_t)G * R;
  if (rows == 0) return ok();
  if (!tokens || !masked) return fail(BDA_EINVAL, "tokens and masked must be non-NULL");
  const size_t lbytes = rows * V * (dtype == BDA_BF16 ? 2 : 4);
  if (overlap(tokens, rows * 8, logits, lbytes) || overlap(masked, rows, logits, lbytes) ||
      overlap(tokens, rows * 8, masked, rows))
    return fail(BDA_EINVAL, "tokens, masked and logits must not overlap");
  bda::CommitPlan p;
  bda::commit_make_plan(G, R, V, dtype, &p);
  if (p.ws_bytes > bda::kCommitNoAllocBytes)
    return fail(BDA_EWORKSPACE, "G x R x V = %d x %d x %d needs %zu bytes of scratch, above the %zu bytes of "
                "the static scratch; use bda_commit with a workspace", G, R, V, p.ws_bytes,
                bda::kCommitNoAllocBytes);
  void* scratch = nullptr;
  hipError_t e = bda::commit_noalloc_scratch(&scratch);
  if (e != hipSuccess) return fail(BDA_EHIP, "static scratch address: %s", hipGetErrorString(e));
  e = bda::commit_launch(p, logits, tokens, masked, threshold, k_min, scratch, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t bda_verify_workspace_bytes(int B, int R, int V) { return bda_commit_workspace_bytes(B, R, V); }

size_t bda_commit_entropy_workspace_bytes(int G, int R, int V) { return bda_commit_workspace_bytes(G, R, V); }

int bda_commit_entropy(const void* logits, int dtype, int64_t* tokens, uint8_t* masked, float entropy_bound,
                       float temperature, int k_min, int G, int R, int V, void* workspace, size_t ws_bytes,
                       void* stream) {
  if (int e = check_logits(logits, dtype, G, R, V, "G")) return e;
  if (k_min < 0) return fail(BDA_EINVAL, "k_min must be >= 0");
  if (isnan(entropy_bound)) return fail(BDA_EINVAL, "entropy_bound is NaN");
  if (!(temperature > 0.f) || isinf(temperature)) return fail(BDA_EINVAL, "temperature must be finite and > 0");
  if (R > bda::commit_entropy_max_rows())
    return fail(BDA_EUNSUPPORTED, "R above %d rows per group", bda::commit_entropy_max_rows());
  const size_t rows = (size_t)G * R;
  if (rows == 0) return ok();
  if (!tokens || !masked) return fail(BDA_EINVAL, "tokens and masked must be non-NULL");
  const size_t lbytes = rows * V * (dtype == BDA_BF16 ? 2 : 4);
  if (overlap(tokens, rows * 8, logits, lbytes) || overlap(masked, rows, logits, lbytes) ||
      overlap(tokens, rows * 8, masked, rows))
    return fail(BDA_EINVAL, "tokens, masked and logits must not overlap");
  bda::CommitPlan p;
  bda::commit_make_plan(G, R, V, dtype, &p);
  if (!workspace || ws_bytes < p.ws_bytes)
    return fail(BDA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                workspace ? ws_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(BDA_EINVAL, "workspace must be 16-byte aligned");
  if (overlap(workspace, p.ws_bytes, logits, lbytes) || overlap(workspace, p.ws_bytes, tokens, rows * 8) ||
      overlap(workspace, p.ws_bytes, masked, rows))
    return fail(BDA_EINVAL, "workspace overlaps a tensor argument");
  hipError_t e = bda::commit_entropy_launch(p, logits, tokens, masked, entropy_bound, temperature, k_min, workspace,
                                            (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int bda_adaptive_stop(const int64_t* argmax, int64_t* prev_argmax, int32_t* stable_steps, uint8_t* frozen,
                      const float* mean_entropy, int G, int R, int stability_threshold,
                      float confidence_threshold, int32_t* n_frozen, void* stream) {
  if (G < 0 || R < 0) return fail(BDA_EINVAL, "G and R must be >= 0");
  if (stability_threshold < 0) return fail(BDA_EINVAL, "stability_threshold must be >= 0");
  if (isnan(confidence_threshold)) return fail(BDA_EINVAL, "confidence_threshold is NaN");
  if (G == 0 && !n_frozen) return ok();
  if (G > 0 && (!stable_steps || !frozen || !mean_entropy || (R > 0 && (!argmax || !prev_argmax))))
    return fail(BDA_EINVAL, "argmax, prev_argmax, stable_steps, frozen and mean_entropy must be non-NULL");
  const size_t rows = (size_t)G * R;
  if (((uintptr_t)argmax & 7) || ((uintptr_t)prev_argmax & 7) || ((uintptr_t)stable_steps & 3) ||
      ((uintptr_t)mean_entropy & 3) || ((uintptr_t)n_frozen & 3))
    return fail(BDA_EINVAL, "arguments must be aligned to their element size");
  if (rows && (overlap(prev_argmax, rows * 8, argmax, rows * 8) || overlap(stable_steps, (size_t)G * 4, prev_argmax, rows * 8) ||
               overlap(frozen, (size_t)G, prev_argmax, rows * 8)))
    return fail(BDA_EINVAL, "outputs must not overlap each other or argmax");
  hipError_t e = bda::adaptive_stop_launch(argmax, prev_argmax, stable_steps, frozen, mean_entropy, G, R,
                                           stability_threshold, confidence_threshold, n_frozen, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

static int verify_impl(const void* logits, int dtype, const int64_t* drafts, int64_t* argmax_out,
                       int32_t* accept_len, int32_t* kv_len, int kv_cap, int B, int R, int V, void* workspace,
                       size_t ws_bytes, void* stream) {
  if (int e = check_logits(logits, dtype, B, R, V, "B")) return e;
  if (B == 0) return ok();
  if (!accept_len) return fail(BDA_EINVAL, "accept_len must be non-NULL");
  const size_t rows = (size_t)B * R;
  if (rows && (!drafts || !argmax_out)) return fail(BDA_EINVAL, "drafts and argmax_out must be non-NULL");
  const size_t lbytes = rows * V * (dtype == BDA_BF16 ? 2 : 4);
  if (rows && (overlap(argmax_out, rows * 8, logits, lbytes) || overlap(argmax_out, rows * 8, drafts, rows * 8) ||
               overlap(accept_len, (size_t)B * 4, logits, lbytes) ||
               overlap(accept_len, (size_t)B * 4, argmax_out, rows * 8)))
    return fail(BDA_EINVAL, "outputs must not overlap inputs or each other");
  bda::CommitPlan p;
  bda::commit_make_plan(B, R, V, dtype, &p);
  if (!workspace || ws_bytes < p.ws_bytes)
    return fail(BDA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                workspace ? ws_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(BDA_EINVAL, "workspace must be 16-byte aligned");
  if (kv_len && (((uintptr_t)kv_len & 3) || overlap(kv_len, (size_t)B * 4, accept_len, (size_t)B * 4) ||
                 overlap(kv_len, (size_t)B * 4, logits, lbytes) ||
                 (rows && overlap(kv_len, (size_t)B * 4, argmax_out, rows * 8))))
    return fail(BDA_EINVAL, "kv_len must be 4-byte aligned and must not overlap the other arguments");
  hipError_t e = bda::verify_launch(p, logits, drafts, argmax_out, accept_len, kv_len, kv_cap, workspace,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int bda_verify(const void* logits, int dtype, const int64_t* drafts, int64_t* argmax_out,
               int32_t* accept_len, int B, int R, int V, void* workspace, size_t ws_bytes,
               void* stream) {
  return verify_impl(logits, dtype, drafts, argmax_out, accept_len, nullptr, 0, B, R, V, workspace, ws_bytes,
                     stream);
}

int bda_verify_crop(const void* logits, int dtype, const int64_t* drafts, int64_t* argmax_out,
                    int32_t* accept_len, int32_t* kv_len, int kv_cap, int B, int R, int V, void* workspace,
                    size_t ws_bytes, void* stream) {
  if (!kv_len) return fail(BDA_EINVAL, "kv_len must be non-NULL");
  if (kv_cap < 1) return fail(BDA_EINVAL, "kv_cap must be >= 1");
  return verify_impl(logits, dtype, drafts, argmax_out, accept_len, kv_len, kv_cap, B, R, V, workspace, ws_bytes,
                     stream);
}

int bda_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, const int32_t* kv_len,
                  int B, int Hkv, int L_cap, int n, int d, void* stream) {
  if (B < 0 || Hkv < 1 || n < 1 || L_cap < n) return fail(BDA_EINVAL, "need B >= 0, Hkv >= 1 and 1 <= n <= L_cap");
  if (d != 32 && d != 64 && d != 128) return fail(BDA_EUNSUPPORTED, "d must be 32, 64 or 128");
  if (B == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !kv_len) return fail(BDA_EINVAL, "pointers must be non-NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) || ((uintptr_t)kv_len & 3))
    return fail(BDA_EINVAL, "caches and new rows must be 16-byte aligned, kv_len 4-byte aligned");
  const size_t cb = (size_t)B * Hkv * L_cap * d * 2, nb = (size_t)B * Hkv * n * d * 2;
  if (overlap(k_cache, cb, v_cache, cb) || overlap(k_cache, cb, k_new, nb) || overlap(k_cache, cb, v_new, nb) ||
      overlap(v_cache, cb, k_new, nb) || overlap(v_cache, cb, v_new, nb) ||
      overlap(k_cache, cb, kv_len, (size_t)B * 4) || overlap(v_cache, cb, kv_len, (size_t)B * 4))
    return fail(BDA_EINVAL, "caches overlap each other or an input");
  hipError_t e = bda::kv_append_launch(k_cache, v_cache, k_new, v_new, kv_len, B, Hkv, L_cap, n, d,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t bda_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int block, int mode) {
  if (mode != BDA_MODE_HYBRID || check_attn(B, Hq, Hkv, L, d, block, mode) != BDA_OK) return 0;
  bda::BwdPlan p;
  const char* why = "";
  if (bda::bwd_make_plan(B, Hq, Hkv, L, d, block, &p, &why)) return 0;
  return p.ws_bytes;
}

int bda_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int L, int d,
                 int block, int mode, void* workspace, size_t ws_bytes, void* stream) {
  if (int e = check_attn(B, Hq, Hkv, L, d, block, mode)) return e;
  if (mode != BDA_MODE_HYBRID) return fail(BDA_EUNSUPPORTED, "the backward is implemented for the hybrid form only");
  const void* in[] = {q, k, v, out, dout, lse, dq, dk, dv};
  for (const void* x : in)
    if (!x) return fail(BDA_EINVAL, "q, k, v, out, dout, lse, dq, dk and dv must be non-NULL");
  for (const void* x : in)
    if (!aligned16(x)) return fail(BDA_EINVAL, "all tensors must be 16-byte aligned");
  const size_t S = 2 * (size_t)L;
  const size_t qb = (size_t)B * Hq * S * d * 2, kb = (size_t)B * Hkv * S * d * 2, lb = (size_t)B * Hq * S * 4;
  const void* ins[] = {q, k, v, out, dout, lse};
  const size_t insz[] = {qb, kb, kb, qb, qb, lb};
  void* outs[] = {dq, dk, dv};
  const size_t outsz[] = {qb, kb, kb};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return fail(BDA_EINVAL, "gradients must not overlap inputs");
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return fail(BDA_EINVAL, "gradients must not overlap");
  }
  bda::BwdPlan p;
  const char* why = "";
  if (int e = bda::bwd_make_plan(B, Hq, Hkv, L, d, block, &p, &why))
    return fail(e == 2 ? BDA_EUNSUPPORTED : BDA_EINVAL, "%s", why);
  if (!workspace || ws_bytes < p.ws_bytes)
    return fail(BDA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                workspace ? ws_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(BDA_EINVAL, "workspace must be 16-byte aligned");
  for (int j = 0; j < 6; ++j)
    if (overlap(workspace, p.ws_bytes, ins[j], insz[j])) return fail(BDA_EINVAL, "workspace overlaps an input");
  for (int i = 0; i < 3; ++i)
    if (overlap(workspace, p.ws_bytes, outs[i], outsz[i])) return fail(BDA_EINVAL, "workspace overlaps a gradient");
  hipError_t e = bda::bwd_launch(p, q, k, v, out, dout, lse, dq, dk, dv, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t bda_row_stats_workspace_bytes(int G, int R, int V) { return bda_commit_workspace_bytes(G, R, V); }

int bda_row_stats(const void* logits, int dtype, const uint8_t* masked, float* conf, int64_t* argmax_out,
                  float* entropy, float* mean_entropy, int G, int R, int V, void* workspace,
                  size_t ws_bytes, void* stream) {
  if (int e = check_logits(logits, dtype, G, R, V, "G")) return e;
  if (G == 0) return ok();
  const size_t rows = (size_t)G * R;
  const size_t lbytes = rows * V * (dtype == BDA_BF16 ? 2 : 4);
  if (rows && ((conf && overlap(conf, rows * 4, logits, lbytes)) ||
               (argmax_out && overlap(argmax_out, rows * 8, logits, lbytes)) ||
               (entropy && overlap(entropy, rows * 4, logits, lbytes)) ||
               (conf && argmax_out && overlap(conf, rows * 4, argmax_out, rows * 8)) ||
               (conf && entropy && overlap(conf, rows * 4, entropy, rows * 4)) ||
               (entropy && argmax_out && overlap(entropy, rows * 4, argmax_out, rows * 8))))
    return fail(BDA_EINVAL, "outputs must not overlap the logits or each other");
  if (mean_entropy && (overlap(mean_entropy, (size_t)G * 4, logits, lbytes) ||
                       (conf && overlap(mean_entropy, (size_t)G * 4, conf, rows * 4)) ||
                       (entropy && overlap(mean_entropy, (size_t)G * 4, entropy, rows * 4)) ||
                       (argmax_out && overlap(mean_entropy, (size_t)G * 4, argmax_out, rows * 8))))
    return fail(BDA_EINVAL, "mean_entropy must not overlap the logits or other outputs");
  bda::CommitPlan p;
  bda::commit_make_plan(G, R, V, dtype, &p);
  if (!workspace || ws_bytes < p.ws_bytes)
    return fail(BDA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                workspace ? ws_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(BDA_EINVAL, "workspace must be 16-byte aligned");
  hipError_t e = bda::stats_launch(p, logits, masked, conf, argmax_out, entropy, mean_entropy, workspace,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t bda_row_stats_commit_workspace_bytes(int G, int R, int V) { return bda_commit_workspace_bytes(G, R, V); }

int bda_row_stats_commit(const void* logits, int dtype, int64_t* tokens, uint8_t* masked, float threshold,
                         int k_min, float* conf, int64_t* argmax_out, float* entropy, float* mean_entropy, int G,
                         int R, int V, void* workspace, size_t ws_bytes, void* stream) {
  if (int e = check_logits(logits, dtype, G, R, V, "G")) return e;
  if (k_min < 0) return fail(BDA_EINVAL, "k_min must be >= 0");
  if (isnan(threshold)) return fail(BDA_EINVAL, "threshold is NaN");
  if (G == 0) return ok();
  const size_t rows = (size_t)G * R;
  if (rows && (!tokens || !masked)) return fail(BDA_EINVAL, "tokens and masked must be non-NULL");
  const size_t lbytes = rows * V * (dtype == BDA_BF16 ? 2 : 4);
  struct Buf {
    const void* p;
    size_t n;
  } bufs[] = {{logits, lbytes},       {tokens, rows * 8},  {masked, rows},          {conf, rows * 4},
              {argmax_out, rows * 8}, {entropy, rows * 4}, {mean_entropy, (size_t)G * 4}};
  constexpr int NB = sizeof(bufs) / sizeof(bufs[0]);
  for (int i = 0; i < NB; ++i)
    for (int j = i + 1; j < NB; ++j)
      if (bufs[i].p && bufs[j].p && overlap(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n))
        return fail(BDA_EINVAL, "logits, tokens, masked and the statistics outputs must not overlap");
  bda::CommitPlan p;
  bda::commit_make_plan(G, R, V, dtype, &p);
  if (!workspace || ws_bytes < p.ws_bytes)
    return fail(BDA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                workspace ? ws_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(BDA_EINVAL, "workspace must be 16-byte aligned");
  for (int i = 0; i < NB; ++i)
    if (bufs[i].p && overlap(workspace, p.ws_bytes, bufs[i].p, bufs[i].n))
      return fail(BDA_EINVAL, "workspace overlaps a tensor argument");
  hipError_t e = bda::stats_commit_launch(p, logits, tokens, masked, threshold, k_min, conf, argmax_out, entropy,
                                          mean_entropy, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int bda_sprint_kept_count(int n_image, int n_text, float r_img, float r_text) {
  if (n_image < 0 || n_text < 0 || !(r_img >= 0.f && r_img <= 1.f) || !(r_text >= 0.f && r_text <= 1.f)) return -1;
  return bda::sprint_keep(n_image, r_img) + bda::sprint_keep(n_text, r_text);
}

size_t bda_sprint_workspace_bytes(int B, int L) {
  if (B < 1 || L < 1) return 0;
  return bda::sprint_ws_bytes(B, L);
}

int bda_sprint_prune(const void* k, const void* v, const float* conf, const uint8_t* modality, float alpha,
                     float r_img, float r_text, void* k_out, void* v_out, int cap, int32_t* kept,
                     int32_t* kept_count, float* scores, int B, int Hkv, int L, int d, void* workspace,
                     size_t ws_bytes, void* stream) {
  if (B < 1 || Hkv < 1 || L < 1) return fail(BDA_EINVAL, "B, Hkv and L must be >= 1");
  if (d != 32 && d != 64 && d != 128) return fail(BDA_EUNSUPPORTED, "d must be 32, 64 or 128");
  if (L > 16384) return fail(BDA_EUNSUPPORTED, "L above 16384 is not supported");
  if (!(alpha >= 0.f && alpha <= 1.f) || !(r_img >= 0.f && r_img <= 1.f) || !(r_text >= 0.f && r_text <= 1.f))
    return fail(BDA_EINVAL, "alpha, r_img and r_text must lie in [0, 1]");
  if (cap < 0) return fail(BDA_EINVAL, "cap must be >= 0");
  if (!k || !v || !conf || !modality || !kept) return fail(BDA_EINVAL, "k, v, conf, modality and kept must be non-NULL");
  if (cap > 0 && (!k_out || !v_out)) return fail(BDA_EINVAL, "k_out and v_out must be non-NULL when cap > 0");
  const void* al[] = {k, v, k_out, v_out};
  for (const void* x : al)
    if (x && !aligned16(x)) return fail(BDA_EINVAL, "k, v, k_out and v_out must be 16-byte aligned");
  if (((uintptr_t)conf & 3) || ((uintptr_t)kept & 3) || ((uintptr_t)kept_count & 3) || ((uintptr_t)scores & 3))
    return fail(BDA_EINVAL, "conf, kept, kept_count and scores must be 4-byte aligned");
  const size_t kb = (size_t)B * Hkv * L * d * 2, ob = (size_t)B * Hkv * cap * d * 2, lb = (size_t)B * L * 4;
  if (cap > 0 && (overlap(k_out, ob, k, kb) || overlap(k_out, ob, v, kb) || overlap(v_out, ob, k, kb) ||
                  overlap(v_out, ob, v, kb) || overlap(k_out, ob, v_out, ob)))
    return fail(BDA_EINVAL, "k_out / v_out overlap k, v or each other");
  if (overlap(kept, lb, k, kb) || overlap(kept, lb, v, kb) || (scores && overlap(scores, lb, kept, lb)))
    return fail(BDA_EINVAL, "kept / scores overlap an input");
  const size_t need = bda_sprint_workspace_bytes(B, L);
  if (!workspace || ws_bytes < need)
    return fail(BDA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(BDA_EINVAL, "workspace must be 16-byte aligned");
  hipError_t e = bda::sprint_launch(k, v, conf, modality, alpha, r_img, r_text, k_out, v_out, cap, kept, kept_count,
                                    scores, B, Hkv, L, d, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BDA_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int bda_classify_tile(int mode, int L, int block, int q0, int q1, int k0, int k1) {
  if (mode < 0 || mode > 2 || L < 1 || block < 1 || block > L) return -1;
  const int rows = mode == BDA_MODE_HYBRID ? 2 * L : block;
  const int keys = mode == BDA_MODE_HYBRID ? 2 * L : L;
  if (q0 < 0 || q1 < q0 || q1 > rows || k0 < 0 || k1 < k0 || k1 > keys) return -1;
  return bda::classify_tile(mode, L, block, block, q0, q1, k0, k1);
}

}  // extern "C"
