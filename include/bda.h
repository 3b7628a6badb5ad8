/*
 * bda.h -- block-diffusion attention and the confidence commit on AMD Instinct
 * MI355X (gfx950).  C ABI of libbda.so.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument except `stream` is DEVICE memory owned by the
 *    caller (allocated by whatever the caller uses, e.g. PyTorch).  The
 *    library allocates nothing, frees nothing and keeps no state between
 *    calls (the workspaces below are the caller's too).
 *  - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *    stream).  Calls are asynchronous on that stream; the library never
 *    synchronises.  Faults inside a kernel surface at the caller's next
 *    synchronisation, not here.
 *  - Tensors are dense, row-major, with the last index fastest.  bf16 is the
 *    IEEE bfloat16 bit pattern stored in 16 bits.
 *  - Arguments are validated on the host before any launch.  A non-zero
 *    return is one of the BDA_E* codes below; bda_last_error() then holds a
 *    detail string for the calling thread.  Nothing aborts, throws or prints.
 *  - Outputs must not overlap inputs.  A workspace serves one call at a time.
 *
 * Citations name the pages the operations are defined on:
 *  [NLD-3x]  "Analise do acelero de 3x do Nemotron-Labs-Diffusion-8B-Base"
 *            (doido.pw): sec. 1 Block Diffusion Attention (hybrid mask
 *            M_BD | M_OBC | M_BC, fused flex attention with a block mask),
 *            sec. 2 Linear Speculative Decoding (bidirectional drafting,
 *            causal validation, longest matching prefix).
 *  [LLaDA]   "LLaDA2.0-Uni" summary (discuss.pytorch.kr): training objective
 *            (BDLM conditioning of a noisy block on earlier clean blocks) and
 *            SPRINT (confidence = top-1 softmax probability; accept every
 *            position above tau with a per-step minimum).
 *  [DGemma]  diffusers "DiffusionGemma" pipeline docs: intro (bidirectional
 *            decoder over a canvas and a cached clean prefix), Schedulers
 *            (threshold commit plus an even per-step share), the pipeline
 *            call (logits [batch, canvas, vocab]; LongTensor sequences).
 *  [VLM-8B]  "Nemotron-Labs-Diffusion-VLM-8B" usage page: generate() with
 *            block_size 28 and threshold 0.85.
 */
#ifndef BDA_H
#define BDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { BDA_MODE_HYBRID = 0, BDA_MODE_DECODE = 1, BDA_MODE_CAUSAL = 2 };
enum { BDA_BF16 = 0, BDA_F32 = 1 };
enum {
    BDA_OK = 0,
    BDA_EINVAL = 1,        /* bad pointer, size, shape or parameter          */
    BDA_EUNSUPPORTED = 2,  /* valid request the library does not implement   */
    BDA_EWORKSPACE = 3,    /* workspace missing or smaller than required     */
    BDA_EHIP = 4           /* the HIP runtime reported an error at launch    */
};
enum { BDA_TILE_FULL = 0, BDA_TILE_EMPTY = 1, BDA_TILE_PARTIAL = 2 };

/*
 * Masked attention forward, one kernel family for the three forms.
 * O = softmax(scale * Q K^T restricted to allowed keys) V, scale = 1/sqrt(d),
 * bf16 inputs and output, fp32 accumulation.  Query head h reads kv head
 * h / (Hq/Hkv) (grouped-query attention; Hq % Hkv == 0).  d in {32, 64, 128}.
 *
 * mode = BDA_MODE_HYBRID  ([NLD-3x] sec. 1; conditioning from [LLaDA]):
 *   q, k, v, out are [B, H, 2L, d]; rows 0..L-1 are the noisy copy x_t,
 *   rows L..2L-1 the clean copy x_0.  Positions are cut into blocks of
 *   `block` (1 <= block <= L; the last block may be short).  An x_t query of
 *   block j sees the x_t keys of block j and the x_0 keys of blocks < j; an
 *   x_0 query of block j sees the x_0 keys of blocks <= j; x_0 queries never
 *   see x_t keys.
 * mode = BDA_MODE_DECODE  ([DGemma] intro; drafting in [NLD-3x] sec. 2):
 *   q, out are [B, Hq, n, d] with n = block; k, v are [B, Hkv, L, d] whose
 *   last n rows are the active block.  Every query sees all L keys.
 * mode = BDA_MODE_CAUSAL  (validation in [NLD-3x] sec. 2):
 *   shapes as DECODE; the n queries are the last n of the L positions, so
 *   query i sees keys 0 .. L-n+i.  n = L is ordinary causal attention
 *   (a prefill).
 * workspace: device scratch of at least bda_attn_workspace_bytes(...) bytes
 *   (may be NULL when that is 0); no initial contents are required.
 */
int bda_attn_fwd(const void* q, const void* k, const void* v, void* out,
                 int B, int Hq, int Hkv, int L, int d, int block, int mode,
                 void* workspace, size_t ws_bytes, void* stream);
size_t bda_attn_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int block, int mode);

/*
 * The same forward, also writing lse [B, Hq, Sq] (fp32, device, caller-owned,
 * 16-byte aligned): the natural-log log-sum-exp of each query row's scaled
 * allowed scores, log sum_j exp(scale * q.k_j).  It is what the backward
 * (bda_attn_bwd) takes to rebuild the softmax.  Same workspace as
 * bda_attn_fwd.  lse must not overlap any other argument.
 */
int bda_attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int Hq, int Hkv, int L, int d, int block, int mode,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * DECODE / CAUSAL forward over a cache whose rows hold different numbers of
 * keys: the draft and validation passes of linear speculative decoding
 * ([NLD-3x] sec. 2, "generate and validate") once sequences have accepted
 * different numbers of drafts (its KV-cache strategy crops each cache to
 * what was kept).  k, v are [B, Hkv, L_cap, d] (the capacity is the row
 * stride); kv_len [B] (int32, device, read by the kernels) gives the keys of
 * each batch row, L_b = kv_len[b] clamped to [block, L_cap]; its last `block`
 * keys are the active block.  Row b then behaves exactly as bda_attn_fwd with
 * L = L_b; keys past L_b are never read.  mode must be BDA_MODE_DECODE or
 * BDA_MODE_CAUSAL (else BDA_EUNSUPPORTED).  Workspace as bda_attn_fwd with
 * L = L_cap.  The lengths stay on the device, so a captured graph can replay
 * the call as they change.
 */
int bda_attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, const int32_t* kv_len,
                        int B, int Hq, int Hkv, int L_cap, int d, int block, int mode,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * Writes a block's fresh K/V rows into a cache with per-row lengths (the KV
 * update of [NLD-3x] sec. 2): k_cache[b, h, L_b - n + j] = k_new[b, h, j]
 * for j < n, same for v, with L_b = kv_len[b] clamped to [n, L_cap] as in
 * bda_attn_fwd_varlen.  k_cache, v_cache [B, Hkv, L_cap, d] bf16; k_new,
 * v_new [B, Hkv, n, d] bf16; kv_len [B] int32 (device).  d in {32, 64, 128}.
 */
int bda_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, const int32_t* kv_len,
                  int B, int Hkv, int L_cap, int n, int d, void* stream);

/*
 * Backward of the training form (mode must be BDA_MODE_HYBRID; others return
 * BDA_EUNSUPPORTED) ([NLD-3x] sec. 1 mask; the [LLaDA] BDLM objective trains
 * through it).  For loss = sum(dout * out) with out = bda_attn_fwd(q, k, v):
 *   dq = d loss / d q, dk = d loss / d k, dv = d loss / d v,
 * where the G = Hq/Hkv query heads of a kv head add into its dk, dv.
 * q, out, dout, dq: [B, Hq, 2L, d] bf16; k, v, dk, dv: [B, Hkv, 2L, d] bf16;
 * lse: [B, Hq, 2L] fp32 as written by bda_attn_fwd_lse for the same inputs.
 * Hq/Hkv <= 32.  All device pointers 16-byte aligned; the gradients must not
 * overlap the inputs or each other.  fp32 accumulation; the softmax is
 * rebuilt exactly from lse.
 * workspace: at least bda_attn_bwd_workspace_bytes(...) bytes (per-row
 *   rowsum(dout * out), fp32); no initial contents are required.
 */
int bda_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int L, int d, int block, int mode,
                 void* workspace, size_t ws_bytes, void* stream);
size_t bda_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int block, int mode);

/*
 * Confidence commit ([LLaDA] SPRINT; [DGemma] Schedulers; [VLM-8B]).
 * logits: [G, R, V] of dtype BDA_BF16 or BDA_F32 (G independent groups, e.g.
 *   sequences; R canvas positions; V vocabulary).  Values are finite or
 *   -inf (a banned token, probability 0); every row holds a finite value.
 * masked: [G, R] uint8, 1 = position still masked; updated in place.
 * tokens: [G, R] int64; written only at the positions this call commits.
 * For each group, among masked rows: c_r = largest softmax probability of
 * the row (temperature 1) and a_r = its token (lowest id on ties).  Every row
 * with c_r > threshold (strict, fp32) commits; if fewer than
 * min(k_min, #masked) did, the masked rows with the largest c_r (lower row
 * index first on ties) are added until that many have committed.  A commit
 * sets tokens[g,r] = a_r and masked[g,r] = 0.  k_min >= 0.
 * workspace: at least bda_commit_workspace_bytes(G, R, V) bytes of device
 *   memory; no initial contents are required.
 */
int bda_commit(const void* logits, int dtype, int64_t* tokens, uint8_t* masked,
               float threshold, int k_min, int G, int R, int V,
               void* workspace, size_t ws_bytes, void* stream);
size_t bda_commit_workspace_bytes(int G, int R, int V);

/*
 * bda_commit for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and results as bda_commit, with its scratch in a static
 * array of BDA_COMMIT_NOALLOC_MAX_BYTES bytes that the library holds on each
 * GPU it runs on until the process ends.  No memory is allocated or freed.
 * Calls whose bda_commit_workspace_bytes(G, R, V) exceeds that size return
 * BDA_EWORKSPACE without launching anything (at V = 131072, up to about 7600
 * rows).  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (other streams, other threads) race and must not be
 * issued; calls in one stream are ordered and safe.
 */
#define BDA_COMMIT_NOALLOC_MAX_BYTES (1u << 20)
int bda_commit_noalloc(const void* logits, int dtype, int64_t* tokens, uint8_t* masked,
                       float threshold, int k_min, int G, int R, int V, void* stream);

/*
 * Verify for linear speculative decoding ([NLD-3x] sec. 2).
 * logits [B, R, V] (BDA_BF16 or BDA_F32), drafts [B, R] int64.
 * argmax_out[B, R] int64 = lowest index of each row's largest logit;
 * accept_len[B] int32 = first j with argmax != drafts[b, j], or R if none.
 * workspace: at least bda_verify_workspace_bytes(B, R, V) bytes.
 */
int bda_verify(const void* logits, int dtype, const int64_t* drafts,
               int64_t* argmax_out, int32_t* accept_len, int B, int R, int V,
               void* workspace, size_t ws_bytes, void* stream);
size_t bda_verify_workspace_bytes(int B, int R, int V);

/*
 * bda_verify, then the crop of [NLD-3x]'s KV-cache strategy on the device:
 * kv_len[b] = min(kv_len[b] + accept_len[b], kv_cap) (int32, device,
 * read and written).  With kv_len counting the cached keys plus the block of
 * R drafts (as bda_attn_fwd_varlen takes it), the result counts the kept
 * prefix, now including the accepted drafts, plus room for the next block of
 * R rows; rows of rejected drafts are overwritten by the next bda_kv_append.
 * Same workspace as bda_verify.
 */
int bda_verify_crop(const void* logits, int dtype, const int64_t* drafts, int64_t* argmax_out,
                    int32_t* accept_len, int32_t* kv_len, int kv_cap, int B, int R, int V,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * Entropy-bound commit ([DGemma] Schedulers: the entropy-bound scheduler
 * commits the lowest-entropy positions whose joint entropy stays within a
 * bound, so that roughly independent tokens are accepted together).
 * logits [G, R, V] (BDA_BF16 or BDA_F32, finite or -inf as for bda_commit); masked [G, R] uint8 and
 * tokens [G, R] int64, updated in place as by bda_commit.  For every masked
 * row: H = entropy in nats of softmax(logits / temperature), a = lowest index
 * of the largest logit.  Per group, the masked rows ordered by (H ascending,
 * row ascending) are committed (tokens = a, masked = 0) while the running sum
 * of their H stays <= entropy_bound, and at least min(k_min, #masked) of them.
 * The sum is the joint entropy of positions taken as independent; the
 * scheduler's sampling and its temperature schedule are the caller's (pass
 * the step's temperature).  temperature > 0 and finite, k_min >= 0,
 * R <= 4096 (else BDA_EUNSUPPORTED).  Decisions are taken in fp32.
 * workspace: at least bda_commit_entropy_workspace_bytes(G, R, V) bytes.
 */
int bda_commit_entropy(const void* logits, int dtype, int64_t* tokens, uint8_t* masked,
                       float entropy_bound, float temperature, int k_min, int G, int R, int V,
                       void* workspace, size_t ws_bytes, void* stream);
size_t bda_commit_entropy_workspace_bytes(int G, int R, int V);

/*
 * One step of adaptive stopping ([DGemma] "Adaptive stopping": an example is
 * frozen once its argmax predictions have been stable for stability_threshold
 * steps and its mean per-token entropy is below the confidence threshold;
 * the loop ends when every example is frozen).  Per example g of G (R
 * positions each), on device arrays:
 *   argmax [G, R] int64           this step's argmax (e.g. from bda_row_stats),
 *   prev_argmax [G, R] int64      last step's (in/out; start with -1),
 *   stable_steps [G] int32        consecutive unchanged steps (in/out; start 0),
 *   frozen [G] uint8              in/out (start 0),
 *   mean_entropy [G] float        this step's mean entropy (bda_row_stats).
 * A frozen example keeps its state.  Otherwise stable_steps = (argmax ==
 * prev_argmax at every position) ? stable_steps + 1 : 0, prev_argmax =
 * argmax, and frozen = 1 once stable_steps >= stability_threshold and
 * mean_entropy < confidence_threshold.  n_frozen (int32, device, may be NULL)
 * receives the number of frozen examples after the step.  One kernel.
 */
int bda_adaptive_stop(const int64_t* argmax, int64_t* prev_argmax, int32_t* stable_steps,
                      uint8_t* frozen, const float* mean_entropy, int G, int R,
                      int stability_threshold, float confidence_threshold, int32_t* n_frozen,
                      void* stream);

/*
 * Per-row statistics of a softmax over the vocabulary, for adaptive stopping
 * and entropy-based commits ([DGemma] adaptive stopping: freeze an example
 * once its argmax is stable and its mean per-token entropy is below a
 * confidence threshold; [DGemma] Schedulers: the entropy-bound scheduler
 * commits the lowest-entropy positions) and the SPRINT confidence ([LLaDA]).
 * logits: [G, R, V] of dtype BDA_BF16 or BDA_F32; values finite or -inf (a
 *   banned token: probability 0, no entropy term), at least one finite per row.
 * masked: [G, R] uint8 or NULL.  When given, only rows with masked != 0 are
 *   computed (outputs of the other rows are left untouched); NULL = all rows.
 * For each computed row, with p = softmax(row) at temperature 1:
 *   conf[g,r]    (float, [G,R]) = max p,
 *   argmax[g,r]  (int64, [G,R]) = lowest index of the largest logit,
 *   entropy[g,r] (float, [G,R]) = -sum p log p in nats.
 * mean_entropy[g] (float, [G]) = mean entropy of the group's computed rows
 *   (0 when it has none).  Any of the four outputs may be NULL (not written).
 * workspace: at least bda_row_stats_workspace_bytes(G, R, V) bytes.
 */
int bda_row_stats(const void* logits, int dtype, const uint8_t* masked, float* conf,
                  int64_t* argmax, float* entropy, float* mean_entropy, int G, int R, int V,
                  void* workspace, size_t ws_bytes, void* stream);
size_t bda_row_stats_workspace_bytes(int G, int R, int V);

/*
 * Row statistics and the confidence commit of one denoising step, from one
 * pass over its logits ([DGemma] "Adaptive stopping" and "Schedulers": each
 * step's logits feed both the stopping test and the commit; [LLaDA]
 * SPRINT).  Computes what bda_row_stats(logits, masked = NULL, conf, argmax,
 * entropy, mean_entropy) and then bda_commit(logits, tokens, masked,
 * threshold, k_min) compute: the statistics cover every row, the commit the
 * rows with masked != 0 (tokens and masked updated as bda_commit does).  The
 * logits are read once instead of twice.  Any of conf, argmax, entropy and
 * mean_entropy may be NULL (not written); with R = 0 mean_entropy is 0.  No
 * two of logits, tokens, masked and the outputs may overlap.
 * workspace: at least bda_row_stats_commit_workspace_bytes(G, R, V) bytes.
 */
int bda_row_stats_commit(const void* logits, int dtype, int64_t* tokens, uint8_t* masked,
                         float threshold, int k_min, float* conf, int64_t* argmax,
                         float* entropy, float* mean_entropy, int G, int R, int V,
                         void* workspace, size_t ws_bytes, void* stream);
size_t bda_row_stats_commit_workspace_bytes(int G, int R, int V);

/*
 * SPRINT sparse prefix retention ([LLaDA] "SPRINT"): prune the clean KV
 * prefix once, at the start of a block, to the positions that matter.
 * k, v: [B, Hkv, L, d] bf16 (the prefix cache); conf: [B, L] float, each
 * position's top-1 confidence (e.g. bda_row_stats' conf); modality: [L] uint8
 * device array, 0 = text, nonzero = image (shared by the batch).
 * Score of position i in batch b:
 *   s = alpha * n_i / mean_j n_j + (1 - alpha) * conf[b, i],
 * n_i = L2 norm of the position's keys over all Hkv heads (fp32).  Text
 * positions keep the floor(r_text * n_text + 0.5) best scores and image
 * positions the floor(r_img * n_image + 0.5) best, ties to the lower position.
 * Outputs:
 *   kept [B, L] int32: the kept positions in ascending order, then -1;
 *   kept_count (int32, device, may be NULL): K, the kept count per batch
 *     (equal in every batch; bda_sprint_kept_count gives it on the host);
 *   scores [B, L] float (may be NULL): s;
 *   k_out, v_out [B, Hkv, cap, d] bf16: rows 0..min(K, cap)-1 are the kept
 *     rows of k and v in position order; rows from K on are not written.
 *     cap = 0 skips the gather (k_out, v_out may then be NULL).
 * alpha, r_img, r_text in [0, 1]; d in {32, 64, 128}; L <= 16384.
 * k, v, k_out, v_out and the workspace must be 16-byte aligned, outputs must
 * not overlap inputs.  workspace: bda_sprint_workspace_bytes(B, L) bytes.
 * Three kernels on `stream`: key norms, selection, gather.
 */
int bda_sprint_prune(const void* k, const void* v, const float* conf, const uint8_t* modality,
                     float alpha, float r_img, float r_text, void* k_out, void* v_out, int cap,
                     int32_t* kept, int32_t* kept_count, float* scores, int B, int Hkv, int L, int d,
                     void* workspace, size_t ws_bytes, void* stream);
size_t bda_sprint_workspace_bytes(int B, int L);
/* Host-only: the kept count K for n_image image and n_text text positions
 * (-1 on bad arguments).  Touches no device. */
int bda_sprint_kept_count(int n_image, int n_text, float r_img, float r_text);

/*
 * Host-only tile classifier (the rule the attention kernels use to skip and
 * to take their unmasked fast path).  Rows [q0, q1) of the query tensor and
 * keys [k0, k1) of the key tensor, in the row numbering of bda_attn_fwd for
 * `mode` (HYBRID: L per half; DECODE/CAUSAL: n = block query rows, L keys).
 * Returns BDA_TILE_FULL (every pair allowed), BDA_TILE_EMPTY (none) or
 * BDA_TILE_PARTIAL; -1 on bad arguments.  Touches no device.
 */
int bda_classify_tile(int mode, int L, int block, int q0, int q1, int k0, int k1);

/* Static description of an error code; never NULL. */
const char* bda_strerror(int code);
/* Detail of the calling thread's last failed call ("" if none). */
const char* bda_last_error(void);
/* Library version string. */
const char* bda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BDA_H */
