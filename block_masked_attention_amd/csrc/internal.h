// Host-side plans and launchers shared between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn_index.h"

namespace bda {

// Work decomposition of one attention call.  Both the workspace query and the
// launch derive it from the arguments alone, so they always agree.
struct AttnPlan {
  int mode, B, Hq, Hkv, G, L, n, blk, d;
  int Sq, Sk;           // rows of the query / key tensors
  int nw;               // wavefronts per workgroup
  int stages;           // 4: persistent DMA-fed walk; 2: one item per workgroup
  int qpw;              // query slots per wavefront (32 or 64)
  int rows_per_wg;      // query rows per workgroup (per half in HYBRID)
  int n_qtiles;         // query tiles per (batch, kv head)
  int n_splits;         // key splits (DECODE/CAUSAL only; 1 = no combine)
  int split_keys;       // keys per split, a multiple of the key tile
  int pairs_per_xcd;    // >0: XCD-aware order of workgroups
  long long grid;       // workgroups of the main kernel
  size_t ws_bytes;      // workspace for split partials
};

int attn_make_plan(int B, int Hq, int Hkv, int L, int d, int block, int mode, AttnPlan* p,
                   const char** why);
// The index arguments of the forward kernels for a plan, and the grid of the
// persistent walk on a device of cus compute units (with the XCD-aware
// order's pairs per XCD it can keep, 0 when it cannot).
void attn_fill_index(const AttnPlan& p, AttnIndex* a);
long long attn_persistent_grid(const AttnPlan& p, int cus, int* pairs_per_xcd);
hipError_t attn_launch(const AttnPlan& p, const void* q, const void* k, const void* v, void* out,
                       float* lse, const int32_t* kv_len, void* ws, hipStream_t st);

struct CommitPlan {
  int G, R, V, dtype;
  int chunk;            // vocabulary entries per streaming workgroup
  int n_chunks;         // chunks per row
  size_t ws_bytes;
};

int commit_make_plan(int G, int R, int V, int dtype, CommitPlan* p);
hipError_t commit_launch(const CommitPlan& p, const void* logits, int64_t* tokens, uint8_t* masked,
                         float threshold, int k_min, void* ws, hipStream_t st);
hipError_t stats_launch(const CommitPlan& p, const void* logits, const uint8_t* masked, float* conf,
                        int64_t* argmax_out, float* entropy, float* mean_entropy, void* ws,
                        hipStream_t st);
hipError_t stats_commit_launch(const CommitPlan& p, const void* logits, int64_t* tokens, uint8_t* masked,
                               float threshold, int k_min, float* conf, int64_t* argmax_out, float* entropy,
                               float* mean_entropy, void* ws, hipStream_t st);
hipError_t verify_launch(const CommitPlan& p, const void* logits, const int64_t* drafts,
                         int64_t* argmax_out, int32_t* accept, int32_t* kv_len, int kv_cap, void* ws,
                         hipStream_t st);
hipError_t kv_append_launch(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* kv_len, int B, int Hkv, int L_cap, int n, int d, hipStream_t st);

// Backward of the training form (hybrid mask).
struct BwdPlan {
  int B, Hq, Hkv, G, L, blk, d;
  int nw;               // wavefronts of the dq workgroup
  int rows_per_wg;      // dq: query rows per tile (per half)
  int n_qtiles;         // dq: query tiles per (batch, kv head)
  int nkh;              // dkdv: 128-key tiles per half
  int pairs_per_xcd;    // >0: XCD-aware order
  long long grid_dq, grid_kv;
  size_t ws_bytes;      // per-row delta = rowsum(dO * O), fp32
};

int bwd_make_plan(int B, int Hq, int Hkv, int L, int d, int block, BwdPlan* p, const char** why);
hipError_t bwd_launch(const BwdPlan& p, const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv, void* ws,
                      hipStream_t st);

// The commit over the library's static scratch (no allocation anywhere):
// the scratch's device address on the current device, taken once per device.
constexpr size_t kCommitNoAllocBytes = (size_t)1 << 20;
constexpr int kMaxDevices = 64;
hipError_t commit_noalloc_scratch(void** ptr);

// Entropy-bound commit and adaptive stopping.
hipError_t commit_entropy_launch(const CommitPlan& p, const void* logits, int64_t* tokens, uint8_t* masked,
                                 float bound, float temperature, int k_min, void* ws, hipStream_t st);
int commit_entropy_max_rows();
hipError_t adaptive_stop_launch(const int64_t* argmax, int64_t* prev, int32_t* stable, uint8_t* frozen,
                                const float* mean_entropy, int G, int R, int stability, float conf_thr,
                                int32_t* n_frozen, hipStream_t st);

// SPRINT prefix retention.
int sprint_keep(int n, float r);
size_t sprint_lds_bytes(int L);
size_t sprint_ws_bytes(int B, int L);
hipError_t sprint_launch(const void* k, const void* v, const float* conf, const uint8_t* modality, float alpha,
                         float r_img, float r_text, void* k_out, void* v_out, int cap, int32_t* kept,
                         int32_t* kept_count, float* scores, int B, int Hkv, int L, int d, void* ws,
                         hipStream_t st);

}  // namespace bda
