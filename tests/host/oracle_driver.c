/*
 * Host driver for the sanitizer build of the oracle (test infrastructure).
 * It calls every entry point of oracle/bda_oracle.c on small inputs and on
 * the edge cases of their arguments (one row, block 1 and block = L, a short
 * last block, V = 1, groups with nothing masked, k_min above the masked
 * count, empty SPRINT modalities, rejected arguments), so that an
 * AddressSanitizer / UndefinedBehaviorSanitizer build reports any
 * out-of-bounds access, leak or undefined operation.  Prints "ok" and
 * returns 0 when every call returned as expected.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_mask_shape(int mode, long L, long block, long* rows, long* keys);
int oracle_mask(int mode, long L, long block, uint8_t* M);
int oracle_attention(int mode, const float* q, const float* k, const float* v, double* out, long B, long Hq,
                     long Hkv, long L, long d, long block, const long* sel, long nsel, int nthreads);
int oracle_attention_bwd(int mode, const float* q, const float* k, const float* v, const float* dout, double* dq,
                         double* dk, double* dv, double* lse, long B, long Hq, long Hkv, long L, long d, long block,
                         int nthreads);
int oracle_commit(const float* logits, int64_t* tokens, uint8_t* masked, float threshold, long k_min, long G,
                  long R, long V, double* p64, int64_t* argmax, double* margin, double* gap, int nthreads);
int oracle_verify(const float* logits, const int64_t* drafts, int64_t* argmax_out, int32_t* accept, long B, long R,
                  long V, int nthreads);
int oracle_row_stats(const float* logits, const uint8_t* masked, double* conf, int64_t* argmax, double* entropy,
                     double* mean, long G, long R, long V, int nthreads);
int oracle_commit_entropy(const float* logits, int64_t* tokens, uint8_t* masked, double bound, double temperature,
                          long k_min, long G, long R, long V, double* entropy, int64_t* argmax, int nthreads);
long oracle_sprint(const float* k, const float* conf, const uint8_t* modality, double alpha, double r_img,
                   double r_text, long B, long Hkv, long L, long d, int64_t* kept, double* scores);
int oracle_max_threads(void);

static int failures = 0;
#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static unsigned long long rng = 88172645463325252ull;
static float urand(void) {  /* xorshift64, values in [-2, 2) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (float)((rng >> 11) * (1.0 / 9007199254740992.0)) * 4.0f - 2.0f;
}
static float* fill(long n) {
    float* x = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) x[i] = urand();
    return x;
}

static void attention_case(int mode, long B, long Hq, long Hkv, long L, long d, long block) {
    long rows, keys;
    EXPECT(oracle_mask_shape(mode, L, block, &rows, &keys) == 0);
    uint8_t* M = (uint8_t*)malloc((size_t)(rows * keys));
    EXPECT(oracle_mask(mode, L, block, M) == 0);
    free(M);
    float *q = fill(B * Hq * rows * d), *k = fill(B * Hkv * keys * d), *v = fill(B * Hkv * keys * d);
    float* dout = fill(B * Hq * rows * d);
    double* out = (double*)malloc(sizeof(double) * (size_t)(B * Hq * rows * d));
    EXPECT(oracle_attention(mode, q, k, v, out, B, Hq, Hkv, L, d, block, NULL, 0, 2) == 0);
    long sel[6] = {0, Hq - 1, rows - 1, B - 1, 0, 0};
    double so[2 * 128];
    EXPECT(oracle_attention(mode, q, k, v, so, B, Hq, Hkv, L, d, block, sel, 2, 1) == 0);
    if (mode == 0) {
        double* dq = (double*)malloc(sizeof(double) * (size_t)(B * Hq * rows * d));
        double* dk = (double*)malloc(sizeof(double) * (size_t)(B * Hkv * keys * d));
        double* dv = (double*)malloc(sizeof(double) * (size_t)(B * Hkv * keys * d));
        double* lse = (double*)malloc(sizeof(double) * (size_t)(B * Hq * rows));
        EXPECT(oracle_attention_bwd(mode, q, k, v, dout, dq, dk, dv, lse, B, Hq, Hkv, L, d, block, 2) == 0);
        free(dq); free(dk); free(dv); free(lse);
    }
    free(q); free(k); free(v); free(dout); free(out);
}

static void commit_case(long G, long R, long V, long k_min, float tau, double mask_p) {
    float* lg = fill(G * R * V);
    uint8_t* m = (uint8_t*)malloc((size_t)(G * R + 1));
    int64_t* t = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G * R + 1));
    for (long i = 0; i < G * R; ++i) { m[i] = (urand() + 2.0f) / 4.0f < mask_p; t[i] = -1; }
    double *p64 = (double*)malloc(sizeof(double) * (size_t)(G * R + 1)), *mg = (double*)malloc(sizeof(double) * (size_t)(G * R + 1));
    double* gap = (double*)malloc(sizeof(double) * (size_t)(G + 1));
    int64_t* am = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G * R + 1));
    EXPECT(oracle_commit(lg, t, m, tau, k_min, G, R, V, p64, am, mg, gap, 2) == 0);
    EXPECT(oracle_commit(lg, t, m, tau, k_min, G, R, V, NULL, NULL, NULL, NULL, 1) == 0);
    double *conf = (double*)malloc(sizeof(double) * (size_t)(G * R + 1)), *ent = (double*)malloc(sizeof(double) * (size_t)(G * R + 1));
    double* mean = (double*)malloc(sizeof(double) * (size_t)(G + 1));
    EXPECT(oracle_row_stats(lg, m, conf, am, ent, mean, G, R, V, 2) == 0);
    EXPECT(oracle_row_stats(lg, NULL, conf, am, ent, mean, G, R, V, 1) == 0);
    for (long i = 0; i < G * R; ++i) m[i] = 1;
    EXPECT(oracle_commit_entropy(lg, t, m, 3.0, 0.7, k_min, G, R, V, ent, am, 2) == 0);
    int64_t* dr = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G * R + 1));
    int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (size_t)(G + 1));
    for (long i = 0; i < G * R; ++i) dr[i] = i % V;
    EXPECT(oracle_verify(lg, dr, am, acc, G, R, V, 2) == 0);
    free(lg); free(m); free(t); free(p64); free(mg); free(gap); free(am); free(conf); free(ent); free(mean);
    free(dr); free(acc);
}

static void sprint_case(long B, long Hkv, long L, long d, double alpha, double r_img, double r_text, int all_text) {
    float* k = fill(B * Hkv * L * d);
    float* conf = fill(B * L);
    uint8_t* mod = (uint8_t*)malloc((size_t)L);
    for (long i = 0; i < L; ++i) mod[i] = all_text ? 0 : (uint8_t)(i % 3 == 0);
    int64_t* kept = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B * L));
    double* sc = (double*)malloc(sizeof(double) * (size_t)(B * L));
    EXPECT(oracle_sprint(k, conf, mod, alpha, r_img, r_text, B, Hkv, L, d, kept, sc) >= 0);
    free(k); free(conf); free(mod); free(kept); free(sc);
}

int main(void) {
    /* attention: every mode, block 1, block = L, short last block, GQA, d 32..128 */
    attention_case(0, 1, 2, 1, 1, 32, 1);
    attention_case(0, 2, 4, 2, 13, 32, 1);
    attention_case(0, 1, 4, 1, 13, 64, 5);
    attention_case(0, 1, 2, 2, 16, 128, 16);
    attention_case(1, 2, 4, 2, 17, 32, 3);
    attention_case(1, 1, 2, 1, 5, 64, 5);
    attention_case(2, 2, 4, 2, 19, 32, 4);
    attention_case(2, 1, 2, 1, 9, 128, 9);
    attention_case(2, 1, 2, 1, 1, 32, 1);
    /* rejected arguments */
    long rows, keys;
    EXPECT(oracle_mask_shape(3, 4, 1, &rows, &keys) != 0);
    EXPECT(oracle_mask_shape(0, 4, 5, &rows, &keys) != 0);
    EXPECT(oracle_mask_shape(1, 0, 1, &rows, &keys) != 0);
    EXPECT(oracle_attention(0, NULL, NULL, NULL, NULL, 1, 3, 2, 4, 32, 1, NULL, 0, 1) != 0);
    /* commit family: V = 1, one row, nothing masked, k_min above the masked count, ragged V */
    commit_case(1, 1, 1, 1, 0.5f, 1.0);
    commit_case(2, 5, 7, 9, 0.1f, 0.5);
    commit_case(3, 12, 1000, 2, 0.85f, 0.7);
    commit_case(1, 4, 3, 0, 0.99f, 0.0);
    EXPECT(oracle_commit(NULL, NULL, NULL, 0.5f, -1, 1, 1, 1, NULL, NULL, NULL, NULL, 1) != 0);
    EXPECT(oracle_commit_entropy(NULL, NULL, NULL, 1.0, 0.0, 0, 1, 1, 1, NULL, NULL, 1) != 0);
    /* SPRINT: mixed modalities, all text, keep nothing / everything */
    sprint_case(2, 2, 37, 32, 0.5, 0.8, 1.0, 0);
    sprint_case(1, 1, 1, 64, 1.0, 0.0, 1.0, 0);
    sprint_case(1, 3, 20, 128, 0.0, 0.0, 0.0, 1);
    EXPECT(oracle_max_threads() >= 1);
    if (failures) return 1;
    printf("ok\n");
    return 0;
}
