/*
 * Reference (oracle) for block-diffusion attention and the confidence commit.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain CPU definition that
 * the HIP library is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the library never does.  It shares
 * no source, header, table or helper with the HIP path.
 *
 * Everything is computed in double precision.  Inputs arrive as float32 arrays
 * (bf16 and fp32 values are exactly representable there) and are widened to
 * double before any arithmetic.
 *
 * Sources (pages as titled):
 *  [NLD-3x]  "Analise do acelero de 3x do Nemotron-Labs-Diffusion-8B-Base"
 *            (doido.pw), sec. 1 "Block Diffusion Attention" (the three mask
 *            names M_BD, M_OBC, M_BC) and sec. 2 "Linear Speculative Decoding"
 *            (bidirectional drafting, causal validation, longest matching
 *            prefix).
 *  [LLaDA]   "LLaDA2.0-Uni" summary (discuss.pytorch.kr), "Training objective"
 *            (BDLM: block k of x_t is predicted from the clean blocks x_0,<k
 *            and its own noisy block x_t,k) and "SPRINT" (confidence c_i is the
 *            top-1 softmax probability; the accepted set is every position with
 *            c_n > tau, with at least a per-step quota of acceptances).
 *  [DGemma]  diffusers "DiffusionGemma" pipeline docs, "Usage"/intro (causal
 *            encoder fills the KV cache; bidirectional decoder over the canvas
 *            and that cache) and "Schedulers" (BlockRefinementScheduler commits
 *            the most confident tokens above a threshold plus a per-step even
 *            share).
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes): sequence order [x_t ; x_0]; x_0 queries never see x_t keys; the last
 * block may be short (block id = floor(position / b)); the query head h uses
 * kv head floor(h * Hkv / Hq); scale 1/sqrt(d), no bias; decode keys include
 * the active block as the last n rows; causal is bottom-right aligned
 * (query i sees keys 0 .. L-n+i); threshold test is strict (c > tau) and taken
 * in fp32 (the kernel's precision) on the fp64 value rounded to fp32; argmax
 * ties go to the lowest vocab id, ranking ties to the lowest row index.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_HYBRID = 0, OR_DECODE = 1, OR_CAUSAL = 2 };

/* Threads of one call: nthreads when positive, else the OpenMP default.  The
 * count is given to each parallel region, so a call never changes the
 * process-wide default that later calls see. */
static int thread_count(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* ---------------------------------------------------------------------- */
/* Mask                                                                     */
/* ---------------------------------------------------------------------- */

/* Training form, [NLD-3x] sec. 1 with the BDLM conditioning of [LLaDA]:
 * positions 0..L-1 are the noisy copy x_t, L..2L-1 the clean copy x_0.
 *   x_t query, x_t key : same block                 (M_BD, block-diagonal)
 *   x_t query, x_0 key : key block strictly earlier (M_OBC, offset block-causal)
 *   x_0 query, x_0 key : key block same or earlier  (M_BC, block-causal)
 *   x_0 query, x_t key : never                                             */
static int allowed_hybrid(long i, long j, long L, long b)
{
    int qi_noisy = i < L, kj_noisy = j < L;
    long bq = (qi_noisy ? i : i - L) / b;
    long bk = (kj_noisy ? j : j - L) / b;
    if (qi_noisy && kj_noisy) return bq == bk;
    if (qi_noisy && !kj_noisy) return bk < bq;
    if (!qi_noisy && !kj_noisy) return bk <= bq;
    return 0;
}

/* Decode form ([DGemma] intro; [NLD-3x] sec. 2 drafting): the n active
 * queries see every one of the L keys (clean prefix + their own block). */
static int allowed_decode(long i, long j, long L, long n)
{
    (void)i; (void)j; (void)L; (void)n;
    return 1;
}

/* Verify form ([NLD-3x] sec. 2): causal, with the n queries being the last n
 * of the L key positions, so query i sees keys 0 .. L-n+i. */
static int allowed_causal(long i, long j, long L, long n)
{
    return j <= L - n + i;
}

static int allowed(int mode, long i, long j, long L, long n, long b)
{
    if (mode == OR_HYBRID) return allowed_hybrid(i, j, L, b);
    if (mode == OR_DECODE) return allowed_decode(i, j, L, n);
    return allowed_causal(i, j, L, n);
}

/* Rows and key count of the dense mask for a mode.  HYBRID: L is the per-half
 * length, rows = keys = 2L.  DECODE/CAUSAL: L keys, n = block query rows. */
static void mask_shape(int mode, long L, long block, long* rows, long* keys)
{
    if (mode == OR_HYBRID) { *rows = 2 * L; *keys = 2 * L; }
    else { *rows = block; *keys = L; }
}

int oracle_mask_shape(int mode, long L, long block, long* rows, long* keys)
{
    if (mode < 0 || mode > 2 || L <= 0 || block <= 0) return 1;
    if (mode == OR_HYBRID && block > L) return 1;
    if (mode != OR_HYBRID && block > L) return 1;
    mask_shape(mode, L, block, rows, keys);
    return 0;
}

/* Dense mask M[rows][keys] (1 = the query may attend to the key). */
int oracle_mask(int mode, long L, long block, uint8_t* M)
{
    long rows, keys;
    if (oracle_mask_shape(mode, L, block, &rows, &keys)) return 1;
    for (long i = 0; i < rows; ++i)
        for (long j = 0; j < keys; ++j)
            M[i * keys + j] = (uint8_t)allowed(mode, i, j, L, block, block);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Attention                                                                */
/* ---------------------------------------------------------------------- */

/* One output row: softmax over the allowed keys of scale * q.k, then the
 * weighted sum of the allowed value rows.  All in double. */
static void attend_row(const float* qrow, const float* K, const float* Vv, const uint8_t* Mrow,
                       long keys, long d, double scale, double* out, double* s)
{
    double m = -INFINITY;
    for (long j = 0; j < keys; ++j) {
        if (!Mrow[j]) continue;
        const float* kr = K + j * d;
        double acc = 0.0;
        for (long c = 0; c < d; ++c) acc += (double)qrow[c] * (double)kr[c];
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
    }
    double Z = 0.0;
    for (long j = 0; j < keys; ++j) {
        if (!Mrow[j]) continue;
        s[j] = exp(s[j] - m);
        Z += s[j];
    }
    for (long c = 0; c < d; ++c) out[c] = 0.0;
    for (long j = 0; j < keys; ++j) {
        if (!Mrow[j]) continue;
        const float* vr = Vv + j * d;
        double w = s[j] / Z;
        for (long c = 0; c < d; ++c) out[c] += w * (double)vr[c];
    }
}

/*
 * Attention with an explicit dense mask.
 *   q   [B, Hq,  rows, d]    k, v [B, Hkv, keys, d]   (float32, row-major)
 *   out [B, Hq,  rows, d] double, or, when sel != NULL, [nsel, d] for the
 *       listed (b, h, i) triples in sel[3*t .. 3*t+2].
 * Returns 0, or 1 on a bad argument.
 */
int oracle_attention(int mode, const float* q, const float* k, const float* v, double* out,
                     long B, long Hq, long Hkv, long L, long d, long block,
                     const long* sel, long nsel, int nthreads)
{
    long rows, keys;
    if (oracle_mask_shape(mode, L, block, &rows, &keys)) return 1;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv) return 1;
    uint8_t* M = (uint8_t*)malloc((size_t)rows * (size_t)keys);
    if (!M) return 1;
    oracle_mask(mode, L, block, M);
    double scale = 1.0 / sqrt((double)d);
    long group = Hq / Hkv;
    long total = sel ? nsel : B * Hq * rows;
    const int nt = thread_count(nthreads);
    int fail = 0;
#pragma omp parallel num_threads(nt)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)keys);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long t = 0; t < total; ++t) {
                long b, h, i;
                if (sel) { b = sel[3 * t]; h = sel[3 * t + 1]; i = sel[3 * t + 2]; }
                else { b = t / (Hq * rows); h = (t / rows) % Hq; i = t % rows; }
                long g = h / group;
                const float* qrow = q + ((b * Hq + h) * rows + i) * d;
                const float* K = k + (b * Hkv + g) * keys * d;
                const float* Vv = v + (b * Hkv + g) * keys * d;
                attend_row(qrow, K, Vv, M + i * keys, keys, d, scale, out + t * d, s);
            }
            free(s);
        }
    }
    free(M);
    return fail;
}

/*
 * Gradients of the masked attention above (the training form's backward;
 * the BDLM objective of [LLaDA] trains through this attention).  With
 * loss = sum(dout * out), for every (b, h) and query row i with allowed set
 * A_i, s_ij = scale q_i.k_j, p_ij = softmax_j(s_i), o_i = sum_j p_ij v_j:
 *   dv_j   += p_ij dout_i                            (summed over rows, heads)
 *   dP_ij   = dout_i . v_j
 *   dS_ij   = p_ij (dP_ij - dout_i . o_i)
 *   dq_i    = scale sum_j dS_ij k_j
 *   dk_j   += scale dS_ij q_i                        (summed over rows, heads)
 * and lse_i = log sum_{j in A_i} exp(s_ij).  dq: [B,Hq,rows,d]; dk, dv:
 * [B,Hkv,keys,d]; lse: [B,Hq,rows] (may be NULL).  The G = Hq/Hkv query
 * heads of a kv head accumulate into its dk, dv; each (b, kv head) is one
 * task, so the sums run in a fixed order.
 */
int oracle_attention_bwd(int mode, const float* q, const float* k, const float* v, const float* dout,
                         double* dq, double* dk, double* dv, double* lse, long B, long Hq, long Hkv,
                         long L, long d, long block, int nthreads)
{
    long rows, keys;
    if (oracle_mask_shape(mode, L, block, &rows, &keys)) return 1;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv) return 1;
    uint8_t* M = (uint8_t*)malloc((size_t)rows * (size_t)keys);
    if (!M) return 1;
    oracle_mask(mode, L, block, M);
    const double scale = 1.0 / sqrt((double)d);
    const long group = Hq / Hkv;
    const int nt = thread_count(nthreads);
    int fail = 0;
#pragma omp parallel num_threads(nt)
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)keys);
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
        if (!p || !o) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long t = 0; t < B * Hkv; ++t) {
                const long b = t / Hkv, g = t % Hkv;
                const float* K = k + (b * Hkv + g) * keys * d;
                const float* Vv = v + (b * Hkv + g) * keys * d;
                double* dK = dk + (b * Hkv + g) * keys * d;
                double* dV = dv + (b * Hkv + g) * keys * d;
                for (long x = 0; x < keys * d; ++x) { dK[x] = 0.0; dV[x] = 0.0; }
                for (long h = g * group; h < (g + 1) * group; ++h) {
                    for (long i = 0; i < rows; ++i) {
                        const float* qi = q + ((b * Hq + h) * rows + i) * d;
                        const float* gi = dout + ((b * Hq + h) * rows + i) * d;
                        double* dqi = dq + ((b * Hq + h) * rows + i) * d;
                        const uint8_t* Mi = M + i * keys;
                        double m = -INFINITY;
                        for (long j = 0; j < keys; ++j) {
                            p[j] = 0.0;
                            if (!Mi[j]) continue;
                            double acc = 0.0;
                            for (long c = 0; c < d; ++c) acc += (double)qi[c] * (double)K[j * d + c];
                            p[j] = acc * scale;
                            if (p[j] > m) m = p[j];
                        }
                        double Z = 0.0;
                        for (long j = 0; j < keys; ++j)
                            if (Mi[j]) { p[j] = exp(p[j] - m); Z += p[j]; }
                        for (long c = 0; c < d; ++c) o[c] = 0.0;
                        for (long j = 0; j < keys; ++j) {
                            if (!Mi[j]) continue;
                            p[j] /= Z;
                            for (long c = 0; c < d; ++c) o[c] += p[j] * (double)Vv[j * d + c];
                        }
                        if (lse) lse[(b * Hq + h) * rows + i] = m + log(Z);
                        double Di = 0.0;
                        for (long c = 0; c < d; ++c) Di += (double)gi[c] * o[c];
                        for (long c = 0; c < d; ++c) dqi[c] = 0.0;
                        for (long j = 0; j < keys; ++j) {
                            if (!Mi[j]) continue;
                            double dP = 0.0;
                            for (long c = 0; c < d; ++c) dP += (double)gi[c] * (double)Vv[j * d + c];
                            const double dS = p[j] * (dP - Di);
                            for (long c = 0; c < d; ++c) {
                                dqi[c] += scale * dS * (double)K[j * d + c];
                                dK[j * d + c] += scale * dS * (double)qi[c];
                                dV[j * d + c] += p[j] * (double)gi[c];
                            }
                        }
                    }
                }
            }
        }
        free(p);
        free(o);
    }
    free(M);
    return fail;
}

/* ---------------------------------------------------------------------- */
/* Confidence commit ([LLaDA] SPRINT; [DGemma] Schedulers)                  */
/* ---------------------------------------------------------------------- */

/* Row statistics on the stored values: the largest logit m, its lowest index
 * a, and Z = sum_v exp(l_v - m), so the top-1 softmax probability is 1/Z. */
static void row_stats(const float* row, long V, double* m_out, long* a_out, double* Z_out)
{
    double m = (double)row[0];
    long a = 0;
    for (long j = 1; j < V; ++j)
        if ((double)row[j] > m) { m = (double)row[j]; a = j; }
    double Z = 0.0;
    for (long j = 0; j < V; ++j) Z += exp((double)row[j] - m);
    *m_out = m; *a_out = a; *Z_out = Z;
}

/*
 * Commit on logits [G, R, V] (float32 holding bf16/fp32 values).
 * For every group g, among rows r with masked[g,r] = 1:
 *   p_r  = top-1 softmax probability (double), decided on (float)p_r;
 *   C    = { r : (float)p_r > threshold }  (strict, fp32);
 *   need = min(k_min, #masked) - |C|; if need > 0, the `need` masked rows not
 *          in C with the largest (float)p_r join C (ties: lower row first);
 *   for r in C: tokens[g,r] = argmax_r, masked[g,r] = 0.  Other rows untouched.
 * Diagnostics (may be NULL): p64[G*R] (NaN for rows not masked on entry),
 * argmax[G*R] (-1 likewise), margin[G*R] = |p64 - threshold| (NaN likewise),
 * gap[G] = (float)p of the last row taken by the fallback minus that of the
 * first masked row left out (INFINITY when no fallback choice was made).
 */
int oracle_commit(const float* logits, int64_t* tokens, uint8_t* masked, float threshold, long k_min,
                  long G, long R, long V, double* p64, int64_t* argmax, double* margin, double* gap,
                  int nthreads)
{
    if (G < 0 || R < 0 || V <= 0 || k_min < 0) return 1;
    if (isnan(threshold)) return 1;
    double* p = (double*)malloc(sizeof(double) * (size_t)(G * R + 1));
    long* a = (long*)malloc(sizeof(long) * (size_t)(G * R + 1));
    if (!p || !a) { free(p); free(a); return 1; }
    const int nt = thread_count(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (long t = 0; t < G * R; ++t) {
        p[t] = NAN; a[t] = -1;
        if (!masked[t]) continue;
        double m, Z;
        long idx;
        row_stats(logits + t * V, V, &m, &idx, &Z);
        p[t] = 1.0 / Z;
        a[t] = idx;
    }
    double tau64 = (double)threshold;
    for (long g = 0; g < G; ++g) {
        const long base = g * R;
        long nmasked = 0;
        for (long r = 0; r < R; ++r) nmasked += masked[base + r] != 0;
        uint8_t* take = (uint8_t*)calloc((size_t)R + 1, 1);
        if (!take) { free(p); free(a); return 1; }
        long ntake = 0;
        for (long r = 0; r < R; ++r)
            if (masked[base + r] && (float)p[base + r] > threshold) { take[r] = 1; ++ntake; }
        long quota = k_min < nmasked ? k_min : nmasked;
        long need = quota - ntake;
        float last_in = NAN;
        for (long step = 0; step < need; ++step) {
            long best = -1;
            for (long r = 0; r < R; ++r) {
                if (!masked[base + r] || take[r]) continue;
                if (best < 0 || (float)p[base + r] > (float)p[base + best]) best = r;
            }
            take[best] = 1; ++ntake;
            last_in = (float)p[base + best];
        }
        if (gap) {
            gap[g] = INFINITY;
            if (need > 0) {
                long first_out = -1;
                for (long r = 0; r < R; ++r) {
                    if (!masked[base + r] || take[r]) continue;
                    if (first_out < 0 || (float)p[base + r] > (float)p[base + first_out]) first_out = r;
                }
                if (first_out >= 0) gap[g] = (double)last_in - (double)(float)p[base + first_out];
            }
        }
        for (long r = 0; r < R; ++r) {
            long t = base + r;
            if (p64) p64[t] = p[t];
            if (argmax) argmax[t] = a[t];
            if (margin) margin[t] = masked[t] ? fabs(p[t] - tau64) : NAN;
        }
        for (long r = 0; r < R; ++r) {
            if (!take[r]) continue;
            tokens[base + r] = a[base + r];
            masked[base + r] = 0;
        }
        free(take);
    }
    free(p);
    free(a);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Verify ([NLD-3x] sec. 2)                                                 */
/* ---------------------------------------------------------------------- */

/* argmax_out[b,j] = lowest index of the largest logit of row (b, j);
 * accept[b] = first j with argmax != drafts[b,j], or R when all agree. */
int oracle_verify(const float* logits, const int64_t* drafts, int64_t* argmax_out, int32_t* accept,
                  long B, long R, long V, int nthreads)
{
    if (B < 0 || R < 0 || V <= 0) return 1;
    const int nt = thread_count(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (long t = 0; t < B * R; ++t) {
        const float* row = logits + t * V;
        double m = (double)row[0];
        long idx = 0;
        for (long j = 1; j < V; ++j)
            if ((double)row[j] > m) { m = (double)row[j]; idx = j; }
        argmax_out[t] = idx;
    }
    for (long b = 0; b < B; ++b) {
        long acc = R;
        for (long j = 0; j < R; ++j)
            if (argmax_out[b * R + j] != drafts[b * R + j]) { acc = j; break; }
        accept[b] = (int32_t)acc;
    }
    return 0;
}

/*
 * Per-row softmax statistics ([DGemma] "Adaptive stopping": the mean
 * per-token entropy of the predicted distribution; "Schedulers": the
 * entropy-bound scheduler ranks positions by entropy; [LLaDA] SPRINT:
 * confidence = top-1 probability).  For each selected row (masked == NULL or
 * masked[t] != 0): p_j = exp(l_j) / sum_k exp(l_k) at temperature 1,
 * conf = max_j p_j, argmax = lowest j reaching the largest logit, and the
 * entropy -sum_j p_j log p_j in nats, written term by term (p_j = 0 adds
 * nothing).  mean[g] = mean entropy over the group's selected rows, 0 if
 * none.  Unselected rows are left untouched.
 */
int oracle_row_stats(const float* logits, const uint8_t* masked, double* conf, int64_t* argmax,
                     double* entropy, double* mean, long G, long R, long V, int nthreads)
{
    if (G < 0 || R < 0 || V <= 0) return 1;
    const int nt = thread_count(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (long t = 0; t < G * R; ++t) {
        if (masked && !masked[t]) continue;
        const float* row = logits + t * V;
        double m = (double)row[0];
        long idx = 0;
        for (long j = 1; j < V; ++j)
            if ((double)row[j] > m) { m = (double)row[j]; idx = j; }
        double Z = 0.0;
        for (long j = 0; j < V; ++j) Z += exp((double)row[j] - m);
        double H = 0.0;
        for (long j = 0; j < V; ++j) {
            const double pj = exp((double)row[j] - m) / Z;
            if (pj > 0.0) H -= pj * log(pj);
        }
        conf[t] = 1.0 / Z;
        argmax[t] = idx;
        entropy[t] = H;
    }
    for (long g = 0; g < G; ++g) {
        double sum = 0.0;
        long n = 0;
        for (long r = 0; r < R; ++r) {
            const long t = g * R + r;
            if (masked && !masked[t]) continue;
            sum += entropy[t];
            ++n;
        }
        mean[g] = n > 0 ? sum / (double)n : 0.0;
    }
    return 0;
}

/*
 * Entropy-bound commit ([DGemma] "Schedulers", EntropyBoundScheduler: commit
 * the lowest-entropy positions whose joint entropy stays within the bound).
 * For each masked row t of group g: p_j = softmax(l_j / T) with T =
 * temperature, H_t = -sum_j p_j log p_j in nats (term by term), a_t = lowest
 * j reaching the largest logit.  The group's masked rows are ordered by
 * (H ascending, row ascending); with S_j the sum of the first j entropies,
 * the first n rows are committed, n = max(min(k_min, #masked),
 * max{ j : S_j <= bound }): tokens = a, masked = 0.  Joint entropy is read as
 * the sum of the per-position entropies (independent positions).
 * entropy[t] / argmax[t] are written for masked rows.  Returns 0, 1 on a bad
 * argument.
 */
static const double *g_ent_key;
static int ent_cmp(const void *x, const void *y)
{
    const long a = *(const long *)x, b = *(const long *)y;
    const double ha = g_ent_key[a], hb = g_ent_key[b];
    if (ha < hb) return -1;
    if (ha > hb) return 1;
    return (a > b) - (a < b);
}

int oracle_commit_entropy(const float* logits, int64_t* tokens, uint8_t* masked, double bound, double temperature,
                          long k_min, long G, long R, long V, double* entropy, int64_t* argmax, int nthreads)
{
    if (G < 0 || R < 0 || V <= 0 || k_min < 0 || !(temperature > 0.0)) return 1;
    const int nt = thread_count(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (long t = 0; t < G * R; ++t) {
        if (!masked[t]) continue;
        const float* row = logits + t * V;
        double m = (double)row[0];
        long idx = 0;
        for (long j = 1; j < V; ++j)
            if ((double)row[j] > m) { m = (double)row[j]; idx = j; }
        double Z = 0.0;
        for (long j = 0; j < V; ++j) Z += exp(((double)row[j] - m) / temperature);
        double H = 0.0;
        for (long j = 0; j < V; ++j) {
            const double pj = exp(((double)row[j] - m) / temperature) / Z;
            if (pj > 0.0) H -= pj * log(pj);
        }
        entropy[t] = H;
        argmax[t] = idx;
    }
    long* order = (long*)malloc(sizeof(long) * (size_t)(R > 0 ? R : 1));
    if (!order) return 1;
    for (long g = 0; g < G; ++g) {
        long n = 0;
        for (long r = 0; r < R; ++r)
            if (masked[g * R + r]) order[n++] = g * R + r;
        g_ent_key = entropy;
        qsort(order, (size_t)n, sizeof(long), ent_cmp);
        long take = 0;
        double sum = 0.0;
        for (long j = 0; j < n; ++j) {
            sum += entropy[order[j]];
            if (sum <= bound) take = j + 1;
            else break;
        }
        if (take < (k_min < n ? k_min : n)) take = k_min < n ? k_min : n;
        for (long j = 0; j < take; ++j) {
            tokens[order[j]] = argmax[order[j]];
            masked[order[j]] = 0;
        }
    }
    free(order);
    return 0;
}

/*
 * SPRINT sparse prefix retention ([LLaDA] "SPRINT": the cache is pruned once
 * at the start of a block).  For batch b and prefix position i:
 *   n_i   = || k_{b,.,i,.} ||_2 over all kv heads and channels,
 *   I_i   = n_i / ((1/L) sum_j n_j)                 (mean-normalised key norm),
 *   s_i   = alpha * I_i + (1 - alpha) * conf[b,i]    (composite score),
 * then, separately for image positions (modality 1) and text positions (0),
 * the keep_m = floor(r_m * count_m + 0.5) positions with the largest s_i are
 * kept (ties: lower position first).  kept[b, 0..K) lists the kept positions
 * in increasing order, -1 after; scores[b, i] = s_i.  Returns K (the same
 * for every batch), or -1 on a bad argument.
 */
long oracle_sprint(const float* k, const float* conf, const uint8_t* modality, double alpha, double r_img,
                   double r_text, long B, long Hkv, long L, long d, int64_t* kept, double* scores)
{
    if (B <= 0 || Hkv <= 0 || L <= 0 || d <= 0) return -1;
    long cnt[2] = {0, 0};
    for (long i = 0; i < L; ++i) cnt[modality[i] ? 1 : 0]++;
    const long keep[2] = {(long)floor(r_text * (double)cnt[0] + 0.5), (long)floor(r_img * (double)cnt[1] + 0.5)};
    if (keep[0] < 0 || keep[0] > cnt[0] || keep[1] < 0 || keep[1] > cnt[1]) return -1;
    double* nrm = (double*)malloc(sizeof(double) * (size_t)L);
    long* order = (long*)malloc(sizeof(long) * (size_t)L);
    uint8_t* take = (uint8_t*)malloc((size_t)L);
    if (!nrm || !order || !take) { free(nrm); free(order); free(take); return -1; }
    for (long b = 0; b < B; ++b) {
        double mean = 0.0;
        for (long i = 0; i < L; ++i) {
            double ss = 0.0;
            for (long h = 0; h < Hkv; ++h)
                for (long c = 0; c < d; ++c) {
                    const double x = (double)k[((b * Hkv + h) * L + i) * d + c];
                    ss += x * x;
                }
            nrm[i] = sqrt(ss);
            mean += nrm[i];
        }
        mean /= (double)L;
        double* sc = scores + b * L;
        for (long i = 0; i < L; ++i)
            sc[i] = alpha * (nrm[i] / mean) + (1.0 - alpha) * (double)conf[b * L + i];
        for (long i = 0; i < L; ++i) take[i] = 0;
        for (int m = 0; m < 2; ++m) {
            /* selection: repeatedly take the best remaining position of modality m */
            for (long t = 0; t < keep[m]; ++t) {
                long best = -1;
                for (long i = 0; i < L; ++i) {
                    if ((modality[i] ? 1 : 0) != m || take[i]) continue;
                    if (best < 0 || sc[i] > sc[best]) best = i;
                }
                take[best] = 1;
            }
        }
        long K = 0;
        for (long i = 0; i < L; ++i)
            if (take[i]) kept[b * L + K++] = i;
        for (long j = K; j < L; ++j) kept[b * L + j] = -1;
    }
    free(nrm); free(order); free(take);
    return keep[0] + keep[1];
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
