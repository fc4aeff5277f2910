/*
 * dsa_oracle.c -- plain, slow CPU oracle for the DeepSeek Sparse Attention
 * (DSA) forward path: pooled lightning-indexer scores, per-query top-k pool
 * selection, and softmax attention restricted to the selected tokens.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load or call
 * this library: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * helper with the GPU library; both sides only consume the same seeded
 * input arrays.
 *
 * What is computed, and where it comes from (SkyRL blog, "Scaling Training
 * to 1M Token Context on GLM-5.3-Flash"):
 *   - section "DeepSeek Sparse Attention (DSA) Optimizations": an indexer
 *     rates, for each query, each pool of 4 tokens lying wholly before it;
 *     attention then reads the chosen tokens alone (2048 = 512 pools x 4);
 *   - section "Making Sparse Attention Actually Sparse": NoPE heads (no
 *     rotary channels, so narrower heads) and 2,051 selected keys;
 *   - section "Splitting the DSA Indexer / Over Time: Chunking": scores are
 *     fp32, formed and selected for chunks of hundreds of queries;
 *   - section "Across GPUs: Sharding": selected pool indices are int32.
 * The page prints no formula for the indexer score.  The reading used here
 * is the standard lightning-indexer form: a head-weighted sum of ReLU'd dot
 * products of the query's indexer heads with the mean-pooled key,
 *     s(t,p) = sum_h w[t,h] * max(0, sum_d q_idx[t,h,d] * kbar_p[d]),
 *     kbar_p[d] = (k[4p][d] + k[4p+1][d] + k[4p+2][d] + k[4p+3][d]) / 4,
 * with no extra scale factor, ties in the top-k broken towards the lower
 * pool index.
 *
 * Readings of points the page leaves open (each one also pinned by tests):
 *   - "earlier pool" is strict: pool p is eligible for the query at
 *     position t iff all of its tokens precede t, i.e. p < floor(t/4)
 *     (and p < P = floor(S_k/4));
 *   - kbar is kept exact (fp64); each score is rounded once to fp32 and the
 *     ranking (and its tie-break) is taken on that fp32 value; a zero score
 *     is canonicalised to +0;
 *   - the selected pool ids are emitted in ascending order, padded with -1
 *     when fewer than k pools are eligible;
 *   - the 2,051 keys are 512 pools x 4 tokens plus up to 3 tokens of the
 *     query's own unfinished pool that precede it ("tail"); no query attends
 *     to itself;
 *   - attention logits are scaled by a caller-given factor (1/sqrt(D) by
 *     default); an empty token set gives output 0 and lse = -inf;
 *   - fp8 variant (OCP E4M3, "e4m3fn"): q and k arrive as codes with
 *     per-tensor fp32 scales.  The pooled key is re-quantised per pool to
 *     E4M3 with a power-of-two scale 2^e, e the smallest integer with
 *     max_d |mean code value| <= 448 * 2^e, so that the quantisation is a
 *     round-to-nearest-even of an exactly scaled value and no precision
 *     choice can change a code;
 *   - gated pooling (section "DSA: Gather by Token Position" mentions
 *     per-token gate scores applied to the keys inside each pool; it prints
 *     no normalisation): with a per-token gate array g the pooled key is the plain
 *     gate-weighted sum kbar_p = sum_r g[4p+r] * k[4p+r], the caller
 *     supplying normalised gates.  Without gates the mean is used, which is
 *     the gated sum with every gate equal to 1/4.
 *
 *   - backward of the attention (the pages' setting is training; they print
 *     no backward): the exact gradient of the forward's definition for the
 *     loss sum dout . o, D taken from the exact fp64 forward.
 *
 * Everything is accumulated in fp64 in plain loops; no blocking, fusion or
 * reordering beyond the definitions above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_IDX (-2)
#define ORACLE_ERR_MEM (-3)

/* ------------------------------------------------------------------ */
/* Number formats                                                     */
/* ------------------------------------------------------------------ */

/* bfloat16 is the upper half of an IEEE-754 binary32; widening is exact. */
double dsa_oracle_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * No infinities; S.1111.111 is NaN; exponent field 0 holds subnormals
 * m * 2^-9; the largest finite magnitude is 1.75 * 2^8 = 448. */
double dsa_oracle_e4m3_value(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest E4M3 code to x, ties to the even mantissa, magnitudes beyond 448
 * saturate to 448.  Written as a search over all finite codes: obviously
 * correct, not fast. */
uint8_t dsa_oracle_e4m3_encode(double x)
{
    double a = fabs(x);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double err = fabs(dsa_oracle_e4m3_value((uint8_t)c) - a);
        /* codes are visited in increasing magnitude; on an exact tie keep
         * the one whose mantissa (lowest code bit) is even */
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    if (a > 448.0)
        best = 0x7E;
    return (uint8_t)(best | ((x < 0.0 || (x == 0.0 && signbit(x))) ? 0x80 : 0));
}

/* ------------------------------------------------------------------ */
/* Shared definitions                                                 */
/* ------------------------------------------------------------------ */

/* Number of pools eligible for the query at position t. */
static int64_t eligible_pools(int64_t t, int pool, int64_t n_pools)
{
    int64_t n = t / pool;
    return n < n_pools ? n : n_pools;
}

static float canonical_f32(double s)
{
    float f = (float)s;
    return f == 0.0f ? 0.0f : f;
}

/* Pooled keys in fp64 from bf16 keys: kbar[p][d] = mean of the pool's rows,
 * or, with gates, sum_r gate[p*pool + r] * k[p*pool + r][d]. */
static void pool_keys_bf16(const uint16_t *k_idx, const float *gate, int64_t n_pools,
                           int d_idx, int pool, double *kbar)
{
    for (int64_t p = 0; p < n_pools; ++p)
        for (int d = 0; d < d_idx; ++d) {
            double sum = 0.0;
            for (int r = 0; r < pool; ++r) {
                double x = dsa_oracle_bf16_value(k_idx[(p * pool + r) * d_idx + d]);
                sum += gate ? (double)gate[p * pool + r] * x : x;
            }
            kbar[p * d_idx + d] = gate ? sum : sum / pool;
        }
}

/* fp8 pooled keys: mean (or gate-weighted sum) of the pool's code values,
 * re-quantised per pool to E4M3 with a power-of-two scale.  kbar8 receives
 * the fp64 value of the re-quantised codes times 2^e (the per-tensor k scale
 * is applied by the caller); codes and exponents are returned for
 * inspection when non-NULL. */
static void pool_keys_fp8(const uint8_t *k8, const float *gate, int64_t n_pools, int d_idx,
                          int pool, double *kbar8, uint8_t *codes, int32_t *exps)
{
    double *m = (double *)malloc(sizeof(double) * (size_t)d_idx);
    for (int64_t p = 0; p < n_pools; ++p) {
        double amax = 0.0;
        for (int d = 0; d < d_idx; ++d) {
            double sum = 0.0;
            for (int r = 0; r < pool; ++r) {
                double x = dsa_oracle_e4m3_value(k8[(p * pool + r) * d_idx + d]);
                sum += gate ? (double)gate[p * pool + r] * x : x;
            }
            m[d] = gate ? sum : sum / pool;
            if (fabs(m[d]) > amax)
                amax = fabs(m[d]);
        }
        int e = 0;
        if (amax > 0.0) {
            e = (int)floor(log2(amax / 448.0)) - 2;
            while (amax > ldexp(448.0, e))
                ++e;
        }
        for (int d = 0; d < d_idx; ++d) {
            uint8_t c = dsa_oracle_e4m3_encode(ldexp(m[d], -e));
            if (codes)
                codes[p * d_idx + d] = c;
            kbar8[p * d_idx + d] = ldexp(dsa_oracle_e4m3_value(c), e);
        }
        if (exps)
            exps[p] = e;
    }
    free(m);
}

/* s(t,p) in fp64 for one query (q_t widened to fp64, [h_idx][d_idx]). */
static double score_one(const double *q_t, const double *kbar_p, const double *w_t,
                        int h_idx, int d_idx, double qk_scale)
{
    double s = 0.0;
    for (int h = 0; h < h_idx; ++h) {
        double dot = 0.0;
        for (int d = 0; d < d_idx; ++d)
            dot += q_t[h * d_idx + d] * kbar_p[d];
        dot *= qk_scale;
        double relu = dot > 0.0 ? dot : 0.0;
        s += w_t[h] * relu;
    }
    return s;
}

typedef struct {
    float s;
    int32_t p;
} scored_pool;

/* Descending score, then ascending pool id (ties to the lower index). */
static int by_score_then_index(const void *a, const void *b)
{
    const scored_pool *x = (const scored_pool *)a, *y = (const scored_pool *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->p > y->p) - (x->p < y->p);
}

static int by_index(const void *a, const void *b)
{
    const scored_pool *x = (const scored_pool *)a, *y = (const scored_pool *)b;
    return (x->p > y->p) - (x->p < y->p);
}

/* Scores of every pool for the listed rows (fp32; -inf where not eligible),
 * and/or the top-k selection.  q is given either as bf16 bits or as fp8
 * codes; kbar is the fp64 pooled key table already built by the caller. */
static int score_and_select(const uint16_t *q_bf16, const uint8_t *q_fp8, double q_scale,
                            const double *kbar, double qk_scale, const float *w,
                            int64_t w_stride, int64_t s_q, int64_t q_pos0, int64_t n_pools,
                            int h_idx, int d_idx, int pool, int k_pools,
                            const int64_t *rows, int64_t n_rows, float *scores_out,
                            int32_t *idx_out, float *sel_scores_out)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t i = rows[r];
        if (i < 0 || i >= s_q) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        int64_t t = q_pos0 + i;
        int64_t n = eligible_pools(t, pool, n_pools);
        double *q_t = (double *)malloc(sizeof(double) * (size_t)h_idx * d_idx);
        double *w_t = (double *)malloc(sizeof(double) * (size_t)h_idx);
        scored_pool *sp = (scored_pool *)malloc(sizeof(scored_pool) * (size_t)(n > 0 ? n : 1));
        for (int e = 0; e < h_idx * d_idx; ++e)
            q_t[e] = q_bf16 ? dsa_oracle_bf16_value(q_bf16[i * h_idx * d_idx + e])
                            : q_scale * dsa_oracle_e4m3_value(q_fp8[i * h_idx * d_idx + e]);
        for (int h = 0; h < h_idx; ++h)
            w_t[h] = (double)w[i * w_stride + h];
        for (int64_t p = 0; p < n; ++p) {
            sp[p].s = canonical_f32(score_one(q_t, kbar + p * d_idx, w_t, h_idx, d_idx, qk_scale));
            sp[p].p = (int32_t)p;
        }
        if (scores_out) {
            for (int64_t p = 0; p < n_pools; ++p)
                scores_out[r * n_pools + p] = p < n ? sp[p].s : -INFINITY;
        }
        if (idx_out) {
            int64_t take = n;
            if (n > k_pools) {
                qsort(sp, (size_t)n, sizeof(scored_pool), by_score_then_index);
                take = k_pools;
            }
            qsort(sp, (size_t)take, sizeof(scored_pool), by_index);
            for (int j = 0; j < k_pools; ++j) {
                idx_out[r * k_pools + j] = j < take ? sp[j].p : -1;
                if (sel_scores_out)
                    sel_scores_out[r * k_pools + j] = j < take ? sp[j].s : -INFINITY;
            }
        }
        free(q_t);
        free(w_t);
        free(sp);
    }
    return bad ? ORACLE_ERR_ARG : ORACLE_OK;
}

static int check_index_args(int64_t s_q, int64_t s_k, int64_t q_pos0, int h_idx, int d_idx,
                            int pool, int k_pools, int64_t n_rows)
{
    if (s_q < 0 || s_k < 0 || q_pos0 < 0 || h_idx <= 0 || d_idx <= 0 || pool <= 0 ||
        k_pools <= 0 || n_rows < 0)
        return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Public entry points (bf16 indexer)                                 */
/* ------------------------------------------------------------------ */

/* Pooled keys in fp64, [floor(s_k/pool), d_idx]; gate [s_k] or NULL (mean). */
int dsa_oracle_pool_keys(const uint16_t *k_idx, const float *gate, int64_t s_k, int d_idx,
                         int pool, double *kbar)
{
    if (s_k < 0 || d_idx <= 0 || pool <= 0 || !kbar)
        return ORACLE_ERR_ARG;
    pool_keys_bf16(k_idx, gate, s_k / pool, d_idx, pool, kbar);
    return ORACLE_OK;
}

/* Dense fp32 scores for the listed rows: out[r][p], p < P; -inf where the
 * pool is not eligible for that row's query. */
int dsa_oracle_index_scores(const uint16_t *q_idx, const uint16_t *k_idx, const float *gate,
                            const float *w,
                            int64_t w_stride, int64_t s_q, int64_t s_k, int64_t q_pos0,
                            int h_idx, int d_idx, int pool, const int64_t *rows,
                            int64_t n_rows, float *out)
{
    if (check_index_args(s_q, s_k, q_pos0, h_idx, d_idx, pool, 1, n_rows) || !out)
        return ORACLE_ERR_ARG;
    int64_t n_pools = s_k / pool;
    double *kbar = (double *)malloc(sizeof(double) * (size_t)(n_pools > 0 ? n_pools : 1) * d_idx);
    if (!kbar)
        return ORACLE_ERR_MEM;
    pool_keys_bf16(k_idx, gate, n_pools, d_idx, pool, kbar);
    int rc = score_and_select(q_idx, NULL, 1.0, kbar, 1.0, w, w_stride, s_q, q_pos0, n_pools,
                              h_idx, d_idx, pool, 1, rows, n_rows, out, NULL, NULL);
    free(kbar);
    return rc;
}

/* Top-k pool selection for the listed rows: idx_out[r][0..k) ascending
 * pool ids, -1 padded; sel_scores_out (optional) the matching fp32 scores,
 * -inf for padding. */
int dsa_oracle_index_topk(const uint16_t *q_idx, const uint16_t *k_idx, const float *gate,
                          const float *w,
                          int64_t w_stride, int64_t s_q, int64_t s_k, int64_t q_pos0,
                          int h_idx, int d_idx, int pool, int k_pools, const int64_t *rows,
                          int64_t n_rows, int32_t *idx_out, float *sel_scores_out)
{
    if (check_index_args(s_q, s_k, q_pos0, h_idx, d_idx, pool, k_pools, n_rows) || !idx_out)
        return ORACLE_ERR_ARG;
    int64_t n_pools = s_k / pool;
    double *kbar = (double *)malloc(sizeof(double) * (size_t)(n_pools > 0 ? n_pools : 1) * d_idx);
    if (!kbar)
        return ORACLE_ERR_MEM;
    pool_keys_bf16(k_idx, gate, n_pools, d_idx, pool, kbar);
    int rc = score_and_select(q_idx, NULL, 1.0, kbar, 1.0, w, w_stride, s_q, q_pos0, n_pools,
                              h_idx, d_idx, pool, k_pools, rows, n_rows, NULL, idx_out,
                              sel_scores_out);
    free(kbar);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Public entry points (fp8 E4M3 indexer)                             */
/* ------------------------------------------------------------------ */

/* Re-quantised pooled keys: codes [P, d_idx] and per-pool exponents [P]. */
int dsa_oracle_pool_keys_fp8(const uint8_t *k8, const float *gate, int64_t s_k, int d_idx,
                             int pool, uint8_t *codes, int32_t *exps)
{
    if (s_k < 0 || d_idx <= 0 || pool <= 0 || !codes || !exps)
        return ORACLE_ERR_ARG;
    int64_t n_pools = s_k / pool;
    double *kbar8 = (double *)malloc(sizeof(double) * (size_t)(n_pools > 0 ? n_pools : 1) * d_idx);
    if (!kbar8)
        return ORACLE_ERR_MEM;
    pool_keys_fp8(k8, gate, n_pools, d_idx, pool, kbar8, codes, exps);
    free(kbar8);
    return ORACLE_OK;
}

/* fp8 scores: s = sum_h w * relu(q_scale * k_scale * q8 . (2^e_p * kbar8_p)). */
int dsa_oracle_index_scores_fp8(const uint8_t *q8, const uint8_t *k8, const float *gate,
                                float q_scale,
                                float k_scale, const float *w, int64_t w_stride, int64_t s_q,
                                int64_t s_k, int64_t q_pos0, int h_idx, int d_idx, int pool,
                                const int64_t *rows, int64_t n_rows, float *out)
{
    if (check_index_args(s_q, s_k, q_pos0, h_idx, d_idx, pool, 1, n_rows) || !out)
        return ORACLE_ERR_ARG;
    int64_t n_pools = s_k / pool;
    double *kbar8 = (double *)malloc(sizeof(double) * (size_t)(n_pools > 0 ? n_pools : 1) * d_idx);
    if (!kbar8)
        return ORACLE_ERR_MEM;
    pool_keys_fp8(k8, gate, n_pools, d_idx, pool, kbar8, NULL, NULL);
    int rc = score_and_select(NULL, q8, (double)q_scale, kbar8, (double)k_scale, w, w_stride, s_q,
                              q_pos0, n_pools, h_idx, d_idx, pool, 1, rows, n_rows, out, NULL,
                              NULL);
    free(kbar8);
    return rc;
}

int dsa_oracle_index_topk_fp8(const uint8_t *q8, const uint8_t *k8, const float *gate,
                              float q_scale, float k_scale,
                              const float *w, int64_t w_stride, int64_t s_q, int64_t s_k,
                              int64_t q_pos0, int h_idx, int d_idx, int pool, int k_pools,
                              const int64_t *rows, int64_t n_rows, int32_t *idx_out,
                              float *sel_scores_out)
{
    if (check_index_args(s_q, s_k, q_pos0, h_idx, d_idx, pool, k_pools, n_rows) || !idx_out)
        return ORACLE_ERR_ARG;
    int64_t n_pools = s_k / pool;
    double *kbar8 = (double *)malloc(sizeof(double) * (size_t)(n_pools > 0 ? n_pools : 1) * d_idx);
    if (!kbar8)
        return ORACLE_ERR_MEM;
    pool_keys_fp8(k8, gate, n_pools, d_idx, pool, kbar8, NULL, NULL);
    int rc = score_and_select(NULL, q8, (double)q_scale, kbar8, (double)k_scale, w, w_stride, s_q,
                              q_pos0, n_pools, h_idx, d_idx, pool, k_pools, rows, n_rows, NULL,
                              idx_out, sel_scores_out);
    free(kbar8);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Sparse attention                                                   */
/* ------------------------------------------------------------------ */

/* The token set T(t) of the query at position t (see the attention section
 * below): the tokens of every pool listed in idx row `row` (strictly
 * ascending ids in [0, n), then only -1), followed, when n_tail > 0, by the
 * up to n_tail tokens of t's own pool that precede t.  Writes the token
 * positions to tok (room for k_pools * pool + pool entries) and their number
 * to *n_tok; returns ORACLE_ERR_IDX for a malformed row. */
static int token_set(const int32_t *row, int k_pools, int pool, int64_t n, int64_t t,
                     int n_tail, int64_t s_k, int64_t *tok, int64_t *n_tok)
{
    int64_t cnt = 0, prev = -1;
    int ended = 0;
    for (int j = 0; j < k_pools; ++j) {
        int64_t p = row[j];
        if (p < 0) {
            if (p != -1)
                return ORACLE_ERR_IDX;
            ended = 1;
            continue;
        }
        if (ended || p <= prev || p >= n)
            return ORACLE_ERR_IDX;
        prev = p;
        for (int u = 0; u < pool; ++u)
            tok[cnt++] = p * pool + u;
    }
    if (n_tail > 0) {
        int64_t start = (t / pool) * pool;
        if (t - n_tail > start)
            start = t - n_tail;
        for (int64_t j = start; j < t && j < s_k; ++j)
            tok[cnt++] = j;
    }
    *n_tok = cnt;
    return ORACLE_OK;
}

/* For each listed row r (query position t = q_pos0 + rows[r]) and head h:
 *   T(t)  = tokens {pool*p .. pool*p+pool-1} of every pool p >= 0 in
 *           idx[r][0..k_pools) (which must be strictly ascending, eligible,
 *           and followed only by -1), plus, when n_tail > 0, the up to
 *           n_tail tokens of t's own pool that precede t;
 *   l_j   = scale * q[t,h,:] . k[j,:]            for j in T(t)
 *   o     = sum_j exp(l_j - m) v[j,:] / sum_j exp(l_j - m),  m = max_j l_j
 *   lse   = m + log(sum_j exp(l_j - m))
 * An empty T(t) gives o = 0 and lse = -inf.  o is [n_rows, h, dv], lse
 * [n_rows, h], both fp64.  Returns ORACLE_ERR_IDX for a malformed idx row. */
int dsa_oracle_sparse_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const int32_t *idx, int64_t s_q, int64_t s_k, int64_t q_pos0,
                           int h, int d, int dv, int k_pools, int pool, int n_tail,
                           double scale, const int64_t *rows, int64_t n_rows, double *o,
                           double *lse)
{
    if (s_q < 0 || s_k < 0 || q_pos0 < 0 || h <= 0 || d <= 0 || dv <= 0 || k_pools <= 0 ||
        pool <= 0 || n_tail < 0 || n_tail >= pool || n_rows < 0 || !o || !lse)
        return ORACLE_ERR_ARG;
    int64_t n_pools = s_k / pool;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t i = rows[r];
        if (i < 0 || i >= s_q) {
#pragma omp atomic write
            bad = ORACLE_ERR_ARG;
            continue;
        }
        int64_t t = q_pos0 + i;
        int64_t n = eligible_pools(t, pool, n_pools);
        const int32_t *row = idx + r * k_pools;
        int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k_pools * pool + pool));
        int64_t n_tok = 0;
        int row_bad = token_set(row, k_pools, pool, n, t, n_tail, s_k, tok, &n_tok);
        if (row_bad) {
#pragma omp atomic write
            bad = ORACLE_ERR_IDX;
            free(tok);
            continue;
        }
        double *logit = (double *)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1));
        for (int hh = 0; hh < h; ++hh) {
            double *o_th = o + (r * h + hh) * dv;
            if (n_tok == 0) {
                for (int e = 0; e < dv; ++e)
                    o_th[e] = 0.0;
                lse[r * h + hh] = -INFINITY;
                continue;
            }
            const uint16_t *q_th = q + (i * h + hh) * d;
            double m = -INFINITY;
            for (int64_t a = 0; a < n_tok; ++a) {
                double dot = 0.0;
                for (int e = 0; e < d; ++e)
                    dot += dsa_oracle_bf16_value(q_th[e]) * dsa_oracle_bf16_value(k[tok[a] * d + e]);
                logit[a] = scale * dot;
                if (logit[a] > m)
                    m = logit[a];
            }
            double z = 0.0;
            for (int64_t a = 0; a < n_tok; ++a)
                z += exp(logit[a] - m);
            for (int e = 0; e < dv; ++e) {
                double acc = 0.0;
                for (int64_t a = 0; a < n_tok; ++a)
                    acc += exp(logit[a] - m) * dsa_oracle_bf16_value(v[tok[a] * dv + e]);
                o_th[e] = acc / z;
            }
            lse[r * h + hh] = m + log(z);
        }
        free(logit);
        free(tok);
    }
    return bad;
}

/* Gradients of the sparse attention above.  The pages' setting is training
 * (section "Activation Recompute": each layer's forward is rerun in the
 * backward pass); the page prints no backward, so this is the gradient of
 * the forward's definition written out.  For the loss L = sum dout . o over
 * the listed rows (equivalently: dout set to zero on every other row), per
 * listed row r (position t, query row i = rows[r]) and head h, with P_j the
 * softmax weights of T(t):
 *   dP_j = dout[i,h,:] . v[j,:]
 *   D    = sum_j P_j dP_j                  (= dout[i,h,:] . o[i,h,:])
 *   dS_j = P_j (dP_j - D)                  (gradient of L wrt logit l_j)
 *   dq[r,h,:]  = scale * sum_j dS_j k[j,:]
 *   dk[j,:]   += scale * dS_j q[i,h,:]     for every j in T(t)
 *   dv[j,:]   += P_j dout[i,h,:]
 * dq is [n_rows, h, d]; dk [s_k, d] and dv [s_k, dv] cover every key row
 * (rows no listed query attends stay 0).  All fp64.
 *
 * Optional magnitudes (any of dq_mag, dk_mag, dv_mag may be NULL), the same
 * sums over absolute values, from which a floating-point error bound of an
 * implementation that rounds the weights or the stored output follows:
 *   Dabs  = sum_e |dout[i,h,e]| sum_j P_j |v[j,e]|
 *   m_j   = |dS_j| + P_j Dabs
 *   dq_mag[r,h,:] = scale * sum_j m_j |k[j,:]|
 *   dk_mag[j,:]  += scale * m_j |q[i,h,:]|
 *   dv_mag[j,:]  += P_j |dout[i,h,:]|
 * Rows are processed in the listed order, heads and tokens in increasing
 * order.  Returns ORACLE_ERR_IDX for a malformed idx row (outputs are then
 * incomplete). */
int dsa_oracle_sparse_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const int32_t *idx, const uint16_t *dout, int64_t s_q,
                               int64_t s_k, int64_t q_pos0, int h, int d, int dv, int k_pools,
                               int pool, int n_tail, double scale, const int64_t *rows,
                               int64_t n_rows, double *dq, double *dk, double *dvv,
                               double *dq_mag, double *dk_mag, double *dv_mag)
{
    if (s_q < 0 || s_k < 0 || q_pos0 < 0 || h <= 0 || d <= 0 || dv <= 0 || k_pools <= 0 ||
        pool <= 0 || n_tail < 0 || n_tail >= pool || n_rows < 0 || !dq || !dk || !dvv)
        return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= s_q)
            return ORACLE_ERR_ARG;
    int64_t n_pools = s_k / pool;
    memset(dk, 0, sizeof(double) * (size_t)(s_k * d));
    memset(dvv, 0, sizeof(double) * (size_t)(s_k * dv));
    if (dk_mag)
        memset(dk_mag, 0, sizeof(double) * (size_t)(s_k * d));
    if (dv_mag)
        memset(dv_mag, 0, sizeof(double) * (size_t)(s_k * dv));
    int64_t cap = (int64_t)k_pools * pool + pool;
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
    /* per head: P_j, dS_j, m_j of the current row */
    double *pw = (double *)malloc(sizeof(double) * (size_t)(h * cap));
    double *ds = (double *)malloc(sizeof(double) * (size_t)(h * cap));
    double *mj = (double *)malloc(sizeof(double) * (size_t)(h * cap));
    if (!tok || !pw || !ds || !mj) {
        free(tok);
        free(pw);
        free(ds);
        free(mj);
        return ORACLE_ERR_MEM;
    }
    int rc = ORACLE_OK;
    for (int64_t r = 0; r < n_rows && rc == ORACLE_OK; ++r) {
        int64_t i = rows[r];
        int64_t t = q_pos0 + i;
        int64_t n_tok = 0;
        if (token_set(idx + r * k_pools, k_pools, pool, eligible_pools(t, pool, n_pools), t,
                      n_tail, s_k, tok, &n_tok)) {
            rc = ORACLE_ERR_IDX;
            break;
        }
        /* per head: softmax weights, dS, magnitudes and dq (heads are
         * independent; each writes only its own slices) */
#pragma omp parallel for schedule(static)
        for (int hh = 0; hh < h; ++hh) {
            const uint16_t *q_th = q + (i * h + hh) * d;
            const uint16_t *do_th = dout + (i * h + hh) * dv;
            double *P = pw + (int64_t)hh * cap, *dS = ds + (int64_t)hh * cap;
            double *M = mj + (int64_t)hh * cap;
            double *dq_th = dq + (r * h + hh) * d;
            for (int e = 0; e < d; ++e) {
                dq_th[e] = 0.0;
                if (dq_mag)
                    dq_mag[(r * h + hh) * d + e] = 0.0;
            }
            if (n_tok == 0)
                continue;
            double m = -INFINITY;
            for (int64_t a = 0; a < n_tok; ++a) {
                double dot = 0.0;
                for (int e = 0; e < d; ++e)
                    dot += dsa_oracle_bf16_value(q_th[e]) * dsa_oracle_bf16_value(k[tok[a] * d + e]);
                P[a] = scale * dot;
                if (P[a] > m)
                    m = P[a];
            }
            double z = 0.0;
            for (int64_t a = 0; a < n_tok; ++a)
                z += exp(P[a] - m);
            for (int64_t a = 0; a < n_tok; ++a)
                P[a] = exp(P[a] - m) / z;
            double D = 0.0;
            for (int64_t a = 0; a < n_tok; ++a) {
                double dp = 0.0;
                for (int e = 0; e < dv; ++e)
                    dp += dsa_oracle_bf16_value(do_th[e]) * dsa_oracle_bf16_value(v[tok[a] * dv + e]);
                dS[a] = dp;  /* dP_j for now */
                D += P[a] * dp;
            }
            for (int64_t a = 0; a < n_tok; ++a)
                dS[a] = P[a] * (dS[a] - D);
            double dabs = 0.0;
            for (int e = 0; e < dv; ++e) {
                double pv = 0.0;
                for (int64_t a = 0; a < n_tok; ++a)
                    pv += P[a] * fabs(dsa_oracle_bf16_value(v[tok[a] * dv + e]));
                dabs += fabs(dsa_oracle_bf16_value(do_th[e])) * pv;
            }
            for (int64_t a = 0; a < n_tok; ++a)
                M[a] = fabs(dS[a]) + P[a] * dabs;
            for (int e = 0; e < d; ++e) {
                double acc = 0.0, mag = 0.0;
                for (int64_t a = 0; a < n_tok; ++a) {
                    double kv = dsa_oracle_bf16_value(k[tok[a] * d + e]);
                    acc += dS[a] * kv;
                    mag += M[a] * fabs(kv);
                }
                dq_th[e] = scale * acc;
                if (dq_mag)
                    dq_mag[(r * h + hh) * d + e] = scale * mag;
            }
        }
        /* key and value gradients: each element's sum runs over rows, then
         * tokens, then heads, in that order; columns are independent */
#pragma omp parallel for schedule(static)
        for (int e = 0; e < d; ++e)
            for (int64_t a = 0; a < n_tok; ++a)
                for (int hh = 0; hh < h; ++hh) {
                    double qv = dsa_oracle_bf16_value(q[(i * h + hh) * d + e]);
                    dk[tok[a] * d + e] += scale * ds[(int64_t)hh * cap + a] * qv;
                    if (dk_mag)
                        dk_mag[tok[a] * d + e] += scale * mj[(int64_t)hh * cap + a] * fabs(qv);
                }
#pragma omp parallel for schedule(static)
        for (int e = 0; e < dv; ++e)
            for (int64_t a = 0; a < n_tok; ++a)
                for (int hh = 0; hh < h; ++hh) {
                    double g = dsa_oracle_bf16_value(dout[(i * h + hh) * dv + e]);
                    dvv[tok[a] * dv + e] += pw[(int64_t)hh * cap + a] * g;
                    if (dv_mag)
                        dv_mag[tok[a] * dv + e] += pw[(int64_t)hh * cap + a] * fabs(g);
                }
    }
    free(tok);
    free(pw);
    free(ds);
    free(mj);
    return rc;
}

/* Token count |T(t)| for each listed row given its idx row (used to size
 * work when timing the oracle on a sample). */
int64_t dsa_oracle_token_count(const int32_t *idx, int64_t q_pos0, int64_t s_k, int k_pools,
                               int pool, int n_tail, const int64_t *rows, int64_t n_rows)
{
    int64_t total = 0;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t t = q_pos0 + rows[r];
        for (int j = 0; j < k_pools; ++j)
            if (idx[r * k_pools + j] >= 0)
                total += pool;
        if (n_tail > 0) {
            int64_t start = (t / pool) * pool;
            if (t - n_tail > start)
                start = t - n_tail;
            for (int64_t j = start; j < t && j < s_k; ++j)
                ++total;
        }
    }
    return total;
}
