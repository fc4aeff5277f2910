/* Runs every entry point of oracle/dsa_oracle.c on small and edge-case
 * shapes, for a build under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py).  Inputs come from a fixed linear congruential
 * generator; the driver checks return codes only (the values are pinned by
 * the other tests).  Exit status 0: every call returned what it should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double dsa_oracle_bf16_value(uint16_t bits);
double dsa_oracle_e4m3_value(uint8_t code);
uint8_t dsa_oracle_e4m3_encode(double x);
int dsa_oracle_pool_keys(const uint16_t *k_idx, const float *gate, int64_t s_k, int d_idx,
                         int pool, double *kbar);
int dsa_oracle_pool_keys_fp8(const uint8_t *k8, const float *gate, int64_t s_k, int d_idx,
                             int pool, uint8_t *codes, int32_t *exps);
int dsa_oracle_index_scores(const uint16_t *q_idx, const uint16_t *k_idx, const float *gate,
                            const float *w, int64_t w_stride, int64_t s_q, int64_t s_k,
                            int64_t q_pos0, int h_idx, int d_idx, int pool, const int64_t *rows,
                            int64_t n_rows, float *out);
int dsa_oracle_index_topk(const uint16_t *q_idx, const uint16_t *k_idx, const float *gate,
                          const float *w, int64_t w_stride, int64_t s_q, int64_t s_k,
                          int64_t q_pos0, int h_idx, int d_idx, int pool, int k_pools,
                          const int64_t *rows, int64_t n_rows, int32_t *idx_out,
                          float *sel_scores_out);
int dsa_oracle_index_scores_fp8(const uint8_t *q8, const uint8_t *k8, const float *gate,
                                float q_scale, float k_scale, const float *w, int64_t w_stride,
                                int64_t s_q, int64_t s_k, int64_t q_pos0, int h_idx, int d_idx,
                                int pool, const int64_t *rows, int64_t n_rows, float *out);
int dsa_oracle_index_topk_fp8(const uint8_t *q8, const uint8_t *k8, const float *gate,
                              float q_scale, float k_scale, const float *w, int64_t w_stride,
                              int64_t s_q, int64_t s_k, int64_t q_pos0, int h_idx, int d_idx,
                              int pool, int k_pools, const int64_t *rows, int64_t n_rows,
                              int32_t *idx_out, float *sel_scores_out);
int dsa_oracle_sparse_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const int32_t *idx, int64_t s_q, int64_t s_k, int64_t q_pos0, int h,
                           int d, int dv, int k_pools, int pool, int n_tail, double scale,
                           const int64_t *rows, int64_t n_rows, double *o, double *lse);
int dsa_oracle_sparse_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const int32_t *idx, const uint16_t *dout, int64_t s_q,
                               int64_t s_k, int64_t q_pos0, int h, int d, int dv, int k_pools,
                               int pool, int n_tail, double scale, const int64_t *rows,
                               int64_t n_rows, double *dq, double *dk, double *dvv,
                               double *dq_mag, double *dk_mag, double *dv_mag);
int64_t dsa_oracle_token_count(const int32_t *idx, int64_t q_pos0, int64_t s_k, int k_pools,
                               int pool, int n_tail, const int64_t *rows, int64_t n_rows);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void)
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_state >> 33);
}
/* bf16 bit pattern of a value in about (-2, 2) */
static uint16_t rand_bf16(void) { return (uint16_t)(0x3F00u + (next32() & 0xFFu)) ^ (uint16_t)((next32() & 1u) << 15); }
static uint8_t rand_e4m3(void) { return (uint8_t)((next32() % 0x7Eu) | ((next32() & 1u) << 7)); }
static float rand_unit(void) { return (float)(next32() & 0xFFFFu) / 65536.0f; }

static int failures = 0;
#define EXPECT(call, want)                                                                  \
    do {                                                                                    \
        long long got_ = (long long)(call);                                                 \
        if (got_ != (long long)(want)) {                                                    \
            fprintf(stderr, "%s:%d: %s returned %lld, expected %lld\n", __FILE__, __LINE__, \
                    #call, got_, (long long)(want));                                        \
            ++failures;                                                                     \
        }                                                                                   \
    } while (0)

static void *xcalloc(size_t n, size_t sz) { void *p = calloc(n ? n : 1, sz ? sz : 1); if (!p) abort(); return p; }

static void run_shape(int64_t s_q, int64_t s_k, int64_t q_pos0, int h_idx, int d_idx, int k_pools,
                      int h, int d, int dv, int n_tail, int gated, int per_query_w)
{
    const int pool = 4;
    const int64_t n_pools = s_k / pool;
    uint16_t *qi = xcalloc((size_t)(s_q * h_idx * d_idx), 2), *ki = xcalloc((size_t)(s_k * d_idx), 2);
    uint8_t *q8 = xcalloc((size_t)(s_q * h_idx * d_idx), 1), *k8 = xcalloc((size_t)(s_k * d_idx), 1);
    float *w = xcalloc((size_t)(s_q * h_idx), 4), *gate = xcalloc((size_t)s_k, 4);
    uint16_t *q = xcalloc((size_t)(s_q * h * d), 2), *k = xcalloc((size_t)(s_k * d), 2);
    uint16_t *v = xcalloc((size_t)(s_k * dv), 2), *dout = xcalloc((size_t)(s_q * h * dv), 2);
    for (int64_t i = 0; i < s_q * h_idx * d_idx; ++i) { qi[i] = rand_bf16(); q8[i] = rand_e4m3(); }
    for (int64_t i = 0; i < s_k * d_idx; ++i) { ki[i] = rand_bf16(); k8[i] = rand_e4m3(); }
    for (int64_t i = 0; i < s_q * h_idx; ++i) w[i] = rand_unit();
    for (int64_t i = 0; i < s_k; ++i) gate[i] = 0.25f * rand_unit();
    for (int64_t i = 0; i < s_q * h * d; ++i) q[i] = rand_bf16();
    for (int64_t i = 0; i < s_k * d; ++i) k[i] = rand_bf16();
    for (int64_t i = 0; i < s_k * dv; ++i) v[i] = rand_bf16();
    for (int64_t i = 0; i < s_q * h * dv; ++i) dout[i] = rand_bf16();
    const float *g = gated ? gate : NULL;
    const int64_t ws = per_query_w ? h_idx : 0;
    int64_t *rows = xcalloc((size_t)s_q, 8);
    for (int64_t r = 0; r < s_q; ++r) rows[r] = s_q - 1 - r;  /* every row, in reverse */

    double *kbar = xcalloc((size_t)(n_pools * d_idx), 8);
    uint8_t *codes = xcalloc((size_t)(n_pools * d_idx), 1);
    int32_t *exps = xcalloc((size_t)n_pools, 4);
    EXPECT(dsa_oracle_pool_keys(ki, g, s_k, d_idx, pool, kbar), 0);
    EXPECT(dsa_oracle_pool_keys_fp8(k8, g, s_k, d_idx, pool, codes, exps), 0);

    float *sc = xcalloc((size_t)(s_q * (n_pools ? n_pools : 1)), 4);
    int32_t *idx = xcalloc((size_t)(s_q * k_pools), 4);
    float *sel = xcalloc((size_t)(s_q * k_pools), 4);
    EXPECT(dsa_oracle_index_scores(qi, ki, g, w, ws, s_q, s_k, q_pos0, h_idx, d_idx, pool, rows, s_q, sc), 0);
    EXPECT(dsa_oracle_index_scores_fp8(q8, k8, g, 0.5f, -2.0f, w, ws, s_q, s_k, q_pos0, h_idx, d_idx, pool, rows, s_q, sc), 0);
    EXPECT(dsa_oracle_index_topk_fp8(q8, k8, g, 1.0f, 1.0f, w, ws, s_q, s_k, q_pos0, h_idx, d_idx, pool, k_pools, rows, s_q, idx, sel), 0);
    EXPECT(dsa_oracle_index_topk(qi, ki, g, w, ws, s_q, s_k, q_pos0, h_idx, d_idx, pool, k_pools, rows, s_q, idx, NULL), 0);
    EXPECT(dsa_oracle_index_topk(qi, ki, g, w, ws, s_q, s_k, q_pos0, h_idx, d_idx, pool, k_pools, rows, s_q, idx, sel), 0);

    /* attention takes one id row per listed row, in the listed order (as
       the selection returns them) */
    const int32_t *idx_rows = idx;
    double *o = xcalloc((size_t)(s_q * h * dv), 8), *lse = xcalloc((size_t)(s_q * h), 8);
    EXPECT(dsa_oracle_sparse_attn(q, k, v, idx_rows, s_q, s_k, q_pos0, h, d, dv, k_pools, pool, n_tail,
                                  1.0 / sqrt((double)d), rows, s_q, o, lse), 0);
    double *dq = xcalloc((size_t)(s_q * h * d), 8), *dk = xcalloc((size_t)(s_k * d), 8);
    double *dvv = xcalloc((size_t)(s_k * dv), 8), *dqm = xcalloc((size_t)(s_q * h * d), 8);
    double *dkm = xcalloc((size_t)(s_k * d), 8), *dvm = xcalloc((size_t)(s_k * dv), 8);
    EXPECT(dsa_oracle_sparse_attn_bwd(q, k, v, idx_rows, dout, s_q, s_k, q_pos0, h, d, dv, k_pools, pool,
                                      n_tail, 0.125, rows, s_q, dq, dk, dvv, dqm, dkm, dvm), 0);
    EXPECT(dsa_oracle_sparse_attn_bwd(q, k, v, idx_rows, dout, s_q, s_k, q_pos0, h, d, dv, k_pools, pool,
                                      n_tail, 0.125, rows, s_q, dq, dk, dvv, NULL, NULL, NULL), 0);
    if (dsa_oracle_token_count(idx_rows, q_pos0, s_k, k_pools, pool, n_tail, rows, s_q) < 0) {
        fprintf(stderr, "token count failed\n");
        ++failures;
    }
    if (s_q > 0 && n_pools > 3) {
        /* a malformed row is rejected, not read out of bounds: row 0 of the
           list (query s_q - 1) with an id past the last pool */
        int32_t *bad = xcalloc((size_t)k_pools, 4);
        memcpy(bad, idx_rows, sizeof(int32_t) * (size_t)k_pools);
        bad[0] = (int32_t)(n_pools + 5);
        if (dsa_oracle_sparse_attn(q, k, v, bad, s_q, s_k, q_pos0, h, d, dv, k_pools, pool, n_tail, 0.1,
                                   rows, 1, o, lse) == 0) {
            fprintf(stderr, "an out-of-range id was accepted\n");
            ++failures;
        }
        free(bad);
    }
    free(qi); free(ki); free(q8); free(k8); free(w); free(gate); free(q); free(k); free(v); free(dout);
    free(rows); free(kbar); free(codes); free(exps); free(sc); free(idx); free(sel);
    free(o); free(lse); free(dq); free(dk); free(dvv); free(dqm); free(dkm); free(dvm);
}

int main(void)
{
    /* value helpers over their whole domains */
    for (uint32_t b = 0; b < 65536; ++b) (void)dsa_oracle_bf16_value((uint16_t)b);
    for (uint32_t c = 0; c < 256; ++c) (void)dsa_oracle_e4m3_value((uint8_t)c);
    for (int i = -2000; i <= 2000; ++i) (void)dsa_oracle_e4m3_encode(i * 0.25);
    /* s_q, s_k, q_pos0, h_idx, d_idx, k, h, d, dv, n_tail, gated, per-query w */
    run_shape(37, 37, 0, 4, 64, 3, 2, 64, 64, 0, 0, 0);
    run_shape(21, 61, 40, 8, 96, 5, 3, 96, 128, 3, 1, 1);
    run_shape(9, 130, 121, 16, 128, 40, 1, 128, 96, 1, 0, 1);  /* k > n for some rows */
    run_shape(6, 3, 0, 4, 64, 2, 2, 64, 64, 2, 1, 0);          /* fewer keys than a pool */
    run_shape(1, 4, 3, 4, 64, 1, 1, 64, 64, 3, 0, 0);          /* t = 3: tail only */
    /* argument checks */
    EXPECT(dsa_oracle_pool_keys(NULL, NULL, 8, 64, 4, NULL) != 0, 1);
    EXPECT(dsa_oracle_index_topk(NULL, NULL, NULL, NULL, 0, -1, 8, 0, 4, 64, 4, 1, NULL, 0, NULL, NULL) != 0, 1);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    puts("oracle driver: ok");
    return 0;
}
