/*
 * dsa.h -- C ABI of libdsa, the MI355X (gfx950) DeepSeek Sparse Attention
 * (DSA) forward path.
 *
 * The method (SkyRL blog, "Scaling Training to 1M Token Context on
 * GLM-5.3-Flash"):
 *   section "DeepSeek Sparse Attention (DSA) Optimizations" -- a small
 *     indexer rates each query's whole causal past, 4 tokens (one pool) at
 *     a time, keeps the highest-rated pools, and attention then touches
 *     only 2048 tokens (512 pools x 4);
 *   section "Making Sparse Attention Actually Sparse" -- NoPE heads are
 *     narrower than the rotary shapes and the pooled selection can return
 *     2,051 keys; unsupported shapes must not silently fall back to dense;
 *   section "Splitting the DSA Indexer / Over Time: Chunking" -- queries are
 *     scored and selected in chunks of hundreds, which bounds the indexer's
 *     memory whatever the context length;
 *   section "Across GPUs: Sharding" -- the selected pool ids are small and
 *     are handed on as int32.
 * The page prints no score formula; the library computes the standard
 * lightning-indexer form
 *     s(t,p) = sum_h w[t,h] * max(0, q_idx[t,h,:] . kbar_p),
 *     kbar_p = mean of key rows 4p .. 4p+3,
 * for every pool p with 4p+3 < t (strictly earlier), keeps the k_pools best
 * (ties to the lower pool id) and attends, with softmax, to the 4 tokens of
 * each kept pool (plus up to n_tail tokens of t's own unfinished pool that
 * precede t).
 *
 * Conventions for every call:
 *   - Device pointers are device memory on the current HIP device, 16-byte
 *     aligned, row-major and contiguous in the shapes given.  The caller owns
 *     all memory; the library allocates none and keeps no state beyond
 *     cached device properties, optional profiling events and a per-thread
 *     error message.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; DSA_OK means the launches were enqueued.
 *   - On any error, nothing is launched, outputs are left untouched, and
 *     dsa_last_error() describes the failure.  No call ever falls back to a
 *     different algorithm: shapes outside the supported set return
 *     DSA_ERR_UNSUPPORTED.
 *   - Results are deterministic: identical inputs give identical outputs,
 *     bit for bit (no floating-point atomics).
 *   - Positions: query row i (0 <= i < s_q) sits at sequence position
 *     t = q_pos0 + i; key row j is position j; P = floor(s_k / 4) pools;
 *     query t sees n(t) = min(floor(t/4), P) pools.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1, /* null pointer, misalignment, negative size, ... */
    DSA_ERR_UNSUPPORTED = 2, /* a shape outside the supported set */
    DSA_ERR_WORKSPACE = 3,   /* workspace missing or too small */
    DSA_ERR_HIP = 4          /* a HIP runtime call failed */
} dsa_status;

typedef enum {
    DSA_BF16 = 0,    /* indexer q/k in bfloat16 */
    DSA_FP8_E4M3 = 1 /* indexer q/k as OCP FP8 E4M3 codes with fp32 scales */
} dsa_dtype;

/* Library version, major * 10000 + minor * 100 + patch. */
int dsa_version(void);

/* Message describing the last failed call on this thread ("" if none). */
const char *dsa_last_error(void);

/*
 * Bytes of device workspace dsa_index_score_topk needs.  Holds the pooled
 * key table (bf16: hi = bf16(mean) plus the residual as E4M3 codes with a
 * per-pool power-of-two scale and two per-pool error-bound factors; fp8: E4M3
 * codes plus per-pool factors), for the bf16 indexer the chunk's queries and
 * head weights packed in scoring tiles (with E4M3 copies of the queries for
 * the correction term) and two per-query error-bound factors, and the per-chunk
 * fp32 score buffer of chunk_q x round_up(P, 512) entries ("Over Time:
 * Chunking": the buffer is constant in s_q).  chunk_q = 0 picks the
 * library's default for these shapes (the value is returned through
 * *chunk_q_used when that pointer is non-NULL).
 * Pure host computation; valid without a GPU.
 */
dsa_status dsa_index_workspace_size(int64_t s_q, int64_t s_k, int h_idx, int d_idx,
                                    int k_pools, int pool_size, int64_t chunk_q, int dtype,
                                    size_t *bytes, int64_t *chunk_q_used);

/*
 * Pooling, chunked indexer scoring and top-k selection (sections "DeepSeek
 * Sparse Attention (DSA) Optimizations", "Over Time: Chunking", "Across
 * GPUs: Sharding").
 *   q_idx    [s_q, h_idx, d_idx]   bf16, or E4M3 codes when dtype = DSA_FP8_E4M3
 *   k_idx    [s_k, d_idx]          bf16, or E4M3 codes
 *   q_scale, k_scale               fp8 only: device pointers to one fp32 scale
 *                                  each (NULL = 1.0); must be NULL for bf16
 *   w        [s_q, h_idx] fp32 with row stride w_stride_q elements
 *                                  (w_stride_q = 0: one [h_idx] row for all queries)
 *   pool_size                      must be 4
 *   k_pools                        pools kept per query, 1 .. 2048
 *   chunk_q                        queries per chunk (0 = default; a multiple of 64)
 *   idx_out  [s_q, k_pools] int32  kept pool ids, ascending, padded with -1
 *                                  when n(t) < k_pools
 *   score_out [s_q, k_pools] fp32  optional (NULL): the kept pools' scores,
 *                                  -inf for padding
 *   workspace                      >= dsa_index_workspace_size(...) bytes
 * Supported: h_idx in {4, 8, 16, 32}; d_idx in {64, 96, 128}; s_q, s_k < 2^31;
 * q_pos0 < 2^40.
 * The fp32 score of a pool is a +0.0 when zero (never -0.0).
 * bf16 indexer: the score of a pool is q . hi on bf16 matrix cores plus the
 * correction q . lo on scaled E4M3 matrix cores, exactly as
 * dsa_index_scores returns it, and the kept set is exactly the top k_pools
 * of those scores.  (The chunk is first scored without the correction; a
 * per-pair error bound then decides every pool it can, and only the pools
 * near the k-th score are rescored in full.)
 */
dsa_status dsa_index_score_topk(const void *q_idx, const void *k_idx, const float *q_scale,
                                const float *k_scale, const float *w, int64_t w_stride_q,
                                int64_t s_q, int64_t s_k, int64_t q_pos0, int h_idx, int d_idx,
                                int pool_size, int k_pools, int64_t chunk_q, int dtype,
                                int32_t *idx_out, float *score_out, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * dsa_index_score_topk for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and the same results, bit for bit, with
 * no workspace argument.  The workspace lives in a scratch array of
 * DSA_NOALLOC_SCRATCH_BYTES that is part of the library's device image: each
 * GPU the library runs on holds its own copy from the time the library's
 * code is loaded on it until the process ends.  The call allocates nothing
 * (no hipMalloc, no events: profiling does not record it).
 *   chunk_q   0 = the largest multiple of 64 queries (at most the default of
 *             dsa_index_score_topk) whose workspace fits the scratch array;
 *             a given chunk_q whose workspace does not fit returns
 *             DSA_ERR_WORKSPACE
 * Every other argument is that of dsa_index_score_topk.  Shapes whose pooled
 * key table plus one 64-query chunk exceed the scratch array (beyond about
 * 412K pools, 1.65M keys, at d_idx = 128 with the bf16 indexer; 690K pools
 * with fp8) return DSA_ERR_UNSUPPORTED.  At 128K keys the chunk fits 1728
 * queries, at 1M keys 128.  All calls on one
 * GPU share its scratch array: calls that overlap in time on one GPU (other
 * streams or threads) race and give undefined results; calls ordered on one
 * stream are safe.  The scratch contents left by a call are never read by
 * the next one (every part is written before it is read).
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
dsa_status dsa_index_score_topk_noalloc(const void *q_idx, const void *k_idx,
                                        const float *q_scale, const float *k_scale,
                                        const float *w, int64_t w_stride_q, int64_t s_q,
                                        int64_t s_k, int64_t q_pos0, int h_idx, int d_idx,
                                        int pool_size, int k_pools, int64_t chunk_q, int dtype,
                                        int32_t *idx_out, float *score_out, void *stream);

/*
 * dsa_index_score_topk with gated pooling (section "DSA: Gather by Token
 * Position": per-token k-pool gate scores weight each key within its pool).
 * The pooled key is the gate-weighted sum
 *     kbar_p = sum_{r<4} k_gate[4p + r] * k_idx[4p + r]
 * instead of the mean; the caller supplies normalised gates (gates of 1/4
 * give the mean).
 *   k_gate   [s_k] fp32, device memory, 16-byte aligned; must be non-NULL
 *            when s_k >= 4 (entries past the last whole pool are not read)
 * Every other argument, the workspace size and the error behaviour are those
 * of dsa_index_score_topk.  With the fp8 indexer the gated sum of the code
 * values is formed in fp64 before the per-pool requantisation.
 */
dsa_status dsa_index_score_topk_gated(const void *q_idx, const void *k_idx, const float *k_gate,
                                      const float *q_scale, const float *k_scale, const float *w,
                                      int64_t w_stride_q, int64_t s_q, int64_t s_k,
                                      int64_t q_pos0, int h_idx, int d_idx, int pool_size,
                                      int k_pools, int64_t chunk_q, int dtype, int32_t *idx_out,
                                      float *score_out, void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * Bytes of device workspace dsa_index_scores needs for n_rows query rows:
 * the pooled key table plus, for the bf16 indexer, packed query tiles for up
 * to 4096 rows (the rows are scored 4096 at a time).  Pure host computation.
 */
dsa_status dsa_index_scores_workspace_size(int64_t s_q, int64_t s_k, int h_idx, int d_idx,
                                           int pool_size, int dtype, int64_t n_rows,
                                           size_t *bytes);

/*
 * Dense fp32 indexer scores of query rows [row0, row0 + n_rows) against
 * every pool (testing and inspection): scores_out [n_rows, P], -inf where a
 * pool is not eligible.  Same arguments and support as dsa_index_score_topk;
 * the workspace is sized by dsa_index_scores_workspace_size.
 */
dsa_status dsa_index_scores(const void *q_idx, const void *k_idx, const float *q_scale,
                            const float *k_scale, const float *w, int64_t w_stride_q,
                            int64_t s_q, int64_t s_k, int64_t q_pos0, int h_idx, int d_idx,
                            int pool_size, int dtype, int64_t row0, int64_t n_rows,
                            float *scores_out, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * dsa_index_scores with gated pooled keys, as in dsa_index_score_topk_gated
 * (k_gate [s_k] fp32, non-NULL when s_k >= 4).  Same workspace size.
 */
dsa_status dsa_index_scores_gated(const void *q_idx, const void *k_idx, const float *k_gate,
                                  const float *q_scale, const float *k_scale, const float *w,
                                  int64_t w_stride_q, int64_t s_q, int64_t s_k, int64_t q_pos0,
                                  int h_idx, int d_idx, int pool_size, int dtype, int64_t row0,
                                  int64_t n_rows, float *scores_out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Sparse attention forward over the kept pools (sections "DeepSeek Sparse
 * Attention (DSA) Optimizations" and "Making Sparse Attention Actually
 * Sparse"), with an online softmax.
 *   q    [s_q, h, d]   bf16; h query heads share one key/value head
 *   k    [s_k, d]      bf16
 *   v    [s_k, dv]     bf16 (k == v is allowed)
 *   idx  [s_q, k_pools] int32 pool ids as produced by dsa_index_score_topk;
 *                      entries < 0 or >= P are skipped
 *   n_tail             0 .. pool_size-1: also attend to the last
 *                      min(n_tail, t mod 4) tokens before t (t's own
 *                      unfinished pool); 3 gives the 2,051-key case
 *   softmax_scale      logit scale; <= 0 selects 1/sqrt(d)
 *   out  [s_q, h, dv]  bf16
 *   lse  [s_q, h]      fp32 natural-log sum-exp of the scaled logits, or NULL
 * A query with no token gets out = 0 and lse = -inf.
 * Supported: h in 1 .. 16; d, dv in {64, 96, 128}; pool_size = 4.
 */
dsa_status dsa_sparse_attn_fwd(const void *q, const void *k, const void *v, const int32_t *idx,
                               int64_t s_q, int64_t s_k, int64_t q_pos0, int h, int d, int dv,
                               int k_pools, int pool_size, int n_tail, float softmax_scale,
                               void *out, float *lse, void *stream);

/*
 * Bytes of device workspace dsa_sparse_attn_bwd needs: delta = dout . out
 * per query and head (fp32 [s_q, h], rounded up to 256 bytes), then the
 * bitmap that transposes the queries' selections, chunk_q / 32 rows of
 * ceil(s_k / 4) 32-bit words (rounded up to a multiple of 4) per chunk, for
 * every chunk when that takes at most 1 GiB, else for one chunk (rounded up
 * to 256 bytes), then two arrays of one 32-bit word per pool slot
 * (ceil(s_k / 4) rounded up to a multiple of 4 words each, rounded up to 256
 * bytes): the slots' entry counts and their order, which groups them in fours
 * for the key-major pass.
 * chunk_q = 0
 * picks the default,
 * max(1024, min(1536, 3 P / 32), P / 32) with P = ceil(s_k / 4), rounded up to a
 * multiple of 64, at most 16384
 * and at most s_q rounded up to 64, returned through *chunk_q_used when that
 * pointer is non-NULL; otherwise a multiple of 64 up to 65536 whose bitmap
 * stays within 2 GiB.  Pure host computation.
 */
dsa_status dsa_sparse_attn_bwd_workspace_size(int64_t s_q, int64_t s_k, int h, int64_t chunk_q,
                                              size_t *bytes, int64_t *chunk_q_used);

/*
 * Backward of dsa_sparse_attn_fwd (the pages' setting is training: section
 * "Activation Recompute" reruns the forward inside the backward pass, so the
 * softmax weights are recomputed from the forward's lse rather than stored).
 * Gradients of L = sum dout . out, per query row, head h and attended token j:
 *     D_h  = dout_h . out_h,   P_j = exp(scale q_h . k_j - lse_h),
 *     dS_j = P_j (dout_h . v_j - D_h),
 *     dq_h = scale sum_j dS_j k_j,  dk_j += scale dS_j q_h,  dv_j += P_j dout_h.
 *   q, k, v, idx, s_q .. softmax_scale   as passed to dsa_sparse_attn_fwd;
 *                      every valid id of an idx row must be distinct (as
 *                      dsa_index_score_topk produces them), else the
 *                      gradients are unspecified
 *   out  [s_q, h, dv]  bf16, the forward's output
 *   dout [s_q, h, dv]  bf16, the gradient of L with respect to out
 *   lse  [s_q, h]      fp32, the forward's lse (required)
 *   chunk_q            queries per transposition chunk (0 = default)
 *   dq      [s_q, h, d]  fp32 output
 *   dk      [s_k, d]     fp32 output (every row written; 0 where no query
 *                        attends)
 *   dv_grad [s_k, dv]    fp32 output
 *   workspace          >= dsa_sparse_attn_bwd_workspace_size(...) bytes
 * The key and value gradients are sums over the queries that attend each
 * token; they are formed one chunk of queries at a time, each token's sum in
 * increasing query order, so the results are deterministic.  The products
 * that feed the matrix cores take P and dS rounded to bf16; everything else
 * is fp32.  Supported shapes are those of dsa_sparse_attn_fwd.
 */
dsa_status dsa_sparse_attn_bwd(const void *q, const void *k, const void *v, const int32_t *idx,
                               const void *out, const void *dout, const float *lse, int64_t s_q,
                               int64_t s_k, int64_t q_pos0, int h, int d, int dv, int k_pools,
                               int pool_size, int n_tail, float softmax_scale, int64_t chunk_q,
                               float *dq, float *dk, float *dv_grad, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Per-kernel GPU timing.  While enabled, every kernel launch is bracketed
 * by HIP events on its own stream; dsa_profile_read synchronises on those
 * events and reports, per kernel kind, the number of launches and the summed
 * duration in milliseconds, then clears the record.  Kinds: "pool_keys",
 * "pack_queries", "index_score" (the bf16 scorer of bounded chunks, without
 * the correction term, and the fp8 scorer), "index_score_full" (the bf16
 * scorer with the correction term: chunks of short rows and
 * dsa_index_scores), "topk_select", "sparse_attn", "attn_bwd_dq",
 * "attn_bwd_select", "attn_bwd_dkv".
 */
typedef struct {
    char name[32];
    int64_t launches;
    double total_ms;
} dsa_kernel_stat;

dsa_status dsa_profile_enable(int on);
dsa_status dsa_profile_read(dsa_kernel_stat *stats, int max_stats, int *n_stats);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
