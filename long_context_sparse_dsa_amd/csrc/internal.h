// Internal launchers of the libdsa kernels (host side).  Shapes are checked
// by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Pooled indexer keys kbar (the mean of each pool's 4 rows, or with
// per-token gates [4 * n_pools] fp32 their gate-weighted sum), split as
// hi = bf16(kbar) [P][d] and lo = kbar - hi as E4M3 codes [P][d] with one
// E8M0 power-of-two scale byte per pool.  mu (optional) [P][2] fp32: each
// pool's two factors of the bound on the score error of leaving lo out.
hipError_t launch_pool_keys_bf16(const uint16_t* k_idx, const float* gate, int64_t n_pools,
                                 int d_idx, uint16_t* hi, uint8_t* lo, uint8_t* lo_scale,
                                 float* mu, hipStream_t stream);

// Packed query tiles of the bf16 indexer.  A tile holds 32 (query, head)
// rows r = qi * h_idx + h of 32 / h_idx consecutive chunk queries, laid out
// exactly as the scoring kernel keeps it in LDS:
//   [0, OF8)        bf16 q rows (row stride LB bytes)
//   [OF8, QB)       E4M3 codes of q / 2^e_r (row stride L8 bytes)
//   [QB, QB + 128)  w of each row, fp32
//   [QB + 128, +32) E8M0 byte e_r + 127 of each row
//   [QB + 160, +64) the two error-bound factors of each of the tile's queries, fp32
// Rows are stored in 16-byte pieces.  With d = 128 the piece order within a
// row is XOR-swizzled by the row index so that the MFMA operand reads of 16
// rows at a time hit distinct LDS banks; other widths pad each row by 16
// bytes instead.  Consecutive tiles are TB bytes apart.
struct QueryTileGeom {
    bool swz;
    int lb, l8, of8, qb, tb;
};
inline constexpr QueryTileGeom query_tile_geom(int d) {
    const bool swz = d == 128;
    const int lb = swz ? 2 * d : 2 * d + 16;
    const int l8 = swz ? d : d + 16;
    const int of8 = 32 * lb;
    const int qb = of8 + 32 * l8;
    return QueryTileGeom{swz, lb, l8, of8, qb, (qb + 224 + 127) / 128 * 128};
}
// Byte offset of 16-byte piece c of the bf16 row r / of the E4M3 row r.
inline constexpr int tile_bf16_piece(const QueryTileGeom& g, int r, int c) {
    return r * g.lb + 16 * (g.swz ? (c ^ (r & 15)) : c);
}
inline constexpr int tile_fp8_piece(const QueryTileGeom& g, int r, int c) {
    return g.of8 + r * g.l8 + 16 * (g.swz ? (c ^ ((r & 7) ^ ((r >> 3) & 1))) : c);
}
// Tiles the scoring kernel may read for a chunk of `rows` queries: the
// chunk's own plus three beyond its end (prefetched, never used).
inline constexpr int64_t query_tiles(int64_t rows, int h_idx) {
    return (rows + 32 / h_idx - 1) / (32 / h_idx) + 3;
}

// Rows [row0, row0 + rows) of q_idx and w packed into query tiles; qbound
// (optional) [rows][2] fp32: each query's two factors of the same bound.
hipError_t launch_pack_queries(const uint16_t* q_idx, const float* w, int64_t w_stride,
                               int64_t row0, int rows, int h_idx, int d_idx, uint8_t* tiles,
                               float* qbound, hipStream_t stream);

// Pooled fp8 keys: per pool, E4M3 codes of kbar/2^e and the factor 2^e
// (kbar the mean of the code values, or with gates their gate-weighted sum).
hipError_t launch_pool_keys_fp8(const uint8_t* k8, const float* gate, int64_t n_pools, int d_idx,
                                uint8_t* kbar8, float* pool_scale, hipStream_t stream);

struct ScoreArgs {
    const void* q_idx;        // fp8: [s_q, h_idx, d_idx] E4M3
    const uint8_t* tiles;     // bf16: the chunk's packed query tiles
    const void* kbar;         // bf16: hi [P][d]; fp8: codes [P][d]
    const uint8_t* klo;       // bf16 only: lo codes [P][d]
    const uint8_t* klo_scale; // bf16 only: [P] E8M0
    const float* pool_scale;  // fp8 only: [P] factors 2^e
    const float* q_scale;     // fp8 only: device scalar or null
    const float* k_scale;     // fp8 only: device scalar or null
    const float* w;           // fp8 only (bf16 weights travel in the tiles)
    int64_t w_stride;
    int64_t s_q;
    int64_t row0;             // first query row of the chunk
    int rows;                 // rows in the chunk
    int64_t q_pos0;
    int64_t n_pools;
    int64_t n_chunk;          // pools eligible for the chunk's last query
    int h_idx, d_idx;
    int fp8;
    // exact = 0: buf is a chunk buffer with at least round_up(rows, 8) rows
    // and ld >= round_up(n_chunk, 512); the kernel may write any entry of it
    // (ineligible pools get -inf); with the bf16 indexer and bound factors
    // the scores leave the correction q . lo out (the selection rescores the
    // pools near its threshold).  exact = 1: only the eligible entries of rows
    // [0, rows) are written (a caller's dense [rows, P] layout), with full
    // scores.
    int exact;
    // bf16, exact = 0: bound factors; the buffer receives upper bounds
    // u = fma(A1, m1, fma(A2, m2, score without the correction)) with
    // (A1, A2) = qbound[i] and (m1, m2) = mu[p], or the full scores when
    // qbound is null
    const float* qbound;      // [rows][2]
    const float* mu;          // [n_pools][2]
    float* buf;               // [rows, ld] fp32
    int64_t ld;
};
hipError_t launch_index_score(const ScoreArgs& a, hipStream_t stream);

hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t stream);

struct SelectArgs {
    float* buf;               // [rows, ld] scores of the chunk (rows may be rewritten)
    int64_t ld;
    int64_t row0;
    int rows;
    int64_t q_pos0;
    int64_t n_pools;
    int k_pools;
    int32_t* idx_out;         // [s_q, k_pools]
    float* score_out;         // optional
    // Bounded rows (bf16 indexer): the buffer holds u = s~ + delta with
    // delta = A1 m1 + A2 m2, (A1, A2) = qbound[i], (m1, m2) = mu[p], and s~
    // the score without the correction term, so the full score lies in
    // [u - 2 delta, u]; the selection recomputes it for the pools it cannot
    // decide from the bounds.  qbound == nullptr: the buffer holds the final
    // scores.
    const float* qbound;      // [rows][2] per chunk query
    const float* mu;          // [n_pools][2]
    const uint8_t* tiles;     // the chunk's packed query tiles
    const uint16_t* khi;      // [P][d_idx] bf16
    const uint8_t* klo;       // [P][d_idx] E4M3
    const uint8_t* klo_scale; // [P] E8M0
    int h_idx, d_idx;
};
hipError_t launch_topk_select(const SelectArgs& a, hipStream_t stream);

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* idx;
    int64_t s_q, s_k, q_pos0;
    int h, d, dv, k_pools, n_tail;
    float scale;
    uint16_t* out;
    float* lse;
};
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream);

struct AttnBwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* out;      // forward output [s_q, h, dv]
    const uint16_t* dout;     // its gradient [s_q, h, dv]
    const int32_t* idx;
    const float* lse;         // forward log-sum-exp [s_q, h]
    int64_t s_q, s_k, q_pos0;
    int h, d, dv, k_pools, n_tail;
    float scale;
    float* dq;                // [s_q, h, d]
    float* dk;                // [s_k, d]
    float* dv_grad;           // [s_k, dv]
    float* delta;             // workspace: dout . out per query and head [s_q, h]
    uint32_t* bits;           // workspace: chunk bitmap [chunk / 32][stride] words
    int64_t stride;           // pool slots per bitmap word row: ceil(s_k / 4) rounded up to 4
    uint32_t* slot_counts;    // workspace: entries per pool slot [stride]
    int32_t* slot_perm;       // workspace: pool slots, most entries first [stride]
};
// dq and delta (query-major pass).
hipError_t launch_attn_bwd_dq(const AttnBwdArgs& a, hipStream_t stream);
// ORs the selections of query rows [row0, row0 + rows) into a cleared bitmap.
hipError_t launch_attn_bwd_bits(const AttnBwdArgs& a, int64_t row0, int rows, hipStream_t stream);
// The pool groups of the key-major pass: the pool slots ordered by their
// entries in the current bitmap (rows query rows), most first, in fours.
hipError_t launch_attn_bwd_order(const AttnBwdArgs& a, int rows, hipStream_t stream);
// dk, dv of the chunk's queries: stored (accumulate = 0) or added.
hipError_t launch_attn_bwd_dkv(const AttnBwdArgs& a, int64_t row0, int rows, int accumulate,
                               hipStream_t stream);

}  // namespace dsa
