// Internal launchers of the libdsa kernels (host side).  Shapes are checked
// by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Pooled indexer keys, split as hi = bf16(mean) [P][d] and lo = mean - hi
// as E4M3 codes [P][d] with one E8M0 power-of-two scale byte per pool.
hipError_t launch_pool_keys_bf16(const uint16_t* k_idx, int64_t n_pools, int d_idx,
                                 uint16_t* hi, uint8_t* lo, uint8_t* lo_scale,
                                 hipStream_t stream);

// n_vec query vectors (bf16 [n_vec][d]) as E4M3 codes with one E8M0
// power-of-two scale byte each.
hipError_t launch_quantize_queries(const uint16_t* q_rows, int64_t n_vec, int d_idx,
                                   uint8_t* q8, uint8_t* q_scale, hipStream_t stream);

// Pooled fp8 keys: per pool, E4M3 codes of mean/2^e and the factor 2^e.
hipError_t launch_pool_keys_fp8(const uint8_t* k8, int64_t n_pools, int d_idx, uint8_t* kbar8,
                                float* pool_scale, hipStream_t stream);

struct ScoreArgs {
    const void* q_idx;        // [s_q, h_idx, d_idx] bf16 or E4M3
    const void* kbar;         // bf16: hi [P][d]; fp8: codes [P][d]
    const uint8_t* klo;       // bf16 only: lo codes [P][d]
    const uint8_t* klo_scale; // bf16 only: [P] E8M0
    const uint8_t* q8;        // bf16 only: the chunk's queries as E4M3 [rows][h][d]
    const uint8_t* q8_scale;  // bf16 only: [rows][h] E8M0
    const float* pool_scale;  // fp8 only: [P] factors 2^e
    const float* q_scale;     // fp8 only: device scalar or null
    const float* k_scale;     // fp8 only: device scalar or null
    const float* w;
    int64_t w_stride;
    int64_t s_q;
    int64_t row0;             // first query row of the chunk
    int rows;                 // rows in the chunk
    int64_t q_pos0;
    int64_t n_pools;
    int64_t n_chunk;          // pools eligible for the chunk's last query
    int h_idx, d_idx;
    int fp8;
    float* buf;               // [rows, ld] fp32
    int64_t ld;
};
hipError_t launch_index_score(const ScoreArgs& a, hipStream_t stream);

hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t stream);

struct SelectArgs {
    const float* buf;         // [rows, ld] scores of the chunk
    int64_t ld;
    int64_t row0;
    int rows;
    int64_t q_pos0;
    int64_t n_pools;
    int k_pools;
    int32_t* idx_out;         // [s_q, k_pools]
    float* score_out;         // optional
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

}  // namespace dsa
