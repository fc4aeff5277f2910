// Pooling of the indexer keys and chunked lightning-indexer scoring.
//
// SkyRL blog "Scaling Training to 1M Token Context on GLM-5.3-Flash",
// section "DeepSeek Sparse Attention (DSA) Optimizations": each query gets
// a score for each 4-token pool before it; section "Over Time:
// Chunking": scores are fp32 and are produced a chunk of queries at a time
// into a buffer whose size does not grow with the sequence.
//
// Score (no formula is printed on the page; the standard lightning-indexer
// form): s(t,p) = sum_h w[t,h] * relu(q_idx[t,h,:] . kbar_p), kbar_p the mean
// of key rows 4p..4p+3, for pools with 4p+3 < t.
//
// GEMM view of one chunk: rows = (query, head) pairs, columns = pools,
// contraction = d_idx.  Each workgroup keeps a block of pooled keys resident
// in registers as the MFMA B operand and streams the chunk's queries through
// LDS as the A operand; the head-weighted ReLU reduction runs on the MFMA
// accumulators before anything is stored, so only [query, pool] fp32 scores
// reach memory.
//
// bf16 accuracy: a pooled key rounded once to bf16 perturbs scores by ~1e-3
// relative, enough to move pools across the top-k boundary.  The pooled key
// is therefore split as hi + lo, hi = bf16(mean) and lo = mean - hi (exact in
// fp32, |lo| <= 2^-9 |mean|).  q . hi runs on bf16 MFMAs (exact products);
// the small correction q . lo only needs a few bits, so it runs on scaled fp8
// MFMAs: lo is stored as E4M3 codes with a per-pool power-of-two scale and
// the chunk's queries as E4M3 codes with a per-(query, head) power-of-two
// scale, both handed to the MFMA as its E8M0 block scales, so the correction
// lands in the same accumulators.  The fp8 rounding leaves the correction
// ~5% off, i.e. ~3e-5 of a typical score, far inside the selection's 1e-3
// boundary band.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace dsa {

// ---------------------------------------------------------------- pooling

// ---------------------------------------------------------------- fp8 pooling
//
// OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa
// bits, no infinities, largest finite 448, subnormals m * 2^-9.  A pooled key
// is the mean of its 4 rows' code values (exact in fp32), re-quantised with a
// power-of-two scale 2^e, e the smallest integer with max|mean| <= 448 * 2^e:
// scaling by 2^-e is exact, so the code is the round-to-nearest-even of an
// exact value and does not depend on the precision used.

__device__ __forceinline__ float e4m3_value(uint32_t code) {
    const uint32_t e = (code >> 3) & 15u, m = code & 7u;
    const float mag = e == 0 ? (float)m * 0x1p-9f : ldexpf((float)(8u + m), (int)e - 10);
    return (code & 0x80u) ? -mag : mag;
}

// |x| <= 448; ties to the even mantissa (rintf rounds half to even).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fabsf(x);
    uint32_t code;
    if (a < 0x1p-6f) {
        code = (uint32_t)rintf(a * 512.0f);  // 8 rounds up into the smallest normal, 0x08
    } else {
        const int E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
        uint32_t mm = (uint32_t)rintf(ldexpf(a, 3 - E)) - 8u;  // 0..8
        uint32_t ee = (uint32_t)(E + 7);
        if (mm == 8u) {
            mm = 0u;
            ++ee;
        }
        code = (ee << 3) | mm;
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return code | sign;
}

// The same rounding from an fp64 value: |x| <= 448, ties to even.
__device__ __forceinline__ uint32_t e4m3_code_f64(double x) {
    const uint32_t sign = x < 0.0 ? 0x80u : 0u;
    const double a = fabs(x);
    uint32_t code;
    if (a < 0x1p-6) {
        code = (uint32_t)rint(a * 512.0);
    } else {
        int E;
        (void)frexp(a, &E);  // a = f * 2^E, f in [0.5, 1)
        E -= 1;              // a in [2^E, 2^(E+1))
        uint32_t mm = (uint32_t)rint(ldexp(a, 3 - E)) - 8u;
        uint32_t ee = (uint32_t)(E + 7);
        if (mm == 8u) {
            mm = 0u;
            ++ee;
        }
        code = (ee << 3) | mm;
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return code | sign;
}

// Gated fp8 pooling: m = sum_r g_r * value(code_r), summed in fp64 in row
// order.  Each product of an fp32 gate and an E4M3 value is exact in fp64,
// so m, the power-of-two scale and the round-to-nearest-even code below do
// not depend on the order of evaluation beyond that of the sum.
template <int DI>
__global__ __launch_bounds__(256) void pool_keys_fp8_gated_kernel(const uint8_t* __restrict__ k8,
                                                                  const float* __restrict__ gate,
                                                                  int64_t n_pools,
                                                                  uint8_t* __restrict__ kbar8,
                                                                  float* __restrict__ pool_scale) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= n_pools) return;
    const f32x4 g = *reinterpret_cast<const f32x4*>(gate + 4 * p);
    double m[DI];
    double amax = 0.0;
#pragma unroll
    for (int c = 0; c < DI / 16; ++c) {
        u32x4 r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = ldg16(k8 + (p * 4 + j) * DI + 16 * c);
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const int word = b >> 2, sh = (b & 3) * 8;
            double s = 0.0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s = __dadd_rn(s, __dmul_rn((double)g[j], (double)e4m3_value((r[j][word] >> sh) & 0xFFu)));
            m[16 * c + b] = s;
            amax = fmax(amax, fabs(s));
        }
    }
    int e = 0;
    if (amax > 0.0) {
        int E;
        (void)frexp(amax / 448.0, &E);
        e = E - 3;
        while (amax > ldexp(448.0, e)) ++e;
    }
#pragma unroll
    for (int c = 0; c < DI / 16; ++c) {
        u32x4 o = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < 16; ++b) o[b >> 2] |= e4m3_code_f64(ldexp(m[16 * c + b], -e)) << ((b & 3) * 8);
        *reinterpret_cast<u32x4*>(kbar8 + p * DI + 16 * c) = o;
    }
    pool_scale[p] = ldexpf(1.0f, e);
}

template <int DI>
__global__ __launch_bounds__(256) void pool_keys_fp8_kernel(const uint8_t* __restrict__ k8,
                                                            int64_t n_pools,
                                                            uint8_t* __restrict__ kbar8,
                                                            float* __restrict__ pool_scale) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= n_pools) return;
    float m[DI];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < DI / 16; ++c) {
        u32x4 r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = ldg16(k8 + (p * 4 + j) * DI + 16 * c);
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const int word = b >> 2, sh = (b & 3) * 8;
            float s = e4m3_value((r[0][word] >> sh) & 0xFFu);
            s += e4m3_value((r[1][word] >> sh) & 0xFFu);
            s += e4m3_value((r[2][word] >> sh) & 0xFFu);
            s += e4m3_value((r[3][word] >> sh) & 0xFFu);
            m[16 * c + b] = s * 0.25f;
            amax = fmaxf(amax, fabsf(m[16 * c + b]));
        }
    }
    int e = 0;
    if (amax > 0.0f) {
        e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 10;
        while (amax > ldexpf(448.0f, e)) ++e;
    }
#pragma unroll
    for (int c = 0; c < DI / 16; ++c) {
        u32x4 o = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < 16; ++b) o[b >> 2] |= e4m3_code(ldexpf(m[16 * c + b], -e)) << ((b & 3) * 8);
        *reinterpret_cast<u32x4*>(kbar8 + p * DI + 16 * c) = o;
    }
    pool_scale[p] = ldexpf(1.0f, e);
}

hipError_t launch_pool_keys_fp8(const uint8_t* k8, const float* gate, int64_t n_pools, int d_idx,
                                uint8_t* kbar8, float* pool_scale, hipStream_t stream) {
    if (n_pools <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n_pools + 255) / 256));
    if (gate) {
        switch (d_idx) {
            case 64: pool_keys_fp8_gated_kernel<64><<<grid, 256, 0, stream>>>(k8, gate, n_pools, kbar8, pool_scale); break;
            case 96: pool_keys_fp8_gated_kernel<96><<<grid, 256, 0, stream>>>(k8, gate, n_pools, kbar8, pool_scale); break;
            case 128: pool_keys_fp8_gated_kernel<128><<<grid, 256, 0, stream>>>(k8, gate, n_pools, kbar8, pool_scale); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (d_idx) {
        case 64: pool_keys_fp8_kernel<64><<<grid, 256, 0, stream>>>(k8, n_pools, kbar8, pool_scale); break;
        case 96: pool_keys_fp8_kernel<96><<<grid, 256, 0, stream>>>(k8, n_pools, kbar8, pool_scale); break;
        case 128: pool_keys_fp8_kernel<128><<<grid, 256, 0, stream>>>(k8, n_pools, kbar8, pool_scale); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- bf16 pooling

// Smallest e with amax <= 448 * 2^e (0 for amax == 0); amax finite.
__device__ __forceinline__ int pow2_scale_exp(float amax) {
    if (!(amax > 0.0f)) return 0;
    int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 10;
    while (amax > ldexpf(448.0f, e)) ++e;
    return e;
}

// One thread per pool: hi = bf16(kbar) [P][DI], lo = E4M3((kbar - hi) / 2^e)
// [P][DI] with one E8M0 byte (e + 127) per pool.  kbar is the mean of the
// pool's 4 rows, or with GATED their gate-weighted sum (fp32).
//
// mu (optional) [P][2] fp32 holds the pool's two factors of the bound on how
// far a score taken with hi alone can be from the score with the E4M3
// correction:
//   m1_p = (1 + 2^-12) ||L8_p||,  m2_p = 2^-10 ||L8_p|| + 2^-14 ||hi_p||
// (both 0 only for a zero pool), L8_p the decoded correction vector.  With
// the query's factors A1 and A2 (pack_queries_kernel),
//   |score(hi) - score(hi + lo)| <= A1 m1_p + A2 m2_p.
// Per head the correction is c_h = Q8_h . L8_p and the ReLU is 1-Lipschitz,
// so the scores differ by at most sum_h |w_h| |c_h| plus rounding.  That sum
// is (sum_h s_h |w_h| Q8_h) . L8_p for the signs s_h of c_h, at most
// ||L8_p|| max over sign vectors of ||sum_h s_h |w_h| Q8_h||, which A1 bounds
// through the Gram matrix of the query's rows.  A2 = (1 + 2^-8) sum_h |w_h|
// max(||q_h||, ||Q8_h||) times m2_p covers fp32 rounding: of the correction
// MFMAs (the 2^-10 term), of the accumulation and the epilogue (the 2^-14
// term, which also covers the chunk path's different order of summing the
// heads), and of s -/+ the bound themselves.  A zero pool scores +0 either way.
template <int DI, bool GATED>
__global__ __launch_bounds__(256) void pool_keys_bf16_kernel(const uint16_t* __restrict__ k,
                                                             const float* __restrict__ gate,
                                                             int64_t n_pools,
                                                             uint16_t* __restrict__ hi_out,
                                                             uint8_t* __restrict__ lo_out,
                                                             uint8_t* __restrict__ lo_scale,
                                                             float* __restrict__ mu) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= n_pools) return;
    f32x4 gw = {0.25f, 0.25f, 0.25f, 0.25f};
    if constexpr (GATED) gw = *reinterpret_cast<const f32x4*>(gate + 4 * p);
    float lo[DI];
    float amax = 0.0f, hi2 = 0.0f;
#pragma unroll
    for (int g = 0; g < DI / 8; ++g) {
        u32x4 r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = ldg16(k + (p * 4 + j) * DI + 8 * g);
        u32x4 hi;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int word = e >> 1, sh = (e & 1) * 16;
            float m;
            if constexpr (GATED) {
                m = gw[0] * bf16_to_f32((r[0][word] >> sh) & 0xFFFFu);
#pragma unroll
                for (int j = 1; j < 4; ++j) m = fmaf(gw[j], bf16_to_f32((r[j][word] >> sh) & 0xFFFFu), m);
            } else {
                float sum = bf16_to_f32((r[0][word] >> sh) & 0xFFFFu);
                sum += bf16_to_f32((r[1][word] >> sh) & 0xFFFFu);
                sum += bf16_to_f32((r[2][word] >> sh) & 0xFFFFu);
                sum += bf16_to_f32((r[3][word] >> sh) & 0xFFFFu);
                m = sum * 0.25f;
            }
            const uint32_t h = f32_to_bf16(m);
            const float hv = bf16_to_f32(h);
            lo[8 * g + e] = m - hv;
            hi2 = fmaf(hv, hv, hi2);
            amax = fmaxf(amax, fabsf(lo[8 * g + e]));
            if ((e & 1) == 0) hi[word] = h;
            else hi[word] |= h << 16;
        }
        *reinterpret_cast<u32x4*>(hi_out + p * DI + 8 * g) = hi;
    }
    const int e = pow2_scale_exp(amax);
    float lo2 = 0.0f;
#pragma unroll
    for (int c = 0; c < DI / 16; ++c) {
        u32x4 o = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const uint32_t code = e4m3_code(ldexpf(lo[16 * c + b], -e));
            const float v = e4m3_value(code);
            lo2 = fmaf(v, v, lo2);
            o[b >> 2] |= code << ((b & 3) * 8);
        }
        *reinterpret_cast<u32x4*>(lo_out + p * DI + 16 * c) = o;
    }
    lo_scale[p] = (uint8_t)(e + 127);
    if (mu) {
        const float nl = ldexpf(sqrtf(lo2), e);
        // m2 > 0 whenever hi is not zero, even with every lo code 0: the
        // chunk path sums the heads in another order than the full score,
        // so its score differs from the full one by rounding (a zero pool
        // scores +0 in every order)
        const f32x2 m = {nl * (1.0f + 0x1p-12f), fmaf(nl, 0x1p-10f, 0x1p-14f * sqrtf(hi2))};
        *reinterpret_cast<f32x2*>(mu + 2 * p) = m;
    }
}

template <bool GATED>
static hipError_t launch_pool_bf16_g(const uint16_t* k_idx, const float* gate, int64_t n_pools,
                                     int d_idx, uint16_t* hi, uint8_t* lo, uint8_t* lo_scale,
                                     float* mu, hipStream_t stream) {
    const dim3 grid((unsigned)((n_pools + 255) / 256));
    switch (d_idx) {
        case 64: pool_keys_bf16_kernel<64, GATED><<<grid, 256, 0, stream>>>(k_idx, gate, n_pools, hi, lo, lo_scale, mu); break;
        case 96: pool_keys_bf16_kernel<96, GATED><<<grid, 256, 0, stream>>>(k_idx, gate, n_pools, hi, lo, lo_scale, mu); break;
        case 128: pool_keys_bf16_kernel<128, GATED><<<grid, 256, 0, stream>>>(k_idx, gate, n_pools, hi, lo, lo_scale, mu); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_pool_keys_bf16(const uint16_t* k_idx, const float* gate, int64_t n_pools,
                                 int d_idx, uint16_t* hi, uint8_t* lo, uint8_t* lo_scale,
                                 float* mu, hipStream_t stream) {
    if (n_pools <= 0) return hipSuccess;
    return gate ? launch_pool_bf16_g<true>(k_idx, gate, n_pools, d_idx, hi, lo, lo_scale, mu, stream)
                : launch_pool_bf16_g<false>(k_idx, gate, n_pools, d_idx, hi, lo, lo_scale, mu, stream);
}

// ---------------------------------------------------------------- query tiles

// Byte offsets inside a packed query tile (layout in internal.h).  LO: the
// E4M3 copies are staged too (else only the bf16 rows and the weights).
template <int DI, bool LO = true>
struct QTile {
    static constexpr QueryTileGeom G = query_tile_geom(DI);
    static constexpr int NPQ = (LO ? G.qb : G.of8) / 16;  // 16-byte pieces of query data
    static constexpr int CPT = (NPQ + 255) / 256;   // pieces per thread when staging
    static constexpr int LDSQ = CPT * 4096;         // LDS bytes for the staged pieces
    static constexpr int LDS_W = LDSQ;              // LDS: w [32] fp32, then scales [32]
    static constexpr int LDSB = LDSQ + 1024;        // LDS bytes per tile buffer
    // piece c (16 bytes) of the bf16 / E4M3 row r
    __device__ static constexpr int bf16_piece(int r, int c) { return tile_bf16_piece(G, r, c); }
    __device__ static constexpr int fp8_piece(int r, int c) { return tile_fp8_piece(G, r, c); }
};

// One workgroup per tile, 8 threads per tile row (query, head), thread c
// holding dims 16c .. 16c + 15: the bf16 row, its E4M3 codes with the
// power-of-two scale 2^e (e the smallest with max|q| <= 448 * 2^e, the row
// maximum combined across the row's 8 threads), and the row's head weight.
// Rows past the chunk are zero with weight 0.
//
// qbound (optional) [rows][2] fp32 receives each query's two factors of the
// score error bound (see pool_keys_bf16_kernel), and the tile a copy:
//   A2 = (1 + 2^-8) sum_h |w_h| max(||q_h||, ||Q8_h||)   (heads in order)
//   A1 = min(A2, (1 + 2^-8) sqrt(S + 2^-14 A2^2)),  S = sum_{h,g} |w_h| |w_g| |G_hg|
// with Q8_h the decoded E4M3 row and G = Q8 Q8^T the Gram matrix of the
// query's rows, taken on the same scaled E4M3 MFMA as the correction term
// (exact products, fp32 accumulation).  For every sign vector s,
// ||sum_h s_h |w_h| Q8_h||^2 = sum_{h,g} s_h s_g |w_h| |w_g| G_hg <= S; the
// 2^-14 A2^2 term covers the accumulation error of G (at most 2^-16
// ||Q8_h|| ||Q8_g|| per entry) and the (1 + 2^-8) factor the rounding of S,
// of the square root and of the products.  Queries with a row scale below
// 2^-48 (products that could leave the fp32 normal range) keep A1 = A2.
template <int HI, int DI>
__global__ __launch_bounds__(256) void pack_queries_kernel(const uint16_t* __restrict__ q,
                                                           const float* __restrict__ w,
                                                           int64_t w_stride, int64_t row0,
                                                           int rows, uint8_t* __restrict__ tiles,
                                                           float* __restrict__ qbound) {
    using T = QTile<DI>;
    constexpr int QPT = 32 / HI;
    constexpr int NSF = (DI + 63) / 64;  // scaled fp8 MFMA steps of the Gram matrix
    __shared__ float rowbound[32];
    // for the Gram matrix: the rows' E4M3 codes (dims past d_idx zero),
    // scale bytes, |w| and tiny-scale flags, and one partial sum per lane
    __shared__ __attribute__((aligned(16))) uint32_t gcode[32][36];
    __shared__ int gsc[32], gtiny[32];
    __shared__ float gw[32], gpart[64];
    const int64_t tile = blockIdx.x;
    const int r = threadIdx.x >> 3, c = threadIdx.x & 7;
    const int64_t i = tile * QPT + r / HI;
    const int h = r % HI;
    const bool in = i < rows, act = c < DI / 16;
    uint8_t* dst = tiles + tile * T::G.tb;
    u32x4 raw[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if (in && act) {
        const uint16_t* src = q + ((row0 + i) * HI + h) * DI + 16 * c;
        raw[0] = ldg16(src);
        raw[1] = ldg16(src + 8);
    }
    float x[16];
    float amax = 0.0f, n2 = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        x[e] = bf16_to_f32((raw[e >> 3][(e & 7) >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
        amax = fmaxf(amax, fabsf(x[e]));
        n2 = fmaf(x[e], x[e], n2);
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
    const int e = pow2_scale_exp(amax);
    float n8 = 0.0f;
    u32x4 o = {0u, 0u, 0u, 0u};
    if (act) {
        *reinterpret_cast<u32x4*>(dst + T::bf16_piece(r, 2 * c)) = raw[0];
        *reinterpret_cast<u32x4*>(dst + T::bf16_piece(r, 2 * c + 1)) = raw[1];
        // v_cvt_pk_fp8_f32 rounds to the nearest E4M3 value, ties to even,
        // exactly as e4m3_code does for |x| <= 448 (the scaled row's range),
        // and v_cvt_f32_fp8 decodes exactly; two codes per conversion
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int wd = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * j], -e), ldexpf(x[4 * j + 1], -e),
                                                     0, false);
            wd = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * j + 2], -e), ldexpf(x[4 * j + 3], -e),
                                                 wd, true);
            o[j] = (uint32_t)wd;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v[4] = {__builtin_amdgcn_cvt_f32_fp8((int)o[j], 0),
                                __builtin_amdgcn_cvt_f32_fp8((int)o[j], 1),
                                __builtin_amdgcn_cvt_f32_fp8((int)o[j], 2),
                                __builtin_amdgcn_cvt_f32_fp8((int)o[j], 3)};
#pragma unroll
            for (int b = 0; b < 4; ++b) n8 = fmaf(v[b], v[b], n8);
        }
        *reinterpret_cast<u32x4*>(dst + T::fp8_piece(r, c)) = o;
    }
    float wr = in ? w[(row0 + i) * w_stride + h] : 0.0f;
    if (c == 0) {
        reinterpret_cast<float*>(dst + T::G.qb)[r] = wr;
        dst[T::G.qb + 128 + r] = (uint8_t)(e + 127);
    }
    if (qbound) {
        n2 += __shfl_xor(n2, 1, 8);
        n2 += __shfl_xor(n2, 2, 8);
        n2 += __shfl_xor(n2, 4, 8);
        n8 += __shfl_xor(n8, 1, 8);
        n8 += __shfl_xor(n8, 2, 8);
        n8 += __shfl_xor(n8, 4, 8);
        if (c == 0) {
            rowbound[r] = fabsf(wr) * fmaxf(sqrtf(n2), ldexpf(sqrtf(n8), e));
            gsc[r] = e + 127;
            gw[r] = fabsf(wr);
            gtiny[r] = amax > 0.0f && e < -48;
        }
        *reinterpret_cast<u32x4*>(&gcode[r][4 * c]) = o;  // zero for pieces past d_idx
        __syncthreads();
        if (threadIdx.x < 64) {
            // G on one wave: lane l holds column l % 32 of rows
            // 8*(v/4) + 4*(l/32) + v%4; only pairs of heads of one query count
            const int lane = threadIdx.x, gr = lane & 31, kb = lane >> 5;
            f32x16 acc;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
            for (int st = 0; st < NSF; ++st) {
                const u32x4 x0 = *reinterpret_cast<const u32x4*>(&gcode[gr][16 * st + 8 * kb]);
                const u32x4 x1 = *reinterpret_cast<const u32x4*>(&gcode[gr][16 * st + 8 * kb + 4]);
                const i32x8 fr = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                  (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr, fr, acc, 0, 0, 0, gsc[gr],
                                                                      0, gsc[gr]);
            }
            float part = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int hr = 8 * (v / 4) + 4 * kb + (v % 4);
                if (hr / HI == gr / HI) part = fmaf(gw[hr], fabsf(acc[v]), part);
            }
            gpart[lane] = part * gw[gr];
        }
        __syncthreads();
        if (threadIdx.x < QPT) {
            const int64_t qi = tile * QPT + threadIdx.x;
            float a = 0.0f, S = 0.0f;
            int tiny = 0;
            for (int hh = 0; hh < HI; ++hh) {
                a += rowbound[threadIdx.x * HI + hh];
                tiny |= gtiny[threadIdx.x * HI + hh];
            }
            a *= 1.0f + 0x1p-8f;
            for (int l = 0; l < 64; ++l)
                if ((l & 31) / HI == (int)threadIdx.x) S += gpart[l];
            const float a1 =
                tiny ? a : fminf(a, (1.0f + 0x1p-8f) * sqrtf(fmaf(0x1p-14f * a, a, S)));
            if (qi < rows) *reinterpret_cast<f32x2*>(qbound + 2 * qi) = f32x2{a1, a};
            reinterpret_cast<f32x2*>(dst + T::G.qb + 160)[threadIdx.x] = f32x2{a1, a};
        }
    }
}

template <int HI>
static hipError_t launch_pack_h(const uint16_t* q, const float* w, int64_t w_stride, int64_t row0,
                                int rows, int d_idx, uint8_t* tiles, float* qbound,
                                hipStream_t stream) {
    const dim3 grid((unsigned)(((int64_t)rows + 32 / HI - 1) / (32 / HI)));
    switch (d_idx) {
        case 64: pack_queries_kernel<HI, 64><<<grid, 256, 0, stream>>>(q, w, w_stride, row0, rows, tiles, qbound); break;
        case 96: pack_queries_kernel<HI, 96><<<grid, 256, 0, stream>>>(q, w, w_stride, row0, rows, tiles, qbound); break;
        case 128: pack_queries_kernel<HI, 128><<<grid, 256, 0, stream>>>(q, w, w_stride, row0, rows, tiles, qbound); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_pack_queries(const uint16_t* q_idx, const float* w, int64_t w_stride,
                               int64_t row0, int rows, int h_idx, int d_idx, uint8_t* tiles,
                               float* qbound, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    switch (h_idx) {
        case 4: return launch_pack_h<4>(q_idx, w, w_stride, row0, rows, d_idx, tiles, qbound, stream);
        case 8: return launch_pack_h<8>(q_idx, w, w_stride, row0, rows, d_idx, tiles, qbound, stream);
        case 16: return launch_pack_h<16>(q_idx, w, w_stride, row0, rows, d_idx, tiles, qbound, stream);
        case 32: return launch_pack_h<32>(q_idx, w, w_stride, row0, rows, d_idx, tiles, qbound, stream);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- fill

__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = v;
}

hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    fill_f32_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(p, n, value);
    return hipGetLastError();
}

// ---------------------------------------------------------------- scoring

struct ScoreK {
    const uint8_t* tiles;       // the chunk's packed query tiles
    const uint16_t* khi;        // [P][DI] bf16
    const uint8_t* klo;         // [P][DI] E4M3
    const uint8_t* klo_scale;   // [P] E8M0
    int64_t row0;
    int rows;
    int gq;          // queries per workgroup (multiple of 32 / HI)
    int64_t q_pos0;
    int64_t n_pools;
    float* buf;
    int64_t ld;
    const float* qbound;        // without the correction: [rows][2] per-query bound factors
    const float* mu;            // and [P][2] per-pool bound factors
};

// bf16 32x32x16 MFMA: lane l supplies A row (l % 32) and B column (l % 32),
// each with 8 contraction elements of half-wave (l / 32); the accumulator
// element v of lane l is row 8*(v/4) + 4*(l/32) + (v%4), column l % 32.  The
// scaled fp8 32x32x64 MFMA has the same row/column lanes and accumulator
// layout with 32 contraction bytes per lane, and takes one E8M0 scale per
// lane for the row (A) or column (B) block that lane holds.
//
// Workgroup = 4 waves; each wave owns NB blocks of 32 consecutive pools
// (hi and lo of the pooled keys resident as B fragments); the workgroup owns
// 128 NB pools and a range of gq chunk rows, walked one packed query tile (32
// (query, head) rows) at a time through double-buffered LDS.  Every thread
// moves the same 16-byte pieces of every tile, from precomputed offsets, two
// tiles ahead in registers and one ahead in LDS; the loop issues the same
// memory operations every tile (prefetches past the last tile read the
// chunk's spare tiles, stores of a chunk buffer are never masked), so its
// memory-counter waits cover only the prefetch they need.
//
// Every workgroup reads each query tile of its rows from L2, so the pools a
// workgroup covers set the L2 traffic per flop: at 256 pools per workgroup
// these re-reads kept the L2 busy about 90% of the scorer's cycles.  The
// bound path at 8 or more heads therefore runs with NB = 4 (512 pools per
// workgroup, 244 VGPRs at d_idx = 128); the full-score path also holds the
// correction's fragments and keeps NB = 2.
//
// EXACT = false: the chunk-buffer contract of ScoreArgs (any entry may be
// written, ineligible pools get -inf).  EXACT = true: only eligible entries of
// rows [0, rows) are stored.  LO = false: the correction q . lo is left out;
// the score s~ from hi alone is within A mu_p of the full score (see
// pool_keys_bf16_kernel), and the buffer receives the upper bound
// u = fma(A, mu_p, s~), from which the selection takes both bounds
// (s~ + A mu_p and u - 2 A mu_p) without reading mu for every pool; it
// rescores the pools near its threshold with the full sequence of MFMAs
// below.  Here A mu_p stands for A1 m1_p + A2 m2_p, formed as
// fma(A1, m1, fma(A2, m2, s~)).
template <int HI, int DI, int NB, bool EXACT, bool LO>
__global__ __launch_bounds__(256, 2) void index_score_bf16_kernel(ScoreK a) {
    static_assert(NB % 2 == 0 && (NB == 2 || (HI != 4 && !LO)),
                  "the epilogue pairs the pool blocks of a wave");
    using T = QTile<DI, LO>;
    constexpr int QPT = 32 / HI;      // queries per tile
    constexpr int NSB = DI / 16;      // bf16 MFMA steps (16 dims each)
    constexpr int NSF = (DI + 63) / 64;  // fp8 MFMA steps (64 dims each)
    constexpr int PW = 32 * NB;       // pools per wave
    constexpr int PB = 4 * PW;        // pools per workgroup
    constexpr int CPT = T::CPT;
    constexpr int NBUF = 4;           // LDS tile buffers (tiles in flight + 1)

    __shared__ __attribute__((aligned(16))) uint8_t lds[NBUF * T::LDSB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;
    int bx, by;
    xcd_block(bx, by);
    const int64_t p_blk = (int64_t)bx * PB;
    const int64_t p_wave = p_blk + wave * PW;

    // rows of this workgroup; skip leading rows that see none of its pools
    int i_begin = by * a.gq;
    const int i_end = min(a.rows, i_begin + a.gq);
    const int64_t first = 4 * (p_blk + 1) - a.q_pos0 - a.row0;
    if (first > i_begin) i_begin = (int)(first < (int64_t)i_end ? first : (int64_t)i_end);
    i_begin = (i_begin / QPT) * QPT;
    if (i_begin >= i_end) return;
    const int n_tiles = (i_end - i_begin + QPT - 1) / QPT;

    // resident pooled keys of pool p_wave + nb*32 + col
    bf16x8 bhi[NB][NSB];
    i32x8 blo[NB][NSF];
    int bsc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t p = p_wave + nb * 32 + col;
        const bool ok = p < a.n_pools;
#pragma unroll
        for (int s = 0; s < NSB; ++s)
            bhi[nb][s] = as_bf16x8(ok ? ldg16(a.khi + p * DI + 16 * s + 8 * half)
                                      : u32x4{0u, 0u, 0u, 0u});
        if constexpr (!LO) continue;
#pragma unroll
        for (int s = 0; s < NSF; ++s) {
            const int d0 = 64 * s + 32 * half;
            u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
            if (ok && d0 < DI) {
                x0 = ldg16(a.klo + p * DI + d0);
                x1 = ldg16(a.klo + p * DI + d0 + 16);
            }
            blo[nb][s] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                               (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
        bsc[nb] = ok ? (int)a.klo_scale[p] : 127;
    }
    // The resident fragments are loaded once; make that explicit so that the
    // tile loop never waits on the memory counter for them.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // Query tiles travel global -> LDS by direct loads (no registers), NBUF
    // buffers deep: the loads for tile j + NBUF - 1 are issued at the start
    // of tile j.  Thread tid moves 16-byte pieces tid + 256u (loads clamped to
    // the last piece; LDS slots past the query data are spare) and one dword
    // of the tail (w at dwords 0-31, scale bytes in 32-39, the queries' bound
    // factor pairs in 40-55).
    // Lane l of a wave lands at the wave's LDS base + l * size, so each
    // instruction fills a contiguous 1 KiB (256 B) slice.
    constexpr int D = NBUF - 1;
    constexpr int NDMA = CPT + 1;                     // direct loads per tile
    constexpr int S = HI == 4 ? 8 : QPT * (NB / 2);   // score stores per tile
    // (wave-uniform tile addresses, per-lane offsets)
    const uint8_t* tile0 = a.tiles + (int64_t)(i_begin / QPT) * T::G.tb;
    uint32_t voff[CPT + 1];
#pragma unroll
    for (int u = 0; u < CPT; ++u) voff[u] = 16u * (uint32_t)min(tid + 256 * u, T::NPQ - 1);
    voff[CPT] = (uint32_t)T::G.qb + 4u * (uint32_t)min(tid, 55);
    const uint32_t lds0 = lds_address(lds) + 1024u * (uint32_t)wave;
    auto fetch = [&](int j, int b) {  // tile j into LDS buffer b = j % NBUF
        const uint8_t* src = tile0 + (int64_t)j * T::G.tb;
        const uint32_t l = lds0 + (uint32_t)(b * T::LDSB);
#pragma unroll
        for (int u = 0; u < CPT; ++u) lds_load16_sv(src, voff[u], l + 4096u * u);
        lds_load4_sv(src, voff[CPT], l + (uint32_t)T::LDS_W - 768u * (uint32_t)wave);
    };
    // Tile j's loads are complete once at most this many later memory
    // operations are outstanding (loads and stores retire in order): the
    // loads of the D - 1 tiles issued after it and the stores of up to D
    // tiles.  With EXACT the stores are conditional and are not counted.
    auto wait_tile = [&](int j) {
        constexpr int base = (D - 1) * NDMA;
        constexpr int full = base + (EXACT ? 0 : D * S);
        static_assert(full < 64, "vmcnt range");
        if (j >= D) __builtin_amdgcn_s_waitcnt(vmcnt_imm(full));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(base));
    };

#pragma unroll
    for (int j = 0; j < D; ++j) fetch(j, j);

    // pool factors of the bound for the columns this lane stores
    const int64_t t_row0 = a.q_pos0 + a.row0;
    f32x2 mu_st[NB] = {};
    // and the first chunk row for which each of those pools is eligible
    // (4p + 3 < t, t = t_row0 + i; never for p >= n_pools), as a 32-bit
    // threshold on the row index: the -inf mask of a store is one compare.
    // (HI >= 8: entry m serves the stores of pool blocks 2m, 2m + 1.)
    int e_st[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t p = HI == 4 ? p_wave + nb * 32 + col : p_wave + 64 * (nb / 2) + lane;
        if constexpr (!LO)
            if (p < a.n_pools) mu_st[nb] = *reinterpret_cast<const f32x2*>(a.mu + 2 * p);
        const int64_t e = p < a.n_pools ? 4 * p + 4 - t_row0 : (int64_t)INT32_MAX;
        e_st[nb] = (int)(e < (int64_t)INT32_MIN ? (int64_t)INT32_MIN
                                                : (e > (int64_t)INT32_MAX ? (int64_t)INT32_MAX : e));
    }
    const uint8_t* Lw = nullptr;  // the current tile's weights/scales/bounds in LDS
    int tile_i0 = 0;
    auto put = [&](int i, int p, float v, f32x2 mu, int e) {
        // row base (wave-uniform where i is) plus a 32-bit byte offset
        float* dst = reinterpret_cast<float*>(reinterpret_cast<char*>(a.buf + (int64_t)i * a.ld) +
                                              (uint32_t)p * 4u);
        if constexpr (EXACT) {
            if (i < i_end && i >= e) *dst = canonical_zero(v);
        } else {
            if constexpr (!LO) {
                // the query's bound factors, staged in LDS with the tile.  A
                // and mu are non-negative, so both products are +0 or
                // positive and u is never -0: it needs no canonicalisation.
                const f32x2 A = reinterpret_cast<const f32x2*>(Lw + 160)[i - tile_i0];
                v = fmaf(A[0], mu[0], fmaf(A[1], mu[1], v));
            } else {
                v = canonical_zero(v);
            }
            *dst = i >= e ? v : -INFINITY;
        }
    };
    // unrolled by NBUF, so that every LDS buffer address is a constant
    // offset from the per-lane operand offsets
    for (int j0 = 0; j0 < n_tiles; j0 += NBUF) {
#pragma unroll
        for (int jj = 0; jj < NBUF; ++jj) {
            const int j = j0 + jj;
            if (j >= n_tiles) break;
            wait_tile(j);
            __syncthreads();
            // every wave is past tile j - 1: its buffer takes tile j + D (tiles
            // past the chunk's end read its spare tiles and are never used)
            fetch(j + D, (jj + D) % NBUF);
            const uint8_t* L = lds + jj * T::LDSB;

            f32x16 acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[nb][v] = 0.0f;

            // all A fragments of the tile first, then q . hi on bf16 MFMAs and
            // q . lo on scaled fp8 MFMAs into the same accumulators
            bf16x8 af[NSB];
            i32x8 af8[NSF];
#pragma unroll
            for (int s = 0; s < NSB; ++s)
                af[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(L + T::bf16_piece(col, 2 * s + half)));
#pragma unroll
            for (int s = 0; s < (LO ? NSF : 0); ++s) {
                // pieces past d_idx (only with d_idx = 96) read row padding or the
                // next row and are zeroed
                const bool in = 64 * s + 32 * half < DI;
                u32x4 x0 = *reinterpret_cast<const u32x4*>(L + T::fp8_piece(col, 4 * s + 2 * half));
                u32x4 x1 = *reinterpret_cast<const u32x4*>(L + T::fp8_piece(col, 4 * s + 2 * half + 1));
                if (!in) x0 = x1 = u32x4{0u, 0u, 0u, 0u};
                af8[s] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                               (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
            }
            const int qsc = LO ? (int)L[T::LDS_W + 128 + col] : 127;
#pragma unroll
            for (int s = 0; s < NSB; ++s)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s], bhi[nb][s], acc[nb], 0, 0, 0);
#pragma unroll
            for (int s = 0; s < (LO ? NSF : 0); ++s)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af8[s], blo[nb][s], acc[nb], 0, 0, 0, qsc, 0, bsc[nb]);
            // keep the LDS reads ahead of the MFMAs
            if constexpr (LO) {
                __builtin_amdgcn_sched_group_barrier(0x100, NSB + 2 * NSF + 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NB * (NSB + NSF), 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(0x100, NSB, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NB * NSB, 0);
            }

            // epilogue: per-lane partial sums w * relu over the rows this lane
            // holds (rows 8*g4 + 4*half + i), then the two half-waves' partials of
            // each column are added
            float wv[16];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 w4 = *reinterpret_cast<const f32x4*>(L + T::LDS_W + 4 * (8 * g4 + 4 * half));
                wv[4 * g4 + 0] = w4[0];
                wv[4 * g4 + 1] = w4[1];
                wv[4 * g4 + 2] = w4[2];
                wv[4 * g4 + 3] = w4[3];
            }
            // (the bound path at 32 heads sums each pool block's 16 rows in
            // two chains of 8, with fewer additions; its order only has to
            // stay within the rounding the bound covers, while full scores
            // keep the order the rescoring reproduces)
            constexpr bool CHAINS = !LO && HI == 32;
            float part[NB][4];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int g4 = 0; g4 < 4; g4 += CHAINS ? 2 : 1) {
                    float sacc = 0.0f;
#pragma unroll
                    for (int i = 0; i < (CHAINS ? 8 : 4); ++i)
                        sacc += wv[4 * g4 + i] * relu(acc[nb][4 * g4 + i]);
                    part[nb][g4] = sacc;
                }
            tile_i0 = i_begin + j * QPT;
            Lw = L + T::LDS_W;
            if constexpr (HI == 4) {
                // rows 8*g4 + 4*half + i are the 4 heads of query 2*g4 + half
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        put(tile_i0 + 2 * g4 + half, (int)p_wave + nb * 32 + col, part[nb][g4],
                            mu_st[nb], e_st[nb]);
            } else {
                // lane l < 32 ends with pool block 2m, lane l >= 32 with block
                // 2m + 1: one store of 64 consecutive pools per query and pair
#pragma unroll
                for (int m = 0; m < NB / 2; ++m)
#pragma unroll
                for (int u = 0; u < QPT; ++u) {
                    const int b0 = 2 * m, b1 = 2 * m + 1;
                    float x0, x1;
                    if constexpr (CHAINS) {
                        x0 = part[b0][0] + part[b0][2];
                        x1 = part[b1][0] + part[b1][2];
                    } else if constexpr (HI == 32) {
                        x0 = (part[b0][0] + part[b0][1]) + (part[b0][2] + part[b0][3]);
                        x1 = (part[b1][0] + part[b1][1]) + (part[b1][2] + part[b1][3]);
                    } else if constexpr (HI == 16) {
                        x0 = part[b0][2 * u] + part[b0][2 * u + 1];
                        x1 = part[b1][2 * u] + part[b1][2 * u + 1];
                    } else {
                        x0 = part[b0][u];
                        x1 = part[b1][u];
                    }
                    put(tile_i0 + u, (int)p_wave + 64 * m + lane, add_halves2(x0, x1), mu_st[b0],
                        e_st[b0]);
                }
            }
        }
    }
    // the direct loads still in flight (spare tiles) write this workgroup's
    // LDS: they must land before the workgroup ends
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

template <int HI, int DI>
static hipError_t launch_score_bf16_t(const ScoreArgs& a, hipStream_t stream) {
    constexpr int NB = 2;
    constexpr int PB = 128 * NB;
    // the bound path at 8+ heads: 4 pool blocks per wave, 512 pools per
    // workgroup, so that each query tile read from L2 serves twice the pools
    constexpr int NBB = HI == 4 ? 2 : 4;
    constexpr int QPT = 32 / HI;
    ScoreK k;
    k.tiles = a.tiles;
    k.khi = static_cast<const uint16_t*>(a.kbar);
    k.klo = a.klo;
    k.klo_scale = a.klo_scale;
    k.row0 = a.row0;
    k.rows = a.rows;
    // queries per workgroup: at d_idx = 128 a workgroup's resident keys (128
    // KiB) are loaded once for 128 query tiles (scoring 1-3% faster than 64
    // at 32k, 128k and the 1M share; 32, 192 and 256 were slower); at 64 and
    // 96, 64 queries
    k.gq = (DI == 128 ? 128 : 64) * QPT;
    k.q_pos0 = a.q_pos0;
    k.n_pools = a.n_pools;
    k.buf = a.buf;
    k.ld = a.ld;
    k.qbound = a.qbound;
    k.mu = a.mu;
    const dim3 grid((unsigned)((a.n_chunk + PB - 1) / PB), (unsigned)((a.rows + k.gq - 1) / k.gq));
    if (grid.x == 0 || grid.y == 0) return hipSuccess;
    // exact (caller-owned) rows get the full scores; the chunk buffer gets
    // the full scores or, with bound factors, the upper bounds of the
    // scores without the correction term
    if (a.exact) index_score_bf16_kernel<HI, DI, NB, true, true><<<grid, 256, 0, stream>>>(k);
    else if (!a.qbound) index_score_bf16_kernel<HI, DI, NB, false, true><<<grid, 256, 0, stream>>>(k);
    else {
        const dim3 gb((unsigned)((a.n_chunk + 128 * NBB - 1) / (128 * NBB)), grid.y);
        index_score_bf16_kernel<HI, DI, NBB, false, false><<<gb, 256, 0, stream>>>(k);
    }
    return hipGetLastError();
}

struct ScoreK8 {
    const uint8_t* q8;
    const uint8_t* kbar8;
    const float* pool_scale;
    const float* q_scale;
    const float* k_scale;
    const float* w;
    int64_t w_stride;
    int64_t s_q;
    int64_t row0;
    int rows;
    int gq;
    int64_t q_pos0;
    int64_t n_pools;
    float* buf;
    int64_t ld;
};

// fp8 E4M3 scoring with the 32x32x64 f8f6f4 MFMA (unit block scales): lane l
// supplies A row / B column l % 32 and 32 contraction bytes of half-wave
// l / 32; the accumulator layout is that of the 32x32 bf16 MFMA.  Products of
// two E4M3 values are exact in fp32.  The score is
//   s = sum_h w * relu(c_p * q8_h . kbar8_p),   c_p = q_scale * k_scale * 2^e_p,
// computed as |c_p| * sum_h w * relu(sign(c) * acc) (the sign of c is the
// sign of q_scale * k_scale, the same for every pool).  With a negative sign
// w * relu(-x) is taken as (-w) * min(x, 0), one integer min on the bits of
// x (negative floats are the negative ints), so both signs cost one integer
// op and one FMA per element; the sign is a uniform branch per tile.
//
// EXACT = false: the chunk-buffer contract of ScoreArgs (any entry may be
// written, ineligible pools get -inf); EXACT = true: only eligible entries
// of rows [0, rows).
template <int HI, int DI, int NB, bool EXACT>
__global__ __launch_bounds__(256, 2) void index_score_fp8_kernel(ScoreK8 a) {
    static_assert(NB % 2 == 0, "pool blocks are stored in pairs");
    constexpr int QPT = 32 / HI;
    constexpr int NS = (DI + 63) / 64;   // MFMA steps of 64 dims
    constexpr int PW = 32 * NB;
    constexpr int PB = 4 * PW;
    constexpr int LROW = DI + 16;        // LDS row stride in bytes
    constexpr int CHUNKS = 2 * DI;       // 16-byte pieces of a 32-row tile
    constexpr int CPT = (CHUNKS + 255) / 256;

    __shared__ __attribute__((aligned(16))) uint8_t sq[2][32 * LROW];
    __shared__ __attribute__((aligned(16))) float sw[2][32];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;
    int bx, by;
    xcd_block(bx, by);
    const int64_t p_blk = (int64_t)bx * PB;
    const int64_t p_wave = p_blk + wave * PW;

    int i_begin = by * a.gq;
    const int i_end = min(a.rows, i_begin + a.gq);
    const int64_t first = 4 * (p_blk + 1) - a.q_pos0 - a.row0;
    if (first > i_begin) i_begin = (int)(first < (int64_t)i_end ? first : (int64_t)i_end);
    i_begin = (i_begin / QPT) * QPT;
    if (i_begin >= i_end) return;
    const int n_tiles = (i_end - i_begin + QPT - 1) / QPT;

    const float qk = (a.q_scale ? *a.q_scale : 1.0f) * (a.k_scale ? *a.k_scale : 1.0f);
    const bool flip = qk < 0.0f;
    // pools of the stored columns (block 2m in lanes 0-31, 2m + 1 in lanes
    // 32-63) and the first chunk row for which each is eligible (4p + 3 < t),
    // as a 32-bit threshold on the row index
    const int64_t t_row0 = a.q_pos0 + a.row0;
    int e_st[NB / 2];
    float c_st[NB / 2];
#pragma unroll
    for (int m = 0; m < NB / 2; ++m) {
        const int64_t p = p_wave + 64 * m + lane;
        const int64_t e = p < a.n_pools ? 4 * p + 4 - t_row0 : (int64_t)INT32_MAX;
        e_st[m] = (int)(e < (int64_t)INT32_MIN ? (int64_t)INT32_MIN
                                               : (e > (int64_t)INT32_MAX ? (int64_t)INT32_MAX : e));
        c_st[m] = p < a.n_pools ? fabsf(qk) * a.pool_scale[p] : 0.0f;
    }

    // resident pooled keys; contraction bytes 64*s + 32*half .. +32 (zero past DI)
    i32x8 bfr[NB][NS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t p = p_wave + nb * 32 + col;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            u32x4 lo4 = {0u, 0u, 0u, 0u}, hi4 = {0u, 0u, 0u, 0u};
            const int d0 = 64 * s + 32 * half;
            if (p < a.n_pools && d0 < DI) {
                lo4 = ldg16(a.kbar8 + p * DI + d0);
                hi4 = ldg16(a.kbar8 + p * DI + d0 + 16);
            }
            bfr[nb][s] = i32x8{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                               (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): resident loads done before the tile loop

    u32x4 pre[CPT];
    float prew = 0.0f;
    auto fetch = [&](int j) {
        const int64_t qrow0 = a.row0 + i_begin + (int64_t)j * QPT;
        const uint8_t* src = a.q8 + qrow0 * (HI * DI);
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int ch = tid + u * 256;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ch < CHUNKS) {
                const int r = ch / (DI / 16);
                if (qrow0 + r / HI < a.s_q) v = ldg16(src + (int64_t)ch * 16);
            }
            pre[u] = v;
        }
        if (tid < 32) {
            const int64_t qr = qrow0 + tid / HI;
            prew = qr < a.s_q ? a.w[qr * a.w_stride + (tid % HI)] : 0.0f;
        }
    };
    auto stash = [&](int b) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int ch = tid + u * 256;
            if (ch < CHUNKS) {
                const int r = ch / (DI / 16), c16 = ch % (DI / 16);
                *reinterpret_cast<u32x4*>(&sq[b][r * LROW + c16 * 16]) = pre[u];
            }
        }
        if (tid < 32) sw[b][tid] = prew;
    };

    fetch(0);
    stash(0);
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const int cur = j & 1;
        const bool has_next = j + 1 < n_tiles;
        if (has_next) fetch(j + 1);

        f32x16 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[nb][v] = 0.0f;

        const uint8_t* arow = &sq[cur][col * LROW];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int d0 = 64 * s + 32 * half;
            u32x4 lo4 = {0u, 0u, 0u, 0u}, hi4 = {0u, 0u, 0u, 0u};
            if (d0 < DI) {
                lo4 = *reinterpret_cast<const u32x4*>(arow + d0);
                hi4 = *reinterpret_cast<const u32x4*>(arow + d0 + 16);
            }
            const i32x8 af = {(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                              (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bfr[nb][s], acc[nb],
                                                                          0, 0, 0, 127, 0, 127);
        }

        float wv[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(&sw[cur][8 * g4 + 4 * half]);
            wv[4 * g4 + 0] = w4[0];
            wv[4 * g4 + 1] = w4[1];
            wv[4 * g4 + 2] = w4[2];
            wv[4 * g4 + 3] = w4[3];
        }
        const int tile_i0 = i_begin + j * QPT;
        // per-lane partial sums w * relu over the rows this lane holds (rows
        // 8*g4 + 4*half + i of the accumulator)
        float part[NB][4];
        auto head_sums = [&](auto flip_tag) {
            constexpr bool FL = decltype(flip_tag)::value;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    float sacc = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int xb = __float_as_int(acc[nb][4 * g4 + i]);
                        sacc = FL ? fmaf(-wv[4 * g4 + i], __int_as_float(min(xb, 0)), sacc)
                                  : fmaf(wv[4 * g4 + i], __int_as_float(max(xb, 0)), sacc);
                    }
                    part[nb][g4] = sacc;
                }
        };
        if (flip) head_sums(std::true_type{});
        else head_sums(std::false_type{});
        auto put = [&](int i, int m, float v) {
            float* dst = reinterpret_cast<float*>(
                reinterpret_cast<char*>(a.buf + (int64_t)i * a.ld) +
                (uint32_t)(p_wave + 64 * m + lane) * 4u);
            v = canonical_zero(c_st[m] * v);
            if constexpr (EXACT) {
                if (i < i_end && i >= e_st[m]) *dst = v;
            } else {
                *dst = i >= e_st[m] ? v : -INFINITY;
            }
        };
#pragma unroll
        for (int m = 0; m < NB / 2; ++m) {
            // lanes 0-31 end with pool block 2m, lanes 32-63 with block 2m + 1
            if constexpr (HI == 4) {
                // lane half h holds query 2*g4 + h in part[.][g4]; swapping
                // the upper half of block 2m with the lower half of block
                // 2m + 1 gives query 2*g4 in r[0] and query 2*g4 + 1 in r[1]
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const auto r = __builtin_amdgcn_permlane32_swap(
                        __float_as_uint(part[2 * m][g4]), __float_as_uint(part[2 * m + 1][g4]),
                        false, false);
                    put(tile_i0 + 2 * g4, m, __uint_as_float(r[0]));
                    put(tile_i0 + 2 * g4 + 1, m, __uint_as_float(r[1]));
                }
            } else {
#pragma unroll
                for (int u = 0; u < QPT; ++u) {
                    float x0, x1;
                    if constexpr (HI == 32) {
                        x0 = (part[2 * m][0] + part[2 * m][1]) + (part[2 * m][2] + part[2 * m][3]);
                        x1 = (part[2 * m + 1][0] + part[2 * m + 1][1]) +
                             (part[2 * m + 1][2] + part[2 * m + 1][3]);
                    } else if constexpr (HI == 16) {
                        x0 = part[2 * m][2 * u] + part[2 * m][2 * u + 1];
                        x1 = part[2 * m + 1][2 * u] + part[2 * m + 1][2 * u + 1];
                    } else {
                        x0 = part[2 * m][u];
                        x1 = part[2 * m + 1][u];
                    }
                    put(tile_i0 + u, m, add_halves2(x0, x1));
                }
            }
        }

        if (has_next) stash(cur ^ 1);
        __syncthreads();
    }
}

template <int HI, int DI>
static hipError_t launch_score_fp8_t(const ScoreArgs& a, hipStream_t stream) {
    constexpr int NB = 4;
    constexpr int PB = 128 * NB;
    constexpr int QPT = 32 / HI;
    ScoreK8 k;
    k.q8 = static_cast<const uint8_t*>(a.q_idx);
    k.kbar8 = static_cast<const uint8_t*>(a.kbar);
    k.pool_scale = a.pool_scale;
    k.q_scale = a.q_scale;
    k.k_scale = a.k_scale;
    k.w = a.w;
    k.w_stride = a.w_stride;
    k.s_q = a.s_q;
    k.row0 = a.row0;
    k.rows = a.rows;
    k.gq = 64 * QPT;
    k.q_pos0 = a.q_pos0;
    k.n_pools = a.n_pools;
    k.buf = a.buf;
    k.ld = a.ld;
    const dim3 grid((unsigned)((a.n_chunk + PB - 1) / PB), (unsigned)((a.rows + k.gq - 1) / k.gq));
    if (grid.x == 0 || grid.y == 0) return hipSuccess;
    if (a.exact) index_score_fp8_kernel<HI, DI, NB, true><<<grid, 256, 0, stream>>>(k);
    else index_score_fp8_kernel<HI, DI, NB, false><<<grid, 256, 0, stream>>>(k);
    return hipGetLastError();
}

template <int HI>
static hipError_t launch_score_fp8_h(const ScoreArgs& a, hipStream_t stream) {
    switch (a.d_idx) {
        case 64: return launch_score_fp8_t<HI, 64>(a, stream);
        case 96: return launch_score_fp8_t<HI, 96>(a, stream);
        case 128: return launch_score_fp8_t<HI, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int HI>
static hipError_t launch_score_bf16_h(const ScoreArgs& a, hipStream_t stream) {
    switch (a.d_idx) {
        case 64: return launch_score_bf16_t<HI, 64>(a, stream);
        case 96: return launch_score_bf16_t<HI, 96>(a, stream);
        case 128: return launch_score_bf16_t<HI, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t stream) {
    if (a.fp8) {
        switch (a.h_idx) {
            case 4: return launch_score_fp8_h<4>(a, stream);
            case 8: return launch_score_fp8_h<8>(a, stream);
            case 16: return launch_score_fp8_h<16>(a, stream);
            case 32: return launch_score_fp8_h<32>(a, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (a.h_idx) {
        case 4: return launch_score_bf16_h<4>(a, stream);
        case 8: return launch_score_bf16_h<8>(a, stream);
        case 16: return launch_score_bf16_h<16>(a, stream);
        case 32: return launch_score_bf16_h<32>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsa
