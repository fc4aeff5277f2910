// Sparse attention backward: dq, dk, dv of the forward over the kept pools.
//
// SkyRL blog "Scaling Training to 1M Token Context on GLM-5.3-Flash": the
// setting is training, and section "Activation Recompute" reruns each
// layer's forward inside the backward pass, so the softmax weights are not
// stored but recomputed from the forward's log-sum-exp.  The page prints no
// backward; these are the gradients of the forward's definition for
// L = sum dout . out (per query, head h and attended token j):
//   D_h  = dout_h . out_h             (from the stored forward output)
//   P_j  = exp(scale q_h . k_j - lse_h)
//   dS_j = P_j (dout_h . v_j - D_h)
//   dq_h = scale sum_j dS_j k_j,   dk_j += scale dS_j q_h,   dv_j += P_j dout_h
//
// Two passes, both deterministic (no floating-point atomics):
//   1. Query-major, the forward's gather: one wave per query walks its
//      tokens in tiles of 32 slots and forms D and dq.
//   2. Pool-major: the gradient of a key row sums over the queries that
//      attend it.  The selections are transposed into bitmaps [chunk query
//      / 32][pool slot] of 32-bit words by integer atomic OR in LDS (the same
//      bits in any order), those of all chunks at once when they fit the
//      workspace.  The pool slots are ordered by the number of queries of
//      the last chunk that keep them, most first, and taken 4 at a time: a
//      query that keeps one often-kept pool tends to keep others, so a
//      group's visits serve more pools than 4 neighbouring slots would.  One
//      workgroup per group (16 tokens) walks, one chunk of queries at a
//      time, the set bits of its 4 rows in increasing query order,
//      recomputes P and dS for its tokens against each query, and
//      accumulates dk and dv in registers; each chunk's sum is added to dk
//      and dv in chunk order.  The workgroups take the groups in that order,
//      so that those resident together have similar work, walk the chunk's
//      queries together and find each query's rows in the L2.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace dsa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Two fp32 values as packed bf16 (round to nearest even; one instruction).
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

// Element offset of (row r, element e) in an LDS tile of 16-bit rows that
// serves both 16-byte operand reads of 16 consecutive rows and transposed
// reads (ds_read_b64_tr_b16) of 4 consecutive rows without bank conflicts.
// Rows are W + 16 elements apart (W in {64, 96, 128}: 40, 56 or 72 dwords,
// so 8 consecutive rows start on distinct 8-dword bank groups), and the
// 16-byte piece c of row r is stored at piece c ^ b(r) with
// b(r) = ((r >> 2) ^ (r >> 3)) & 1, which separates rows r and r + 4 and
// rows r and r + 8 for the 16-byte reads while keeping the 4 rows of one
// transposed read (same r >> 2) in the same order.
template <int W>
__device__ __forceinline__ int toff(int r, int e) {
    return r * (W + 16) + (((e >> 3) ^ (((r >> 2) ^ (r >> 3)) & 1)) << 3) + (e & 7);
}

// Transposed read of 4 rows of 4 bf16: in each 16-lane group, lane x names
// row base_row + x / 4 and elements e0 + 4 * (x % 4) .. +3, and receives
// element e0 + x of rows base_row + 0..3 (the MFMA operand of a contraction
// over those rows).
template <int W>
__device__ __forceinline__ u32x2 tr_read(const uint16_t* tile, int base_row, int e0, int x) {
    const v4i16 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(tile + toff<W>(base_row + (x >> 2), e0 + 4 * (x & 3))));
    return __builtin_bit_cast(u32x2, t4);
}

// Buffer resource over `bytes` bytes at p (raw, 32-bit offsets; reads at or
// beyond `bytes` return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// The same transposed read at a precomputed element offset.
__device__ __forceinline__ u32x2 tr_at(const uint16_t* p) {
    const v4i16 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
    return __builtin_bit_cast(u32x2, t4);
}

// ---------------------------------------------------------------- pass 1: dq

struct DqK {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* out;
    const uint16_t* dout;
    const int32_t* __restrict__ idx;
    const float* lse;
    int64_t s_q, s_k, q_pos0, n_pools;
    int h, k_pools, n_tail;
    float scale, scale_log2;
    float* dq;      // [s_q, h, d]
    float* delta;   // [s_q, h]
};

// One wave per query (4 per workgroup, independent).  Per 32-slot tile:
//   S^T [32 x 16 heads]  = K_tile . Q^T      (A: key rows from LDS)
//   dP^T[32 x 16 heads]  = V_tile . dout^T   (A: value rows from LDS)
//   dS = P (dP - D), P = exp2(S scale log2e - lse log2e), 0 off the token set
//   dq^T[d x 16 heads]  += K_tile^T . dS^T   (A: key rows read transposed)
// MFMA 16x16x32 bf16: lane l supplies A row l % 16 and B column l % 16 with 8
// contraction elements of group l / 16; accumulator i of lane l is row
// 4 (l / 16) + i, column l % 16.
template <int D, int DV>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(DqK a) {
    constexpr int KS = D / 32, VS = DV / 32, MT = D / 16;
    constexpr int KCH = D / 8, VCH = DV / 8;
    constexpr int KPL = 32 * KCH / 64, VPL = 32 * VCH / 64;
    constexpr int KT = 32 * (D + 16), VT = 32 * (DV + 16);
    __shared__ __attribute__((aligned(16))) uint16_t sk_all[4][KT];
    __shared__ __attribute__((aligned(16))) uint16_t sv_all[4][VT];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t qi = (int64_t)blockIdx.x * 4 + wave;
    if (qi >= a.s_q) return;  // waves are independent: no workgroup barrier below
    uint16_t* sk = sk_all[wave];
    uint16_t* sv = sv_all[wave];
    const int col = lane & 15, grp = lane >> 4;
    const bool head = col < a.h;
    const int64_t t = a.q_pos0 + qi;
    const int n_tail_t = (int)min((int64_t)a.n_tail, t & 3);
    const int n_pool_slots = 4 * a.k_pools;
    const int n_slots = n_pool_slots + n_tail_t;
    const int n_tiles = (n_slots + 31) / 32;
    const int n_full = a.k_pools / 8;
    const int32_t* irow = a.idx + qi * a.k_pools;

    // B operands: lane (col = head, grp) holds q / dout of head col, elements
    // 32 s + 8 grp .. +8; the output row in the same layout gives D.
    bf16x8 qf[KS], gf[VS];
    float dsum = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (head) x = ldg16(a.q + (qi * a.h + col) * D + 32 * s + 8 * grp);
        qf[s] = as_bf16x8(x);
    }
#pragma unroll
    for (int s = 0; s < VS; ++s) {
        u32x4 g = {0u, 0u, 0u, 0u}, o = {0u, 0u, 0u, 0u};
        if (head) {
            g = ldg16(a.dout + (qi * a.h + col) * DV + 32 * s + 8 * grp);
            o = ldg16(a.out + (qi * a.h + col) * DV + 32 * s + 8 * grp);
        }
        gf[s] = as_bf16x8(g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            dsum += bf16_to_f32(g[j] & 0xFFFFu) * bf16_to_f32(o[j] & 0xFFFFu);
            dsum += bf16_to_f32(g[j] >> 16) * bf16_to_f32(o[j] >> 16);
        }
    }
    dsum += __shfl_xor(dsum, 16);
    dsum += __shfl_xor(dsum, 32);
    const float delta = dsum;
    const float lse2 = head ? a.lse[qi * a.h + col] * kLog2e : 0.0f;
    if (head && grp == 0) a.delta[qi * a.h + col] = delta;

    struct Tile {
        u32x4 k[KPL];
        u32x4 v[VPL];
        uint32_t valid;   // bit s: slot s holds a real token
    };
    // 8 whole pools: wave-uniform pool ids; ids outside [0, P) read pool 0
    // (a real row) and are masked out.
    auto load_full = [&](int tile, Tile& T) {
        int32_t pid[8];
        uint32_t valid = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int32_t p = irow[tile * 8 + j];
            const bool ok = p >= 0 && (int64_t)p < a.n_pools;
            valid |= ok ? 0xFu << (4 * j) : 0u;
            pid[j] = ok ? p : 0;
        }
        T.valid = valid;
        auto pool_of = [&](int r, int ch, int slot) -> int32_t {
            const int p0 = 64 * r / (4 * ch);
            return (slot >> 2) == p0 ? pid[p0] : pid[p0 + 1 < 8 ? p0 + 1 : p0];
        };
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
            const int g = lane + 64 * r, slot = g / KCH;
            T.k[r] = ldg16(a.k + (4 * (int64_t)pool_of(r, KCH, slot) + (slot & 3)) * D + 8 * (g % KCH));
        }
#pragma unroll
        for (int r = 0; r < VPL; ++r) {
            const int g = lane + 64 * r, slot = g / VCH;
            T.v[r] = ldg16(a.v + (4 * (int64_t)pool_of(r, VCH, slot) + (slot & 3)) * DV + 8 * (g % VCH));
        }
    };
    // A partial pool tile and/or the own-pool tail: per-slot tokens, zeros
    // for empty slots.  Every lane calls token_of (shuffle inside).
    auto token_of = [&](int slot_in_tile, int tile, int32_t pid) -> int64_t {
        const int slot = tile * 32 + slot_in_tile;
        const int32_t p = __shfl(pid, (slot_in_tile >> 2) & 7);
        if (slot < n_pool_slots) {
            if (p >= 0 && (int64_t)p < a.n_pools) return 4 * (int64_t)p + (slot & 3);
            return -1;
        }
        const int j = slot - n_pool_slots;
        if (j < n_tail_t) {
            const int64_t tok = t - n_tail_t + j;
            if (tok >= 0 && tok < a.s_k) return tok;
        }
        return -1;
    };
    auto load_general = [&](int tile, Tile& T) {
        const int pi = tile * 8 + (lane & 7);
        const int32_t pid = pi < a.k_pools ? irow[pi] : -1;
        const int64_t vt = token_of(lane & 31, tile, pid);
        T.valid = (uint32_t)__ballot(vt >= 0);
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
            const int g = lane + 64 * r;
            const int64_t tok = token_of(g / KCH, tile, pid);
            u32x4 x = {0u, 0u, 0u, 0u};
            if (tok >= 0) x = ldg16(a.k + tok * D + 8 * (g % KCH));
            T.k[r] = x;
        }
#pragma unroll
        for (int r = 0; r < VPL; ++r) {
            const int g = lane + 64 * r;
            const int64_t tok = token_of(g / VCH, tile, pid);
            u32x4 x = {0u, 0u, 0u, 0u};
            if (tok >= 0) x = ldg16(a.v + tok * DV + 8 * (g % VCH));
            T.v[r] = x;
        }
    };
    auto load_tile = [&](int tile, Tile& T) {
        if (tile < n_full) load_full(tile, T);
        else load_general(tile, T);
    };
    auto stash = [&](const Tile& T) {
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
            const int g = lane + 64 * r;
            *reinterpret_cast<u32x4*>(sk + toff<D>(g / KCH, 8 * (g % KCH))) = T.k[r];
        }
#pragma unroll
        for (int r = 0; r < VPL; ++r) {
            const int g = lane + 64 * r;
            *reinterpret_cast<u32x4*>(sv + toff<DV>(g / VCH, 8 * (g % VCH))) = T.v[r];
        }
    };

    f32x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    Tile cur;
    if (n_tiles > 0) load_tile(0, cur);
    for (int tile = 0; tile < n_tiles; ++tile) {
        stash(cur);
        const uint32_t valid = cur.valid;
        if (tile + 1 < n_tiles) load_tile(tile + 1, cur);

        f32x4 sacc[2], pacc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            sacc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            pacc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(sk + toff<D>(16 * u + col, 32 * s + 8 * grp));
                sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), qf[s], sacc[u], 0, 0, 0);
            }
#pragma unroll
            for (int s = 0; s < VS; ++s) {
                const u32x4 vf = *reinterpret_cast<const u32x4*>(sv + toff<DV>(16 * u + col, 32 * s + 8 * grp));
                pacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf), gf[s], pacc[u], 0, 0, 0);
            }
        }
        // this lane holds slots 16u + 4 grp + i of head col
        float ds[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int slot = 16 * u + 4 * grp + i;
                const float p = (head && ((valid >> slot) & 1u))
                                    ? __builtin_amdgcn_exp2f(sacc[u][i] * a.scale_log2 - lse2)
                                    : 0.0f;
                ds[u][i] = p * (pacc[u][i] - delta);
            }
        // dS^T fragment: contraction slots {4 grp .. +3, 16 + 4 grp .. +3}
        u32x4 dw;
#pragma unroll
        for (int j = 0; j < 4; ++j) dw[j] = pack2(ds[j >> 1][(j & 1) * 2], ds[j >> 1][(j & 1) * 2 + 1]);
        const bf16x8 dsf = as_bf16x8(dw);
        // K^T fragments: row = dim 16 m + col, the same contraction slots
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const u32x2 lo = tr_read<D>(sk, 4 * grp, 16 * m, col);
            const u32x2 hi = tr_read<D>(sk, 16 + 4 * grp, 16 * m, col);
            const u32x4 kw = {lo[0], lo[1], hi[0], hi[1]};
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kw), dsf, acc[m], 0, 0, 0);
        }
    }
    if (head) {
        float* row = a.dq + (qi * a.h + col) * D;
#pragma unroll
        for (int m = 0; m < MT; ++m)
            *reinterpret_cast<f32x4*>(row + 16 * m + 4 * grp) = acc[m] * a.scale;
    }
}

// ---------------------------------------------------------------- transposed selection

// Chunk bitmap, word-major: bit (r % 32) of word [r / 32][slot] (row stride
// `stride` slots, a multiple of 4) is set when chunk query row r attends a
// token of pool slot `slot` -- a kept pool id in [0, P), or its own pool when
// it has tail tokens there.  One workgroup per (word column c, range of
// `range` slots): its 32 query rows OR their bits into an LDS copy of the
// range with LDS atomics (the same bits in any order), then it writes every
// word of the range, zeros included, so the bitmap needs no clearing.  The
// launcher narrows the range (16384 slots, 64 KiB of LDS, down to 2048) until
// the launch has about a thousand workgroups; every workgroup reads all ids
// of its 32 rows and keeps those in its range.
constexpr int BITS_RANGE_MAX = 16384;
constexpr int BITS_RANGE_MIN = 2048;

__global__ __launch_bounds__(256) void bwd_select_bits_kernel(
    const int32_t* __restrict__ idx, int k_pools, int64_t row0, int rows, int64_t q_pos0,
    int64_t n_pools, int64_t s_k, int n_tail, uint32_t* bits, int64_t stride, int range) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lw[];  // range words
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = (int)blockIdx.x;
    const int64_t s0 = (int64_t)blockIdx.y * range;
    const int64_t s1 = s0 + range < stride ? s0 + range : stride;
    const int width = (int)(s1 - s0);  // a multiple of 4
    const int64_t p_end = s1 < n_pools ? s1 : n_pools;  // kept ids in [s0, p_end) count
    // rows 32 c + 8 wave .. +7 of the chunk: the first 512 ids of all 8 rows
    // (8 per lane and row) are loaded at once, while the range is cleared and
    // before the first atomic; ids past 512 follow row by row, 8 per lane at
    // a time
    int32_t pv[8][8];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        const int row = 32 * c + 8 * wave + rr;
        const int32_t* irow = idx + (row0 + row) * k_pools;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = lane + 64 * u;
            pv[rr][u] = row < rows && j < k_pools ? irow[j] : -1;
        }
    }
    for (int e = 4 * tid; e < width; e += 4 * 256)
        *reinterpret_cast<u32x4*>(lw + e) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        const int r = 8 * wave + rr;
        const int row = 32 * c + r;
        if (row >= rows) break;
        const int64_t i = row0 + row;
        const uint32_t bit = 1u << r;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (pv[rr][u] >= s0 && pv[rr][u] < p_end) atomicOr(&lw[pv[rr][u] - s0], bit);
        const int32_t* irow = idx + i * k_pools;
        for (int j0 = 512; j0 < k_pools; j0 += 512) {
            int32_t pw[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + lane + 64 * u;
                pw[u] = j < k_pools ? irow[j] : -1;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (pw[u] >= s0 && pw[u] < p_end) atomicOr(&lw[pw[u] - s0], bit);
        }
        const int64_t t = q_pos0 + i;
        const int64_t own = t >> 2;
        if (lane == 0 && n_tail > 0 && (t & 3) != 0 && 4 * own < s_k && own >= s0 && own < s1)
            atomicOr(&lw[own - s0], bit);
    }
    __syncthreads();
    uint32_t* dst = bits + (int64_t)c * stride + s0;
    for (int e = 4 * tid; e < width; e += 4 * 256)
        *reinterpret_cast<u32x4*>(dst + e) = *reinterpret_cast<const u32x4*>(lw + e);
}

// Entries per pool slot in nw word rows of the bitmap (32 queries each).
__global__ __launch_bounds__(256) void bwd_slot_counts_kernel(const uint32_t* __restrict__ bits,
                                                              int64_t stride, int nw,
                                                              uint32_t* counts) {
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (s >= stride) return;
    uint32_t c = 0;
#pragma unroll 8
    for (int w = 0; w < nw; ++w) c += __popc(bits[(int64_t)w * stride + s]);
    counts[s] = c;
}

// The pool slots in decreasing order of their entry counts (of `rows`
// queries), in ORDER_BUCKETS equal bands of the count, and in increasing slot
// order inside a band: a stable split, so the order is a function of the
// counts alone.  One workgroup of 16 waves takes 1024 slots at a time; a
// slot's place is its band's start, plus the band's slots of earlier tiles
// and earlier waves of this tile, plus its rank among the lanes of its wave
// in the same band (found by ballots, one per band present in the wave).
constexpr int ORDER_BUCKETS = 64;

__global__ __launch_bounds__(1024) void bwd_slot_order_kernel(const uint32_t* __restrict__ counts,
                                                              int64_t stride, int rows,
                                                              int32_t* perm) {
    constexpr int NB = ORDER_BUCKETS;
    static_assert(NB == 64, "one band per lane when a wave clears its counts");
    __shared__ uint32_t base[NB];       // next place of each band
    __shared__ uint32_t wcnt[16][NB];   // this tile: slots per wave and band, then their offsets
    __shared__ uint32_t tile_n[NB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // band 0 holds the most entries
    auto band = [&](uint32_t c) {
        const uint64_t b = (uint64_t)c * NB / ((uint64_t)rows + 1);
        return NB - 1 - (int)(b < NB ? b : NB - 1);
    };
    if (tid < NB) base[tid] = 0u;
    __syncthreads();
    for (int64_t s = tid; s < stride; s += 1024) atomicAdd(&base[band(counts[s])], 1u);
    __syncthreads();
    if (tid == 0) {
        uint32_t sum = 0u;
        for (int b = 0; b < NB; ++b) {
            const uint32_t n = base[b];
            base[b] = sum;
            sum += n;
        }
    }
    for (int64_t t0 = 0; t0 < stride; t0 += 1024) {
        wcnt[wave][lane] = 0u;
        __syncthreads();
        const int64_t s = t0 + tid;
        const bool valid = s < stride;
        const int b = valid ? band(counts[s]) : -1;
        int rank = 0;
        for (uint64_t todo = __ballot(valid); todo;) {
            const int lead = __builtin_ctzll(todo);
            const int lb = __builtin_amdgcn_readlane(b, lead);
            const uint64_t m = __ballot(b == lb);
            if (b == lb) rank = __popcll(m & ((1ull << lane) - 1ull));
            if (lane == lead) wcnt[wave][lb] = (uint32_t)__popcll(m);
            todo &= ~m;
        }
        __syncthreads();
        if (tid < NB) {
            uint32_t run = 0u;
            for (int w = 0; w < 16; ++w) {
                const uint32_t n = wcnt[w][tid];
                wcnt[w][tid] = run;
                run += n;
            }
            tile_n[tid] = run;
        }
        __syncthreads();
        if (valid) perm[base[b] + wcnt[wave][b] + rank] = (int32_t)s;
        __syncthreads();
        if (tid < NB) base[tid] += tile_n[tid];
    }
}

// ---------------------------------------------------------------- pass 2: dk, dv

struct DkvK {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const float* lse;
    const float* delta;
    const int32_t* perm;    // [stride] pool slots; group g holds perm[4 g .. 4 g + 3]
    const uint32_t* bits;   // [chunk / 32][stride]
    int64_t stride;
    int64_t s_k, q_pos0, row0;
    int rows;
    int64_t slots;          // pool slots: ceil(s_k / 4)
    int h, n_tail;
    float scale, scale_log2;
    int accumulate;         // 0: store the chunk's sum; 1: add it
    float* dk;              // [s_k, d]
    float* dv;              // [s_k, dv]
};

// One workgroup (4 waves) per 4 pool slots = 16 tokens.  The chunk's
// entries are the set bits of the OR of the 4 bitmap rows, in increasing
// query order; entry pair n (entries 2n, 2n + 1) belongs to wave n % 4.  For
// the two queries A, B of a pair:
//   S_X [16 heads x 16 tokens] = Q_X . K^T          (A: q rows from LDS)
//   dP_X[16 x 16]              = dout_X . V^T       (A: dout rows from LDS)
//   P, dS as in pass 1, zero for tokens the query does not attend
//   dV[16 tokens x dv] += P^T . dout,  dK[16 x d] += dS^T . Q
// where the last two contract over the 32 (query, head) pairs of A and B;
// the contraction order of lane group g is heads 4g .. 4g+3 of A, then of B,
// which is exactly what the S accumulators of the lane hold, and what the
// transposed reads of the q and dout rows return.  The 4 waves' partial sums
// are added in wave order at the end.
template <int D, int DV>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkv_kernel(DkvK a) {
    constexpr int KS = D / 32, VS = DV / 32, MK = D / 16, MV = DV / 16;
    constexpr int QT = 16 * (D + 16), OT = 16 * (DV + 16);      // one query's rows
    constexpr int STAGE = 2 * QT + 2 * OT;                         // per wave, elements
    constexpr int QCH = D / 8, OCH = DV / 8;                       // pieces per row
    constexpr int QPL = 16 * QCH / 64, OPL = 16 * OCH / 64;        // pieces per lane per query
    constexpr int RED = D + DV + 4;                                // reduction row stride (fp32)
    static_assert(4 * STAGE * 2 >= 4 * 16 * RED * 4, "reduction area exceeds the staging area");
    __shared__ __attribute__((aligned(16))) uint16_t stage_all[4 * STAGE];
    __shared__ __attribute__((aligned(16))) float sl_all[4][64];   // lse, delta of a pair

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int col = lane & 15, grp = lane >> 4;
    // the group's 4 pool slots (slots >= a.slots pad the order and hold no
    // tokens); its token 4 j + r is token r of slot j
    int64_t slot[4];
    int64_t tmin = INT64_MAX;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        slot[j] = a.perm[4 * (int64_t)blockIdx.x + j];
        if (slot[j] < a.slots && 4 * slot[j] < tmin) tmin = 4 * slot[j];
    }
    const int64_t t_last = a.q_pos0 + a.row0 + a.rows - 1;
    // row of token 4 j + r (r < 4) in k, v, dk and dv; -1 past s_k
    auto token_row = [&](int tok) -> int64_t {
        const int j = tok >> 2;
        const int64_t sj = j == 0 ? slot[0] : j == 1 ? slot[1] : j == 2 ? slot[2] : slot[3];
        const int64_t t = 4 * sj + (tok & 3);
        return sj < a.slots && t < a.s_k ? t : -1;
    };
    bool found = false;     // this wave had an entry
    uint16_t* st = stage_all + wave * STAGE;
    uint16_t* sq[2] = {st, st + QT};
    uint16_t* so[2] = {st + 2 * QT, st + 2 * QT + OT};
    float* sl = sl_all[wave];

    f32x4 dka[MK], dva[MV];
#pragma unroll
    for (int m = 0; m < MK; ++m) dka[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < MV; ++m) dva[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // a token is attended only by queries after it
    if (tmin < t_last) {
        // rows of heads >= h stay zero in LDS (never written below)
        if (a.h < 16) {
            for (int e = lane * 8; e < STAGE; e += 64 * 8)
                *reinterpret_cast<u32x4*>(st + e) = u32x4{0u, 0u, 0u, 0u};
        }
        // ---- entry scan.  Windows of 64 bitmap words (2048 chunk queries):
        // lane L holds word wbase + L of the 4 rows; a wave-wide prefix sum of
        // the per-word entry counts gives every entry its global index, and
        // lane L keeps in `mine` the bits of its word that are entries of this
        // wave.  The words of the next window are loaded while this one is
        // consumed.
        // token masks of the 4 slots (slots past s_k hold fewer or no tokens)
        uint32_t slot_tokens = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t left = slot[j] < a.slots ? a.s_k - 4 * slot[j] : 0;
            const uint32_t m = left >= 4 ? 0xFu : (left > 0 ? (1u << left) - 1u : 0u);
            slot_tokens |= m << (4 * j);
        }
        const int nw = (a.rows + 31) / 32;
        // the 4 slots' words of word row wb + lane (the padding slots'
        // columns hold zeros)
        auto load_words = [&](int wb, uint32_t (&dst)[4]) {
            const uint32_t* brow = a.bits + (int64_t)(wb + lane) * a.stride;
            const bool ok = wb + lane < nw;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[j] = ok ? brow[slot[j]] : 0u;
        };
        uint32_t ww[4], pw[4];
        load_words(0, pw);
        int wbase = -64;
        int base_n = 0;           // entries before the current window
        uint32_t mine = 0;        // per lane
        uint64_t lanes = 0;       // lanes with entries of this wave left
        int cl = 0;               // current lane (word)
        uint32_t cbits = 0, cw[4] = {0u, 0u, 0u, 0u};
        auto next_window = [&]() -> bool {
            wbase += 64;
            if (wbase >= nw) return false;
#pragma unroll
            for (int j = 0; j < 4; ++j) ww[j] = pw[j];
            if (wbase + 64 < nw) load_words(wbase + 64, pw);
            const uint32_t u = ww[0] | ww[1] | ww[2] | ww[3];
            const int c = __popc(u);
            int incl = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off);
                if (lane >= off) incl += y;
            }
            int idx = base_n + incl - c;
            mine = 0;
            for (uint32_t r = u; r; r &= r - 1, ++idx)
                if (((idx >> 1) & 3) == wave) mine |= r & (0u - r);
            base_n += __shfl(incl, 63);
            lanes = __ballot(mine != 0);
            return true;
        };
        // next entry of this wave: chunk row and 16-bit token mask; false at the end
        auto next_entry = [&](int& row, uint32_t& mask) -> bool {
            while (cbits == 0) {
                if (lanes == 0) {
                    if (!next_window()) return false;
                    continue;
                }
                cl = __builtin_ctzll(lanes);
                lanes &= lanes - 1;
                cbits = __builtin_amdgcn_readlane(mine, cl);
#pragma unroll
                for (int j = 0; j < 4; ++j) cw[j] = __builtin_amdgcn_readlane(ww[j], cl);
            }
            const int b = __builtin_ctz(cbits);
            cbits &= cbits - 1;
            row = 32 * (wbase + cl) + b;
            // the entry's 4 slot bits, spread to nibbles, times the slots'
            // token masks
            const uint32_t b4 = ((cw[0] >> b) & 1u) | (((cw[1] >> b) & 1u) << 1) |
                                (((cw[2] >> b) & 1u) << 2) | (((cw[3] >> b) & 1u) << 3);
            const uint32_t spread = (b4 & 1u) | ((b4 & 2u) << 3) | ((b4 & 4u) << 6) | ((b4 & 8u) << 9);
            mask = (spread * 0xFu) & slot_tokens;
            const int64_t t = a.q_pos0 + a.row0 + row;
            const int64_t own = t >> 2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (slot[j] == own) {
                    // the query's own pool is in this group (its bit comes
                    // from the tail only): the tail tokens before t
                    const int r = (int)(t & 3);
                    const int u0 = max(0, r - a.n_tail);
                    const uint32_t tail = ((1u << r) - 1u) & ~((1u << u0) - 1u);
                    mask &= ~((~tail & 0xFu) << (4 * j));
                }
            }
            return true;
        };

        // staged rows of one pair, in registers while the previous pair computes
        struct Pair {
            u32x4 q[2][QPL];
            u32x4 o[2][OPL];
            float ld;         // lane l: (l < 32 ? A : B), (l & 16 ? delta : lse), head l & 15
            uint32_t mask[2];
        };
        // A query's q (and dout) rows are h x 2W contiguous bytes, and lane
        // L's piece r is byte 16 (L + 64 r) of them: one buffer load with a
        // scalar base per query, whose range ends with the h rows (pieces of
        // heads >= h read as zero).  Its LDS place toff(g / CH, 8 (g % CH)),
        // g = L + 64 r, is fixed per lane: at W = 128 it is base_b + 4 r
        // (W + 16) with b = (r ^ r / 2) & 1 choosing one of two lane bases;
        // at other widths one precomputed offset per piece.
        constexpr bool ROWS128 = D == 128 && DV == 128;
        const uint32_t goff = 16u * (uint32_t)lane;
        const uint32_t qbytes = (uint32_t)(a.h * D * 2), obytes = (uint32_t)(a.h * DV * 2);
        const int tbase = (lane >> 4) * (D + 16);
        const int sbase0 = tbase + ((lane & 15) << 3), sbase1 = tbase + (((lane & 15) ^ 1) << 3);
        int qst[ROWS128 ? 1 : QPL], ost[ROWS128 ? 1 : OPL];
        // Lane offsets of the reads, fixed per lane: the A-operand piece of
        // step s is toff(col, 32 s + 8 grp) = col (W + 16) + 32 s + 8 (grp ^
        // b(col)); the transposed read of rows 4 grp .. +3 at element 16 m is
        // toff(4 grp + col / 4, 16 m + 4 (col % 4)) = tr + 16 m.
        const int bsw = ((col >> 2) ^ (col >> 3)) & 1;
        const int qrd = col * (D + 16) + 8 * (grp ^ bsw);
        const int ord = col * (DV + 16) + 8 * (grp ^ bsw);
        const int trow = 4 * grp + (col >> 2), c3 = col & 3;
        const int btr = ((trow >> 2) ^ (trow >> 3)) & 1;
        const int qtr = trow * (D + 16) + 8 * ((c3 >> 1) ^ btr) + 4 * (c3 & 1);
        const int otr = trow * (DV + 16) + 8 * ((c3 >> 1) ^ btr) + 4 * (c3 & 1);
        if constexpr (!ROWS128) {
#pragma unroll
            for (int r = 0; r < QPL; ++r) {
                const int g = lane + 64 * r;
                qst[r] = toff<D>(g / QCH, 8 * (g % QCH));
            }
#pragma unroll
            for (int r = 0; r < OPL; ++r) {
                const int g = lane + 64 * r;
                ost[r] = toff<DV>(g / OCH, 8 * (g % OCH));
            }
        }
        auto load_pair = [&](int rowA, uint32_t mA, int rowB, uint32_t mB, Pair& P) {
            P.mask[0] = mA;
            P.mask[1] = mB;
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int64_t qi = a.row0 + (x ? rowB : rowA);
                const __amdgpu_buffer_rsrc_t rq = rsrc_of(a.q + qi * a.h * D, qbytes);
                const __amdgpu_buffer_rsrc_t ro = rsrc_of(a.dout + qi * a.h * DV, obytes);
#pragma unroll
                for (int r = 0; r < QPL; ++r)
                    P.q[x][r] = __builtin_amdgcn_raw_buffer_load_b128(rq, goff + 1024u * r, 0, 0);
#pragma unroll
                for (int r = 0; r < OPL; ++r)
                    P.o[x][r] = __builtin_amdgcn_raw_buffer_load_b128(ro, goff + 1024u * r, 0, 0);
            }
            const int64_t ql = a.row0 + ((lane >> 5) ? rowB : rowA);
            const int hl = lane & 15;
            const float* src = (lane & 16) ? a.delta : a.lse;
            P.ld = hl < a.h ? src[ql * a.h + hl] : 0.0f;
        };
        auto stash_pair = [&](const Pair& P) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                if constexpr (ROWS128) {
#pragma unroll
                    for (int r = 0; r < QPL; ++r)
                        *reinterpret_cast<u32x4*>(sq[x] + (((r ^ (r >> 1)) & 1) ? sbase1 : sbase0) +
                                                  4 * r * (D + 16)) = P.q[x][r];
#pragma unroll
                    for (int r = 0; r < OPL; ++r)
                        *reinterpret_cast<u32x4*>(so[x] + (((r ^ (r >> 1)) & 1) ? sbase1 : sbase0) +
                                                  4 * r * (DV + 16)) = P.o[x][r];
                } else {
                    // (pieces of heads >= h hold zeros: their rows stay zero)
#pragma unroll
                    for (int r = 0; r < QPL; ++r)
                        *reinterpret_cast<u32x4*>(sq[x] + qst[r]) = P.q[x][r];
#pragma unroll
                    for (int r = 0; r < OPL; ++r)
                        *reinterpret_cast<u32x4*>(so[x] + ost[r]) = P.o[x][r];
                }
            }
            sl[lane] = P.ld;
        };
        // the next pair of this wave; a lone last entry is paired with itself
        // under an empty mask (its rows are real, so everything stays finite)
        auto fetch = [&](Pair& P) -> bool {
            int ra, rb;
            uint32_t ma, mb;
            if (!next_entry(ra, ma)) return false;
            if (!next_entry(rb, mb)) {
                rb = ra;
                mb = 0;
            }
            load_pair(ra, ma, rb, mb, P);
            return true;
        };

        Pair nxt;
        bool have = fetch(nxt);
        found = have;
        // B operands of S and dP: lane (col = token, grp) holds key / value
        // row of token col, elements 32 s + 8 grp .. +8 (zero past s_k)
        bf16x8 kf[KS], vf[VS];
        if (have) {
            const int64_t tr = token_row(col);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                u32x4 x = {0u, 0u, 0u, 0u};
                if (tr >= 0) x = ldg16(a.k + tr * D + 32 * s + 8 * grp);
                kf[s] = as_bf16x8(x);
            }
#pragma unroll
            for (int s = 0; s < VS; ++s) {
                u32x4 x = {0u, 0u, 0u, 0u};
                if (tr >= 0) x = ldg16(a.v + tr * DV + 32 * s + 8 * grp);
                vf[s] = as_bf16x8(x);
            }
        }
        while (have) {
            stash_pair(nxt);
            uint32_t mask[2] = {nxt.mask[0], nxt.mask[1]};
            have = fetch(nxt);

            float pv[2][4], dsv[2][4];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f}, pacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const u32x4 qa = *reinterpret_cast<const u32x4*>(sq[x] + qrd + 32 * s);
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa), kf[s], sacc, 0, 0, 0);
                }
#pragma unroll
                for (int s = 0; s < VS; ++s) {
                    const u32x4 oa = *reinterpret_cast<const u32x4*>(so[x] + ord + 32 * s);
                    pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(oa), vf[s], pacc, 0, 0, 0);
                }
                // accumulator i: head 4 grp + i, token col
                const bool on = (mask[x] >> col) & 1u;
                const f32x4 lsx = *reinterpret_cast<const f32x4*>(sl + 32 * x + 4 * grp);
                const f32x4 dlx = *reinterpret_cast<const f32x4*>(sl + 32 * x + 16 + 4 * grp);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = on && 4 * grp + i < a.h;
                    const float p = ok ? __builtin_amdgcn_exp2f(sacc[i] * a.scale_log2 - lsx[i] * kLog2e) : 0.0f;
                    pv[x][i] = p;
                    dsv[x][i] = p * (pacc[i] - dlx[i]);
                }
            }
            // A operands over the 32 (query, head) pairs: heads 4 grp .. +3 of A, then of B
            const u32x4 pw = {pack2(pv[0][0], pv[0][1]), pack2(pv[0][2], pv[0][3]),
                              pack2(pv[1][0], pv[1][1]), pack2(pv[1][2], pv[1][3])};
            const u32x4 dw = {pack2(dsv[0][0], dsv[0][1]), pack2(dsv[0][2], dsv[0][3]),
                              pack2(dsv[1][0], dsv[1][1]), pack2(dsv[1][2], dsv[1][3])};
            const bf16x8 pf = as_bf16x8(pw), df = as_bf16x8(dw);
#pragma unroll
            for (int m = 0; m < MV; ++m) {
                const u32x2 x0 = tr_at(so[0] + otr + 16 * m);
                const u32x2 x1 = tr_at(so[1] + otr + 16 * m);
                const u32x4 ow = {x0[0], x0[1], x1[0], x1[1]};
                dva[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, as_bf16x8(ow), dva[m], 0, 0, 0);
            }
#pragma unroll
            for (int m = 0; m < MK; ++m) {
                const u32x2 x0 = tr_at(sq[0] + qtr + 16 * m);
                const u32x2 x1 = tr_at(sq[1] + qtr + 16 * m);
                const u32x4 qw = {x0[0], x0[1], x1[0], x1[1]};
                dka[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(df, as_bf16x8(qw), dka[m], 0, 0, 0);
            }
        }
    }
    // a group without entries in this chunk has nothing to add
    if (!__syncthreads_or(found ? 1 : 0) && a.accumulate) return;

    // ---- sum of the 4 waves in wave order, then store or add
    float* red = reinterpret_cast<float*>(stage_all);
    // accumulator i of lane (col, grp): token 4 grp + i, column 16 m + col
#pragma unroll
    for (int m = 0; m < MK; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * grp + i) * RED + 16 * m + col] = dka[m][i];
#pragma unroll
    for (int m = 0; m < MV; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * grp + i) * RED + D + 16 * m + col] = dva[m][i];
    __syncthreads();
    constexpr int C4 = (D + DV) / 4;
    for (int e = threadIdx.x; e < 16 * C4; e += 256) {
        const int tok = e / C4, c = 4 * (e % C4);
        const int64_t tr = token_row(tok);
        if (tr < 0) continue;
        f32x4 s = *reinterpret_cast<const f32x4*>(red + tok * RED + c);
#pragma unroll
        for (int wv = 1; wv < 4; ++wv) s += *reinterpret_cast<const f32x4*>(red + (wv * 16 + tok) * RED + c);
        float* dst = c < D ? a.dk + tr * D + c : a.dv + tr * DV + (c - D);
        if (c < D) s *= a.scale;
        if (a.accumulate) s += *reinterpret_cast<const f32x4*>(dst);
        *reinterpret_cast<f32x4*>(dst) = s;
    }
}

template <int D>
hipError_t launch_dq_d(const DqK& k, int dv, dim3 grid, hipStream_t s) {
    switch (dv) {
        case 64: attn_bwd_dq_kernel<D, 64><<<grid, 256, 0, s>>>(k); break;
        case 96: attn_bwd_dq_kernel<D, 96><<<grid, 256, 0, s>>>(k); break;
        case 128: attn_bwd_dq_kernel<D, 128><<<grid, 256, 0, s>>>(k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_dkv_d(const DkvK& k, int dv, dim3 grid, hipStream_t s) {
    switch (dv) {
        case 64: attn_bwd_dkv_kernel<D, 64><<<grid, 256, 0, s>>>(k); break;
        case 96: attn_bwd_dkv_kernel<D, 96><<<grid, 256, 0, s>>>(k); break;
        case 128: attn_bwd_dkv_kernel<D, 128><<<grid, 256, 0, s>>>(k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_dq(const AttnBwdArgs& a, hipStream_t stream) {
    if (a.s_q <= 0) return hipSuccess;
    DqK k;
    k.q = a.q;
    k.k = a.k;
    k.v = a.v;
    k.out = a.out;
    k.dout = a.dout;
    k.idx = a.idx;
    k.lse = a.lse;
    k.s_q = a.s_q;
    k.s_k = a.s_k;
    k.q_pos0 = a.q_pos0;
    k.n_pools = a.s_k / 4;
    k.h = a.h;
    k.k_pools = a.k_pools;
    k.n_tail = a.n_tail;
    k.scale = a.scale;
    k.scale_log2 = a.scale * kLog2e;
    k.dq = a.dq;
    k.delta = a.delta;
    const dim3 grid((unsigned)((a.s_q + 3) / 4));
    switch (a.d) {
        case 64: return launch_dq_d<64>(k, a.dv, grid, stream);
        case 96: return launch_dq_d<96>(k, a.dv, grid, stream);
        case 128: return launch_dq_d<128>(k, a.dv, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn_bwd_bits(const AttnBwdArgs& a, int64_t row0, int rows, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const int64_t cols = (rows + 31) / 32;
    int range = BITS_RANGE_MAX;
    while (range > BITS_RANGE_MIN && cols * ((a.stride + range - 1) / range) < 1024) range /= 2;
    const dim3 grid((unsigned)cols, (unsigned)((a.stride + range - 1) / range));
    bwd_select_bits_kernel<<<grid, 256, (size_t)range * 4u, stream>>>(
        a.idx, a.k_pools, row0, rows, a.q_pos0, a.s_k / 4, a.s_k, a.n_tail, a.bits, a.stride,
        range);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_order(const AttnBwdArgs& a, int rows, hipStream_t stream) {
    if (a.stride <= 0 || rows <= 0) return hipSuccess;
    bwd_slot_counts_kernel<<<(unsigned)((a.stride + 255) / 256), 256, 0, stream>>>(
        a.bits, a.stride, (rows + 31) / 32, a.slot_counts);
    bwd_slot_order_kernel<<<1, 1024, 0, stream>>>(a.slot_counts, a.stride, rows, a.slot_perm);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_dkv(const AttnBwdArgs& a, int64_t row0, int rows, int accumulate,
                               hipStream_t stream) {
    const int64_t slots = (a.s_k + 3) / 4;
    if (slots <= 0) return hipSuccess;
    DkvK k;
    k.q = a.q;
    k.k = a.k;
    k.v = a.v;
    k.dout = a.dout;
    k.lse = a.lse;
    k.delta = a.delta;
    k.perm = a.slot_perm;
    k.bits = a.bits;
    k.stride = a.stride;
    k.s_k = a.s_k;
    k.q_pos0 = a.q_pos0;
    k.row0 = row0;
    k.rows = rows;
    k.slots = slots;
    k.h = a.h;
    k.n_tail = a.n_tail;
    k.scale = a.scale;
    k.scale_log2 = a.scale * kLog2e;
    k.accumulate = accumulate;
    k.dk = a.dk;
    k.dv = a.dv_grad;
    const dim3 grid((unsigned)((slots + 3) / 4));
    switch (a.d) {
        case 64: return launch_dkv_d<64>(k, a.dv, grid, stream);
        case 96: return launch_dkv_d<96>(k, a.dv, grid, stream);
        case 128: return launch_dkv_d<128>(k, a.dv, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsa
