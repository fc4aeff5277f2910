// Sparse attention forward over the kept pools, online softmax.
//
// SkyRL blog "Scaling Training to 1M Token Context on GLM-5.3-Flash",
// section "DeepSeek Sparse Attention (DSA) Optimizations": attention reads
// only the selected tokens (2048 = 512 pools x 4), so its cost is linear in
// the sequence; section "Making Sparse Attention Actually Sparse": NoPE heads
// (head dim 96 here, natively, no padding) and 2,051 keys, read as the 512
// pools plus up to 3 tokens of the query's own unfinished pool before it.
//
// One wave per query; all query heads (<= 16) share the single key/value
// head, so every gathered key/value row serves every head.  Tokens are
// processed in tiles of 32 slots (8 pools).  Per tile:
//   S^T[32 tokens x 16 heads] = K_tile . Q^T      2 x (d/32) MFMA 16x16x32 bf16
//     (key rows pass through a per-wave LDS tile: an operand load would
//      touch 16 tokens' half cache lines, a tile load reads whole pools)
//   online softmax per head (fp32, exp2 domain)
//   O^T[dv x 16 heads] += V_tile^T . P^T           dv/16 MFMA 16x16x32 bf16
//     (P^T comes straight from the S^T accumulators; V goes through a
//      per-wave LDS tile because its token axis is the contraction axis, and
//      comes back transposed by ds_read_b64_tr_b16)
// The next tile's key/value rows are loaded into registers (whole pools per
// load) while the current tile is computed.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace dsa {

namespace {

struct AttnK {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* __restrict__ idx;
    int64_t s_q, s_k, q_pos0, n_pools;
    int h, k_pools, n_tail;
    float scale_log2;  // softmax scale * log2(e)
    uint16_t* out;
    float* lse;
};

// 16x16x32 bf16 MFMA: lane l supplies A row (l % 16) and B column (l % 16),
// each with 8 contraction elements of group (l / 16); accumulator element i
// of lane l is row 4*(l/16) + i, column l % 16.
// Two fp32 values as packed bf16 (round to nearest even; one instruction).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

template <int D, int DV>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(AttnK a) {
    constexpr int KS = D / 32;             // QK contraction steps
    constexpr int MT = DV / 16;            // O^T row tiles
    constexpr int KCH = D / 8;             // 16-byte pieces per key row
    constexpr int VCH = DV / 8;            // 16-byte pieces per value row
    constexpr int KPL = 32 * KCH / 64;     // key pieces per lane per tile
    constexpr int VPL = 32 * VCH / 64;     // value pieces per lane per tile
    // LDS row strides (bf16).  Keys: D + 8, so the 16-byte operand reads of
    // 16 consecutive rows fall on distinct banks.  Values: DV + 16, so rows
    // stay 16-byte aligned and the 4 rows x 32 bytes of one transposed read
    // of a 16-lane group hit distinct banks (stride = 8 dwords mod 32).
    constexpr int KROW = D + 8;
    constexpr int VROW = DV + 16;
    __shared__ __attribute__((aligned(16))) uint16_t sk_all[4][32 * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t sv_all[4][32 * VROW];

    const int lane = threadIdx.x & 63;
    // wave-uniform: everything derived from the query row stays scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t qi = (int64_t)blockIdx.x * 4 + wave;
    if (qi >= a.s_q) return;  // waves are independent: no workgroup barrier below
    uint16_t* sk = sk_all[wave];
    uint16_t* sv = sv_all[wave];
    const int col = lane & 15, grp = lane >> 4;
    const int64_t t = a.q_pos0 + qi;
    const int n_tail_t = (int)min((int64_t)a.n_tail, t & 3);
    const int n_pool_slots = 4 * a.k_pools;
    const int n_slots = n_pool_slots + n_tail_t;
    const int n_tiles = (n_slots + 31) / 32;
    const int n_full = a.k_pools / 8;      // tiles of 8 whole pools
    const int32_t* irow = a.idx + qi * a.k_pools;

    // Q^T fragments: head = col, dims 32*s + 8*grp .. +8
    bf16x8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (col < a.h) v = ldg16(a.q + (qi * a.h + col) * D + 32 * s + 8 * grp);
        qf[s] = as_bf16x8(v);
    }

    // Tile registers: lane L moves 16-byte piece g = L + 64r of the tile's
    // key rows (slot g / KCH, piece g % KCH) and of its value rows.  Rows of
    // one pool are contiguous in memory, so every load reads whole cache
    // lines of at most two pools.
    struct Tile {
        u32x4 k[KPL];
        u32x4 v[VPL];
        uint32_t valid;   // bit s: slot s holds a real token
    };

    // A tile of 8 whole pools: the pool ids are wave-uniform scalars.  Ids
    // outside [0, P) are replaced by pool 0 (a real row, so no load strays)
    // and their slots are masked out of the softmax.  A load touches one
    // pool when a row has 16 pieces (then its address is scalar), else two.
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
            const int p0 = 64 * r / (4 * ch);  // first pool load r touches
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

    // General tile (a partial last pool tile and/or the unfinished-pool
    // tail): per-slot tokens; invalid slots load zeros.  Every lane must call
    // token_of (shuffle inside); pid holds the tile's pool ids in lanes 0..7.
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
            u32x4 v = {0u, 0u, 0u, 0u};
            if (tok >= 0) v = ldg16(a.k + tok * D + 8 * (g % KCH));
            T.k[r] = v;
        }
#pragma unroll
        for (int r = 0; r < VPL; ++r) {
            const int g = lane + 64 * r;
            const int64_t tok = token_of(g / VCH, tile, pid);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (tok >= 0) v = ldg16(a.v + tok * DV + 8 * (g % VCH));
            T.v[r] = v;
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
            *reinterpret_cast<u32x4*>(sk + (g / KCH) * KROW + 8 * (g % KCH)) = T.k[r];
        }
#pragma unroll
        for (int r = 0; r < VPL; ++r) {
            const int g = lane + 64 * r;
            *reinterpret_cast<u32x4*>(sv + (g / VCH) * VROW + 8 * (g % VCH)) = T.v[r];
        }
    };

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 oacc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) oacc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // One set of tile registers: tile j goes to LDS before tile j + 1 is
    // loaded over it, so the next tile's loads overlap this tile's MFMAs and
    // softmax.
    Tile cur;
    if (n_tiles > 0) load_tile(0, cur);

    for (int tile = 0; tile < n_tiles; ++tile) {
        stash(cur);
        const uint32_t valid = cur.valid;
        if (tile + 1 < n_tiles) load_tile(tile + 1, cur);

        // S^T for the two 16-slot halves; A = key rows from LDS: lane
        // (col, grp) reads slot 16u + col, dims 32s + 8grp .. +8
        f32x4 sacc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            sacc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(sk + (16 * u + col) * KROW + 32 * s + 8 * grp);
                sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), qf[s], sacc[u], 0, 0, 0);
            }
        }

        // online softmax; this lane holds slots 16u + 4*grp + i of head col
        float x[2][4];
        float mt = -INFINITY;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int slot = 16 * u + 4 * grp + i;
                x[u][i] = ((valid >> slot) & 1u) ? sacc[u][i] * a.scale_log2 : -INFINITY;
                mt = fmaxf(mt, x[u][i]);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // Lazy rescaling: the running maximum moves only when the tile's
        // maximum exceeds it by more than 2^8, so probabilities stay <= 256
        // (harmless in fp32 and bf16) and the accumulators are rescaled only
        // on the rare tiles where some head's maximum jumps.  l and O stay
        // consistent with the same m_run, so the result is unchanged.
        const bool jump = mt > m_run + 8.0f;
        float alpha = 1.0f;
        if (jump) {
            alpha = __builtin_amdgcn_exp2f(m_run - mt);  // 0 when m_run = -inf
            m_run = mt;
        }
        float p[2][4];
        float ps = 0.0f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // no valid token seen yet: m_run = -inf, every p is 0
                p[u][i] = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[u][i] - m_run);
                ps += p[u][i];
            }
        l_run = l_run * alpha + ps;
        if (__ballot(jump)) {
#pragma unroll
            for (int m = 0; m < MT; ++m) oacc[m] *= alpha;
        }

        // P^T fragment: contraction slots {4g..4g+3, 16+4g..16+4g+3}
        u32x4 pw;
#pragma unroll
        for (int j = 0; j < 4; ++j) pw[j] = pack_bf16x2(p[j >> 1][(j & 1) * 2], p[j >> 1][(j & 1) * 2 + 1]);
        const bf16x8 pf = as_bf16x8(pw);

        // V^T fragments from LDS: row = dim 16m + col, the same contraction
        // slots.  ds_read_b64_tr_b16: in each 16-lane group, lane r names a
        // row of 4 bf16 and receives element r % 4 of the rows named by lanes
        // r/4, r/4 + 4, r/4 + 8, r/4 + 12.  Lane x of group grp names slot
        // 16u + 4*grp + x/4, dims 16m + 4*(x%4) .. +3, so lane (col, grp)
        // receives dim 16m + col of slots 16u + 4*grp + 0..3.
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            u32x4 vw;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int slot = 16 * u + 4 * grp + (col >> 2);
                const v4i16 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16*)(sv + slot * VROW + 16 * m + 4 * (col & 3)));
                const u32x2 w2 = __builtin_bit_cast(u32x2, t4);
                vw[2 * u] = w2[0];
                vw[2 * u + 1] = w2[1];
            }
            oacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vw), pf, oacc[m], 0, 0, 0);
        }
    }

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (col < a.h) {
        uint16_t* orow = a.out + (qi * a.h + col) * DV;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint32_t w0 = f32_to_bf16(oacc[m][0] * inv) | (f32_to_bf16(oacc[m][1] * inv) << 16);
            const uint32_t w1 = f32_to_bf16(oacc[m][2] * inv) | (f32_to_bf16(oacc[m][3] * inv) << 16);
            *reinterpret_cast<u32x2*>(orow + 16 * m + 4 * grp) = u32x2{w0, w1};
        }
        if (a.lse && grp == 0)
            a.lse[qi * a.h + col] =
                l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
}

template <int D>
hipError_t launch_d(const AttnK& k, int dv, dim3 grid, hipStream_t stream) {
    switch (dv) {
        case 64: sparse_attn_kernel<D, 64><<<grid, 256, 0, stream>>>(k); break;
        case 96: sparse_attn_kernel<D, 96><<<grid, 256, 0, stream>>>(k); break;
        case 128: sparse_attn_kernel<D, 128><<<grid, 256, 0, stream>>>(k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream) {
    if (a.s_q <= 0) return hipSuccess;
    AttnK k;
    k.q = a.q;
    k.k = a.k;
    k.v = a.v;
    k.idx = a.idx;
    k.s_q = a.s_q;
    k.s_k = a.s_k;
    k.q_pos0 = a.q_pos0;
    k.n_pools = a.s_k / 4;
    k.h = a.h;
    k.k_pools = a.k_pools;
    k.n_tail = a.n_tail;
    k.scale_log2 = a.scale * 1.4426950408889634f;
    k.out = a.out;
    k.lse = a.lse;
    const dim3 grid((unsigned)((a.s_q + 3) / 4));
    switch (a.d) {
        case 64: return launch_d<64>(k, a.dv, grid, stream);
        case 96: return launch_d<96>(k, a.dv, grid, stream);
        case 128: return launch_d<128>(k, a.dv, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsa
