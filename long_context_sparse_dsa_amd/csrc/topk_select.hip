// Per-query top-k pool selection over one chunk's fp32 score rows.
//
// SkyRL blog "Scaling Training to 1M Token Context on GLM-5.3-Flash",
// section "DeepSeek Sparse Attention (DSA) Optimizations": each query keeps
// its best pools (512 pools = 2048 tokens); section "Over Time: Chunking":
// pools are scored and selected a chunk of queries at a time; section
// "Across GPUs: Sharding": the kept pool ids are int32.
//
// Rule: keep the k largest fp32 scores among the n(t) eligible pools, ties
// broken towards the lower pool id; emit the ids in ascending order, padded
// with -1 when n(t) < k.  Exact and deterministic: every decision is taken on
// the 32-bit order key of the fp32 score (larger float <=> larger key), with
// integer counting only.
//
// One workgroup (4 waves) per query row:
//   n <= k       every eligible pool, no scores read;
//   n <= CAP     the whole row goes to an LDS list (key, id) in id order;
//   n >  CAP     a 2048-element sample of the row (128 cache-line blocks)
//                gives a threshold tau that about 2-4x k elements exceed;
//                one coalesced pass compacts {key >= tau} into the LDS list,
//                keeping id order; if fewer than k or more than CAP elements
//                qualify, an exact multi-pass radix over the row in global
//                memory takes over (slow path, still exact).
// On a list, a radix-16 refinement narrows a key range [lo, hi] until the
// elements above hi plus the in-range ones are exactly decided: everything
// above hi is kept, and in-range elements are kept in id order while fewer
// than `remaining` have been kept.  Counting uses per-thread LDS counters
// (one slot per digit and thread) so that skewed score distributions cause
// no atomic contention.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace dsa {

namespace {

constexpr int NT = 256;
constexpr int CAP = 4096;
constexpr int SAMPLE_BLOCKS = 128;
constexpr int SAMPLE_LEN = 16;
constexpr int SAMPLE_N = SAMPLE_BLOCKS * SAMPLE_LEN;
// per-thread digit counters, one row of NT per digit, padded so that the
// transposed reduction (16 digits x 16 partial sums per wave) is free of
// bank conflicts
constexpr int CNT_STRIDE = NT + 16;

struct SelShared {
    alignas(16) uint32_t key[CAP];
    alignas(16) int32_t id[CAP];
    uint32_t cnt[16 * CNT_STRIDE];
    uint32_t hist[16];
    uint32_t tmp[8];
    uint32_t wtot[8 * (NT / 64)];
};

// Wave-level inclusive scans on DPP: row shifts 1, 2, 4, 8 within each row
// of 16 lanes, then row broadcasts of lanes 15 and 31 into the later rows.
// Lanes without a source take the identity `id`.
template <class Op>
__device__ __forceinline__ uint32_t wave_incl_scan_op(uint32_t v, uint32_t id, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xA, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xC, 0xF, false));
    return v;
}

struct AddOp {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct MinOp {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); }
};
struct MaxOp {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); }
};

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int /*lane*/) {
    return wave_incl_scan_op(v, 0u, AddOp{});
}

// Sum over each row of 16 lanes, valid in lane 15 of the row.
__device__ __forceinline__ uint32_t row16_sum(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);
    return v;
}

// Exclusive prefix over the workgroup; *total receives the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, SelShared& sh, uint32_t* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t inc = wave_incl_scan(v, lane);
    if (lane == 63) sh.tmp[wave] = inc;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t x = sh.tmp[w];
        if (w < wave) base += x;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return base + inc - v;
}

// Exclusive prefix over the workgroup of VB counts per thread, ordered
// slot-major: all threads' slot 0, then all threads' slot 1, ...  (the order
// of elements base + (u*NT + tid)*4 + j).  Returns the offsets in `off` and
// the grand total.
template <int VB>
__device__ __forceinline__ uint32_t block_excl_scan_slots(const uint32_t (&c)[VB],
                                                          uint32_t (&off)[VB], SelShared& sh,
                                                          uint32_t* wtot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t inc[VB];
#pragma unroll
    for (int u = 0; u < VB; ++u) {
        inc[u] = wave_incl_scan(c[u], lane);
        if (lane == 63) wtot[u * (NT / 64) + wave] = inc[u];
    }
    __syncthreads();
    uint32_t base = 0;
#pragma unroll
    for (int u = 0; u < VB; ++u) {
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            const uint32_t x = wtot[u * (NT / 64) + w];
            if (w < wave) before += x;
            tot += x;
        }
        off[u] = base + before + inc[u] - c[u];
        base += tot;
    }
    __syncthreads();
    return base;
}

__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, SelShared& sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    mn = wave_incl_scan_op(mn, 0xFFFFFFFFu, MinOp{});
    mx = wave_incl_scan_op(mx, 0u, MaxOp{});
    if (lane == 63) {
        sh.tmp[wave] = mn;
        sh.tmp[4 + wave] = mx;
    }
    __syncthreads();
    mn = min(min(sh.tmp[0], sh.tmp[1]), min(sh.tmp[2], sh.tmp[3]));
    mx = max(max(sh.tmp[4], sh.tmp[5]), max(sh.tmp[6], sh.tmp[7]));
    __syncthreads();
}

// Initial range [lo, hi] from the extreme keys: the aligned block of the
// lowest nibble boundary above their highest differing bit; returns the
// first digit shift (or -1 when all keys are equal).
__device__ __forceinline__ int start_range(uint32_t mn, uint32_t mx, uint32_t& lo, uint32_t& hi) {
    const uint32_t diff = mn ^ mx;
    if (diff == 0) {
        lo = hi = mn;
        return -1;
    }
    const int top = 31 - __clz(diff);
    const int shift = (top / 4) * 4;
    const uint32_t mask = (shift + 4 >= 32) ? 0u : (0xFFFFFFFFu << (shift + 4));
    lo = mn & mask;
    hi = lo | ~mask;
    return shift;
}

// Radix-16 refinement.  Precondition: at least `remaining` keys lie in
// [lo, hi] and every key above hi is already kept.  On return the kept set is
// {key > hi} plus the first `remaining` in-range keys in id order.
template <class KeyAt>
__device__ void refine(KeyAt key_at, int64_t n, int shift, uint32_t& lo, uint32_t& hi,
                       uint32_t& remaining, SelShared& sh) {
    const int tid = threadIdx.x;
    for (; shift >= 0 && lo != hi; shift -= 4) {
#pragma unroll
        for (int d = 0; d < 16; ++d) sh.cnt[d * CNT_STRIDE + tid] = 0;
        for (int64_t e = tid; e < n; e += NT) {
            const uint32_t k = key_at(e);
            if (k >= lo && k <= hi) sh.cnt[((k >> shift) & 15u) * CNT_STRIDE + tid] += 1;
        }
        __syncthreads();
        // digit tid/16 summed over threads (tid%16) + 16u, u = 0..15
        uint32_t s = 0;
        const uint32_t* c = &sh.cnt[(tid >> 4) * CNT_STRIDE + (tid & 15)];
#pragma unroll
        for (int u = 0; u < 16; ++u) s += c[16 * u];
        s = row16_sum(s);
        if ((tid & 15) == 15) sh.hist[tid >> 4] = s;
        __syncthreads();
        uint32_t above = 0, hb = 0;
        int b = 0;
        for (int d = 15; d >= 0; --d) {
            const uint32_t h = sh.hist[d];
            if (above + h >= remaining) {
                b = d;
                hb = h;
                break;
            }
            above += h;
        }
        remaining -= above;
        const uint32_t keep = (shift + 4 >= 32) ? 0u : (lo & (0xFFFFFFFFu << (shift + 4)));
        lo = keep | ((uint32_t)b << shift);
        hi = lo | ((1u << shift) - 1u);
        __syncthreads();
        if (hb == remaining) break;
    }
}

// A key tau with at least r of the SAMPLE_N sample keys (sh.key) >= tau,
// and not many more: a 256-bin histogram linear in the scores' values (not
// in their bit patterns, which would lump the upper tail into one bin) gives
// the highest bin b whose suffix holds r keys; tau is the smallest sample key
// in bins >= b.  Any tau that leaves between k and CAP row elements above it
// serves the compaction; the selection after it is exact.
__device__ uint32_t sample_threshold(uint32_t r, SelShared& sh) {
    constexpr int NBIN = 256;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int e = tid; e < SAMPLE_N; e += NT) {
        mn = min(mn, sh.key[e]);
        mx = max(mx, sh.key[e]);
    }
    block_minmax(mn, mx, sh);
    if (mn == mx) return mn;
    const float vmin = key_to_float(mn), vmax = key_to_float(mx);
    const float scale = (float)NBIN / (vmax - vmin);
    auto bin_of = [&](uint32_t key) {
        const float b = (key_to_float(key) - vmin) * scale;
        return b >= (float)(NBIN - 1) ? NBIN - 1 : (b > 0.0f ? (int)b : 0);
    };
    uint32_t* hist = sh.cnt;  // NBIN counters
    for (int b = tid; b < NBIN; b += NT) hist[b] = 0;
    __syncthreads();
    for (int e = tid; e < SAMPLE_N; e += NT) atomicAdd(&hist[bin_of(sh.key[e])], 1u);
    __syncthreads();
    if (wave == 0) {
        // lane l holds bins 4l .. 4l+3; suffix sums from the top bin down
        uint32_t h[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[j] = hist[4 * lane + j];
            tot += h[j];
        }
        // inclusive scan over lanes in reverse order gives the suffix sum
        const uint32_t rev = wave_incl_scan((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (63 - lane), (int)tot), lane);
        const uint32_t suffix = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (63 - lane), (int)rev);
        // bins of this lane: suffix(4l + j) = suffix - sum of h[0..j)
        uint32_t s_j = suffix;
        int found = -1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (s_j >= r) found = 4 * lane + j;
            s_j -= h[j];
        }
        // the highest bin whose suffix reaches r
        const uint32_t best = wave_incl_scan_op(found < 0 ? 0u : (uint32_t)found + 1u, 0u, MaxOp{});
        if (lane == 63) sh.tmp[0] = best - 1u;
    }
    __syncthreads();
    const int b_min = (int)sh.tmp[0];
    __syncthreads();
    uint32_t kmin = 0xFFFFFFFFu, dummy = 0u;
    for (int e = tid; e < SAMPLE_N; e += NT) {
        const uint32_t key = sh.key[e];
        if (bin_of(key) >= b_min) kmin = min(kmin, key);
    }
    block_minmax(kmin, dummy, sh);
    return kmin;
}

// Radix-256 refinement of a list in LDS: the same contract as refine, with
// 8-bit digits counted by LDS atomics (integer, so the counts do not depend
// on their order) and the digit found by one wave's suffix scan: at most 4
// passes instead of 8.
__device__ void refine256(int m, uint32_t& lo, uint32_t& hi, uint32_t& remaining,
                          SelShared& sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t* hist = sh.cnt;
    const uint32_t diff = lo ^ hi;
    if (diff == 0) return;
    // highest differing bit of the range -> first 8-bit digit
    int shift = ((31 - __clz(diff)) / 8) * 8;
    for (; shift >= 0 && lo != hi; shift -= 8) {
        for (int b = tid; b < 256; b += NT) hist[b] = 0;
        __syncthreads();
        for (int e = tid; e < m; e += NT) {
            const uint32_t k = sh.key[e];
            if (k >= lo && k <= hi) atomicAdd(&hist[(k >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            uint32_t h[4], tot = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[j] = hist[4 * lane + j];
                tot += h[j];
            }
            const uint32_t rev = wave_incl_scan((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (63 - lane), (int)tot), lane);
            const uint32_t suffix = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (63 - lane), (int)rev);
            // digit d: count of in-range keys with digit > d is suffix(d + 1)
            uint32_t s_j = suffix;
            int found = -1;
            uint32_t above_f = 0, h_f = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t above = s_j - h[j];  // keys with a larger digit
                if (above < remaining && s_j >= remaining) {
                    found = 4 * lane + j;
                    above_f = above;
                    h_f = h[j];
                }
                s_j = above;
            }
            // exactly one lane finds the digit
            const uint64_t who = __ballot(found >= 0);
            const int src = (int)__ffsll((unsigned long long)who) - 1;
            const int d = __shfl(found, src);
            const uint32_t ab = (uint32_t)__shfl((int)above_f, src);
            const uint32_t hd = (uint32_t)__shfl((int)h_f, src);
            if (lane == 0) {
                sh.tmp[0] = (uint32_t)d;
                sh.tmp[1] = ab;
                sh.tmp[2] = hd;
            }
        }
        __syncthreads();
        const uint32_t d = sh.tmp[0], above = sh.tmp[1], hd = sh.tmp[2];
        __syncthreads();
        remaining -= above;
        const uint32_t keep = (shift + 8 >= 32) ? 0u : (lo & (0xFFFFFFFFu << (shift + 8)));
        lo = keep | (d << shift);
        hi = lo | ((shift == 0) ? 0u : ((1u << shift) - 1u));
        if (hd == remaining) break;
    }
}

// Emit the kept ids of the LDS list (already in id order) to out[0..k).
__device__ void emit_from_list(int m, uint32_t lo, uint32_t hi, uint32_t remaining,
                               SelShared& sh, int32_t* out, float* score_out, int k_out) {
    const int tid = threadIdx.x;
    // contiguous segments of odd length: a wave's lanes then read LDS words
    // at an odd stride, which touches every bank once
    const int seg = ((m + NT - 1) / NT) | 1;
    const int e0 = min(m, tid * seg), e1 = min(m, e0 + seg);
    uint32_t n_in = 0;
    for (int e = e0; e < e1; ++e) {
        const uint32_t k = sh.key[e];
        n_in += (k >= lo && k <= hi);
    }
    uint32_t tot;
    uint32_t rank = block_excl_scan(n_in, sh, &tot);
    uint32_t n_sel = 0;
    {
        uint32_t r = rank;
        for (int e = e0; e < e1; ++e) {
            const uint32_t k = sh.key[e];
            if (k > hi) {
                ++n_sel;
            } else if (k >= lo) {
                n_sel += (r < remaining);
                ++r;
            }
        }
    }
    uint32_t pos = block_excl_scan(n_sel, sh, &tot);
    for (int e = e0; e < e1; ++e) {
        const uint32_t k = sh.key[e];
        bool take = false;
        if (k > hi) {
            take = true;
        } else if (k >= lo) {
            take = rank < remaining;
            ++rank;
        }
        if (take) {
            if (pos < (uint32_t)k_out) {
                out[pos] = sh.id[e];
                if (score_out) score_out[pos] = key_to_float(k);
            }
            ++pos;
        }
    }
}

__device__ __forceinline__ f32x4 load_row4(const float* row, int64_t e, int64_t n) {
    // row is 16-byte aligned and padded to a multiple of 4 elements
    f32x4 v = *reinterpret_cast<const f32x4*>(row + e);
#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (e + u >= n) v[u] = -INFINITY;
    return v;
}

// Exact selection directly over the row in global memory.
__device__ void select_global(const float* row, int64_t n, int k, SelShared& sh, int32_t* out,
                              float* score_out) {
    const int tid = threadIdx.x;
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int64_t e = tid; e < n; e += NT) {
        const uint32_t kk = order_key(row[e]);
        mn = min(mn, kk);
        mx = max(mx, kk);
    }
    block_minmax(mn, mx, sh);
    uint32_t lo, hi, remaining = (uint32_t)k;
    const int shift = start_range(mn, mx, lo, hi);
    refine([&](int64_t e) { return order_key(row[e]); }, n, shift, lo, hi, remaining, sh);

    // ordered emission, one 4-element group per thread per tile
    uint32_t rank_base = 0, pos_base = 0;
    for (int64_t base = 0; base < n; base += 4 * NT) {
        const int64_t e0 = base + 4 * tid;
        uint32_t kk[4];
        uint32_t n_in = 0;
        if (e0 < n) {
            const f32x4 v = load_row4(row, e0, n);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                kk[u] = (e0 + u < n) ? order_key(v[u]) : 0u;
                n_in += (e0 + u < n) && kk[u] >= lo && kk[u] <= hi;
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) kk[u] = 0u;
        }
        uint32_t tot_in;
        uint32_t rank = rank_base + block_excl_scan(n_in, sh, &tot_in);
        bool take[4];
        uint32_t n_sel = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            take[u] = false;
            if (e0 + u < n) {
                if (kk[u] > hi) {
                    take[u] = true;
                } else if (kk[u] >= lo) {
                    take[u] = rank < remaining;
                    ++rank;
                }
            }
            n_sel += take[u];
        }
        uint32_t tot_sel;
        uint32_t pos = pos_base + block_excl_scan(n_sel, sh, &tot_sel);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (take[u]) {
                if (pos < (uint32_t)k) {
                    out[pos] = (int32_t)(e0 + u);
                    if (score_out) score_out[pos] = key_to_float(kk[u]);
                }
                ++pos;
            }
        rank_base += tot_in;
        pos_base += tot_sel;
    }
}

__global__ __launch_bounds__(NT, 3) void topk_select_kernel(SelectArgs a) {
    __shared__ SelShared sh;
    const int tid = threadIdx.x;
    const int i = blockIdx.x;
    const int64_t qrow = a.row0 + i;
    const int64_t t = a.q_pos0 + qrow;
    const int64_t n = (t >> 2) < a.n_pools ? (t >> 2) : a.n_pools;
    const int k = a.k_pools;
    int32_t* out = a.idx_out + qrow * k;
    float* sout = a.score_out ? a.score_out + qrow * k : nullptr;
    const float* row = a.buf + (int64_t)i * a.ld;

    if (n <= k) {
        for (int j = tid; j < k; j += NT) {
            out[j] = j < n ? j : -1;
            if (sout) sout[j] = j < n ? row[j] : -INFINITY;
        }
        return;
    }

    int m = 0;  // list length
    if (n <= CAP) {
        // whole row into the list; rows are 16-byte aligned and padded to 4
        for (int e = 4 * tid; e < (int)n; e += 4 * NT) {
            const f32x4 v = load_row4(row, e, n);
            *reinterpret_cast<u32x4*>(&sh.key[e]) =
                u32x4{order_key(v[0]), order_key(v[1]), order_key(v[2]), order_key(v[3])};
            *reinterpret_cast<u32x4*>(&sh.id[e]) =
                u32x4{(uint32_t)e, (uint32_t)e + 1, (uint32_t)e + 2, (uint32_t)e + 3};
        }
        m = (int)n;
        __syncthreads();
    } else {
        // threshold from a sample of SAMPLE_BLOCKS cache-line blocks
        for (int s4 = tid; s4 < SAMPLE_N / 4; s4 += NT) {
            const int b = (4 * s4) / SAMPLE_LEN, u = (4 * s4) % SAMPLE_LEN;
            const int64_t start = ((int64_t)b * n / SAMPLE_BLOCKS) & ~(int64_t)(SAMPLE_LEN - 1);
            const f32x4 v = *reinterpret_cast<const f32x4*>(row + start + u);
            *reinterpret_cast<u32x4*>(&sh.key[4 * s4]) =
                u32x4{order_key(v[0]), order_key(v[1]), order_key(v[2]), order_key(v[3])};
        }
        __syncthreads();
        const float mu = (float)k * (float)SAMPLE_N / (float)n;
        uint32_t r = (uint32_t)ceilf(mu + 4.0f * sqrtf(mu) + 4.0f);
        if (r > (uint32_t)SAMPLE_N) r = SAMPLE_N;
        const uint32_t tau = sample_threshold(r, sh);  // at least r sample keys are >= tau
        __syncthreads();

        // ordered compaction of {key >= tau}: batches of VB 16-byte loads per
        // thread, the next batch in flight while the current one is compacted
        constexpr int VB = 4;
        constexpr int BATCH = 4 * NT * VB;
        f32x4 cur[VB], nxt[VB];
        auto fetch = [&](int64_t base, f32x4 (&v)[VB]) {
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                const int64_t e = base + (int64_t)(u * NT + tid) * 4;
                v[u] = e < n ? *reinterpret_cast<const f32x4*>(row + e)
                             : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            }
        };
        const float tau_f = key_to_float(tau);
        uint32_t count = 0;
        fetch(0, cur);
        for (int64_t base = 0; base < n; base += BATCH) {
            if (base + BATCH < n) fetch(base + BATCH, nxt);
            uint32_t c[VB], off[VB];
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                const int64_t e = base + (int64_t)(u * NT + tid) * 4;
                uint32_t cc = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) cc += (e + j < n) && cur[u][j] >= tau_f;
                c[u] = cc;
            }
            const uint32_t tot = block_excl_scan_slots<VB>(c, off, sh, sh.wtot);
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                if (!c[u]) continue;
                const int64_t e = base + (int64_t)(u * NT + tid) * 4;
                uint32_t pos = count + off[u];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (e + j < n && cur[u][j] >= tau_f) {
                        if (pos < (uint32_t)CAP) {
                            sh.key[pos] = order_key(cur[u][j]);
                            sh.id[pos] = (int32_t)(e + j);
                        }
                        ++pos;
                    }
                }
            }
            count += tot;
#pragma unroll
            for (int u = 0; u < VB; ++u) cur[u] = nxt[u];
        }
        __syncthreads();
        if (count < (uint32_t)k || count > (uint32_t)CAP) {
            select_global(row, n, k, sh, out, sout);
            return;
        }
        m = (int)count;
    }

    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int e = tid; e < m; e += NT) {
        mn = min(mn, sh.key[e]);
        mx = max(mx, sh.key[e]);
    }
    block_minmax(mn, mx, sh);
    uint32_t lo = mn, hi = mx, remaining = (uint32_t)k;
    refine256(m, lo, hi, remaining, sh);
    emit_from_list(m, lo, hi, remaining, sh, out, sout, k);
}

}  // namespace

hipError_t launch_topk_select(const SelectArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    topk_select_kernel<<<dim3((unsigned)a.rows), NT, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
