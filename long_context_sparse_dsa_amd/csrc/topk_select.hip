// Per-query top-k pool selection over one chunk's fp32 score rows.
//
// SkyRL blog "Scaling Training to 1M Token Context on GLM-5.3-Flash",
// section "DeepSeek Sparse Attention (DSA) Optimizations": each query keeps
// its best pools (512 pools = 2048 tokens); section "Over Time: Chunking":
// pools are scored and selected a chunk of queries at a time; section
// "Across GPUs: Sharding": the kept pool ids are int32.
//
// Rule: keep the k largest scores among the n(t) eligible pools, ties broken
// towards the lower pool id; emit the ids in ascending order, padded with -1
// when n(t) < k.  Exact and deterministic: every decision is taken on the
// 32-bit order key of an fp32 value (larger float <=> larger key), with
// integer counting only.
//
// Approximate rows (bf16 indexer): the row holds s~_p, the score taken with
// the bf16 pooled key hi_p alone, and the selection is made on the full score
// s_p (hi_p plus the E4M3 correction lo_p) that the scoring kernel would give
// with the correction.  Every |s~_p - s_p| <= delta_p = A * mu_p (A per query,
// mu_p per pool; see the pooling and packing kernels), so with
//   l_p = s~_p - delta_p,  u_p = s~_p + delta_p,
//   L = k-th largest l,    U = k-th largest u,
// the k-th largest full score lies in [L, U]: pools with l_p > U are kept for
// certain, pools with u_p < L are dropped for certain, and only the pools in
// between (the band, typically about k of them) are rescored, by the same
// MFMA sequence the scoring kernel uses with the correction, so the result is
// bit for bit the selection over the full scores.  Pools with delta_p = 0
// (zero pools only) already hold their full score, +0.  Final rows (fp8 indexer) are the case
// delta = 0: the band is the set of keys equal to the k-th.
//
// One workgroup (4 waves) per query row:
//   n <= k       every eligible pool;
//   n <= WHOLE   the whole row goes to an LDS list (id, score, delta);
//                WHOLE is the list's capacity for approximate rows (3072
//                or 4096 pools, see CAP_SHORT), 2048 for final ones
//   n >  WHOLE   a sample of the row (blocks of 16 contiguous pools: 128 for
//                bounded rows up to 64k pools, 384 beyond, half that for final
//                rows) gives a threshold tau on the l keys; one coalesced pass keeps
//                {u >= tau} in the LDS list (at most its capacity), in
//                id order.  The list then holds every pool that can matter
//                when at least k of its l keys are >= tau and it fits;
//                otherwise the row is handled in
//                global memory (slow path, still exact): L' and U' from the
//                same histograms over the row, the band rescored in place,
//                and an exact radix selection over the row.
// On a list, safe bounds L' <= L and U' >= U come from 256-bin histograms
// linear in value, and the kept band members from a radix selection over
// their full scores.
#include <math.h>
#include <stddef.h>

#include "common.h"
#include "internal.h"

namespace dsa {

namespace {

constexpr int NT = 256;
// list capacity: rows of up to LONG_ROW pools use a 3072-entry list, whose
// 38 KiB of LDS lets 4 workgroups share a CU, where the kernel then fits 128
// VGPRs (D_I = 64, or 96 with at least 16 heads); longer rows, whose sampled
// lists are larger, and the other shapes a 4096-entry list (3 per CU)
constexpr int CAP = 4096;
constexpr int CAP_SHORT = 3072;
constexpr int SAMPLE_LEN = 32;  // one 128-byte line of fp32 scores per block
// sample blocks of SAMPLE_LEN: more for long rows, where k is a smaller
// fraction of the row, and twice as many for bounded rows, whose threshold
// takes a wider margin (the sample lives in the three list arrays)
constexpr int SAMPLE_BLOCKS_SHORT = 64;
constexpr int SAMPLE_BLOCKS_LONG = 192;
constexpr int64_t LONG_ROW = 65536;
// rows up to this many pools go whole to the list (bounded rows: the list's
// capacity), longer ones take the sample; the sample's blocks then lie
// inside the row and apart
constexpr int WHOLE_FINAL = 2048;
static_assert(WHOLE_FINAL <= CAP_SHORT, "a whole row must fit the list");
static_assert(SAMPLE_BLOCKS_SHORT * SAMPLE_LEN <= CAP_SHORT, "sample blocks overlap");
static_assert(SAMPLE_BLOCKS_SHORT / 2 * SAMPLE_LEN <= WHOLE_FINAL, "sample blocks overlap");
static_assert(SAMPLE_BLOCKS_LONG * SAMPLE_LEN <= 3 * CAP, "the sample lives in the list");
static_assert(SAMPLE_BLOCKS_SHORT * SAMPLE_LEN <= 3 * CAP_SHORT, "the sample lives in the list");

// list entry tags: id in bits 0-28 (ids < 2^29), class in bits 29-30, and
// bit 31 set when the entry's full score must be computed
constexpr uint32_t ID_MASK = (1u << 29) - 1u;
constexpr uint32_t C_OUT = 0u, C_IN = 1u, C_BAND = 2u;
constexpr uint32_t RESCORE = 1u << 31;
__device__ __forceinline__ uint32_t cls_of(uint32_t t) { return (t >> 29) & 3u; }

// The workgroup's LDS, for a list of LCAP entries.  d is last: rows of final
// scores never touch it, and their kernel is launched without it (fewer
// bytes, more workgroups per CU).
template <int LCAP>
struct SelSharedT {
    static constexpr int CAP = LCAP;
    uint32_t hist[512];
    float w[32];  // head weights of the row's query tile (approximate rows)
    uint32_t tmp[8];
    uint32_t wtot[8 * (NT / 64)];  // per-slot wave totals of block_excl_scan_slots (<= 8 slots)
    union {
        struct {
            alignas(16) uint32_t idc[LCAP];  // tagged pool ids
            alignas(16) float s[LCAP];       // scores: approximate, then full where rescored
            alignas(16) float d[LCAP];       // bounds delta; then the entries to rescore
        };
        alignas(16) uint32_t sample[3 * LCAP];  // sample keys, before the list is built
    };
};
using SelShared = SelSharedT<CAP>;
using SelSharedShort = SelSharedT<CAP_SHORT>;
template <int LCAP>
constexpr size_t lds_bounded() { return sizeof(SelSharedT<LCAP>); }
template <int LCAP>
constexpr size_t lds_final() { return sizeof(SelSharedT<LCAP>) - LCAP * sizeof(float); }
static_assert(offsetof(SelShared, d) == lds_final<CAP>(), "d must be the last member");
static_assert(offsetof(SelSharedShort, d) == lds_final<CAP_SHORT>(), "d must be the last member");
static_assert(lds_bounded<CAP>() <= 64 * 1024, "dynamic LDS beyond 64 KiB needs an opt-in");
static_assert(4 * lds_bounded<CAP_SHORT>() <= 160 * 1024, "4 short-list workgroups per CU");
// the sample of a row of final scores lies below d
static_assert(SAMPLE_BLOCKS_LONG / 2 * SAMPLE_LEN <= 2 * CAP, "final-row sample beyond idc and s");

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

// Exclusive prefix over the workgroup; *total receives the sum.
template <class SH>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, SH& sh, uint32_t* total) {
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
template <int VB, int NW, class SH>
__device__ __forceinline__ uint32_t block_excl_scan_slots(const uint32_t (&c)[VB],
                                                          uint32_t (&off)[VB], SH& sh,
                                                          uint32_t (&wtot)[NW]) {
    static_assert(VB * (NT / 64) <= NW, "one wave total per slot and wave");
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

template <class SH>
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, SH& sh) {
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


// Sum over the workgroup.
template <class SH>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, SH& sh) {
    uint32_t tot;
    (void)block_excl_scan(v, sh, &tot);
    return tot;
}

// One wave's search of a 256-bin digit histogram (lane l holds bins
// 4l .. 4l+3): the digit d whose in-range keys reach `remaining` when counted
// from the top, with the count of keys above it and in it.  Exactly one lane
// finds it when at least `remaining` keys are in range.
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t remaining, uint32_t& dg,
                                           uint32_t& above_out, uint32_t& in_out) {
    const int lane = threadIdx.x & 63;
    uint32_t h[4], tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = hist[4 * lane + j];
        tot += h[j];
    }
    const uint32_t rev = wave_incl_scan((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (63 - lane), (int)tot), lane);
    const uint32_t suffix = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (63 - lane), (int)rev);
    // digit d: the in-range keys with a digit above d number suffix(d + 1)
    uint32_t s_j = suffix;
    int found = -1;
    uint32_t above_f = 0, h_f = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t above = s_j - h[j];
        if (above < remaining && s_j >= remaining) {
            found = 4 * lane + j;
            above_f = above;
            h_f = h[j];
        }
        s_j = above;
    }
    const uint64_t who = __ballot(found >= 0);
    const int src = who ? (int)__ffsll((unsigned long long)who) - 1 : 0;
    dg = (uint32_t)__shfl(found, src);
    above_out = (uint32_t)__shfl((int)above_f, src);
    in_out = (uint32_t)__shfl((int)h_f, src);
}

// Digit shifts: the first 8-bit digit ends at the highest bit where lo and
// hi differ (so the keys of one row, which share their top bits, spread over
// all 256 bins), then 8 bits lower each pass, the last one clipped at bit 0
// (its bins above the remaining bits are then constant).  -1: done.
__device__ __forceinline__ int first_shift(uint32_t lo, uint32_t hi) {
    const uint32_t diff = lo ^ hi;
    if (diff == 0) return -1;
    const int top = 31 - __clz(diff);
    return top >= 7 ? top - 7 : 0;
}
__device__ __forceinline__ int next_shift(int shift) {
    return shift >= 8 ? shift - 8 : (shift > 0 ? 0 : -1);
}

// Narrow [lo, hi] to digit dg at `shift` (the bits of lo above the digit
// are shared by every in-range key).
__device__ __forceinline__ void narrow(uint32_t& lo, uint32_t& hi, int shift, uint32_t dg) {
    const uint32_t keep = (shift + 8 >= 32) ? 0u : (lo & (0xFFFFFFFFu << (shift + 8)));
    lo = keep | (dg << shift);
    hi = lo | ((shift == 0) ? 0u : ((1u << shift) - 1u));
}

// Radix-256 narrowing over the keys of the member elements e < n of any
// source: key_at(e, &key) returns whether e is a member.  Precondition: at
// least `remaining` member keys lie in [lo, hi] and every member key above hi
// is kept.  On return the kept set is {key > hi} plus the first `remaining`
// member keys in [lo, hi] in element order.  With to_end the range is
// narrowed to a single key (lo == hi, the k-th largest); otherwise it stops
// as soon as every in-range key is kept.  Digits are counted with LDS
// atomics (integer, so the counts do not depend on their order) and found by
// one wave's suffix scan.
template <class KeyAt, class SH>
__device__ void radix_narrow(int64_t n, KeyAt key_at, uint32_t& lo, uint32_t& hi,
                             uint32_t& remaining, bool to_end, SH& sh) {
    const int tid = threadIdx.x, wave = tid >> 6;
    uint32_t* hist = sh.hist;
    for (int shift = first_shift(lo, hi); shift >= 0 && lo != hi; shift = next_shift(shift)) {
        for (int b = tid; b < 256; b += NT) hist[b] = 0;
        __syncthreads();
        for (int64_t e = tid; e < n; e += NT) {
            uint32_t k;
            if (key_at(e, k) && k >= lo && k <= hi) atomicAdd(&hist[(k >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            uint32_t dg, ab, hd;
            find_digit(hist, remaining, dg, ab, hd);
            if ((tid & 63) == 0) {
                sh.tmp[0] = dg;
                sh.tmp[1] = ab;
                sh.tmp[2] = hd;
            }
        }
        __syncthreads();
        const uint32_t dg = sh.tmp[0], above = sh.tmp[1], hd = sh.tmp[2];
        __syncthreads();
        remaining -= above;
        narrow(lo, hi, shift, dg);
        if (!to_end && hd == remaining) break;
    }
}

// The highest bin b of a 256-bin histogram (one wave, lane l holding bins
// 4l .. 4l+3) whose suffix sum (bins b .. 255) reaches r; -1 if none.
__device__ __forceinline__ int top_bin(const uint32_t* hist, uint32_t r) {
    const int lane = threadIdx.x & 63;
    uint32_t h[4], tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = hist[4 * lane + j];
        tot += h[j];
    }
    // inclusive scan over lanes in reverse order gives the suffix sums
    const uint32_t rev = wave_incl_scan((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (63 - lane), (int)tot), lane);
    const uint32_t suffix = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (63 - lane), (int)rev);
    uint32_t s_j = suffix;
    int found = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (s_j >= r) found = 4 * lane + j;
        s_j -= h[j];
    }
    const uint32_t best = wave_incl_scan_op(found < 0 ? 0u : (uint32_t)found + 1u, 0u, MaxOp{});
    return (int)__shfl((int)best, 63) - 1;
}

// Bin of a value in a 256-bin histogram linear in value from vmin (scale =
// 256 / range); monotone non-decreasing in the value.
__device__ __forceinline__ int value_bin(float x, float vmin, float scale) {
    const float b = (x - vmin) * scale;
    return b >= 255.0f ? 255 : (b > 0.0f ? (int)b : 0);
}

// Safe bounds on the k-th largest l and u keys of the list (at least k
// entries): Lk <= the k-th largest l and Uk >= the k-th largest u.  One
// sweep for the value range, one filling a 256-bin histogram of each,
// linear in value, and one for the smallest l in the bins that hold the k
// largest l and the largest u in the bins up to the one holding the k-th
// largest u.  The bins widen the band by at most one bin each way.
template <class Key2At, class SH>
__device__ void band_bounds(int m, Key2At key2_at, uint32_t k, uint32_t& Lk, uint32_t& Uk,
                            SH& sh) {
    const int tid = threadIdx.x, wave = tid >> 6;
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int e = tid; e < m; e += NT) {
        uint32_t lk, uk;
        key2_at(e, lk, uk);
        mn = min(mn, lk);
        mx = max(mx, uk);
    }
    block_minmax(mn, mx, sh);
    const float vmin = key_to_float(mn), vmax = key_to_float(mx);
    const float scale = 256.0f / (vmax - vmin);
    for (int b = tid; b < 512; b += NT) sh.hist[b] = 0;
    __syncthreads();
    for (int e = tid; e < m; e += NT) {
        uint32_t lk, uk;
        key2_at(e, lk, uk);
        atomicAdd(&sh.hist[value_bin(key_to_float(lk), vmin, scale)], 1u);
        atomicAdd(&sh.hist[256 + value_bin(key_to_float(uk), vmin, scale)], 1u);
    }
    __syncthreads();
    if (wave < 2) {
        const int b = top_bin(sh.hist + 256 * wave, k);
        if ((tid & 63) == 0) sh.tmp[wave] = (uint32_t)b;
    }
    __syncthreads();
    const int bl = (int)sh.tmp[0], bu = (int)sh.tmp[1];
    __syncthreads();
    uint32_t lmin = 0xFFFFFFFFu, umax = 0u;
    for (int e = tid; e < m; e += NT) {
        uint32_t lk, uk;
        key2_at(e, lk, uk);
        if (value_bin(key_to_float(lk), vmin, scale) >= bl) lmin = min(lmin, lk);
        if (value_bin(key_to_float(uk), vmin, scale) <= bu) umax = max(umax, uk);
    }
    block_minmax(lmin, umax, sh);
    Lk = lmin;
    Uk = umax;
}

// Smallest and largest member key (min = 0xFFFFFFFF, max = 0 when none).
template <class KeyAt, class SH>
__device__ void member_minmax(int64_t n, KeyAt key_at, uint32_t& mn, uint32_t& mx, SH& sh) {
    mn = 0xFFFFFFFFu;
    mx = 0u;
    for (int64_t e = threadIdx.x; e < n; e += NT) {
        uint32_t k;
        if (key_at(e, k)) {
            mn = min(mn, k);
            mx = max(mx, k);
        }
    }
    block_minmax(mn, mx, sh);
}

// A key tau with at least r of the ns sample keys (sh.sample) >= tau,
// and not many more: a 256-bin histogram linear in the sampled values (not
// in their bit patterns, which would lump the upper tail into one bin) gives
// the highest bin b whose suffix holds r keys; tau is the smallest sample key
// in bins >= b.
template <class SH>
__device__ uint32_t sample_threshold(int ns, uint32_t r, SH& sh) {
    constexpr int NBIN = 256;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int e = tid; e < ns; e += NT) {
        mn = min(mn, sh.sample[e]);
        mx = max(mx, sh.sample[e]);
    }
    block_minmax(mn, mx, sh);
    if (mn == mx) return mn;
    const float vmin = key_to_float(mn), vmax = key_to_float(mx);
    const float scale = (float)NBIN / (vmax - vmin);
    auto bin_of = [&](uint32_t key) {
        const float b = (key_to_float(key) - vmin) * scale;
        return b >= (float)(NBIN - 1) ? NBIN - 1 : (b > 0.0f ? (int)b : 0);
    };
    uint32_t* hist = sh.hist;
    for (int b = tid; b < NBIN; b += NT) hist[b] = 0;
    __syncthreads();
    for (int e = tid; e < ns; e += NT) atomicAdd(&hist[bin_of(sh.sample[e])], 1u);
    __syncthreads();
    if (wave == 0) {
        // lane l holds bins 4l .. 4l+3; suffix sums from the top bin down
        uint32_t h[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[j] = hist[4 * lane + j];
            tot += h[j];
        }
        const uint32_t rev = wave_incl_scan((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (63 - lane), (int)tot), lane);
        const uint32_t suffix = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (63 - lane), (int)rev);
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
    for (int e = tid; e < ns; e += NT) {
        const uint32_t key = sh.sample[e];
        if (bin_of(key) >= b_min) kmin = min(kmin, key);
    }
    block_minmax(kmin, dummy, sh);
    return kmin;
}

// Ordered compaction: entries with flag(e) for e < n in element order go to
// slots [0, count) through put(slot, e); returns count.  Thread tid takes a
// contiguous segment of odd length, so that a wave's LDS reads at that
// stride touch every bank once.
template <class Flag, class Put, class SH>
__device__ uint32_t compact(int n, Flag flag, Put put, SH& sh) {
    const int tid = threadIdx.x;
    const int seg = ((n + NT - 1) / NT) | 1;
    const int e0 = min(n, tid * seg), e1 = min(n, e0 + seg);
    uint32_t c = 0;
    for (int e = e0; e < e1; ++e) c += flag(e);
    uint32_t tot;
    uint32_t pos = block_excl_scan(c, sh, &tot);
    for (int e = e0; e < e1; ++e)
        if (flag(e)) put(pos++, e);
    return tot;
}

// ---------------------------------------------------------------- rescoring

// The full score of pools for one query, with the scoring kernel's MFMA
// sequence and epilogue (so that the value is bit for bit the one the
// scoring kernel stores when it includes the correction): per lane
// (col = lane % 32, half = lane / 32) the A operand is row col of the
// query's packed tile, the B operand pool cand[col]; 8 (d / 16) bf16 MFMAs
// with hi, then the scaled E4M3 MFMAs with lo, into one 32 x 32 accumulator;
// then per query sum_h w_h relu(acc), the rows of the query summed in the
// scoring kernel's order.  One wave scores 32 pools at a time.  Both
// operands are loaded for every block (the tile stays in cache), so that
// nothing is live across blocks and every load of a block is in flight
// before its first MFMA: a gather costs one memory latency, not one per
// MFMA.
template <int HI, int DI, bool SPLIT = false>
struct Rescorer {
    static constexpr QueryTileGeom G = query_tile_geom(DI);
    static constexpr int QPT = 32 / HI;
    static constexpr int NSB = DI / 16;
    static constexpr int NSF = (DI + 63) / 64;
    const uint8_t* tile;
    int qi;

    __device__ void init(const uint8_t* tiles, int64_t i) {
        tile = tiles + (i / QPT) * G.tb;
        qi = (int)(i % QPT);
    }

    // the 32 head weights of row i's query tile
    static __device__ const float* weights(const uint8_t* tiles, int64_t i) {
        return reinterpret_cast<const float*>(tiles + (i / QPT) * G.tb + G.qb);
    }

    // Score of pool p (this lane's column); the value is valid on lane
    // owner() of each column (col or col + 32).  w: the tile's 32 head
    // weights, staged in LDS.
    __device__ float score(const uint16_t* khi, const uint8_t* klo, const uint8_t* klo_scale,
                           int64_t p, const float* w) const {
        const int lane = threadIdx.x & 63, col = lane & 31, half = lane >> 5;
        // SPLIT: half the bf16 steps' operands (and the fp8 ones) load first,
        // the other half while their MFMAs run (fewer registers live)
        constexpr int H1 = SPLIT ? NSB / 2 : NSB;
        bf16x8 af[NSB], bhi[NSB];
        i32x8 af8[NSF], blo[NSF];
#pragma unroll
        for (int s = 0; s < H1; ++s) {
            af[s] = as_bf16x8(ldg16(tile + tile_bf16_piece(G, col, 2 * s + half)));
            bhi[s] = as_bf16x8(ldg16(khi + p * DI + 16 * s + 8 * half));
        }
#pragma unroll
        for (int s = 0; s < NSF; ++s) {
            u32x4 a0 = {0u, 0u, 0u, 0u}, a1 = {0u, 0u, 0u, 0u};
            u32x4 b0 = {0u, 0u, 0u, 0u}, b1 = {0u, 0u, 0u, 0u};
            const int d0 = 64 * s + 32 * half;
            if (d0 < DI) {
                a0 = ldg16(tile + tile_fp8_piece(G, col, 4 * s + 2 * half));
                a1 = ldg16(tile + tile_fp8_piece(G, col, 4 * s + 2 * half + 1));
                b0 = ldg16(klo + p * DI + d0);
                b1 = ldg16(klo + p * DI + d0 + 16);
            }
            af8[s] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                           (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            blo[s] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                           (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
        }
        const int qsc = (int)tile[G.qb + 128 + col];
        const int bsc = (int)klo_scale[p];
        f32x16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
        if constexpr (SPLIT) {
#pragma unroll
            for (int s = 0; s < H1; ++s)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s], bhi[s], acc, 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 2 * H1 + 4 * NSF + 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, H1, 0);
#pragma unroll
            for (int s = H1; s < NSB; ++s) {
                af[s] = as_bf16x8(ldg16(tile + tile_bf16_piece(G, col, 2 * s + half)));
                bhi[s] = as_bf16x8(ldg16(khi + p * DI + 16 * s + 8 * half));
            }
        }
        // (the same MFMA sequence either way: the score is bit for bit the
        // scoring kernel's)
#pragma unroll
        for (int s = SPLIT ? H1 : 0; s < NSB; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s], bhi[s], acc, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < NSF; ++s)
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af8[s], blo[s], acc, 0, 0, 0, qsc,
                                                                  0, bsc);
        // every load first, then the MFMAs
        __builtin_amdgcn_sched_group_barrier(0x020, 2 * (NSB - (SPLIT ? H1 : 0)) + (SPLIT ? 0 : 4 * NSF + 2), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NSB - (SPLIT ? H1 : 0) + NSF, 0);
        float part[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(w + 8 * g4 + 4 * half);
            float sacc = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc += w4[i] * relu(acc[4 * g4 + i]);
            part[g4] = sacc;
        }
        // (selects, not an indexed register array)
        auto pick = [&](int j) {
            return j == 0 ? part[0] : j == 1 ? part[1] : j == 2 ? part[2] : part[3];
        };
        float v;
        if constexpr (HI == 4) {
            // rows 8*g4 + 4*half + i are the 4 heads of query 2*g4 + half
            v = pick(qi >> 1);
        } else if constexpr (HI == 32) {
            v = add_halves((part[0] + part[1]) + (part[2] + part[3]));
        } else if constexpr (HI == 16) {
            v = add_halves(qi == 0 ? part[0] + part[1] : part[2] + part[3]);
        } else {
            v = add_halves(pick(qi));
        }
        return canonical_zero(v);
    }

    // the lane that holds column col's value
    __device__ int owner(int col) const { return HI == 4 ? col + 32 * (qi & 1) : col; }
};

// Rescore the entries j < nr whose tag tag_of(j) has the RESCORE bit: the
// tag's id bits name the pool, and its full score goes to put(j, value).
// The 4 waves take blocks of 32 entries in turn and skip blocks with nothing
// to rescore.  Called by the whole workgroup after a barrier that follows
// the staging of the tile's head weights in sh.w at the kernel's start.
template <int HI, int DI, class TagOf, class Put, class SH>
__device__ void rescore(uint32_t nr, TagOf tag_of, Put put, const SelectArgs& a, int64_t i,
                        SH& sh) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 31;
    // the short-list kernel runs 4 workgroups per CU: operands in two rounds
    Rescorer<HI, DI, SH::CAP == CAP_SHORT> r;
    r.init(a.tiles, i);
    const float* w = sh.w;
    const uint32_t nblk = (nr + 31) / 32;
    if ((uint32_t)wave >= nblk) return;
    const int own = r.owner(col);
    for (uint32_t b = wave; b < nblk; b += 4) {
        const uint32_t j = 32 * b + col;
        // columns past the end score entry 32 b (any valid pool) and are dropped
        const uint32_t t = tag_of(j < nr ? j : 32 * b);
        const bool keep = j < nr && (t & RESCORE) != 0u;
        if (__ballot(keep) == 0) continue;
        const float v = r.score(a.khi, a.klo, a.klo_scale, (int64_t)(t & ID_MASK), w);
        if (lane == own && keep) put(j, v);
    }
}

// ---------------------------------------------------------------- emission

// Emit the kept ids of the list (in id order) to out[0..k): every C_IN
// entry, and the C_BAND entries with key > hi plus the first `remaining`
// with key in [lo, hi].  ALL_BAND: every entry is a band entry (untagged).
template <bool ALL_BAND, class SH>
__device__ void emit_list(int m, uint32_t lo, uint32_t hi, uint32_t remaining, SH& sh,
                          int32_t* out, float* score_out, int k_out) {
    const int tid = threadIdx.x;
    const int seg = ((m + NT - 1) / NT) | 1;
    const int e0 = min(m, tid * seg), e1 = min(m, e0 + seg);
    uint32_t n_in = 0;
    for (int e = e0; e < e1; ++e) {
        const uint32_t k = order_key(sh.s[e]);
        n_in += (ALL_BAND || cls_of(sh.idc[e]) == C_BAND) && k >= lo && k <= hi;
    }
    uint32_t tot;
    const uint32_t rank0 = block_excl_scan(n_in, sh, &tot);
    auto take = [&](int e, uint32_t& r) {
        const uint32_t c = ALL_BAND ? C_BAND : cls_of(sh.idc[e]);
        if (c == C_IN) return true;
        if (c != C_BAND) return false;
        const uint32_t k = order_key(sh.s[e]);
        if (k > hi) return true;
        if (k < lo) return false;
        return r++ < remaining;
    };
    uint32_t n_sel = 0;
    {
        uint32_t r = rank0;
        for (int e = e0; e < e1; ++e) n_sel += take(e, r);
    }
    uint32_t pos = block_excl_scan(n_sel, sh, &tot);
    uint32_t r = rank0;
    for (int e = e0; e < e1; ++e) {
        if (take(e, r)) {
            if (pos < (uint32_t)k_out) {
                out[pos] = (int32_t)(sh.idc[e] & ID_MASK);
                if (score_out) score_out[pos] = sh.s[e];
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

// Exact selection directly over a row of final scores in global memory.
template <class SH>
__device__ void select_row(const float* row, int64_t n, int k, SH& sh, int32_t* out,
                           float* score_out) {
    const int tid = threadIdx.x;
    auto key_at = [&](int64_t e, uint32_t& key) {
        key = order_key(row[e]);
        return true;
    };
    uint32_t lo, hi, remaining = (uint32_t)k;
    member_minmax(n, key_at, lo, hi, sh);
    radix_narrow(n, key_at, lo, hi, remaining, false, sh);

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
        bool tk[4];
        uint32_t n_sel = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            tk[u] = false;
            if (e0 + u < n) {
                if (kk[u] > hi) {
                    tk[u] = true;
                } else if (kk[u] >= lo) {
                    tk[u] = rank < remaining;
                    ++rank;
                }
            }
            n_sel += tk[u];
        }
        uint32_t tot_sel;
        uint32_t pos = pos_base + block_excl_scan(n_sel, sh, &tot_sel);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (tk[u]) {
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

// The half-width of pool p's score interval for a query with bound factors
// A: A1 m1 + A2 m2 (the chunk buffer holds the interval's upper end).
__device__ __forceinline__ float bound_delta(f32x2 A, const float* mu, int64_t p) {
    const f32x2 m = *reinterpret_cast<const f32x2*>(mu + 2 * p);
    return fmaf(A[0], m[0], A[1] * m[1]);
}

// Slow path for an approximate row that does not fit the list: L and U by
// radix over the row, every pool that needs its full score rescored in place
// (the band; with score_out also the certain ones), then the exact selection
// over the row.  Pools outside the band keep their approximate scores, which
// lie strictly above U (kept) or below L (dropped) and so cannot change the
// set.
template <int HI, int DI, class SH>
__device__ void select_row_bounded(const SelectArgs& a, int64_t i, float* row, int64_t n, f32x2 A,
                                   SH& sh, int32_t* out, float* score_out) {
    const int tid = threadIdx.x;
    uint32_t Lk, Uk;
    band_bounds((int)n, [&](int64_t e, uint32_t& lk, uint32_t& uk) {
        const float x = row[e];
        lk = order_key(x - 2.0f * bound_delta(A, a.mu, e));
        uk = order_key(x);
    }, (uint32_t)a.k_pools, Lk, Uk, sh);
    uint32_t* ids = reinterpret_cast<uint32_t*>(sh.d);
    for (int64_t base = 0; base < n; base += SH::CAP) {
        const int w = (int)min((int64_t)SH::CAP, n - base);
        // this window's pools in LDS first: the rescoring below writes the row
        for (int e = tid; e < w; e += NT) {
            const float x = row[base + e], dl = bound_delta(A, a.mu, base + e);
            const uint32_t lk = order_key(x - 2.0f * dl), uk = order_key(x);
            const bool band = uk >= Lk && lk <= Uk;
            const bool in = lk > Uk;
            sh.idc[e] = (dl > 0.0f && (band || (in && score_out))) ? 1u : 0u;
        }
        __syncthreads();
        const uint32_t nr = compact(w, [&](int e) { return sh.idc[e] != 0u; },
                                    [&](uint32_t slot, int e) { ids[slot] = (uint32_t)(base + e); },
                                    sh);
        __syncthreads();
        rescore<HI, DI>(nr, [&](uint32_t j) { return ids[j] | RESCORE; },
                        [&](uint32_t j, float v) { row[ids[j]] = v; }, a, i, sh);
        __threadfence_block();
        __syncthreads();
    }
    select_row(row, n, a.k_pools, sh, out, score_out);
}

template <int HI, int DI, bool BOUNDS, int LCAP>
// Approximate rows: 4 workgroups per CU with the short list (38 KiB of LDS,
// 128 VGPRs), 3 with the long one (LDS and registers).  Rows of final scores
// need neither the bounds array nor the rescoring: 4 workgroups per CU.
__global__ __launch_bounds__(NT, BOUNDS && LCAP == CAP ? 3 : 4) void topk_select_kernel(SelectArgs a) {
    using SH = SelSharedT<LCAP>;
    extern __shared__ __align__(16) uint8_t sel_lds[];
    SH& sh = *reinterpret_cast<SH*>(sel_lds);
    const int tid = threadIdx.x;
    const int i = blockIdx.x;
    const int64_t qrow = a.row0 + i;
    const int64_t t = a.q_pos0 + qrow;
    const int64_t n = (t >> 2) < a.n_pools ? (t >> 2) : a.n_pools;
    const int k = a.k_pools;
    int32_t* out = a.idx_out + qrow * k;
    float* sout = a.score_out ? a.score_out + qrow * k : nullptr;
    float* row = a.buf + (int64_t)i * a.ld;
    const f32x2 A = BOUNDS ? *reinterpret_cast<const f32x2*>(a.qbound + 2 * i) : f32x2{0.0f, 0.0f};
    auto delta = [&](int64_t p) { return BOUNDS ? bound_delta(A, a.mu, p) : 0.0f; };
    // read by the rescoring, always after at least one barrier
    if (BOUNDS && tid < 32) sh.w[tid] = Rescorer<HI, DI>::weights(a.tiles, i)[tid];

    if (n <= k) {
        for (int j = tid; j < k; j += NT) out[j] = j < n ? j : -1;
        if (!sout) return;
        // the scores of every eligible pool, rescored where they are approximate
        for (int j = tid; j < (int)n; j += NT) {
            sh.s[j] = row[j];
            sh.idc[j] = (BOUNDS && delta(j) > 0.0f) ? 1u : 0u;
        }
        __syncthreads();
        if constexpr (BOUNDS) {
            uint32_t* ids = reinterpret_cast<uint32_t*>(sh.d);
            const uint32_t nr = compact((int)n, [&](int e) { return sh.idc[e] != 0u; },
                                        [&](uint32_t slot, int e) { ids[slot] = (uint32_t)e; }, sh);
            __syncthreads();
            rescore<HI, DI>(nr, [&](uint32_t j) { return ids[j] | RESCORE; },
                            [&](uint32_t j, float v) { sh.s[ids[j]] = v; }, a, i, sh);
            __syncthreads();
        }
        for (int j = tid; j < k; j += NT) sout[j] = j < n ? sh.s[j] : -INFINITY;
        return;
    }

    int m = 0;  // list length
    if (n <= (BOUNDS ? LCAP : WHOLE_FINAL)) {
        // the whole row; rows are 16-byte aligned and padded to 4
        for (int e = 4 * tid; e < (int)n; e += 4 * NT) {
            const f32x4 v = load_row4(row, e, n);
            *reinterpret_cast<f32x4*>(&sh.s[e]) = v;
            *reinterpret_cast<u32x4*>(&sh.idc[e]) =
                u32x4{(uint32_t)e, (uint32_t)e + 1, (uint32_t)e + 2, (uint32_t)e + 3};
            if constexpr (BOUNDS) {
#pragma unroll
                for (int u = 0; u < 4; ++u) sh.d[e + u] = e + u < n ? delta(e + u) : 0.0f;
            }
        }
        m = (int)n;
        __syncthreads();
    } else {
        // threshold on the l keys from nb blocks of SAMPLE_LEN
        // (the short list's launcher keeps its rows within LONG_ROW pools)
        const int nb = (LCAP == CAP && n > LONG_ROW ? SAMPLE_BLOCKS_LONG : SAMPLE_BLOCKS_SHORT) /
                       (BOUNDS ? 1 : 2);
        const int ns = nb * SAMPLE_LEN;
        // b n / nb for the four block counts (a uniform branch; constant
        // divisors become shifts and multiplications)
        auto blk_start = [&](int64_t bn) -> int64_t {
            switch (nb) {
                case SAMPLE_BLOCKS_LONG: return bn / SAMPLE_BLOCKS_LONG;
                case SAMPLE_BLOCKS_LONG / 2: return bn / (SAMPLE_BLOCKS_LONG / 2);
                case SAMPLE_BLOCKS_SHORT: return bn / SAMPLE_BLOCKS_SHORT;
                default: return bn / (SAMPLE_BLOCKS_SHORT / 2);
            }
        };
        // SU 16-byte pieces per thread in flight at once (ns / 4 is a
        // multiple of NT; the blocks lie inside the row)
        constexpr int SU = LCAP == CAP ? 6 : 4;
        for (int s0 = 0; s0 < ns / 4; s0 += SU * NT) {
            f32x4 v[SU], mv[SU][2];
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int s4 = s0 + u * NT + tid;
                if (s4 >= ns / 4) continue;
                const int b = (4 * s4) / SAMPLE_LEN, o = (4 * s4) % SAMPLE_LEN;
                const int64_t e = (blk_start((int64_t)b * n) & ~(int64_t)(SAMPLE_LEN - 1)) + o;
                v[u] = *reinterpret_cast<const f32x4*>(row + e);
                if constexpr (BOUNDS) {
                    mv[u][0] = *reinterpret_cast<const f32x4*>(a.mu + 2 * e);
                    mv[u][1] = *reinterpret_cast<const f32x4*>(a.mu + 2 * e + 4);
                }
            }
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int s4 = s0 + u * NT + tid;
                if (s4 >= ns / 4) continue;
                u32x4 kk;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float dl = BOUNDS ? fmaf(A[0], mv[u][j >> 1][2 * (j & 1)],
                                                   A[1] * mv[u][j >> 1][2 * (j & 1) + 1])
                                            : 0.0f;
                    kk[j] = order_key(v[u][j] - 2.0f * dl);
                }
                *reinterpret_cast<u32x4*>(&sh.sample[4 * s4]) = kk;
            }
        }
        __syncthreads();
        // expected sample keys above the k-th; the margin of a bounded row
        // also covers the l keys' shift below the scores
        const float mu = (float)k * (float)ns / (float)n;
        uint32_t r = (uint32_t)ceilf(BOUNDS ? mu + 5.0f * sqrtf(mu) + 8.0f : mu + 4.0f * sqrtf(mu) + 4.0f);
        if (r > (uint32_t)ns) r = ns;
        // the first compaction batch does not depend on tau: its loads are
        // in flight while the threshold is found
        constexpr int VB = 8;
        constexpr int BATCH = 4 * NT * VB;
        const int64_t last = (n - 1) & ~(int64_t)3;
        f32x4 v[VB];
        auto load_batch = [&](int64_t base) {
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                const int64_t e = base + (int64_t)(u * NT + tid) * 4;
                v[u] = *reinterpret_cast<const f32x4*>(row + (e < n ? e : last));
            }
        };
        load_batch(0);
        const uint32_t tau = sample_threshold(ns, r, sh);  // at least r sample l keys are >= tau
        __syncthreads();

        // ordered compaction of {u key >= tau} (rows hold u): batches of VB
        // 16-byte pieces per thread, all loads of a batch in flight at once
        // (pieces past the row read its last piece and are masked).  Rows
        // hold no -0, so order_key(x) >= tau is x >= ftau.
        const float ftau = key_to_float(tau);
        uint32_t count = 0, cnt_l = 0;
        for (int64_t base = 0; base < n; base += BATCH) {
            if (base > 0) load_batch(base);
            int lim[VB];  // elements of piece u below lim[u] lie in the row
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                const int64_t e = base + (int64_t)(u * NT + tid) * 4;
                lim[u] = e + 4 <= n ? 4 : (e < n ? (int)(n - e) : 0);
            }
            uint32_t c[VB], off[VB];
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                uint32_t cc = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) cc += (j < lim[u]) & (v[u][j] >= ftau);
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
                    if ((j < lim[u]) & (v[u][j] >= ftau)) {
                        if (pos < (uint32_t)LCAP) {
                            sh.s[pos] = v[u][j];
                            sh.idc[pos] = (uint32_t)(e + j);
                        }
                        ++pos;
                    }
                }
            }
            count += tot;
        }
        __syncthreads();
        // the bounds of the kept entries, and how many have l key >= tau
        if constexpr (BOUNDS) {
            // every gather of the thread in flight at once (mm <= LCAP)
            const int mm = (int)min(count, (uint32_t)LCAP);
            constexpr int GU = LCAP / NT;
            float dl[GU];
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int e = u * NT + tid;
                dl[u] = e < mm ? delta(sh.idc[e]) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int e = u * NT + tid;
                if (e < mm) {
                    sh.d[e] = dl[u];
                    cnt_l += order_key(sh.s[e] - 2.0f * dl[u]) >= tau;
                }
            }
            cnt_l = block_sum(cnt_l, sh);
        } else {
            cnt_l = count;
        }
        __syncthreads();
        if (count > (uint32_t)LCAP || cnt_l < (uint32_t)k) {
            if constexpr (BOUNDS) {
                if (A[1] > 0.0f) {
                    select_row_bounded<HI, DI>(a, i, row, n, A, sh, out, sout);
                    return;
                }
            }
            select_row(row, n, k, sh, out, sout);
            return;
        }
        m = (int)count;
    }

    if constexpr (!BOUNDS) {
        // final scores: one selection over the whole list
        auto key_at = [&](int64_t e, uint32_t& key) {
            key = order_key(sh.s[e]);
            return true;
        };
        uint32_t lo, hi, remaining = (uint32_t)k;
        member_minmax(m, key_at, lo, hi, sh);
        radix_narrow(m, key_at, lo, hi, remaining, false, sh);
        emit_list<true>(m, lo, hi, remaining, sh, out, sout, k);
        return;
    }
    // bounds on L and U over the list
    uint32_t Lk, Uk;
    band_bounds(m, [&](int64_t e, uint32_t& lk, uint32_t& uk) {
        const float x = sh.s[e];
        lk = order_key(x - 2.0f * sh.d[e]);
        uk = order_key(x);
    }, (uint32_t)k, Lk, Uk, sh);
    // classify: certain (l > U), band (u >= L, l <= U), dropped (u < L)
    uint32_t n_in = 0;
    for (int e = tid; e < m; e += NT) {
        const float x = sh.s[e], dl = sh.d[e];
        const uint32_t lk = order_key(x - 2.0f * dl), uk = order_key(x);
        const uint32_t c = lk > Uk ? C_IN : (uk >= Lk ? C_BAND : C_OUT);
        const bool need = dl > 0.0f && (c == C_BAND || (c == C_IN && sout));
        sh.idc[e] |= (c << 29) | (need ? RESCORE : 0u);
        n_in += c == C_IN;
    }
    n_in = block_sum(n_in, sh);
    __syncthreads();
    // the band and the entries to rescore, in list order
    uint32_t* pos = reinterpret_cast<uint32_t*>(sh.d);
    const uint32_t np = compact(m, [&](int e) {
        const uint32_t t = sh.idc[e];
        return cls_of(t) == C_BAND || (t & RESCORE) != 0u;
    }, [&](uint32_t slot, int e) { pos[slot] = (uint32_t)e; }, sh);
    __syncthreads();
    rescore<HI, DI>(np, [&](uint32_t j) { return sh.idc[pos[j]]; },
                    [&](uint32_t j, float v) { sh.s[pos[j]] = v; }, a, i, sh);
    __syncthreads();
    // the remaining k - n_in from the band, by full score, ties to the lower id
    auto band_key = [&](int64_t j, uint32_t& key) {
        key = order_key(sh.s[pos[j]]);
        return cls_of(sh.idc[pos[j]]) == C_BAND;
    };
    uint32_t lo, hi, remaining = (uint32_t)k - n_in;
    member_minmax(np, band_key, lo, hi, sh);
    radix_narrow(np, band_key, lo, hi, remaining, false, sh);
    emit_list<false>(m, lo, hi, remaining, sh, out, sout, k);
}

// Shapes whose short-list kernel fits 128 VGPRs without spilling (the
// rescoring's operands grow with D_I and, below 16 heads, take more lanes).
template <int HI, int DI>
constexpr bool short_list_fits() { return DI == 64 || (DI == 96 && HI >= 16); }

template <int HI, int DI>
hipError_t launch_bounded_di(const SelectArgs& a, bool long_rows, hipStream_t stream) {
    const dim3 grid((unsigned)a.rows);
    if constexpr (short_list_fits<HI, DI>()) {
        if (!long_rows) {
            topk_select_kernel<HI, DI, true, CAP_SHORT>
                <<<grid, NT, lds_bounded<CAP_SHORT>(), stream>>>(a);
            return hipGetLastError();
        }
    }
    topk_select_kernel<HI, DI, true, CAP><<<grid, NT, lds_bounded<CAP>(), stream>>>(a);
    return hipGetLastError();
}

// The short list when it fits and no row of the chunk has more than
// LONG_ROW pools.
template <int HI>
hipError_t launch_bounded_h(const SelectArgs& a, hipStream_t stream) {
    const int64_t t_last = a.q_pos0 + a.row0 + a.rows - 1;
    const int64_t n_max = (t_last >> 2) < a.n_pools ? (t_last >> 2) : a.n_pools;
    const bool long_rows = n_max > LONG_ROW;
    switch (a.d_idx) {
        case 64: return launch_bounded_di<HI, 64>(a, long_rows, stream);
        case 96: return launch_bounded_di<HI, 96>(a, long_rows, stream);
        case 128: return launch_bounded_di<HI, 128>(a, long_rows, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_topk_select(const SelectArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (!a.qbound) {
        topk_select_kernel<32, 128, false, CAP><<<dim3((unsigned)a.rows), NT, lds_final<CAP>(), stream>>>(a);
        return hipGetLastError();
    }
    switch (a.h_idx) {
        case 4: return launch_bounded_h<4>(a, stream);
        case 8: return launch_bounded_h<8>(a, stream);
        case 16: return launch_bounded_h<16>(a, stream);
        case 32: return launch_bounded_h<32>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsa
