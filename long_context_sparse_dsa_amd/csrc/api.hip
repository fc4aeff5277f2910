// C ABI of libdsa: argument checks, workspace layout, the query-chunk loop
// and per-kernel timing.  Every entry point validates all arguments before
// enqueuing anything; on failure nothing is launched and dsa_last_error()
// holds the reason.  There is no fallback path: unsupported shapes are
// rejected (SkyRL blog "Scaling Training to 1M Token Context on
// GLM-5.3-Flash", section "Making Sparse Attention Actually Sparse", on how
// a silent dense fallback looked like a memory problem rather than a bug).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "dsa.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

constexpr int64_t kMaxKPools = 2048;
constexpr int64_t kDefaultChunkMax = 8192;
constexpr int64_t kDefaultBufferBudget = int64_t(3) << 29;  // 1.5 GiB
// Top-k workgroups resident at once on MI355X for rows of long-list shapes:
// 256 CUs x 3.  Default chunks that the buffer budget limits (long rows) are
// a multiple of it, so that no selection launch ends on a partial wave.
constexpr int64_t kSelectWave = 768;
constexpr int64_t kMaxChunk = 1 << 16;
constexpr int64_t kScoreBufferCap = int64_t(2) << 30;  // per chunk, as the page keeps it

// ------------------------------------------------------------ profiling

enum Kind {
    K_POOL = 0, K_PACK, K_SCORE, K_SELECT, K_ATTN, K_BWD_DQ, K_BWD_BITS, K_BWD_DKV,
    K_SCORE_FULL, K_COUNT
};
// index_score: the bf16 scorer without the correction term (bounded chunks)
// and the fp8 scorer; index_score_full: the bf16 scorer with it (chunks of
// short rows, and the dense-score entry point), a separate kernel
const char* kKindName[K_COUNT] = {"pool_keys", "pack_queries", "index_score", "topk_select",
                                  "sparse_attn", "attn_bwd_dq", "attn_bwd_select",
                                  "attn_bwd_dkv", "index_score_full"};

struct Rec {
    int kind;
    hipEvent_t a, b;
};

struct Prof {
    std::mutex mu;
    bool on = false;
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;
} g_prof;

// Set while the no-allocation entry point runs on this thread: no profiling
// events are created or recorded (creating one allocates).
thread_local bool t_no_events = false;

hipEvent_t take_event() {
    if (!g_prof.pool.empty()) {
        hipEvent_t e = g_prof.pool.back();
        g_prof.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Brackets one launch with events when profiling is on.
struct Timed {
    int kind;
    hipStream_t s;
    hipEvent_t a = nullptr, b = nullptr;
    Timed(int k, hipStream_t st) : kind(k), s(st) {
        if (t_no_events) return;
        std::lock_guard<std::mutex> lk(g_prof.mu);
        if (!g_prof.on) return;
        a = take_event();
        b = take_event();
        if (a && b) (void)hipEventRecord(a, s);
    }
    ~Timed() {
        if (!a || !b) return;
        (void)hipEventRecord(b, s);
        std::lock_guard<std::mutex> lk(g_prof.mu);
        g_prof.recs.push_back(Rec{kind, a, b});
    }
};

dsa_status hip_fail(hipError_t e, const char* what) {
    return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ------------------------------------------------------------ indexer checks

struct IndexShape {
    int64_t s_q, s_k, q_pos0;
    int h_idx, d_idx, pool_size, k_pools, dtype;
    int64_t n_pools;
};

dsa_status check_index_shape(const IndexShape& sh, bool need_k) {
    if (sh.s_q < 0 || sh.s_k < 0 || sh.q_pos0 < 0)
        return fail(DSA_ERR_INVALID_ARG, "negative size or position (s_q=%lld s_k=%lld q_pos0=%lld)",
                    (long long)sh.s_q, (long long)sh.s_k, (long long)sh.q_pos0);
    if (sh.s_k >= (int64_t(1) << 31) || sh.s_q >= (int64_t(1) << 31) ||
        sh.q_pos0 >= (int64_t(1) << 40))
        return fail(DSA_ERR_UNSUPPORTED,
                    "s_q and s_k must be below 2^31 and q_pos0 below 2^40 (s_q=%lld s_k=%lld "
                    "q_pos0=%lld)", (long long)sh.s_q, (long long)sh.s_k, (long long)sh.q_pos0);
    if (sh.pool_size != 4)
        return fail(DSA_ERR_UNSUPPORTED, "pool_size %d: only pools of 4 tokens are supported",
                    sh.pool_size);
    if (sh.h_idx != 4 && sh.h_idx != 8 && sh.h_idx != 16 && sh.h_idx != 32)
        return fail(DSA_ERR_UNSUPPORTED, "h_idx %d: supported indexer heads are 4, 8, 16, 32",
                    sh.h_idx);
    if (sh.d_idx != 64 && sh.d_idx != 96 && sh.d_idx != 128)
        return fail(DSA_ERR_UNSUPPORTED, "d_idx %d: supported indexer dims are 64, 96, 128",
                    sh.d_idx);
    if (sh.dtype != DSA_BF16 && sh.dtype != DSA_FP8_E4M3)
        return fail(DSA_ERR_INVALID_ARG, "unknown dtype %d", sh.dtype);
    if (need_k && (sh.k_pools < 1 || sh.k_pools > kMaxKPools))
        return fail(DSA_ERR_UNSUPPORTED, "k_pools %d: supported range is 1..%lld", sh.k_pools,
                    (long long)kMaxKPools);
    return DSA_OK;
}

// Row stride of the chunk score buffer: a multiple of the pools one scoring
// workgroup covers, so that its stores never need a column mask.
int64_t score_ld(const IndexShape& sh) { return round_up(sh.n_pools > 0 ? sh.n_pools : 1, 512); }

// bf16 indexer: score a chunk without the correction term and rescore only
// the pools near each row's k-th score (bounded), or score it in full?  The
// rescoring costs about k pools per row whatever the row's length, the
// correction term a share of every pool, so the bounds pay once the rows see
// more than about 16 k pools (measured on MI355X at k = 512 with 8192-query
// chunks: 8, 12, 16 and 24 k per row were within 1% of each other at 32k
// and 128k, 16 k the fastest at 128k).
bool bounded_chunk(const IndexShape& sh, int64_t t_first, int64_t t_last) {
    const int64_t n_first = (t_first / 4) < sh.n_pools ? (t_first / 4) : sh.n_pools;
    const int64_t n_last = (t_last / 4) < sh.n_pools ? (t_last / 4) : sh.n_pools;
    return n_first + n_last > 2 * 16 * (int64_t)sh.k_pools;
}

// Rows per scoring launch of the dense-score entry point (bounds its workspace).
constexpr int64_t kDenseRows = 4096;

dsa_status resolve_chunk(const IndexShape& sh, int64_t chunk_q, int64_t* out) {
    if (chunk_q < 0) return fail(DSA_ERR_INVALID_ARG, "chunk_q %lld < 0", (long long)chunk_q);
    if (chunk_q == 0) {
        // at most 8192 queries (and no more than the queries there are);
        // when the 1.5 GiB buffer budget is what limits the chunk (long
        // rows), the largest multiple of 768 within it, else of 64
        chunk_q = kDefaultBufferBudget / (score_ld(sh) * 4);
        const bool by_budget = chunk_q < kDefaultChunkMax;
        if (chunk_q > kDefaultChunkMax) chunk_q = kDefaultChunkMax;
        if (chunk_q > round_up(sh.s_q, 64)) chunk_q = round_up(sh.s_q, 64);
        chunk_q = by_budget && chunk_q >= kSelectWave && sh.s_q > kSelectWave
                      ? chunk_q / kSelectWave * kSelectWave
                      : chunk_q / 64 * 64;
        if (chunk_q < 64) chunk_q = 64;
    } else if (chunk_q % 64 != 0 || chunk_q > kMaxChunk) {
        return fail(DSA_ERR_UNSUPPORTED, "chunk_q %lld must be a multiple of 64 up to %lld",
                    (long long)chunk_q, (long long)kMaxChunk);
    }
    if (chunk_q * score_ld(sh) * 4 > kScoreBufferCap)
        return fail(DSA_ERR_UNSUPPORTED,
                    "chunk_q %lld x %lld pools x 4 B exceeds the 2 GiB per-chunk buffer cap",
                    (long long)chunk_q, (long long)sh.n_pools);
    *out = chunk_q;
    return DSA_OK;
}

// Workspace layout, every part starting on a 256-byte boundary:
//   bf16 indexer: hi [P][d] bf16 | lo [P][d] E4M3 | lo scales [P] E8M0 |
//                 bound factors mu [P][2] fp32 | the chunk's packed query tiles |
//                 bound factors A [rows][2] fp32 | score buffer [rows][ld] fp32
//   fp8 indexer:  codes [P][d] | per-pool factors [P] fp32 | score buffer
struct Layout {
    int64_t hi = 0, lo = 0, lo_scale = 0, mu = 0, tiles = 0, qbound = 0, buf = 0, total = 0;
};

Layout layout(const IndexShape& sh, int64_t rows, bool with_buffer) {
    Layout L;
    const int64_t P = sh.n_pools, d = sh.d_idx;
    int64_t off = 0;
    if (sh.dtype == DSA_BF16) {
        L.hi = off;        off += round_up(P * d * 2, 256);
        L.lo = off;        off += round_up(P * d, 256);
        L.lo_scale = off;  off += round_up(P, 256);
        L.mu = off;        off += round_up(P * 8, 256);
        L.tiles = off;
        off += round_up(dsa::query_tiles(rows, sh.h_idx) * dsa::query_tile_geom((int)d).tb, 256);
        L.qbound = off;    off += round_up(rows * 8, 256);
    } else {
        L.hi = off;        off += round_up(P * d, 256);
        L.lo_scale = off;  off += round_up(P * 4, 256);  // fp32 factors 2^e
    }
    L.buf = off;
    if (with_buffer) off += round_up(rows * score_ld(sh) * 4, 256);
    L.total = off;
    return L;
}

dsa_status index_workspace(const IndexShape& sh, int64_t chunk_q, size_t* bytes) {
    *bytes = (size_t)layout(sh, chunk_q, true).total;
    return DSA_OK;
}

dsa_status check_index_ptrs(const void* q_idx, const void* k_idx, const float* q_scale,
                            const float* k_scale, const float* w, int64_t w_stride,
                            const IndexShape& sh) {
    if (sh.s_q > 0 && (!q_idx || !w))
        return fail(DSA_ERR_INVALID_ARG, "q_idx and w must be non-null");
    if (sh.n_pools > 0 && !k_idx) return fail(DSA_ERR_INVALID_ARG, "k_idx must be non-null");
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w))
        return fail(DSA_ERR_INVALID_ARG, "q_idx, k_idx and w must be 16-byte aligned");
    if (w_stride < 0 || (w_stride != 0 && w_stride < sh.h_idx))
        return fail(DSA_ERR_INVALID_ARG, "w_stride_q %lld must be 0 or >= h_idx",
                    (long long)w_stride);
    if (sh.dtype == DSA_BF16 && (q_scale || k_scale))
        return fail(DSA_ERR_INVALID_ARG, "q_scale/k_scale apply to the fp8 indexer only");
    if ((reinterpret_cast<uintptr_t>(q_scale) & 3u) || (reinterpret_cast<uintptr_t>(k_scale) & 3u))
        return fail(DSA_ERR_INVALID_ARG, "q_scale and k_scale must be 4-byte aligned");
    return DSA_OK;
}

dsa_status check_gate(const float* k_gate) {
    if (!aligned16(k_gate)) return fail(DSA_ERR_INVALID_ARG, "k_gate must be 16-byte aligned");
    return DSA_OK;
}

hipError_t launch_pool(const IndexShape& sh, const Layout& L, const void* k_idx,
                       const float* k_gate, void* ws, hipStream_t s) {
    Timed tm(K_POOL, s);
    char* w = static_cast<char*>(ws);
    if (sh.dtype == DSA_BF16)
        return dsa::launch_pool_keys_bf16(static_cast<const uint16_t*>(k_idx), k_gate, sh.n_pools,
                                          sh.d_idx, reinterpret_cast<uint16_t*>(w + L.hi),
                                          reinterpret_cast<uint8_t*>(w + L.lo),
                                          reinterpret_cast<uint8_t*>(w + L.lo_scale),
                                          reinterpret_cast<float*>(w + L.mu), s);
    return dsa::launch_pool_keys_fp8(static_cast<const uint8_t*>(k_idx), k_gate, sh.n_pools,
                                     sh.d_idx, reinterpret_cast<uint8_t*>(w + L.hi),
                                     reinterpret_cast<float*>(w + L.lo_scale), s);
}

// bf16 indexer: pack query rows [row0, row0 + rows) and their weights into
// the tiles the scoring kernel streams (with_bound: and each query's bound
// factor, for the selection).
hipError_t launch_pack(const IndexShape& sh, const Layout& L, const void* q_idx, const float* w,
                       int64_t w_stride, int64_t row0, int64_t rows, bool with_bound, void* ws,
                       hipStream_t s) {
    if (sh.dtype != DSA_BF16) return hipSuccess;
    Timed tm(K_PACK, s);
    char* base = static_cast<char*>(ws);
    return dsa::launch_pack_queries(static_cast<const uint16_t*>(q_idx), w, w_stride, row0,
                                    (int)rows, sh.h_idx, sh.d_idx,
                                    reinterpret_cast<uint8_t*>(base + L.tiles),
                                    with_bound ? reinterpret_cast<float*>(base + L.qbound) : nullptr,
                                    s);
}

void fill_score_args(dsa::ScoreArgs& a, const IndexShape& sh, const Layout& L,
                     const void* q_idx, void* ws, const float* q_scale, const float* k_scale,
                     const float* w, int64_t w_stride) {
    char* base = static_cast<char*>(ws);
    a.q_idx = q_idx;
    a.kbar = base + L.hi;
    if (sh.dtype == DSA_BF16) {
        a.klo = reinterpret_cast<const uint8_t*>(base + L.lo);
        a.klo_scale = reinterpret_cast<const uint8_t*>(base + L.lo_scale);
        a.tiles = reinterpret_cast<const uint8_t*>(base + L.tiles);
        a.pool_scale = nullptr;
    } else {
        a.pool_scale = reinterpret_cast<const float*>(base + L.lo_scale);
    }
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.w = w;
    a.w_stride = w_stride;
    a.s_q = sh.s_q;
    a.q_pos0 = sh.q_pos0;
    a.n_pools = sh.n_pools;
    a.h_idx = sh.h_idx;
    a.d_idx = sh.d_idx;
    a.fp8 = sh.dtype == DSA_FP8_E4M3;
}

// Shape checks shared by the attention forward and backward.
dsa_status check_attn_shape(int64_t s_q, int64_t s_k, int64_t q_pos0, int h, int d, int dv,
                            int k_pools, int pool_size, int n_tail, float softmax_scale) {
    if (s_q < 0 || s_k < 0 || q_pos0 < 0)
        return fail(DSA_ERR_INVALID_ARG, "negative size or position");
    if (s_k >= (int64_t(1) << 31) || s_q >= (int64_t(1) << 31))
        return fail(DSA_ERR_UNSUPPORTED, "s_q and s_k must be below 2^31");
    if (pool_size != 4) return fail(DSA_ERR_UNSUPPORTED, "pool_size %d: only 4 is supported", pool_size);
    if (h < 1 || h > 16)
        return fail(DSA_ERR_UNSUPPORTED, "h %d: 1..16 query heads per key/value head", h);
    if ((d != 64 && d != 96 && d != 128) || (dv != 64 && dv != 96 && dv != 128))
        return fail(DSA_ERR_UNSUPPORTED, "d %d / dv %d: supported head dims are 64, 96, 128", d, dv);
    if (k_pools < 1 || k_pools > kMaxKPools)
        return fail(DSA_ERR_UNSUPPORTED, "k_pools %d: supported range is 1..%lld", k_pools,
                    (long long)kMaxKPools);
    if (n_tail < 0 || n_tail >= pool_size)
        return fail(DSA_ERR_INVALID_ARG, "n_tail %d outside 0..%d", n_tail, pool_size - 1);
    if (!(softmax_scale == softmax_scale)) return fail(DSA_ERR_INVALID_ARG, "softmax_scale is NaN");
    return DSA_OK;
}

// Backward: queries per transposition chunk (a multiple of 64), and the
// workspace: delta [s_q, h] fp32, then the bitmaps [chunk / 32][ceil(s_k / 4)]
// words of every chunk when they fit kBwdBitmapAll (else of one chunk), then
// the pool slots' entry counts and order.  Default chunk: max(1024,
// min(1536, 3 slots / 32), slots / 32), at most 16384.  Every chunk pays a
// pass of the key-major kernel over all pool slots, so the chunk grows with
// them; smaller chunks keep more of a chunk's query rows in the L2s.
// (Measured best of 768 .. 2048 with the slots grouped by count: 1024 at 8K
// slots, 1536 at 16K and 32K; of 2048 .. 16384 before: 8192 to 16384 at
// 262144.)
constexpr int64_t kBwdChunkMin = 1024;
constexpr int64_t kBwdChunkMid = 1536;
// The bitmaps of all chunks are built by one launch when together they take
// at most this many bytes (else one chunk's bitmap at a time).
constexpr int64_t kBwdBitmapAll = int64_t(1) << 30;
constexpr int64_t kBwdChunkMax = 16384;
constexpr int64_t kBwdBitmapCap = int64_t(2) << 30;

dsa_status bwd_layout(int64_t s_q, int64_t s_k, int h, int64_t chunk_q, int64_t* chunk_used,
                      int64_t* delta_bytes, int64_t* bits_bytes) {
    if (chunk_q < 0) return fail(DSA_ERR_INVALID_ARG, "chunk_q %lld < 0", (long long)chunk_q);
    const int64_t slots = (s_k + 3) / 4;
    if (chunk_q == 0) {
        int64_t c = 3 * slots / 32 < kBwdChunkMid ? 3 * slots / 32 : kBwdChunkMid;
        if (c < kBwdChunkMin) c = kBwdChunkMin;
        if (slots / 32 > c) c = slots / 32;
        c = round_up(c, 64);
        if (c > kBwdChunkMax) c = kBwdChunkMax;
        const int64_t all = round_up(s_q > 0 ? s_q : 1, 64);
        chunk_q = c < all ? c : all;
    }
    if (chunk_q % 64 != 0 || chunk_q > kMaxChunk)
        return fail(DSA_ERR_UNSUPPORTED, "chunk_q %lld: must be a multiple of 64 up to %lld",
                    (long long)chunk_q, (long long)kMaxChunk);
    const int64_t bits = round_up(slots, 4) * (chunk_q / 32) * 4;
    if (bits > kBwdBitmapCap)
        return fail(DSA_ERR_UNSUPPORTED, "chunk_q %lld: the chunk bitmap (%lld bytes) exceeds 2 GiB",
                    (long long)chunk_q, (long long)bits);
    const int64_t nchunks = s_q > 0 ? (s_q + chunk_q - 1) / chunk_q : 1;
    const int64_t all = bits * nchunks;
    *chunk_used = chunk_q;
    *delta_bytes = round_up(s_q * h * 4, 256);
    // the bitmap (of every chunk when that fits kBwdBitmapAll), then the pool
    // slots' entry counts and their order
    *bits_bytes = round_up(all <= kBwdBitmapAll ? all : bits, 256) +
                  2 * round_up(round_up(slots, 4) * 4, 256);
    return DSA_OK;
}

// ------------------------------------------------------------ scratch

// The workspace of dsa_index_score_topk_noalloc (declared at file scope
// below): the largest chunk of a multiple of 64 queries whose workspace fits
// in max_bytes, or the caller's chunk_q if it fits.
dsa_status chunk_within(const IndexShape& sh, int64_t chunk_q, int64_t max_bytes, int64_t* out) {
    int64_t cq = 0;
    dsa_status st = resolve_chunk(sh, chunk_q, &cq);
    if (st != DSA_OK) return st;
    if (chunk_q != 0) {
        const int64_t need = layout(sh, cq, true).total;
        if (need > max_bytes)
            return fail(DSA_ERR_WORKSPACE,
                        "chunk_q %lld needs %lld bytes of scratch; the no-allocation entry "
                        "point has %lld (pass chunk_q = 0 to fit the chunk to it)",
                        (long long)chunk_q, (long long)need, (long long)max_bytes);
    } else {
        cq = cq / 64 * 64;
        while (cq > 64 && layout(sh, cq, true).total > max_bytes) cq -= 64;
        const int64_t need = layout(sh, cq, true).total;
        if (need > max_bytes)
            return fail(DSA_ERR_UNSUPPORTED,
                        "these shapes need %lld bytes of scratch (pooled keys and one chunk of "
                        "64 queries); the no-allocation entry point has %lld",
                        (long long)need, (long long)max_bytes);
    }
    *out = cq;
    return DSA_OK;
}

}  // namespace

// Scratch memory of dsa_index_score_topk_noalloc: one copy per GPU in the
// library's device image, allocated with the code object on each device the
// library runs on and held until the process ends.  In host code `scratch`
// only names the symbol; its device address comes from hipGetSymbolAddress.
constexpr int64_t kScratchBytes = int64_t(256) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (the first call on it) with that device current.
dsa_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned no address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DSA_OK;
}

struct NoEvents {
    NoEvents() { t_no_events = true; }
    ~NoEvents() { t_no_events = false; }
};

}  // namespace

extern "C" {

int dsa_version(void) { return 100; }

const char* dsa_last_error(void) { return g_err; }

dsa_status dsa_index_workspace_size(int64_t s_q, int64_t s_k, int h_idx, int d_idx, int k_pools,
                                    int pool_size, int64_t chunk_q, int dtype, size_t* bytes,
                                    int64_t* chunk_q_used) {
    g_err[0] = 0;
    if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes must be non-null");
    IndexShape sh{s_q, s_k, 0, h_idx, d_idx, pool_size, k_pools, dtype, s_k / 4};
    dsa_status st = check_index_shape(sh, true);
    if (st != DSA_OK) return st;
    int64_t cq = 0;
    if ((st = resolve_chunk(sh, chunk_q, &cq)) != DSA_OK) return st;
    if (chunk_q_used) *chunk_q_used = cq;
    return index_workspace(sh, cq, bytes);
}

dsa_status dsa_index_scores_workspace_size(int64_t s_q, int64_t s_k, int h_idx, int d_idx,
                                           int pool_size, int dtype, int64_t n_rows,
                                           size_t* bytes) {
    g_err[0] = 0;
    if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes must be non-null");
    IndexShape sh{s_q, s_k, 0, h_idx, d_idx, pool_size, 1, dtype, s_k / 4};
    dsa_status st = check_index_shape(sh, false);
    if (st != DSA_OK) return st;
    if (n_rows < 0 || n_rows > s_q) return fail(DSA_ERR_INVALID_ARG, "n_rows outside [0, s_q]");
    *bytes = (size_t)layout(sh, n_rows < kDenseRows ? n_rows : kDenseRows, false).total;
    return DSA_OK;
}

static dsa_status index_score_topk(const void* q_idx, const void* k_idx, const float* k_gate,
                                   const float* q_scale, const float* k_scale, const float* w,
                                   int64_t w_stride_q, int64_t s_q, int64_t s_k, int64_t q_pos0,
                                   int h_idx, int d_idx, int pool_size, int k_pools,
                                   int64_t chunk_q, int dtype, int32_t* idx_out,
                                   float* score_out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    g_err[0] = 0;
    IndexShape sh{s_q, s_k, q_pos0, h_idx, d_idx, pool_size, k_pools, dtype, s_k / 4};
    dsa_status st = check_index_shape(sh, true);
    if (st != DSA_OK) return st;
    if ((st = check_index_ptrs(q_idx, k_idx, q_scale, k_scale, w, w_stride_q, sh)) != DSA_OK)
        return st;
    if ((st = check_gate(k_gate)) != DSA_OK) return st;
    if (s_q > 0 && !idx_out) return fail(DSA_ERR_INVALID_ARG, "idx_out must be non-null");
    if (!aligned16(idx_out) || !aligned16(score_out))
        return fail(DSA_ERR_INVALID_ARG, "idx_out and score_out must be 16-byte aligned");
    int64_t cq = 0;
    if ((st = resolve_chunk(sh, chunk_q, &cq)) != DSA_OK) return st;
    size_t need = 0;
    index_workspace(sh, cq, &need);
    if (s_q == 0) return DSA_OK;
    if (!workspace || workspace_bytes < need)
        return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    const Layout L = layout(sh, cq, true);
    float* buf = reinterpret_cast<float*>(ws + L.buf);
    const int64_t ld = score_ld(sh);
    hipError_t e;
    if (sh.n_pools > 0) {
        e = launch_pool(sh, L, k_idx, k_gate, ws, s);
        if (e != hipSuccess) return hip_fail(e, "pool_keys launch");
    }
    for (int64_t c0 = 0; c0 < s_q; c0 += cq) {
        const int rows = (int)(s_q - c0 < cq ? s_q - c0 : cq);
        const int64_t t_last = q_pos0 + c0 + rows - 1;
        const int64_t n_chunk = (t_last / 4) < sh.n_pools ? (t_last / 4) : sh.n_pools;
        const bool bounded = dtype == DSA_BF16 && bounded_chunk(sh, q_pos0 + c0, t_last);
        if (n_chunk > 0 && (n_chunk > k_pools || score_out)) {
            e = launch_pack(sh, L, q_idx, w, w_stride_q, c0, rows, bounded, ws, s);
            if (e != hipSuccess) return hip_fail(e, "pack_queries launch");
            dsa::ScoreArgs a{};
            fill_score_args(a, sh, L, q_idx, ws, q_scale, k_scale, w, w_stride_q);
            a.row0 = c0;
            a.rows = rows;
            a.n_chunk = n_chunk;
            a.buf = buf;
            a.ld = ld;
            if (bounded) {
                a.qbound = reinterpret_cast<const float*>(ws + L.qbound);
                a.mu = reinterpret_cast<const float*>(ws + L.mu);
            }
            Timed tm(bounded || dtype != DSA_BF16 ? K_SCORE : K_SCORE_FULL, s);
            e = dsa::launch_index_score(a, s);
            if (e != hipSuccess) return hip_fail(e, "index_score launch");
        }
        dsa::SelectArgs b{};
        b.buf = buf;
        b.ld = ld;
        b.row0 = c0;
        b.rows = rows;
        b.q_pos0 = q_pos0;
        b.n_pools = sh.n_pools;
        b.k_pools = k_pools;
        b.idx_out = idx_out;
        b.score_out = score_out;
        b.h_idx = h_idx;
        b.d_idx = d_idx;
        if (bounded) {
            // bounds of the scores without the correction term: the
            // selection rescores the pools its bound cannot decide
            b.qbound = reinterpret_cast<const float*>(ws + L.qbound);
            b.mu = reinterpret_cast<const float*>(ws + L.mu);
            b.tiles = reinterpret_cast<const uint8_t*>(ws + L.tiles);
            b.khi = reinterpret_cast<const uint16_t*>(ws + L.hi);
            b.klo = reinterpret_cast<const uint8_t*>(ws + L.lo);
            b.klo_scale = reinterpret_cast<const uint8_t*>(ws + L.lo_scale);
        }
        Timed tm(K_SELECT, s);
        e = dsa::launch_topk_select(b, s);
        if (e != hipSuccess) return hip_fail(e, "topk_select launch");
    }
    return DSA_OK;
}

static dsa_status index_scores(const void* q_idx, const void* k_idx, const float* k_gate,
                               const float* q_scale, const float* k_scale, const float* w,
                               int64_t w_stride_q, int64_t s_q, int64_t s_k, int64_t q_pos0,
                               int h_idx, int d_idx, int pool_size, int dtype, int64_t row0,
                               int64_t n_rows, float* scores_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    IndexShape sh{s_q, s_k, q_pos0, h_idx, d_idx, pool_size, 1, dtype, s_k / 4};
    dsa_status st = check_index_shape(sh, false);
    if (st != DSA_OK) return st;
    if ((st = check_index_ptrs(q_idx, k_idx, q_scale, k_scale, w, w_stride_q, sh)) != DSA_OK)
        return st;
    if ((st = check_gate(k_gate)) != DSA_OK) return st;
    if (row0 < 0 || n_rows < 0 || row0 + n_rows > s_q)
        return fail(DSA_ERR_INVALID_ARG, "rows [%lld, %lld) outside [0, %lld)", (long long)row0,
                    (long long)(row0 + n_rows), (long long)s_q);
    if (n_rows > (int64_t(1) << 20))
        return fail(DSA_ERR_UNSUPPORTED, "at most 2^20 rows per call");
    if (n_rows > 0 && !scores_out) return fail(DSA_ERR_INVALID_ARG, "scores_out must be non-null");
    if (!aligned16(scores_out)) return fail(DSA_ERR_INVALID_ARG, "scores_out must be 16-byte aligned");
    const Layout L = layout(sh, n_rows < kDenseRows ? n_rows : kDenseRows, false);
    const size_t need = (size_t)L.total;
    if (n_rows == 0 || sh.n_pools == 0) return DSA_OK;  // nothing to write
    if (!workspace || workspace_bytes < need)
        return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = dsa::launch_fill_f32(scores_out, n_rows * sh.n_pools, -INFINITY, s);
    if (e != hipSuccess) return hip_fail(e, "fill launch");
    e = launch_pool(sh, L, k_idx, k_gate, workspace, s);
    if (e != hipSuccess) return hip_fail(e, "pool_keys launch");
    for (int64_t r0 = row0; r0 < row0 + n_rows; r0 += kDenseRows) {
        const int64_t rows = row0 + n_rows - r0 < kDenseRows ? row0 + n_rows - r0 : kDenseRows;
        const int64_t t_last = q_pos0 + r0 + rows - 1;
        const int64_t n_chunk = (t_last / 4) < sh.n_pools ? (t_last / 4) : sh.n_pools;
        if (n_chunk == 0) continue;
        e = launch_pack(sh, L, q_idx, w, w_stride_q, r0, rows, false, workspace, s);
        if (e != hipSuccess) return hip_fail(e, "pack_queries launch");
        dsa::ScoreArgs a{};
        fill_score_args(a, sh, L, q_idx, workspace, q_scale, k_scale, w, w_stride_q);
        a.row0 = r0;
        a.rows = (int)rows;
        a.n_chunk = n_chunk;
        a.exact = 1;
        a.buf = scores_out + (r0 - row0) * sh.n_pools;
        a.ld = sh.n_pools;
        Timed tm(dtype == DSA_BF16 ? K_SCORE_FULL : K_SCORE, s);
        e = dsa::launch_index_score(a, s);
        if (e != hipSuccess) return hip_fail(e, "index_score launch");
    }
    return DSA_OK;
}

dsa_status dsa_index_score_topk(const void* q_idx, const void* k_idx, const float* q_scale,
                                const float* k_scale, const float* w, int64_t w_stride_q,
                                int64_t s_q, int64_t s_k, int64_t q_pos0, int h_idx, int d_idx,
                                int pool_size, int k_pools, int64_t chunk_q, int dtype,
                                int32_t* idx_out, float* score_out, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return index_score_topk(q_idx, k_idx, nullptr, q_scale, k_scale, w, w_stride_q, s_q, s_k,
                            q_pos0, h_idx, d_idx, pool_size, k_pools, chunk_q, dtype, idx_out,
                            score_out, workspace, workspace_bytes, stream);
}

dsa_status dsa_index_score_topk_noalloc(const void* q_idx, const void* k_idx,
                                        const float* q_scale, const float* k_scale,
                                        const float* w, int64_t w_stride_q, int64_t s_q,
                                        int64_t s_k, int64_t q_pos0, int h_idx, int d_idx,
                                        int pool_size, int k_pools, int64_t chunk_q, int dtype,
                                        int32_t* idx_out, float* score_out, void* stream) {
    g_err[0] = 0;
    IndexShape sh{s_q, s_k, q_pos0, h_idx, d_idx, pool_size, k_pools, dtype, s_k / 4};
    dsa_status st = check_index_shape(sh, true);
    if (st != DSA_OK) return st;
    if ((st = check_index_ptrs(q_idx, k_idx, q_scale, k_scale, w, w_stride_q, sh)) != DSA_OK)
        return st;
    if (s_q > 0 && !idx_out) return fail(DSA_ERR_INVALID_ARG, "idx_out must be non-null");
    if (!aligned16(idx_out) || !aligned16(score_out))
        return fail(DSA_ERR_INVALID_ARG, "idx_out and score_out must be 16-byte aligned");
    int64_t cq = 0;
    if ((st = chunk_within(sh, chunk_q, kScratchBytes, &cq)) != DSA_OK) return st;
    if (s_q == 0) return DSA_OK;
    void* ws = nullptr;
    if ((st = scratch_address(&ws)) != DSA_OK) return st;
    NoEvents quiet;
    return index_score_topk(q_idx, k_idx, nullptr, q_scale, k_scale, w, w_stride_q, s_q, s_k,
                            q_pos0, h_idx, d_idx, pool_size, k_pools, cq, dtype, idx_out,
                            score_out, ws, (size_t)kScratchBytes, stream);
}

dsa_status dsa_index_score_topk_gated(const void* q_idx, const void* k_idx, const float* k_gate,
                                      const float* q_scale, const float* k_scale, const float* w,
                                      int64_t w_stride_q, int64_t s_q, int64_t s_k,
                                      int64_t q_pos0, int h_idx, int d_idx, int pool_size,
                                      int k_pools, int64_t chunk_q, int dtype, int32_t* idx_out,
                                      float* score_out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
    if (!k_gate && s_k / 4 > 0) {
        g_err[0] = 0;
        return fail(DSA_ERR_INVALID_ARG, "k_gate must be non-null");
    }
    return index_score_topk(q_idx, k_idx, k_gate, q_scale, k_scale, w, w_stride_q, s_q, s_k,
                            q_pos0, h_idx, d_idx, pool_size, k_pools, chunk_q, dtype, idx_out,
                            score_out, workspace, workspace_bytes, stream);
}

dsa_status dsa_index_scores(const void* q_idx, const void* k_idx, const float* q_scale,
                            const float* k_scale, const float* w, int64_t w_stride_q,
                            int64_t s_q, int64_t s_k, int64_t q_pos0, int h_idx, int d_idx,
                            int pool_size, int dtype, int64_t row0, int64_t n_rows,
                            float* scores_out, void* workspace, size_t workspace_bytes,
                            void* stream) {
    return index_scores(q_idx, k_idx, nullptr, q_scale, k_scale, w, w_stride_q, s_q, s_k, q_pos0,
                        h_idx, d_idx, pool_size, dtype, row0, n_rows, scores_out, workspace,
                        workspace_bytes, stream);
}

dsa_status dsa_index_scores_gated(const void* q_idx, const void* k_idx, const float* k_gate,
                                  const float* q_scale, const float* k_scale, const float* w,
                                  int64_t w_stride_q, int64_t s_q, int64_t s_k, int64_t q_pos0,
                                  int h_idx, int d_idx, int pool_size, int dtype, int64_t row0,
                                  int64_t n_rows, float* scores_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (!k_gate && s_k / 4 > 0) {
        g_err[0] = 0;
        return fail(DSA_ERR_INVALID_ARG, "k_gate must be non-null");
    }
    return index_scores(q_idx, k_idx, k_gate, q_scale, k_scale, w, w_stride_q, s_q, s_k, q_pos0,
                        h_idx, d_idx, pool_size, dtype, row0, n_rows, scores_out, workspace,
                        workspace_bytes, stream);
}

dsa_status dsa_sparse_attn_fwd(const void* q, const void* k, const void* v, const int32_t* idx,
                               int64_t s_q, int64_t s_k, int64_t q_pos0, int h, int d, int dv,
                               int k_pools, int pool_size, int n_tail, float softmax_scale,
                               void* out, float* lse, void* stream) {
    g_err[0] = 0;
    dsa_status st = check_attn_shape(s_q, s_k, q_pos0, h, d, dv, k_pools, pool_size, n_tail,
                                     softmax_scale);
    if (st != DSA_OK) return st;
    if (s_q > 0 && (!q || !idx || !out))
        return fail(DSA_ERR_INVALID_ARG, "q, idx and out must be non-null");
    if (s_k > 0 && s_q > 0 && (!k || !v)) return fail(DSA_ERR_INVALID_ARG, "k and v must be non-null");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(idx) || !aligned16(out) ||
        !aligned16(lse))
        return fail(DSA_ERR_INVALID_ARG, "all buffers must be 16-byte aligned");
    if (s_q == 0) return DSA_OK;
    const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)d);
    dsa::AttnArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.idx = idx;
    a.s_q = s_q;
    a.s_k = s_k;
    a.q_pos0 = q_pos0;
    a.h = h;
    a.d = d;
    a.dv = dv;
    a.k_pools = k_pools;
    a.n_tail = n_tail;
    a.scale = scale;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Timed tm(K_ATTN, s);
    hipError_t e = dsa::launch_sparse_attn(a, s);
    if (e != hipSuccess) return hip_fail(e, "sparse_attn launch");
    return DSA_OK;
}

dsa_status dsa_sparse_attn_bwd_workspace_size(int64_t s_q, int64_t s_k, int h, int64_t chunk_q,
                                              size_t* bytes, int64_t* chunk_q_used) {
    g_err[0] = 0;
    if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes must be non-null");
    if (s_q < 0 || s_k < 0) return fail(DSA_ERR_INVALID_ARG, "negative size");
    if (h < 1 || h > 16)
        return fail(DSA_ERR_UNSUPPORTED, "h %d: 1..16 query heads per key/value head", h);
    int64_t cq, db, bb;
    dsa_status st = bwd_layout(s_q, s_k, h, chunk_q, &cq, &db, &bb);
    if (st != DSA_OK) return st;
    *bytes = (size_t)(db + bb);
    if (chunk_q_used) *chunk_q_used = cq;
    return DSA_OK;
}

dsa_status dsa_sparse_attn_bwd(const void* q, const void* k, const void* v, const int32_t* idx,
                               const void* out, const void* dout, const float* lse, int64_t s_q,
                               int64_t s_k, int64_t q_pos0, int h, int d, int dv, int k_pools,
                               int pool_size, int n_tail, float softmax_scale, int64_t chunk_q,
                               float* dq, float* dk, float* dv_grad, void* workspace,
                               size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    dsa_status st = check_attn_shape(s_q, s_k, q_pos0, h, d, dv, k_pools, pool_size, n_tail,
                                     softmax_scale);
    if (st != DSA_OK) return st;
    if (s_q > 0 && (!q || !idx || !out || !dout || !lse || !dq))
        return fail(DSA_ERR_INVALID_ARG, "q, idx, out, dout, lse and dq must be non-null");
    if (s_k > 0 && (!dk || !dv_grad)) return fail(DSA_ERR_INVALID_ARG, "dk and dv must be non-null");
    if (s_k > 0 && s_q > 0 && (!k || !v)) return fail(DSA_ERR_INVALID_ARG, "k and v must be non-null");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(idx) || !aligned16(out) ||
        !aligned16(dout) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv_grad) || !aligned16(workspace))
        return fail(DSA_ERR_INVALID_ARG, "all buffers must be 16-byte aligned");
    int64_t cq, db, bb;
    st = bwd_layout(s_q, s_k, h, chunk_q, &cq, &db, &bb);
    if (st != DSA_OK) return st;
    if (s_q > 0 && (!workspace || workspace_bytes < (size_t)(db + bb)))
        return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %lld needed",
                    workspace_bytes, (long long)(db + bb));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (s_q == 0) {
        // no query: the key and value gradients are zero
        hipError_t e = dsa::launch_fill_f32(dk, s_k * d, 0.0f, s);
        if (e == hipSuccess) e = dsa::launch_fill_f32(dv_grad, s_k * dv, 0.0f, s);
        if (e != hipSuccess) return hip_fail(e, "fill launch");
        return DSA_OK;
    }
    dsa::AttnBwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.out = static_cast<const uint16_t*>(out);
    a.dout = static_cast<const uint16_t*>(dout);
    a.idx = idx;
    a.lse = lse;
    a.s_q = s_q;
    a.s_k = s_k;
    a.q_pos0 = q_pos0;
    a.h = h;
    a.d = d;
    a.dv = dv;
    a.k_pools = k_pools;
    a.n_tail = n_tail;
    a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)d);
    a.dq = dq;
    a.dk = dk;
    a.dv_grad = dv_grad;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    a.delta = reinterpret_cast<float*>(ws);
    a.bits = reinterpret_cast<uint32_t*>(ws + db);
    a.stride = round_up((s_k + 3) / 4, 4);
    const int64_t chunk_bits = a.stride * (cq / 32) * 4;
    const int64_t nchunks = (s_q + cq - 1) / cq;
    const bool all_bits = chunk_bits * nchunks <= kBwdBitmapAll;
    const int64_t bitmap_bytes = round_up(all_bits ? chunk_bits * nchunks : chunk_bits, 256);
    const int64_t slot_bytes = round_up(a.stride * 4, 256);
    a.slot_counts = reinterpret_cast<uint32_t*>(ws + db + bitmap_bytes);
    a.slot_perm = reinterpret_cast<int32_t*>(ws + db + bitmap_bytes + slot_bytes);
    {
        Timed tm(K_BWD_DQ, s);
        hipError_t e = dsa::launch_attn_bwd_dq(a, s);
        if (e != hipSuccess) return hip_fail(e, "attn_bwd_dq launch");
    }
    if (s_k == 0) return DSA_OK;
    // the bitmap word rows of chunk query rows from r0 on (every chunk's
    // rows in one array when they fit, else the one chunk's)
    uint32_t* const bits0 = a.bits;
    auto chunk_bits_at = [&](int64_t r0) {
        return all_bits ? bits0 + (r0 / 32) * a.stride : bits0;
    };
    {
        // every chunk's bitmap when they fit (one launch); the pool groups
        // (slots in fours, those kept by the most queries first) come from
        // the selections of the last chunk_q queries
        // (from a word boundary: they see every pool the others see, and a
        // short last chunk does not make the order arbitrary), built on their
        // own when the bitmaps do not fit
        Timed tm(K_BWD_BITS, s);
        const int64_t w0 = s_q > cq ? round_up(s_q - cq, 32) : 0;
        hipError_t e;
        if (all_bits) {
            a.bits = bits0;
            e = dsa::launch_attn_bwd_bits(a, 0, (int)s_q, s);
            a.bits = bits0 + (w0 / 32) * a.stride;
        } else {
            a.bits = bits0;
            e = dsa::launch_attn_bwd_bits(a, w0, (int)(s_q - w0), s);
        }
        if (e == hipSuccess) e = dsa::launch_attn_bwd_order(a, (int)(s_q - w0), s);
        if (e != hipSuccess) return hip_fail(e, "attn_bwd_select launch");
    }
    for (int64_t r0 = 0, c = 0; r0 < s_q; r0 += cq, ++c) {
        const int rows = (int)(s_q - r0 < cq ? s_q - r0 : cq);
        a.bits = chunk_bits_at(r0);
        if (!all_bits) {
            Timed tm(K_BWD_BITS, s);
            hipError_t e = dsa::launch_attn_bwd_bits(a, r0, rows, s);
            if (e != hipSuccess) return hip_fail(e, "attn_bwd_select launch");
        }
        Timed tm(K_BWD_DKV, s);
        hipError_t e = dsa::launch_attn_bwd_dkv(a, r0, rows, c > 0 ? 1 : 0, s);
        if (e != hipSuccess) return hip_fail(e, "attn_bwd_dkv launch");
    }
    return DSA_OK;
}

dsa_status dsa_profile_enable(int on) {
    g_err[0] = 0;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.on = on != 0;
    return DSA_OK;
}

dsa_status dsa_profile_read(dsa_kernel_stat* stats, int max_stats, int* n_stats) {
    g_err[0] = 0;
    if (!n_stats || (max_stats > 0 && !stats) || max_stats < 0)
        return fail(DSA_ERR_INVALID_ARG, "bad output arguments");
    std::vector<Rec> recs;
    {
        std::lock_guard<std::mutex> lk(g_prof.mu);
        recs.swap(g_prof.recs);
    }
    int64_t launches[K_COUNT] = {0};
    double total[K_COUNT] = {0};
    dsa_status st = DSA_OK;
    for (const Rec& r : recs) {
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess && st == DSA_OK) st = hip_fail(e, "profile event");
        launches[r.kind] += 1;
        total[r.kind] += ms;
    }
    {
        std::lock_guard<std::mutex> lk(g_prof.mu);
        for (const Rec& r : recs) {
            g_prof.pool.push_back(r.a);
            g_prof.pool.push_back(r.b);
        }
    }
    int n = 0;
    for (int kd = 0; kd < K_COUNT; ++kd) {
        if (launches[kd] == 0) continue;
        if (n < max_stats) {
            memset(&stats[n], 0, sizeof stats[n]);
            strncpy(stats[n].name, kKindName[kd], sizeof stats[n].name - 1);
            stats[n].launches = launches[kd];
            stats[n].total_ms = total[kd];
        }
        ++n;
    }
    *n_stats = n < max_stats ? n : max_stats;
    return st;
}

}  // extern "C"
