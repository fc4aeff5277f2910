// Host-side paths of the libdsa C ABI (workspace sizing, argument checks,
// profiling bookkeeping, the no-allocation entry point's size checks), for a
// build whose host code runs under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  No call here reaches
// a kernel launch: every rejected call returns before touching the device,
// and the pointers passed are never dereferenced.  Exit status 0: every call
// returned the expected status.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dsa.h"

static int failures = 0;
#define EXPECT(call, want)                                                                    \
    do {                                                                                      \
        const int got_ = (int)(call);                                                         \
        if (got_ != (int)(want)) {                                                            \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__,  \
                    #call, got_, (int)(want), dsa_last_error());                              \
            ++failures;                                                                       \
        }                                                                                     \
    } while (0)

int main() {
    void* p = reinterpret_cast<void*>(uintptr_t(4096));  // aligned, never dereferenced
    const float* f = static_cast<const float*>(p);
    size_t bytes = 0;
    int64_t cq = 0;
    // workspace sizing over the supported shapes and the 1M-token cap
    const int heads[] = {4, 8, 16, 32}, dims[] = {64, 96, 128};
    for (int h : heads)
        for (int d : dims)
            for (int dt = 0; dt < 2; ++dt) {
                EXPECT(dsa_index_workspace_size(131072, 131072, h, d, 512, 4, 0, dt, &bytes, &cq), DSA_OK);
                EXPECT(dsa_index_workspace_size(131072, 1 << 20, h, d, 512, 4, 0, dt, &bytes, &cq), DSA_OK);
                EXPECT(dsa_index_scores_workspace_size(1000, 5000, h, d, 4, dt, 1000, &bytes), DSA_OK);
            }
    EXPECT(dsa_index_workspace_size(64, 1 << 20, 32, 128, 512, 4, 2112, 0, &bytes, &cq), DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_index_workspace_size(-1, 100, 32, 128, 512, 4, 0, 0, &bytes, &cq), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_index_workspace_size(64, 100, 32, 128, 512, 4, 0, 0, nullptr, &cq), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_sparse_attn_bwd_workspace_size(131072, 131072, 16, 0, &bytes, &cq), DSA_OK);
    EXPECT(dsa_sparse_attn_bwd_workspace_size(131072, 131072, 17, 0, &bytes, &cq), DSA_ERR_UNSUPPORTED);
    // rejected before any launch
    EXPECT(dsa_index_score_topk(p, p, nullptr, nullptr, f, 0, 64, 4096, 0, 12, 128, 4, 16, 0, 0,
                                static_cast<int32_t*>(p), nullptr, p, 1 << 20, nullptr),
           DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_index_score_topk(p, p, nullptr, nullptr, f, 0, 64, 4096, 0, 32, 128, 4, 16, 0, 0,
                                static_cast<int32_t*>(p), nullptr, p, 16, nullptr),
           DSA_ERR_WORKSPACE);
    EXPECT(dsa_index_score_topk(nullptr, p, nullptr, nullptr, f, 0, 64, 4096, 0, 32, 128, 4, 16, 0,
                                0, static_cast<int32_t*>(p), nullptr, p, 1 << 30, nullptr),
           DSA_ERR_INVALID_ARG);
    EXPECT(dsa_index_score_topk_gated(p, p, nullptr, nullptr, nullptr, f, 0, 64, 4096, 0, 32, 128,
                                      4, 16, 0, 0, static_cast<int32_t*>(p), nullptr, p, 1 << 30,
                                      nullptr),
           DSA_ERR_INVALID_ARG);
    EXPECT(dsa_index_scores(p, p, nullptr, nullptr, f, 0, 64, 4096, 0, 32, 128, 4, 0, 60, 10,
                            static_cast<float*>(p), p, 1 << 30, nullptr),
           DSA_ERR_INVALID_ARG);
    EXPECT(dsa_sparse_attn_fwd(p, p, p, static_cast<const int32_t*>(p), 64, 4096, 0, 17, 128, 128,
                               512, 4, 0, 0.0f, p, nullptr, nullptr),
           DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_sparse_attn_fwd(p, p, p, static_cast<const int32_t*>(p), 64, 4096, 0, 16, 128, 128,
                               512, 4, 4, 0.0f, p, nullptr, nullptr),
           DSA_ERR_INVALID_ARG);
    EXPECT(dsa_sparse_attn_bwd(p, p, p, static_cast<const int32_t*>(p), p, p, nullptr, 64, 4096,
                               0, 16, 128, 128, 512, 4, 0, 0.0f, 0, static_cast<float*>(p),
                               static_cast<float*>(p), static_cast<float*>(p), p, 1 << 30, nullptr),
           DSA_ERR_INVALID_ARG);
    // no query: nothing to launch
    EXPECT(dsa_index_score_topk(p, p, nullptr, nullptr, f, 0, 0, 4096, 0, 32, 128, 4, 16, 0, 0,
                                nullptr, nullptr, nullptr, 0, nullptr),
           DSA_OK);
    // the no-allocation entry point: its size checks come first
    EXPECT(dsa_index_score_topk_noalloc(p, p, nullptr, nullptr, f, 0, 64, 1 << 21, 0, 32, 128, 4,
                                        512, 0, 0, static_cast<int32_t*>(p), nullptr, nullptr),
           DSA_ERR_UNSUPPORTED);
    EXPECT(dsa_index_score_topk_noalloc(p, p, nullptr, nullptr, f, 0, 8192, 131072, 0, 32, 128, 4,
                                        512, 8192, 0, static_cast<int32_t*>(p), nullptr, nullptr),
           DSA_ERR_WORKSPACE);
    // an error message longer than the buffer is truncated, not overrun
    char big[64];
    memset(big, 'x', sizeof big);
    EXPECT(dsa_index_workspace_size(64, 100, 32, 128, 512, 4, -64, 0, &bytes, &cq), DSA_ERR_INVALID_ARG);
    if (strlen(dsa_last_error()) == 0) ++failures;
    // profiling bookkeeping without any launch
    dsa_kernel_stat st[8];
    int n = -1;
    EXPECT(dsa_profile_enable(1), DSA_OK);
    EXPECT(dsa_profile_read(st, 8, &n), DSA_OK);
    EXPECT(n, 0);
    EXPECT(dsa_profile_read(nullptr, 8, &n), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_profile_enable(0), DSA_OK);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    puts("abi driver: ok");
    return 0;
}
