// Peak probes for the measurement (not part of the DSA path): the rates the
// chip sustains on this machine, next to the published ones.
//   mfma loop  -- back-to-back matrix-core instructions, bf16 32x32x16 or
//                 scaled fp8 32x32x64, four independent accumulator chains
//                 per wave so that no instruction waits on another, on every
//                 SIMD (four waves per SIMD); operands vary by lane.
//   copy       -- a 16-byte-per-lane device copy, src -> dst.
//   read       -- 16-byte-per-lane reads of a buffer, `passes` times over;
//                 a buffer that fits the L2s (each XCD keeps the part its
//                 workgroups read) measures L2 read bandwidth, a large one
//                 read once measures memory read bandwidth.
// The caller times one launch with events on `stream`; the library returns
// the algorithmic work of that launch.
//   e4m3       -- not a rate: the matrix-core E4M3 conversions the query
//                 packing uses (v_cvt_pk_fp8_f32, v_cvt_f32_fp8) applied to
//                 a caller's list of floats, for a test against the
//                 definition of the format.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;
constexpr int kWorkgroups = 1024;  // 256 CUs x 4 workgroups of 4 waves

template <bool FP8>
__global__ __launch_bounds__(256) void mfma_loop(int iters, float* sink) {
    const uint32_t lane = threadIdx.x & 63;
    // small finite operands that differ by lane: bf16 1 + lane/256, or E4M3
    // codes near 1; the sums stay far from overflow
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
    if constexpr (FP8) {
        const uint32_t b = 0x38u + (lane & 7u);  // E4M3 1.0 .. 1.875
        const int w = (int)(b | (b << 8) | (b << 16) | (b << 24));
        const i32x8 a8 = {w, w, w, w, w, w, w, w};
        const i32x8 b8 = {w ^ 0x01010101, w, w, w, w, w, w, w ^ 0x01010101};
        for (int i = 0; i < iters; ++i)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 0, 0, 0,
                                                                         121, 0, 121);
    } else {
        const uint32_t h = 0x3F80u + lane;  // bf16 1 + lane / 128
        const uint32_t w = h | (h << 16);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w, w, w, w});
        const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{w ^ 1u, w, w, w ^ 0x10000u});
        for (int i = 0; i < iters; ++i)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[c][v];
    if (s == -1.0f) sink[blockIdx.x * 256 + threadIdx.x] = s;  // never true; keeps the loop
}

__global__ __launch_bounds__(256) void copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                              int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read16(const u32x4* __restrict__ src, int64_t n, int passes,
                                              uint32_t* sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int p = 0; p < passes; ++p) {
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
             i += (int64_t)gridDim.x * 256)
            acc += src[i];
        asm volatile("" ::: "memory");  // every pass reads again
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9E3779B9u) sink[threadIdx.x] = acc[0];
}

// code[i] = the E4M3 code v_cvt_pk_fp8_f32 gives x[i]; value[i] = that
// code decoded by v_cvt_f32_fp8.
__global__ __launch_bounds__(256) void e4m3_round_trip(const float* x, uint8_t* code,
                                                       float* value, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int c = __builtin_amdgcn_cvt_pk_fp8_f32(x[i], 0.0f, 0, false) & 0xFF;
        code[i] = (uint8_t)c;
        value[i] = __builtin_amdgcn_cvt_f32_fp8(c, 0);
    }
}

}  // namespace

extern "C" {

// kind 0: bf16, 1: fp8.  sink: device memory of 1024 x 256 floats (never
// written in practice).  *flops receives the launch's matrix-core flops.
int dsa_probe_mfma(int kind, int iters, float* sink, double* flops, void* stream) {
    if ((kind != 0 && kind != 1) || iters < 1 || !sink || !flops) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (kind == 0) mfma_loop<false><<<kWorkgroups, 256, 0, s>>>(iters, sink);
    else mfma_loop<true><<<kWorkgroups, 256, 0, s>>>(iters, sink);
    const double per = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
    *flops = per * kChains * (double)iters * kWorkgroups * 4;
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// bytes: a multiple of 16; src, dst 16-byte aligned device buffers.
int dsa_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (!src || !dst || bytes <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) ||
        (reinterpret_cast<uintptr_t>(dst) & 15))
        return 1;
    copy16<<<256 * 16, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// bytes: a multiple of 16; src 16-byte aligned; sink: 256 uint32 of device
// memory (never written in practice).  Reads the buffer `passes` times.
int dsa_probe_read(const void* src, int64_t bytes, int passes, uint32_t* sink, void* stream) {
    if (!src || !sink || bytes <= 0 || (bytes & 15) || passes < 1 ||
        (reinterpret_cast<uintptr_t>(src) & 15))
        return 1;
    read16<<<256 * 8, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(src), bytes / 16, passes, sink);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// x: n floats; code: n bytes; value: n floats (device memory).
int dsa_probe_e4m3(const float* x, uint8_t* code, float* value, int64_t n, void* stream) {
    if (!x || !code || !value || n < 0) return 1;
    if (n == 0) return 0;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    e4m3_round_trip<<<(unsigned)blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(x, code, value, n);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
