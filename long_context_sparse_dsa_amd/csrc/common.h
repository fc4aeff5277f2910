// Device-side helpers shared by the libdsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ldg16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Orderable key of an fp32 value: larger float <=> larger unsigned key.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
    uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(b);
}

// A zero score is stored as +0.0 so that its order key is unique.
__device__ __forceinline__ float canonical_zero(float x) { return x == 0.0f ? 0.0f : x; }

// max(x, 0) as one integer max: a non-negative float's bits are a
// non-negative int, a negative float's (and -0.0's) a negative one.
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// x[l] + x[l ^ 32] on every lane l (both halves add low half + high half).
__device__ __forceinline__ float add_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt immediate that waits until at most n vector memory operations
// are outstanding (0 <= n < 64), leaving the other counters alone.
__host__ __device__ constexpr int vmcnt_imm(int n) {
    return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00;
}

// Byte address of an LDS object in the LDS aperture.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global -> LDS loads: lane l of the wave reads `size` bytes at its
// own global address and writes them to LDS at lds + l * size (lds is
// wave-uniform).  Issued as inline assembly so that the compiler does not
// serialise them against later LDS reads and barriers; the caller orders
// them with explicit memory-counter waits.  M0 takes the LDS base (one
// wait state between the M0 write and the load).
__device__ __forceinline__ void lds_load16(const void* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void lds_load4(const void* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// The same with a wave-uniform base address (SGPR pair) and a 32-bit
// per-lane offset, so that moving to the next tile is scalar arithmetic.
__device__ __forceinline__ void lds_load16_sv(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void lds_load4_sv(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// XCD-aware workgroup order.  The dispatcher deals workgroups of a launch to
// the chip's 8 XCDs round-robin by linear id, and each XCD has its own L2.
// The logical id returned here makes every XCD walk one contiguous range of
// the launch (x fastest): workgroups that share input rows (same y) then run
// on the same XCD and share its L2.  Bijective for any grid size.
__device__ __forceinline__ void xcd_block(int& bx, int& by) {
    const int gx = (int)gridDim.x;
    const int n = gx * (int)gridDim.y;
    const int h = (int)blockIdx.y * gx + (int)blockIdx.x;
    const int q = n >> 3, r = n & 7, k = h & 7;
    const int logical = k * q + min(k, r) + (h >> 3);
    bx = logical % gx;
    by = logical / gx;
}

// Two half-wave sums at once: lanes 0-31 get x0[l] + x0[l + 32], lanes 32-63
// get x1[l - 32] + x1[l] (the swap exchanges x0's upper half with x1's lower).
__device__ __forceinline__ float add_halves2(float x0, float x1) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x1),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace dsa
