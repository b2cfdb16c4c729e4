// fa_common.h -- types and wavefront helpers shared by the gfx950 attention kernels.
//
// MFMA operand layouts used throughout (gfx950, wave64; checked on hardware):
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l%32][(l/32)*8 + j], j = 0..7   (8 bf16)
//     B: lane l holds B[(l/32)*8 + j][l%32], j = 0..7   (8 bf16)
//     C: lane l, register i holds C[8*(i/4) + 4*(l/32) + i%4][l%32], i = 0..15
//   v_mfma_f32_32x32x2_f32    C[32x32] += A[32x2] * B[2x32]
//     A: lane l holds A[l%32][l/32];  B: lane l holds B[l/32][l%32];  C as above.
//
// Every kernel computes the TRANSPOSED score tile S^T = K Q^T so that one lane
// column is one query row: a row's statistics live in one lane and its partner
// lane l^32, and the output accumulator O^T = V^T P^T takes P^T straight from
// the score registers (see the key-slot permutation in the forward kernel).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_exp_f32 computes 2^x (exp2(-inf) = 0); v_log_f32 computes log2(x).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Combine a value with the one held by lane l^32 (v_permlane32_swap).  Both
// lanes of a pair see the operands in the same order, so both get bitwise
// identical results.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32_32x32x2(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row (key or query) held by register i of lane half h in a 32x32 C tile.
__device__ __forceinline__ constexpr int c_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// Key-slot permutation inside each group of 16 keys: swap bits 2 and 3.
// The P^T operand of k-step s (16 keys) is taken from score registers whose
// keys are 16s + 8*(j/4) + 4h + j%4; storing V^T at slot(key) makes those eight
// keys contiguous (slots 16s + 8h + j), so one 16-byte LDS read feeds V^T.
__device__ __forceinline__ constexpr int key_slot(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

}  // namespace fa
