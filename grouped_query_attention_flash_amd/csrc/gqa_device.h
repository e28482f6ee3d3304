// Device-side helpers shared by the forward and backward kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;  // log2(e)
constexpr float kLn2 = 0.6931471805599453f;    // ln(2)
// The online softmax moves its reference max only when a row max grows by more
// than this many powers of two, so unnormalised weights stay below 2^8.
constexpr float kRescaleLog2 = 8.0f;

// D = A * B + C on a 32x32 fp32 tile, A 32x16 and B 16x32 in bf16.
// Operand layout (64-wide wave): lane l holds A[l%32][8*(l/32) .. +7] and
// B[8*(l/32) .. +7][l%32]; result register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator tile held by register r of a lane in half c (= lane / 32).
__device__ __forceinline__ constexpr int acc_row(int r, int c) { return 8 * (r >> 2) + 4 * c + (r & 3); }

// XOR swizzle of 16-byte chunks inside one LDS row of CPR chunks. Rows
// r..r+15 (aligned) map one logical chunk to 16 distinct chunk slots, and
// 4 consecutive rows x 4 consecutive chunks (the transpose-read footprint)
// land in distinct 64-byte bank groups.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CPR >= 16)
        return ((r & 3) << 2) | ((r >> 2) & 3);
    else
        return ((r & 3) << 1) | ((r >> 2) & 1);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group,
// lane j receives element (j % 4) of the 4-element chunks addressed by the
// group's lanes j/4, 4 + j/4, 8 + j/4 and 12 + j/4, in that order.
__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

// Two 4 x 16-bit transpose-read results as one 8-element bf16 MFMA operand
// (whole-vector bit casts; lo fills elements 0..3, hi 4..7).
__device__ __forceinline__ bf16x8 join_bf16x8(const s16x4 &lo, const s16x4 &hi) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const i32x2 a = __builtin_bit_cast(i32x2, lo);
    const i32x2 b = __builtin_bit_cast(i32x2, hi);
    const i32x4 w = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
    return x;
}

}  // namespace gqa
