// Shared device helpers for the gfx950 kernels (64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace minikv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Copy an element of these vectors to a scalar before __builtin_bit_cast: with
// the element expression itself as the operand (bit_cast(float, v[1])), this
// compiler has been seen to read element 0.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kGroup = 32;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// fp16 bits -> fp32 (exact, subnormals kept)
__device__ __forceinline__ float half_bits_to_f32(uint32_t h16) {
    __half h;
    __builtin_memcpy(&h, &h16, 2);
    return __half2float(h);
}

// fp32 -> fp16 bits, IEEE round-half-even, subnormals kept
__device__ __forceinline__ uint32_t f32_to_half_bits_rn(float f) {
    __half h = __float2half_rn(f);
    uint16_t b;
    __builtin_memcpy(&b, &h, 2);
    return b;
}

// Value of lane (lane ^ 32): one permlane32 swap.
__device__ __forceinline__ float swap_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Sum over aligned groups of W lanes (W = 2, 4, 8, 16, 32 or 64) with DPP and
// permlane swaps: each step is one VALU op, no LDS crossbar traffic.
template <int W>
__device__ __forceinline__ float dpp_sum(float x) {
    if constexpr (W >= 2)   // xor 1: quad_perm [1,0,3,2]
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    if constexpr (W >= 4)   // xor 2: quad_perm [2,3,0,1]
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    if constexpr (W >= 8)   // other quad of the 8-lane half row: row_half_mirror
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    if constexpr (W >= 16)  // other half of the 16-lane row: row_mirror
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    if constexpr (W >= 32) {  // other 16-lane row of the 32-lane half
        auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
        x += __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
    }
    if constexpr (W >= 64) x += swap_halves(x);
    return x;
}
template <int W>
__device__ __forceinline__ float dpp_max(float x) {
    if constexpr (W >= 2)
        x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false)));
    if constexpr (W >= 4)
        x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)));
    if constexpr (W >= 8)
        x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)));
    if constexpr (W >= 16)
        x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)));
    if constexpr (W >= 32) {
        auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
        x = fmaxf(x, __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]));
    }
    if constexpr (W >= 64) x = fmaxf(x, swap_halves(x));
    return x;
}

// Minimum over aligned 16-lane rows (W = 2, 4, 8 or 16), DPP only.
template <int W>
__device__ __forceinline__ float dpp_min(float x) {
    static_assert(W <= 16, "row-local");
    if constexpr (W >= 2)
        x = fminf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false)));
    if constexpr (W >= 4)
        x = fminf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)));
    if constexpr (W >= 8)
        x = fminf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)));
    if constexpr (W >= 16)
        x = fminf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)));
    return x;
}

// Butterfly reductions over aligned lane groups of width W (W <= 32), via ds_swizzle-free shuffles.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
    return x;
}
template <int W>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
    return x;
}
template <int W>
__device__ __forceinline__ float group_min(float x) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o, kWave));
    return x;
}
template <int W>
__device__ __forceinline__ uint32_t group_or(uint32_t x) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) x |= (uint32_t)__shfl_xor((int)x, o, kWave);
    return x;
}

}  // namespace minikv
