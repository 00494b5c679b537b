// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

// Two fp32 values -> two bf16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// bf16 -> fp32 is exact: the bf16 bits are the upper half of the fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane helpers (wave64).
__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask); }

// DPP row-local exchanges: lanes are paired within rows of 16.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;            // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;            // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;     // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;         // lane i <-> 15-i within 16

// Sum over groups of N consecutive lanes (N in {2,4,8,16}); every lane of the
// group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group size");
    v += dpp_mov<kDppXor1>(v);
    if constexpr (N >= 4) v += dpp_mov<kDppXor2>(v);
    if constexpr (N >= 8) v += dpp_mov<kDppHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_mov<kDppMirror>(v);
    return v;
}

}  // namespace attn
