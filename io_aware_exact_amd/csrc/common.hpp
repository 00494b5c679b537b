// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// Reinterpret one 32-bit word as two bf16 (the word is taken by value: a
// bit_cast applied directly to an ext-vector element lvalue is not safe).
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane helpers (wave64).
__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask); }

// v_permlane32_swap exchanges the two 32-lane halves between its two
// operands; combining both results gives every lane f(x[l], x[l ^ 32]).
__device__ __forceinline__ float half_swap_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                    false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float half_swap_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                    false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero, which gives ragged tiles their zero fill for free.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane from the buffer straight into LDS: lane i's bytes land at
// lds_base + 16 * i (lds_base is wave-uniform); out-of-range offsets write zeros.
__device__ __forceinline__ void buffer_load_lds_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, (int)voff, 0, 0, 0);
}

// The same with the non-temporal cache policy, for data streamed exactly once
// (a decode step's K/V cache): the lines are not kept in L2/MALL.
__device__ __forceinline__ void buffer_load_lds_b128_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, (int)voff, 0, 0, 2 /* nt */);
}

// s_waitcnt vmcnt(N) (other counters untouched); gfx9 encoding of the immediate.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N & 0x30) << 10) | (0x7 << 4) | (0xF << 8));
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 8-byte pieces addressed by lanes 4r + i/4, r = 0..3.
// Four of them, at per-lane LDS addresses a0..a3 plus the immediate offsets
// O0..O3, and the wait for them, in one asm statement: the results are
// complete before the compiler can read or reuse their registers, and the
// outputs are early-clobber so no address register is overwritten while a
// read is in flight.  r0 = (read 0, read 1) and r1 = (read 2, read 3), two
// MFMA operands.  Inline asm because the compiler would otherwise wait for
// every outstanding LDS DMA before each read (it cannot see that the rings'
// stages do not overlap).
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_read_tr16_x4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, u32x4_t& r0,
                                                 u32x4_t& r1) {
    u32x2_t v0, v1, v2, v3;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
        "ds_read_b64_tr_b16 %1, %5 offset:%9\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:%10\n\t"
        "ds_read_b64_tr_b16 %3, %7 offset:%11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "i"(O0), "i"(O1), "i"(O2), "i"(O3));
    r0 = u32x4_t{v0[0], v0[1], v1[0], v1[1]};
    r1 = u32x4_t{v2[0], v2[1], v3[0], v3[1]};
}
// Eight of them and one wait, the same way: r[i] = (read 2i, read 2i + 1).
template <int O0, int O1, int O2, int O3, int O4, int O5, int O6, int O7>
__device__ __forceinline__ void lds_read_tr16_x8(const uint32_t (&a)[8], u32x4_t (&r)[4]) {
    u32x2_t v0, v1, v2, v3, v4, v5, v6, v7;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%17\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%18\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%19\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%20\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%21\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%22\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%23\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6), "=&v"(v7)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(O0), "i"(O1),
          "i"(O2), "i"(O3), "i"(O4), "i"(O5), "i"(O6), "i"(O7));
    r[0] = u32x4_t{v0[0], v0[1], v1[0], v1[1]};
    r[1] = u32x4_t{v2[0], v2[1], v3[0], v3[1]};
    r[2] = u32x4_t{v4[0], v4[1], v5[0], v5[1]};
    r[3] = u32x4_t{v6[0], v6[1], v7[0], v7[1]};
}


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
