// Instruction-mix probes for gfx950 (measurement aids for the benchmark, not
// part of the attention library).  Each kernel runs a loop with no memory
// traffic, so only issue, the VALU, the transcendental unit and the matrix
// pipe bound it.  Each workgroup of 4 waves reserves a share of the 160 KiB
// of LDS per compute unit that lets exactly w workgroups reside on one unit,
// so every SIMD holds w waves at a time however small the register use; the
// grid is many such rounds.  Every wave records the s_memtime (shader clock)
// and s_memrealtime (100 MHz) ticks its loop took, so the host reads the
// clock the loop ran at from their ratio.
//
// Modes (per loop iteration, 16 independent chains where it applies):
//   0  16 x (v_exp_f32 then v_mul_f32)          transcendental rate
//   1  16 x (v_fma_f32 then v_mul_f32)          plain VALU rate
//   2  2 x v_mfma_f32_32x32x16_bf16             matrix-pipe rate
//   3  mode 0 interleaved with 2 MFMAs           MFMA beside exp
//   4  mode 1 interleaved with 2 MFMAs           MFMA beside plain VALU
//   5  one key block of the head-width-64 prefill for 32 query rows, from
//      registers: 8 QK MFMAs, the softmax of 32 scores per lane (FMA, exp2,
//      row-sum adds, bf16 packs) and 8 PV MFMAs, with the kernel's data
//      dependences (the loop-carried accumulators and reference)
//   6  8 ds_read_b128 (1 KiB per wave each, consecutive 16-byte chunks per
//      lane: no bank conflicts) from the workgroup's LDS reservation, the
//      LDS read rate
//   7  the same 8 KiB per wave as 16 ds_read_b64_tr_b16: the transposing
//      read, with the head-width-64 prefill's V operand addressing (a 64-row
//      tile of 128-byte rows, 16-byte chunks XOR-swizzled by row bit 1)
// Issue-port cost (each against mode 13):
//   8  16 independent v_exp_f32                  transcendental rate alone
//   9  mode 8 beside 16 independent v_fma_f32    does the exp share the port
//  10  32 independent v_fma_f32 beside 2 v_mfma_f32_32x32x16_bf16
//  11  the same beside 4 of them                 port time per 32x32x16 MFMA
//  12  the same beside 4 v_mfma_f32_16x16x32_bf16 (half the flops each)
//  13  32 independent v_fma_f32                  the VALU baseline
#include <hip/hip_runtime.h>
#include <stdint.h>

// Every instantiation is compiled for 3 waves per SIMD, so the code is the
// same whatever occupancy the LDS reservation allows; the compiler's note that
// one or two waves per SIMD miss that target is expected.
#pragma clang diagnostic ignored "-Wpass-failed"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// LDS each workgroup reserves so that W (1..3) workgroups fit on a compute
// unit of 160 KiB and one more does not.
constexpr int reserve_floats(int W) { return (W == 1 ? 96 : W == 2 ? 64 : 48) * 256; }

template <int MODE, int W>
__global__ __launch_bounds__(kThreads, 3)
void issue_probe_kernel(int iters, const u32x4_t* __restrict__ operands, float* __restrict__ out,
                        long long* __restrict__ ticks) {
    __shared__ float reserve[reserve_floats(W)];   // occupancy limiter only
    const int tid = threadIdx.x;
    if constexpr (MODE == 6 || MODE == 7) {
        // fill the reservation once: the reads below see defined values
        for (int i = tid; i < reserve_floats(W); i += kThreads) reserve[i] = (float)(i & 255);
        __syncthreads();
    }
    if (iters < 0) {                     // never taken: keeps the reservation
        reserve[tid] = 0.f;
        __syncthreads();
        out[tid] = reserve[(tid + 1) % kThreads];
        return;
    }
    // 20 bf16x8 operands per lane (finite values from the caller)
    bf16x8_t q[4], k[8], v[8];
    const u32x4_t* src = operands + (tid & 63);
#pragma unroll
    for (int t = 0; t < 4; ++t) q[t] = __builtin_bit_cast(bf16x8_t, src[64 * t]);
#pragma unroll
    for (int t = 0; t < 8; ++t) k[t] = __builtin_bit_cast(bf16x8_t, src[64 * (4 + t)]);
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = __builtin_bit_cast(bf16x8_t, src[64 * (12 + t)]);
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = -1e-3f * (float)(tid + i);
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    f32x4_t e0 = {}, e1 = {}, e2 = {}, e3 = {};
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = 2e-3f * (float)(tid + 2 * i);
    float m = 0.5f, l = 0.f;
    const float c = 0.18f;
    const long long r0 = __builtin_amdgcn_s_memrealtime();
    const long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        if constexpr (MODE == 0 || MODE == 3) {
            if constexpr (MODE == 3) c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[0], q[0], c0, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) * -0.5f;
            if constexpr (MODE == 3) c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[1], q[1], c1, 0, 0, 0);
#pragma unroll
            for (int i = 8; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) * -0.5f;
        } else if constexpr (MODE == 1 || MODE == 4) {
            if constexpr (MODE == 4) c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[0], q[0], c0, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], -0.5f, 0.25f) * -0.5f;
            if constexpr (MODE == 4) c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[1], q[1], c1, 0, 0, 0);
#pragma unroll
            for (int i = 8; i < 16; ++i) x[i] = __builtin_fmaf(x[i], -0.5f, 0.25f) * -0.5f;
        } else if constexpr (MODE == 6) {
            // 8 KiB per wave per iteration; the offset walks the reservation
            constexpr int CHUNKS = reserve_floats(W) / 4;          // 16-byte chunks
            const u32x4_t* lds = reinterpret_cast<const u32x4_t*>(reserve);
            const int base = ((tid >> 6) * 512 + it * 64) % CHUNKS;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4_t v = lds[(base + 64 * i + (tid & 63)) % CHUNKS];
                x[2 * i] += __builtin_bit_cast(float, v[0] ^ v[1]);
                x[2 * i + 1] += __builtin_bit_cast(float, v[2] ^ v[3]);
            }
        } else if constexpr (MODE == 7) {
            // lane group lg = lane / 16 and jj = lane % 16 address row
            // 4(lg/2) + jj/4 and columns 32dt + 16(lg%2) + 4(jj%4) of the tile;
            // steps st = 0..3 add 16 rows, the second read of a pair 8 rows
            const int lane = tid & 63, lg = lane >> 4, jj = lane & 15;
            const int row = 4 * (lg >> 1) + (jj >> 2);
            const int tile = ((tid >> 6) + it) % (reserve_floats(W) / 2048);   // 8 KiB tiles
            __attribute__((address_space(3))) char* t0 =
                reinterpret_cast<__attribute__((address_space(3))) char*>(
                    (__attribute__((address_space(3))) float*)reserve) + 8192 * tile;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int st = i >> 2, dt = (i >> 1) & 1, half = i & 1;
                const int col = 32 * dt + 16 * (lg & 1) + 4 * (jj & 3);
                const int off = (16 * st + 8 * half + row) * 128 +
                                ((((col >> 3) ^ (((row >> 1) & 1) << 2)) << 4) | ((col & 4) << 1));
                const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    reinterpret_cast<__attribute__((address_space(3))) i16x4_t*>(t0 + off));
                x[i] += (float)(v[0] ^ v[1] ^ v[2] ^ v[3]);
            }
        } else if constexpr (MODE == 2) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[0], q[0], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[1], q[1], c1, 0, 0, 0);
        } else if constexpr (MODE == 8 || MODE == 9) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                x[i] = __builtin_amdgcn_exp2f(-x[i]);
                if constexpr (MODE == 9) y[i] = __builtin_fmaf(y[i], 0.999f, 1e-4f);
            }
        } else if constexpr (MODE >= 10 && MODE <= 13) {
            if constexpr (MODE == 10 || MODE == 11) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[0], q[0], c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[1], q[1], c1, 0, 0, 0);
            }
            if constexpr (MODE == 11) {
                c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[2], q[2], c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[3], q[3], c3, 0, 0, 0);
            }
            if constexpr (MODE == 12) {
                e0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[0], q[0], e0, 0, 0, 0);
                e1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[1], q[1], e1, 0, 0, 0);
                e2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[2], q[2], e2, 0, 0, 0);
                e3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[3], q[3], e3, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                x[i] = __builtin_fmaf(x[i], 0.999f, 1e-4f);
                y[i] = __builtin_fmaf(y[i], 0.999f, 1e-4f);
            }
        } else {   // 5
            asm volatile("" : "+v"(k[0]), "+v"(k[4]));   // opaque every iteration: nothing is hoisted
            f32x16_t s0 = {}, s1 = {};
#pragma unroll
            for (int t = 0; t < 4; ++t) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[t], q[t], s0, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 4; ++t) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[4 + t], q[t], s1, 0, 0, 0);
            float sv[32];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sv[r] = s0[r];
                sv[16 + r] = s1[r];
            }
            uint32_t pw[16];
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], c, -m));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], c, -m));
                pw[i] = pack2(p0, p1);
                rs += p0 + p1;
            }
            l += rs;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const u32x4_t pv = {pw[4 * st], pw[4 * st + 1], pw[4 * st + 2], pw[4 * st + 3]};
                const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
                c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[2 * st], pb, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[2 * st + 1], pb, c1, 0, 0, 0);
            }
            m += 1e-7f * l;    // loop-carried: the next block's reference depends on this one
        }
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    const long long r1 = __builtin_amdgcn_s_memrealtime();
    float sum = l + m;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += x[i] + y[i] + c0[i] + c1[i] + c2[i] + c3[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) sum += e0[i] + e1[i] + e2[i] + e3[i];
    out[(size_t)blockIdx.x * kThreads + tid] = sum;
    if ((tid & 63) == 0) {
        const size_t w = (size_t)blockIdx.x * (kThreads / 64) + (tid >> 6);
        ticks[2 * w] = t1 - t0;
        ticks[2 * w + 1] = r1 - r0;
    }
}

template <int MODE>
static hipError_t launch_mode(int waves, int blocks, int iters, const u32x4_t* ops, float* out, long long* ticks,
                              hipStream_t stream) {
    if (waves == 1)
        hipLaunchKernelGGL((issue_probe_kernel<MODE, 1>), dim3(blocks), dim3(kThreads), 0, stream, iters, ops, out, ticks);
    else if (waves == 2)
        hipLaunchKernelGGL((issue_probe_kernel<MODE, 2>), dim3(blocks), dim3(kThreads), 0, stream, iters, ops, out, ticks);
    else
        hipLaunchKernelGGL((issue_probe_kernel<MODE, 3>), dim3(blocks), dim3(kThreads), 0, stream, iters, ops, out, ticks);
    return hipGetLastError();
}

}  // namespace

extern "C" {

// Number of modes, and the bf16x8 operand words the caller provides
// (20 per lane of a wave: 20 * 64 * 16 bytes).
int probe_issue_modes(void) { return 14; }
int probe_issue_operand_bytes(void) { return 20 * 64 * 16; }
int probe_issue_threads(void) { return kThreads; }

// Enqueue one launch of mode `mode` on `stream` at `waves` (1..3) waves per
// SIMD: `blocks` workgroups of 256 threads (a multiple of the compute units
// times `waves` fills whole rounds), `iters` loop iterations each; `out`
// holds blocks * 256 floats and `ticks` blocks * 8 long longs (per wave: the
// s_memtime ticks, then the s_memrealtime ticks of its loop).  Returns the
// hipError_t of the launch; invalid arguments are refused before any launch.
int probe_issue(int mode, int waves, int blocks, int iters, const void* operands, float* out, long long* ticks,
                hipStream_t stream) {
    if (mode < 0 || mode > 13 || waves < 1 || waves > 3 || blocks < 1 || iters < 1 || !operands || !out || !ticks)
        return (int)hipErrorInvalidValue;
    const u32x4_t* ops = static_cast<const u32x4_t*>(operands);
    switch (mode) {
        case 0: return (int)launch_mode<0>(waves, blocks, iters, ops, out, ticks, stream);
        case 1: return (int)launch_mode<1>(waves, blocks, iters, ops, out, ticks, stream);
        case 2: return (int)launch_mode<2>(waves, blocks, iters, ops, out, ticks, stream);
        case 3: return (int)launch_mode<3>(waves, blocks, iters, ops, out, ticks, stream);
        case 4: return (int)launch_mode<4>(waves, blocks, iters, ops, out, ticks, stream);
        case 5: return (int)launch_mode<5>(waves, blocks, iters, ops, out, ticks, stream);
        case 6: return (int)launch_mode<6>(waves, blocks, iters, ops, out, ticks, stream);
        case 7: return (int)launch_mode<7>(waves, blocks, iters, ops, out, ticks, stream);
        case 8: return (int)launch_mode<8>(waves, blocks, iters, ops, out, ticks, stream);
        case 9: return (int)launch_mode<9>(waves, blocks, iters, ops, out, ticks, stream);
        case 10: return (int)launch_mode<10>(waves, blocks, iters, ops, out, ticks, stream);
        case 11: return (int)launch_mode<11>(waves, blocks, iters, ops, out, ticks, stream);
        case 12: return (int)launch_mode<12>(waves, blocks, iters, ops, out, ticks, stream);
        default: return (int)launch_mode<13>(waves, blocks, iters, ops, out, ticks, stream);
    }
}

}  // extern "C"
