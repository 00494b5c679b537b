// Matrix-pipe throughput probe for gfx950 (a measurement aid for the
// benchmark, not part of the attention library): every wave issues four
// independent chains of v_mfma_f32_32x32x16_bf16 from register operands, so
// nothing but the matrix pipe and the clock it runs at bounds the rate.  The
// benchmark times a launch of it beside the attention kernels to report the
// bf16 MFMA rate the chip sustains under load, next to the 2.5 PFLOP/s
// quoted at the 2.4 GHz peak clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads)
void mfma_loop_kernel(int iters, float* __restrict__ out) {
    const int tid = threadIdx.x;
    f32x8_t fa, fb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        fa[i] = 1e-3f * (float)((tid + i) & 15);
        fb[i] = 1e-3f * (float)((tid * 3 + i) & 15);
    }
    const bf16x8_t a = __builtin_convertvector(fa, bf16x8_t);
    const bf16x8_t b = __builtin_convertvector(fb, bf16x8_t);
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[(size_t)blockIdx.x * kThreads + tid] = s;   // keeps the chains live
}

}  // namespace

extern "C" {

// Flops of one launch: blocks * (kThreads / 64) waves * iters * 4 MFMAs * 32*32*16*2.
double probe_mfma_loop_flops(int blocks, int iters) {
    return (double)blocks * (kThreads / 64) * (double)iters * 4.0 * 32.0 * 32.0 * 16.0 * 2.0;
}

// Threads per block; `out` must hold blocks * probe_mfma_loop_threads() floats.
int probe_mfma_loop_threads(void) { return kThreads; }

// Enqueue one launch on `stream`; returns the hipError_t of the launch.
int probe_mfma_loop(int blocks, int iters, float* out, hipStream_t stream) {
    if (blocks < 1 || iters < 1 || out == nullptr) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, iters, out);
    return (int)hipGetLastError();
}

}  // extern "C"
