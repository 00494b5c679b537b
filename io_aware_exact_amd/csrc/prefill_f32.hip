// Exact attention forward with fp32 inputs and outputs, gfx950 (the exact
// path: no reduced-precision products anywhere).
//
// One wave per workgroup owns 64 / TPQ query rows (TPQ = 1 lane per row for
// head width <= 64, 2 lanes per row for 128).  Key/value blocks of 64 rows are
// staged in LDS and every lane reads them with broadcast loads; scores are
// formed 16 keys at a time with fp32 FMAs and folded into the running max /
// running sum / running output of "IO-Aware Attention: Tiling the Score
// Matrix Without Materializing It", section "Softmax over blocks, exactly".
// Accumulation and rescaling are fp32 throughout (same article, section
// "Where the approach stops helping", last paragraph).
#include "common.hpp"
#include "launch.hpp"

namespace attn {
namespace {

constexpr int BK = 64;
constexpr int CH = 16;   // keys scored per inner step

template <int D>
__global__ __launch_bounds__(64)
void prefill_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                        const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                        int Tq, int Tkv, int BH, int causal, float c) {
    constexpr int TPQ = (D > 64) ? 2 : 1;
    constexpr int DPT = D / TPQ;
    constexpr int QPW = 64 / TPQ;
    __shared__ __attribute__((aligned(16))) float Ks[BK][D];
    __shared__ __attribute__((aligned(16))) float Vs[BK][D];

    const int lane = threadIdx.x;
    const int bh = blockIdx.x % BH;
    const int qt = blockIdx.x / BH;
    const int q0 = qt * QPW;
    const int qrow = q0 + lane / TPQ;
    const int part = lane % TPQ;
    const int off = Tkv - Tq;

    const size_t qbase = (size_t)bh * Tq * D;
    const size_t kvbase = (size_t)bh * Tkv * D;

    float q[DPT], o[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
        q[i] = (qrow < Tq) ? Q[qbase + (size_t)qrow * D + part * DPT + i] : 0.f;
        o[i] = 0.f;
    }
    float m = kNegInf, l = 0.f;

    const int kend = causal ? min(Tkv, q0 + QPW + off) : Tkv;
    const int lim = causal ? min(Tkv - 1, qrow + off) : Tkv - 1;

    for (int kb = 0; kb < kend; kb += BK) {
        __syncthreads();
        for (int e = lane * 4; e < BK * D; e += 64 * 4) {
            const int row = e / D, col = e % D;
            f32x4_t kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (kb + row < Tkv) {
                kv = *reinterpret_cast<const f32x4_t*>(K + kvbase + (size_t)(kb + row) * D + col);
                vv = *reinterpret_cast<const f32x4_t*>(V + kvbase + (size_t)(kb + row) * D + col);
            }
            *reinterpret_cast<f32x4_t*>(&Ks[row][col]) = kv;
            *reinterpret_cast<f32x4_t*>(&Vs[row][col]) = vv;
        }
        __syncthreads();
        for (int k0 = 0; k0 < BK && kb + k0 < kend; k0 += CH) {
            float s[CH];
            float mx = kNegInf;
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < DPT; ++i) acc = __builtin_fmaf(q[i], Ks[k0 + t][part * DPT + i], acc);
                if constexpr (TPQ == 2) acc += xor_lane(acc, 1);
                s[t] = (kb + k0 + t <= lim) ? acc * c : kNegInf;
                mx = fmaxf(mx, s[t]);
            }
            const float m_new = fmaxf(m, mx);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2(m - m_use);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < DPT; ++i) o[i] *= alpha;
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const float p = fast_exp2(s[t] - m_use);
                l += p;
#pragma unroll
                for (int i = 0; i < DPT; ++i) o[i] = __builtin_fmaf(p, Vs[k0 + t][part * DPT + i], o[i]);
            }
            m = m_new;
        }
    }
    if (qrow < Tq) {
        const float inv = 1.0f / l;
#pragma unroll
        for (int i = 0; i < DPT; ++i) O[qbase + (size_t)qrow * D + part * DPT + i] = o[i] * inv;
        if (LSE != nullptr && part == 0)
            LSE[(size_t)bh * Tq + qrow] = (m + __builtin_log2f(l)) * 0.69314718055994530942f;
    }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
    constexpr int QPW = 64 / ((D > 64) ? 2 : 1);
    const int nqt = (a.Tq + QPW - 1) / QPW;
    const long long grid = (long long)nqt * a.B * a.H;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_f32_kernel<D>), dim3((unsigned)grid), dim3(64), 0, stream,
                       static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.Tq, a.Tkv,
                       a.B * a.H, a.causal ? 1 : 0, a.c);
    return hipGetLastError();
}

}  // namespace

bool prefill_f32_supports(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream, const char** name) {
    switch (a.d) {
        case 16: *name = "prefill_f32_d16<bq=64,bk=64>"; return launch_d<16>(a, stream);
        case 32: *name = "prefill_f32_d32<bq=64,bk=64>"; return launch_d<32>(a, stream);
        case 64: *name = "prefill_f32_d64<bq=64,bk=64>"; return launch_d<64>(a, stream);
        case 128: *name = "prefill_f32_d128<bq=32,bk=64>"; return launch_d<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
