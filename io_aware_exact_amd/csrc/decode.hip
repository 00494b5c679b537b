// Exact attention for one query per (batch, head) against cached keys/values
// (decode), bf16 inputs, head width 64 or 128, gfx950.
//
// With a single query row there is nothing to tile in the query dimension and
// the work is a streaming reduction over the cache, bound by reading K and V
// once ("IO-Aware Attention: Tiling the Score Matrix Without Materializing
// It", section "Where the approach stops helping"; "Attention and Its
// Computational Cost", section "The other shape: one query, many keys").
// The key axis is split into P contiguous partitions, each reduced by its own
// workgroup to a partial output and normaliser, and a second kernel merges the
// partitions with the same rescaling ("IO-Aware Attention", section
// "Parallelism and the cost of the split").
//
// Split kernel, one workgroup per (batch*head, partition):
// * D/8 lanes share one key row: each lane holds 8 elements (16 bytes) of q
//   and of the key, so a wave load instruction reads whole contiguous key rows
//   (non-temporal: every byte is used once).
// * q.k: v_dot2_f32_bf16 on the packed bf16 pairs, then a DPP sum over the
//   D/8 lanes of the row.
// * Each group of D/8 lanes keeps its own running (m, l) and 8-wide output
//   slice, so the key loop has no cross-group traffic at all; groups and waves
//   are merged once at the end through LDS.
// * No LDS staging for K/V: nothing is reused, so loads go straight to VGPRs.
//
// Partial record per (batch*head, partition): o (D floats, not normalised),
// then m (max of scale*log2e*q.k) and l, all fp32.
#include "common.hpp"
#include "launch.hpp"

namespace attn {
namespace {

constexpr int NW = 4;        // waves per workgroup
constexpr int UNROLL = 8;    // key-row loads in flight per lane per operand

template <int D>
struct DecodeShape {
    static constexpr int LPK = D / 8;          // lanes per key row
    static constexpr int KPW = 64 / LPK;       // key rows per wave load
    static constexpr int GROUPS = NW * KPW;    // independent softmax states per workgroup
    static constexpr int STEP = NW * KPW * UNROLL;   // keys per workgroup iteration
};

template <int LPK>
__device__ __forceinline__ float row_sum(float v) { return group_sum<LPK>(v); }

template <int D>
__global__ __launch_bounds__(NW * 64)
void decode_split_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                         const uint16_t* __restrict__ V, float* __restrict__ part,
                         uint16_t* __restrict__ O, float* __restrict__ LSE,
                         int Tkv, int P, float c, int direct) {
    using S = DecodeShape<D>;
    constexpr int LPK = S::LPK, KPW = S::KPW, GROUPS = S::GROUPS, STEP = S::STEP;

    __shared__ float red_o[GROUPS][D];
    __shared__ float red_m[GROUPS];
    __shared__ float red_l[GROUPS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kr = lane / LPK;         // key slot inside one wave load
    const int dc = lane % LPK;         // which 8 elements of the row
    const int grp = wave * KPW + kr;   // softmax-state group

    const int bh = blockIdx.x;
    const int p = blockIdx.y;
    const long long lo = ((long long)p * Tkv) / P;
    const long long hi = ((long long)(p + 1) * Tkv) / P;

    const size_t kvbase = (size_t)bh * Tkv * D;
    const u32x4_t qw = *reinterpret_cast<const u32x4_t*>(Q + (size_t)bh * D + 8 * dc);

    float m = kNegInf, l = 0.f;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;

    for (long long base = lo; base < hi; base += STEP) {
        u32x4_t kw[UNROLL], vw[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const long long key = base + (long long)(wave * UNROLL + u) * KPW + kr;
            if (key < hi) {
                const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(K + kvbase + (size_t)key * D + 8 * dc);
                const u32x4_t* vp = reinterpret_cast<const u32x4_t*>(V + kvbase + (size_t)key * D + 8 * dc);
                kw[u] = __builtin_nontemporal_load(kp);
                vw[u] = __builtin_nontemporal_load(vp);
            } else {
                kw[u] = u32x4_t{0, 0, 0, 0};
                vw[u] = u32x4_t{0, 0, 0, 0};
            }
        }
        float s[UNROLL];
        float mx = kNegInf;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw[u][i]), as_bf16x2(qw[i]), acc, false);
            acc = row_sum<LPK>(acc);
            const long long key = base + (long long)(wave * UNROLL + u) * KPW + kr;
            s[u] = (key < hi) ? acc * c : kNegInf;
            mx = fmaxf(mx, s[u]);
        }
        const float m_new = fmaxf(m, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] *= alpha;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const float pu = fast_exp2(s[u] - m_use);
            l += pu;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[2 * i] = __builtin_fmaf(pu, bf16_lo(vw[u][i]), o[2 * i]);
                o[2 * i + 1] = __builtin_fmaf(pu, bf16_hi(vw[u][i]), o[2 * i + 1]);
            }
        }
        m = m_new;
    }

    // ---- merge the GROUPS states of this workgroup ----
#pragma unroll
    for (int i = 0; i < 8; ++i) red_o[grp][8 * dc + i] = o[i];
    if (dc == 0) {
        red_m[grp] = m;
        red_l[grp] = l;
    }
    __syncthreads();
    for (int d = tid; d < D; d += NW * 64) {
        float M = kNegInf;
        for (int g = 0; g < GROUPS; ++g) M = fmaxf(M, red_m[g]);
        const float Mu = (M == kNegInf) ? 0.f : M;
        float L = 0.f, acc = 0.f;
        for (int g = 0; g < GROUPS; ++g) {
            const float w = fast_exp2(red_m[g] - Mu);
            L += w * red_l[g];
            acc += w * red_o[g][d];
        }
        if (direct) {
            O[(size_t)bh * D + d] = (uint16_t)(pack_bf16x2(acc / L, 0.f) & 0xffffu);
            if (d == 0 && LSE != nullptr) LSE[bh] = (M + __builtin_log2f(L)) * 0.69314718055994530942f;
        } else {
            float* rec = part + ((size_t)bh * P + p) * (D + 2);
            rec[d] = acc;
            if (d == 0) {
                rec[D] = M;
                rec[D + 1] = L;
            }
        }
    }
}

// One workgroup of D threads per (batch, head): merge its P partial records.
template <int D>
__global__ __launch_bounds__(D)
void decode_combine_kernel(const float* __restrict__ part, uint16_t* __restrict__ O,
                           float* __restrict__ LSE, int P) {
    const int bh = blockIdx.x;
    const int d = threadIdx.x;
    const float* rec = part + (size_t)bh * P * (D + 2);
    float M = kNegInf;
    for (int p = 0; p < P; ++p) M = fmaxf(M, rec[(size_t)p * (D + 2) + D]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float L = 0.f, acc = 0.f;
    for (int p = 0; p < P; ++p) {
        const float* r = rec + (size_t)p * (D + 2);
        const float w = fast_exp2(r[D] - Mu);
        L += w * r[D + 1];
        acc += w * r[d];
    }
    O[(size_t)bh * D + d] = (uint16_t)(pack_bf16x2(acc / L, 0.f) & 0xffffu);
    if (d == 0 && LSE != nullptr) LSE[bh] = (M + __builtin_log2f(L)) * 0.69314718055994530942f;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream, const char** name) {
    const int BH = a.B * a.H;
    const bool direct = (a.num_splits == 1);
    hipLaunchKernelGGL((decode_split_kernel<D>), dim3(BH, a.num_splits), dim3(NW * 64), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<float*>(a.workspace),
                       static_cast<uint16_t*>(a.o), a.lse, a.Tkv, a.num_splits, a.c, direct ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || direct) {
        *name = (D == 128) ? "decode_bf16_d128<splits=1,waves=4>" : "decode_bf16_d64<splits=1,waves=4>";
        return e;
    }
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(BH), dim3(D), 0, stream,
                       static_cast<const float*>(a.workspace), static_cast<uint16_t*>(a.o), a.lse, a.num_splits);
    *name = (D == 128) ? "decode_split_bf16_d128<waves=4>+combine" : "decode_split_bf16_d64<waves=4>+combine";
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream, const char** name) {
    if (a.d == 128) return launch_d<128>(a, stream, name);
    return launch_d<64>(a, stream, name);
}

}  // namespace attn
