// Grouped-query decode on the matrix cores, bf16 inputs, head width 64 or
// 128, gfx950 (its own source so that the build can schedule it apart from
// the VALU decode kernel).  With G query heads per key/value head, each score
// of the cache carries G dot products, and the VALU kernel runs out of issue
// slots from G = 4 on.  Here the group's heads (up to 32, zero-padded) are
// the N dimension of two MFMA products per 32-key block:
//
//   S^T (32 keys x 32 heads)  = K_blk Q^T        v_mfma_f32_32x32x16_bf16
//   O^T (d x 32 heads)       += V_blk^T bf16(P)^T
//
// the transposed forms of the prefill kernel, so each lane owns one head
// (lanes l and l + 32 hold the two key halves of head l % 32) and the softmax
// state is per lane.  One wave per workgroup per (batch, kv head, head tile,
// partition): the wave streams its partition's K/V blocks through a private
// NS-stage LDS ring by non-temporal DMA (no barriers), K read as rows, V with
// ds_read_b64_tr_b16.  The reference max is raised lazily as in prefill (when
// either lane's half of a head's block sum would exceed 2^15, so the block
// sum stays within 2^16, or is not finite).  Partial records and the combine
// kernel are those of the VALU kernel (decode.hip).
#include <cstdio>

#include "common.hpp"
#include "launch.hpp"

namespace attn {
namespace {

constexpr int MF_BLK = 32;   // keys per block
constexpr float kMfHalfSumLimit = 32768.0f;   // per lane: half of a head's keys

template <int D>
struct MfGeo;
template <>
struct MfGeo<64> {
    static __device__ __forceinline__ int swz_k(int row) { return (row >> 1) & 7; }
    static __device__ __forceinline__ int swz_v(int row) { return ((row >> 1) & 1) << 2; }
};
template <>
struct MfGeo<128> {
    static __device__ __forceinline__ int swz_k(int row) { return row & 15; }
    static __device__ __forceinline__ int swz_v(int row) { return (row & 3) << 2; }
};

template <int D, int NS>
__global__ __launch_bounds__(64)
void decode_mfma_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, float* __restrict__ part,
                        uint16_t* __restrict__ O, float* __restrict__ LSE,
                        int Hkv, int G, int Tkv, int P, float c, int direct) {
    using Gm = MfGeo<D>;
    constexpr int ROWB = D * 2;
    constexpr int TILEB = MF_BLK * ROWB;      // bytes of one K (or V) block
    constexpr int LI = TILEB / 1024;          // 1 KiB DMA instructions per operand per block
    constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
    constexpr int RPG = 1024 / ROWB;          // rows per DMA instruction
    constexpr int TQ = D / 16;
    constexpr int DT = D / 32;

    __shared__ __attribute__((aligned(1024))) uint8_t ring[NS][2][TILEB];

    const int lane = threadIdx.x;
    const int ln = lane & 31;
    const int hf = lane >> 5;

    const int tiles = (G + 31) / 32;
    const int bkv = blockIdx.x / tiles;
    const int tile = blockIdx.x - bkv * tiles;
    const int b = bkv / Hkv;
    const int hk = bkv - b * Hkv;
    const int h = tile * 32 + ln;             // this lane's head within the group
    const bool valid = h < G;
    const int qh = b * Hkv * G + hk * G + h;  // (batch, query head) row
    const int p = blockIdx.y;
    const int lo = (int)(((long long)p * Tkv) / P);
    const int hi = (int)(((long long)(p + 1) * Tkv) / P);
    const int len = hi - lo;
    const int nblk = (len + MF_BLK - 1) / MF_BLK;

    bf16x8_t qf[TQ];
    if (valid) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(Q + (size_t)qh * D + 8 * hf);
#pragma unroll
        for (int t = 0; t < TQ; ++t) qf[t] = __builtin_bit_cast(bf16x8_t, src[2 * t]);
    } else {
#pragma unroll
        for (int t = 0; t < TQ; ++t) qf[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0});
    }

    const size_t kvoff = ((size_t)bkv * Tkv + lo) * D;
    const uint16_t* Kp = K + kvoff;
    const uint16_t* Vp = V + kvoff;
    // block j goes to stage j % NS; blocks past the end issue with an empty range
    auto issue = [&](int j) {
        const int kb = j * MF_BLK;
        const bool live = j < nblk;
        const uint32_t bytes = live ? (uint32_t)(len - kb) * (uint32_t)ROWB : 0u;
        const size_t eoff = live ? (size_t)kb * D : 0;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kp + eoff, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vp + eoff, bytes);
        uint8_t* st = &ring[j % NS][0][0];
#pragma unroll
        for (int i = 0; i < LI; ++i) {
            const int row = RPG * i + lane / CPR;
            const int slot = lane % CPR;
            buffer_load_lds_b128_stream(rk, (uint32_t)(row * ROWB + ((slot ^ Gm::swz_k(row)) << 4)), st + i * 1024);
            buffer_load_lds_b128_stream(rv, (uint32_t)(row * ROWB + ((slot ^ Gm::swz_v(row)) << 4)),
                                        st + TILEB + i * 1024);
        }
    };

    uint32_t k_roff[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) k_roff[t] = (uint32_t)(ln * ROWB + (((2 * t + hf) ^ Gm::swz_k(ln)) << 4));
    uint32_t v_roff[DT];
    {
        const int lg = lane >> 4, jj = lane & 15;
        const int row = 4 * (lg >> 1) + (jj >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int col = 32 * dt + 16 * (lg & 1) + 4 * (jj & 3);
            v_roff[dt] = (uint32_t)(row * ROWB + ((((col >> 3) ^ Gm::swz_v(row)) << 4) | ((col & 4) << 1)));
        }
    }

    f32x16_t oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m = kNegInf, l = 0.f;

#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue(j);
    for (int j = 0; j < nblk; ++j) {
        wait_vmcnt<2 * LI * (NS - 2)>();      // block j has landed
        asm volatile("" ::: "memory");         // the DMA below must follow the reads of block j - 1
        issue(j + NS - 1);
        const uint8_t* kst = &ring[j % NS][0][0];
        const uint8_t* vst = kst + TILEB;
        f32x16_t s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kst + k_roff[t]);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s, 0, 0, 0);
        }
        const int rem = len - j * MF_BLK;     // keys of this block inside the partition
        if (rem < MF_BLK) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + 4 * hf + (r & 3) >= rem) s[r] = kNegInf;
        }
        uint32_t pw[8];
        float rs = 0.f;
        auto exponentiate = [&](float mref) {
            rs = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p0 = fast_exp2(__builtin_fmaf(s[2 * i], c, -mref));
                const float p1 = fast_exp2(__builtin_fmaf(s[2 * i + 1], c, -mref));
                pw[i] = pack_bf16x2(p0, p1);
                rs = i == 0 ? p0 + p1 : rs + (p0 + p1);   // no add of the zero start value
            }
        };
        exponentiate(m);
        if (__builtin_amdgcn_ballot_w64(!(rs <= kMfHalfSumLimit)) != 0) {
            float mx = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
            mx = half_swap_max(mx);
            const float m_new = fmaxf(m, mx * c);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2(m - m_use);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            m = m_new;
            exponentiate(m_use);
        }
        l += rs;
        const uint32_t vb = lds_addr(vst);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const u32x4_t pv = {pw[4 * st], pw[4 * st + 1], pw[4 * st + 2], pw[4 * st + 3]};
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
#pragma unroll
            for (int d2 = 0; d2 < DT; d2 += 2) {
                const uint32_t va = vb + v_roff[d2], vc = vb + v_roff[d2 + 1];
                u32x4_t a0, a1;
                if (st == 0)
                    lds_read_tr16_x4<0, 8 * ROWB, 0, 8 * ROWB>(va, va, vc, vc, a0, a1);
                else
                    lds_read_tr16_x4<16 * ROWB, 24 * ROWB, 16 * ROWB, 24 * ROWB>(va, va, vc, vc, a0, a1);
                oacc[d2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a0), pb, oacc[d2],
                                                                   0, 0, 0);
                oacc[d2 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a1), pb,
                                                                       oacc[d2 + 1], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();    // no DMA may still be writing LDS when the wave retires

    // lane = head column; element r of tile dt = d 32dt + 8(r/4) + 4hf + r%4
    const float lsum = half_swap_sum(l);
    if (!valid) return;
    if (direct) {
        const float inv = 1.0f / lsum;
        uint16_t* orow = O + (size_t)qh * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2_t w = {pack_bf16x2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv),
                                   pack_bf16x2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv)};
                *reinterpret_cast<u32x2_t*>(orow + 32 * dt + 8 * g + 4 * hf) = w;
            }
        if (LSE != nullptr && hf == 0) LSE[qh] = (m + __builtin_log2f(lsum)) * 0.69314718055994530942f;
    } else {
        float* rec = part + ((size_t)qh * P + p) * (D + 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float4 w;
                w.x = oacc[dt][4 * g];
                w.y = oacc[dt][4 * g + 1];
                w.z = oacc[dt][4 * g + 2];
                w.w = oacc[dt][4 * g + 3];
                // records are (D + 2) floats: 8-byte aligned only, so two 8-byte stores
                *reinterpret_cast<float2*>(rec + 32 * dt + 8 * g + 4 * hf) = make_float2(w.x, w.y);
                *reinterpret_cast<float2*>(rec + 32 * dt + 8 * g + 4 * hf + 2) = make_float2(w.z, w.w);
            }
        if (hf == 0) {
            rec[D] = m;
            rec[D + 1] = lsum;
        }
    }
}


thread_local char g_name[96];

constexpr int kMfmaStages = 3;

template <int D>
hipError_t launch_mfma(const DecodeArgs& a, hipStream_t stream, const char** name) {
    const int G = a.H / a.Hkv;
    const int tiles = (G + 31) / 32;
    const bool direct = (a.num_splits == 1);
    hipLaunchKernelGGL((decode_mfma_kernel<D, kMfmaStages>), dim3(a.B * a.Hkv * tiles, a.num_splits), dim3(64), 0,
                       stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<float*>(a.workspace),
                       static_cast<uint16_t*>(a.o), a.lse, a.Hkv, G, a.Tkv, a.num_splits, a.c, direct ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && !direct) e = launch_decode_combine(a, stream);
    if (direct)
        snprintf(g_name, sizeof g_name, "decode_mfma_bf16_d%d<group=%d,blk=32,stages=%d,splits=1>", D, G, kMfmaStages);
    else
        snprintf(g_name, sizeof g_name, "decode_mfma_bf16_d%d<group=%d,blk=32,stages=%d>+combine", D, G, kMfmaStages);
    *name = g_name;
    return e;
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream, const char** name) {
    if (a.d == 128) return launch_mfma<128>(a, stream, name);
    return launch_mfma<64>(a, stream, name);
}

}  // namespace attn
