// Exact attention for one query per (batch, query head) against cached keys
// and values (decode), bf16 inputs, head width 64 or 128, gfx950.
//
// One query row per head leaves no query axis to block over: a step reads
// every cached K and V row once and folds it into one output, so its time is
// the time to read the cache ("IO-Aware Attention: Tiling the Score Matrix
// Without Materializing It", section "Where the approach stops helping"; "Attention and Its
// Computational Cost", section "The other shape: one query, many keys").
// The key axis is split into P contiguous partitions, each reduced by its own
// workgroup to a partial output and normaliser, and a second kernel merges the
// partitions with the same rescaling ("IO-Aware Attention", section
// "Parallelism and the cost of the split").
//
// Grouped-query attention ("Attention and Its Computational Cost", same
// section: fewer key/value heads than query heads shrink the cache): query
// head h reads key/value head h / G with G = H_q / H_kv.  A workgroup serves
// GT query heads of one group, so every K/V byte it loads is used by GT
// queries; G = 1 is ordinary multi-head decode.
//
// Split kernel, one workgroup per (batch, kv head, head tile, partition):
// * D/8 lanes share one key row: each lane holds 8 elements (16 bytes) of
//   each of its GT queries and of the key, so a wave load instruction reads
//   whole contiguous key rows (non-temporal: every byte is used once).
// * q.k: v_dot2_f32_bf16 on the packed bf16 pairs, then a DPP sum over the
//   D/8 lanes of the row.
// * Each group of D/8 lanes keeps its own running (m, l) and 8-wide output
//   slice per query head, so the key loop has no cross-group traffic at all;
//   groups and waves are merged once at the end through LDS.
// * No LDS staging for K/V: nothing is reused, so loads go straight to VGPRs.
//
// Partial record per (batch*query head, partition): o (D floats, not
// normalised), then m (max of scale*log2e*q.k) and l, all fp32.
#include <algorithm>
#include <cstdio>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace attn {
namespace {

// waves per workgroup: 8 (against 4) gives the same number of waves in flight
// with half the partitions, so batch-1 steps merge half the records; it is
// as fast or faster on every grid measured (batch 1-64, 12-32 heads).
constexpr int NW = 8;
// groups of at least this many query heads per key/value head use the MFMA
// kernel (measured: below 4 the two kernels tie, from 4 on MFMA wins)
constexpr int kMfmaMinGroup = 4;

template <int D, int GT>
struct DecodeShape {
    static constexpr int LPK = D / 8;          // lanes per key row
    static constexpr int KPW = 64 / LPK;       // key rows per wave load
    static constexpr int GROUPS = NW * KPW;    // independent softmax states per workgroup and head
    static constexpr int UNROLL = GT >= 4 ? 4 : 8;   // key-row loads in flight per lane per operand
    static constexpr int STEP = NW * KPW * UNROLL;   // keys per workgroup iteration
    static constexpr int HP = GT < 4 ? GT : 4;       // heads merged per LDS pass
};

template <int D, int GT>
__global__ __launch_bounds__(NW * 64)
void decode_split_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                         const uint16_t* __restrict__ V, float* __restrict__ part,
                         uint16_t* __restrict__ O, float* __restrict__ LSE,
                         int Hkv, int G, int Tkv, int P, float c, int direct) {
    using S = DecodeShape<D, GT>;
    constexpr int LPK = S::LPK, KPW = S::KPW, UNROLL = S::UNROLL, STEP = S::STEP;
    constexpr int HP = S::HP;

    __shared__ float red_o[HP][NW][D];
    __shared__ float red_m[HP][NW];
    __shared__ float red_l[HP][NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kr = lane / LPK;         // key slot inside one wave load
    const int dc = lane % LPK;         // which 8 elements of the row

    // blockIdx.x = (b * Hkv + hk) * (G / GT) + tile
    const int tiles = G / GT;
    const int bkv = blockIdx.x / tiles;
    const int tile = blockIdx.x - bkv * tiles;
    const int b = bkv / Hkv;
    const int hk = bkv - b * Hkv;
    const int Hq = Hkv * G;
    const int qh0 = b * Hq + hk * G + tile * GT;   // first (batch*query head) row of this tile
    const int p = blockIdx.y;
    const long long lo = ((long long)p * Tkv) / P;
    const long long hi = ((long long)(p + 1) * Tkv) / P;

    const size_t kvbase = (size_t)bkv * Tkv * D;
    u32x4_t qw[GT];
#pragma unroll
    for (int t = 0; t < GT; ++t)
        qw[t] = *reinterpret_cast<const u32x4_t*>(Q + (size_t)(qh0 + t) * D + 8 * dc);

    float m[GT], l[GT], o[GT][8];
#pragma unroll
    for (int t = 0; t < GT; ++t) {
        m[t] = kNegInf;
        l[t] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[t][i] = 0.f;
    }

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
        float s[UNROLL][GT];
        float mx[GT];
#pragma unroll
        for (int t = 0; t < GT; ++t) mx[t] = kNegInf;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const long long key = base + (long long)(wave * UNROLL + u) * KPW + kr;
#pragma unroll
            for (int t = 0; t < GT; ++t) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw[u][i]), as_bf16x2(qw[t][i]), acc, false);
                acc = group_sum<LPK>(acc);
                s[u][t] = (key < hi) ? acc * c : kNegInf;
                mx[t] = fmaxf(mx[t], s[u][t]);
            }
        }
        float m_use[GT];
#pragma unroll
        for (int t = 0; t < GT; ++t) {
            const float m_new = fmaxf(m[t], mx[t]);
            m_use[t] = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2(m[t] - m_use[t]);
            l[t] *= alpha;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[t][i] *= alpha;
            m[t] = m_new;
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float vf[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vf[2 * i] = bf16_lo(vw[u][i]);
                vf[2 * i + 1] = bf16_hi(vw[u][i]);
            }
#pragma unroll
            for (int t = 0; t < GT; ++t) {
                const float pu = fast_exp2(s[u][t] - m_use[t]);
                l[t] += pu;
#pragma unroll
                for (int i = 0; i < 8; ++i) o[t][i] = __builtin_fmaf(pu, vf[i], o[t][i]);
            }
        }
    }

    // ---- merge the GROUPS states of this workgroup: first the KPW groups of
    // each wave across lanes (lane bits above the row's LPK lanes), then the
    // NW waves through LDS, HP heads per LDS pass ----
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) {
#pragma unroll
        for (int t = 0; t < GT; ++t) {
            const float mo = __shfl_xor(m[t], x), lo = __shfl_xor(l[t], x);
            const float mm = fmaxf(m[t], mo);
            const float mu = (mm == kNegInf) ? 0.f : mm;
            const float wa = fast_exp2(m[t] - mu), wb = fast_exp2(mo - mu);
            l[t] = wa * l[t] + wb * lo;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[t][i] = wa * o[t][i] + wb * __shfl_xor(o[t][i], x);
            m[t] = mm;
        }
    }
#pragma unroll
    for (int t0 = 0; t0 < GT; t0 += HP) {
        if (t0 > 0) __syncthreads();   // the previous pass has finished reading
        if (kr == 0) {
#pragma unroll
            for (int t = 0; t < HP; ++t) {
#pragma unroll
                for (int i = 0; i < 8; ++i) red_o[t][wave][8 * dc + i] = o[t0 + t][i];
                if (dc == 0) {
                    red_m[t][wave] = m[t0 + t];
                    red_l[t][wave] = l[t0 + t];
                }
            }
        }
        __syncthreads();
        for (int e = tid; e < HP * D; e += NW * 64) {
            const int t = e / D;
            const int d = e - t * D;
            float M = kNegInf;
#pragma unroll
            for (int g = 0; g < NW; ++g) M = fmaxf(M, red_m[t][g]);
            const float Mu = (M == kNegInf) ? 0.f : M;
            float L = 0.f, acc = 0.f;
#pragma unroll
            for (int g = 0; g < NW; ++g) {
                const float w = fast_exp2(red_m[t][g] - Mu);
                L += w * red_l[t][g];
                acc += w * red_o[t][g][d];
            }
            const int row = qh0 + t0 + t;
            if (direct) {
                O[(size_t)row * D + d] = (uint16_t)(pack_bf16x2(acc / L, 0.f) & 0xffffu);
                if (d == 0 && LSE != nullptr) LSE[row] = (M + __builtin_log2f(L)) * 0.69314718055994530942f;
            } else {
                float* rec = part + ((size_t)row * P + p) * (D + 2);
                rec[d] = acc;
                if (d == 0) {
                    rec[D] = M;
                    rec[D + 1] = L;
                }
            }
        }
    }
}

// Merge of each (batch, query head)'s P partial records: M = max_p m_p,
// w_p = 2^(m_p - M), O = sum_p w_p o_p / sum_p w_p l_p and
// LSE = (M + log2 L) ln 2 -- the rescaling merge of "IO-Aware Attention",
// section "Parallelism and the cost of the split".  The merge is bound by the
// latency of reading the records, not by bytes, so NPG adjacent lanes share
// each output element: lane g of the group takes partitions g, g + NPG, ...,
// all its loads in flight together (in groups of CG), and the NPG running
// states are combined by lane exchanges with the same rescaling.
constexpr int CG = 8;
constexpr int NPG = 4;

template <int D>
__global__ __launch_bounds__(D * NPG)
void decode_combine_kernel(const float* __restrict__ part, uint16_t* __restrict__ O,
                           float* __restrict__ LSE, int P) {
    const int bh = blockIdx.x;
    const int g = threadIdx.x % NPG;
    const int d = threadIdx.x / NPG;
    const float* rec = part + (size_t)bh * P * (D + 2);
    float M = kNegInf, L = 0.f, acc = 0.f;
    for (int p0 = g; p0 < P; p0 += NPG * CG) {
        float mk[CG], lk[CG], ok[CG];
#pragma unroll
        for (int i = 0; i < CG; ++i) {
            const int p = min(p0 + NPG * i, P - 1);   // past the last record: weight 0 below
            const float* r = rec + (size_t)p * (D + 2);
            mk[i] = r[D];
            lk[i] = r[D + 1];
            ok[i] = r[d];
        }
        float mg = M;
#pragma unroll
        for (int i = 0; i < CG; ++i)
            if (p0 + NPG * i < P) mg = fmaxf(mg, mk[i]);
        const float mu = (mg == kNegInf) ? 0.f : mg;
        const float alpha = fast_exp2(M - mu);
        L *= alpha;
        acc *= alpha;
#pragma unroll
        for (int i = 0; i < CG; ++i) {
            const float w = (p0 + NPG * i < P) ? fast_exp2(mk[i] - mu) : 0.f;
            L = __builtin_fmaf(w, lk[i], L);
            acc = __builtin_fmaf(w, ok[i], acc);
        }
        M = mg;
    }
    // the NPG lanes of the element (a lane without partitions has M = -inf, L = acc = 0)
#pragma unroll
    for (int x = 1; x < NPG; x <<= 1) {
        const float Mo = __shfl_xor(M, x), Lo = __shfl_xor(L, x), ao = __shfl_xor(acc, x);
        const float mm = fmaxf(M, Mo);
        const float mu = (mm == kNegInf) ? 0.f : mm;
        const float wa = fast_exp2(M - mu), wb = fast_exp2(Mo - mu);
        L = wa * L + wb * Lo;
        acc = wa * acc + wb * ao;
        M = mm;
    }
    if (g == 0) {
        O[(size_t)bh * D + d] = (uint16_t)(pack_bf16x2(acc / L, 0.f) & 0xffffu);
        if (d == 0 && LSE != nullptr) LSE[bh] = (M + __builtin_log2f(L)) * 0.69314718055994530942f;
    }
}

// Largest head tile (8, 4, 2 or 1) that divides the group size.
int head_tile(int G) {
    for (int gt : {8, 4, 2})
        if (G % gt == 0) return gt;
    return 1;
}

thread_local char g_name[96];

template <int D, int GT>
hipError_t launch_dg(const DecodeArgs& a, hipStream_t stream, const char** name) {
    const int G = a.H / a.Hkv;
    const int blocks = a.B * a.Hkv * (G / GT);
    const bool direct = (a.num_splits == 1);
    hipLaunchKernelGGL((decode_split_kernel<D, GT>), dim3(blocks, a.num_splits), dim3(NW * 64), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<float*>(a.workspace),
                       static_cast<uint16_t*>(a.o), a.lse, a.Hkv, G, a.Tkv, a.num_splits, a.c, direct ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && !direct) {
        hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.H), dim3(D * NPG), 0, stream,
                           static_cast<const float*>(a.workspace), static_cast<uint16_t*>(a.o), a.lse,
                           a.num_splits);
        e = hipGetLastError();
    }
    if (direct)
        snprintf(g_name, sizeof g_name, "decode_bf16_d%d<heads=%d,splits=1,waves=%d>", D, GT, NW);
    else
        snprintf(g_name, sizeof g_name, "decode_split_bf16_d%d<heads=%d,waves=%d>+combine", D, GT, NW);
    *name = g_name;
    return e;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream, const char** name) {
    if (a.H / a.Hkv >= kMfmaMinGroup) return launch_decode_mfma(a, stream, name);
    // below kMfmaMinGroup the head tile is 2 (groups of 2) or 1
    if (head_tile(a.H / a.Hkv) == 2) return launch_dg<D, 2>(a, stream, name);
    return launch_dg<D, 1>(a, stream, name);
}

}  // namespace

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream) {
    if (a.d == 128)
        hipLaunchKernelGGL((decode_combine_kernel<128>), dim3(a.B * a.H), dim3(128 * NPG), 0, stream,
                           static_cast<const float*>(a.workspace), static_cast<uint16_t*>(a.o), a.lse,
                           a.num_splits);
    else
        hipLaunchKernelGGL((decode_combine_kernel<64>), dim3(a.B * a.H), dim3(64 * NPG), 0, stream,
                           static_cast<const float*>(a.workspace), static_cast<uint16_t*>(a.o), a.lse,
                           a.num_splits);
    return hipGetLastError();
}

constexpr long long kCUs = 256;   // compute units of an MI355X

int decode_auto_splits(int B, int Hq, int Hkv, int Tkv, int d) {
    // Enough partitions for about 512 workgroups (2 per CU), each holding at
    // least 64 KiB of K and V (256 keys at d = 64, 128 at d = 128); at most 16
    // partitions for the 8-wave VALU kernel and 64 for the 1-wave MFMA kernel.
    // Measured on 12 heads of 64 and 32 heads of 128, groups of 1-32, batch
    // 1-64, 128-16K keys: shorter or more numerous partitions lose to their
    // start-up latency and the merge.  A VALU grid that 16 partitions leave
    // below one workgroup per CU (fewer than 16 head tiles) takes as many as
    // fill the CUs once, up to 64: more than one per CU would leave some CUs
    // a second workgroup to run after the rest have finished (batch 1, 16K
    // keys: 12 heads 12.4 -> 11.8 us at 21 partitions, 8 heads of 128
    // 17.0 -> 13.8 us at 32, 4 heads of 128 26.2 -> 15.7 us at 64).
    const int G = Hq / Hkv;
    const bool mfma = G >= kMfmaMinGroup;
    const long long wgs = mfma ? (long long)B * Hkv * ((G + 31) / 32) : (long long)B * Hkv * (G / head_tile(G));
    const int cap = mfma ? 64 : 16;
    const int min_keys = 16384 / d;
    int p = 1;
    while (p < cap && wgs * p < 512) p *= 2;
    if (!mfma && wgs * p < kCUs) p = (int)std::min<long long>(64, kCUs / wgs);
    p = std::min(p, std::max(1, Tkv / min_keys));
    return p;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream, const char** name) {
    if (a.d == 128) return launch_d<128>(a, stream, name);
    return launch_d<64>(a, stream, name);
}

// Partial-record storage of the allocation-free decode entry point: one
// array per device, part of the library's code object, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host that name is only a stand-in for the device symbol): it takes the
// device address from hipGetSymbolAddress, once per device with that device
// current, and hands that address to the kernels like a caller's workspace.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace attn
