// Exact attention forward (prefill), bf16 inputs, head width 64, gfx950.
//
// One workgroup owns a tile of BQ = 32 * WAVES query rows of one (batch, head)
// and streams the key/value blocks of 64 rows past it ("IO-Aware Attention:
// Tiling the Score Matrix Without Materializing It", section "What has to
// stay in fast memory"; "FlashAttention IO-aware tiling lab", kernel phases
// load Q / score a K tile / update the online softmax / accumulate V / write O
// once).  Per key block j:
//
//   S^T = K_j Q^T                       v_mfma_f32_32x32x16_bf16, fp32 accumulate
//   P   = exp2(S * c - m)               c = scale * log2 e, m = reference max
//   l  += rowsum P (fp32);  O^T += V_j^T bf16(P)^T      (mfma again)
//
// This is the running-max / running-sum recurrence of "IO-Aware Attention",
// section "Softmax over blocks, exactly", in base 2, with one liberty the
// recurrence allows: the reference m is only raised when a block would
// otherwise produce large terms.  The final O / l and m + log2 l do not depend
// on which reference was used (the rescaling factors telescope), so any m not
// far below the running maximum gives the exact result; m is raised (and l, O
// rescaled by exp2(m_old - m_new)) whenever a row's block sum exceeds 2^16 or
// is not finite, which bounds every term by 2^16 and keeps fp32 far from
// overflow.  Blocks therefore cost no row-max in the common case: softmax work
// is one FMA, one exp2 and one add per score and a bf16 pack per pair -- the
// VALU budget is what limits a d = 64 head on CDNA4, since each score carries
// only 4*64 MFMA flops.  (The row sum stays fp32: a sum of the bf16-rounded
// terms would cost the log-sum-exp up to 2^-9 relative on short rows.)
//
// Layout choices for CDNA4:
// * Computing the transposed products puts one query row in each lane (lane
//   l and l+32 hold the two halves of row l % 32), so row sums are lane-local
//   plus one v_permlane32_swap, the softmax rescale is a per-lane scalar, and
//   the fp32 accumulator of the first product is already the B operand of the
//   second (only a bf16 pack in between).
// * Q stays in VGPRs for the whole key loop (16 VGPRs per lane).
// * K blocks are staged row-major in LDS (row pitch 144 B); V blocks are
//   transposed in registers on the way in and staged as V^T (row pitch 136 B)
//   so the PV operand is two 8-byte LDS reads per lane.  Both are double
//   buffered: block j+1 is fetched into registers by buffer loads (whose range
//   check zero-fills the ragged end) while block j is multiplied, then written
//   to the other LDS buffer; one barrier per block.
// * Causal: the key loop stops at the tile's diagonal block; element masks
//   are applied only on blocks that cross a wave's diagonal or the ragged end,
//   and a wave whose rows all lie above a block skips its math for that block.
// * Tiles are launched heaviest-first (last query tiles first) and the
//   linear block id keeps every tile of one (batch, head) on one XCD when the
//   number of heads is a multiple of 8.
#include "common.hpp"
#include "launch.hpp"

namespace attn {
namespace {

constexpr int D = 64;
constexpr int BK = 64;
constexpr int KPITCH = 72;   // bf16 elements per K row in LDS (64 + 8 pad)
constexpr int VPITCH = 68;   // bf16 elements per V^T row in LDS (64 + 4 pad)
constexpr float kSumLimit = 65536.0f;        // 2^16: largest block row sum kept without raising m

template <int WAVES, bool CAUSAL>
__global__ __launch_bounds__(WAVES * 64, 2)
void prefill_bf16_d64_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                             const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                             float* __restrict__ LSE, int Tq, int Tkv, int BH, int nqt, float c) {
    constexpr int BQ = WAVES * 32;
    constexpr int NT = WAVES * 64;
    static_assert(512 % NT == 0 && 256 % NT == 0, "thread count must divide the tile loads");
    constexpr int KCH = 512 / NT;   // 16-byte K chunks per thread per block
    constexpr int VUN = 256 / NT;   // 4x4 V sub-blocks per thread per block

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BK * KPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VPITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 31;
    const int hf = lane >> 5;

    const int id = blockIdx.x;
    const int bh = id % BH;
    const int rank = id / BH;
    const int qt = CAUSAL ? (nqt - 1 - rank) : rank;
    const int q0 = qt * BQ;
    const int off = Tkv - Tq;                 // bottom-right causal alignment

    const size_t qbase = (size_t)bh * Tq * D;
    const size_t kvbase = (size_t)bh * Tkv * D;
    const uint16_t* Kh = K + kvbase;
    const uint16_t* Vh = V + kvbase;

    // ---- Q fragment: row q0 + 32*wave + ln, d = 16t + 8hf + (0..7) ----
    const int qrow = q0 + wave * 32 + ln;
    bf16x8_t qf[4];
    if (qrow < Tq) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(Q + qbase + (size_t)qrow * D + 8 * hf);
#pragma unroll
        for (int t = 0; t < 4; ++t) qf[t] = __builtin_bit_cast(bf16x8_t, src[2 * t]);
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) qf[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0});
    }

    const int kend = CAUSAL ? min(Tkv, q0 + BQ + off) : Tkv;
    const int nblk = (kend + BK - 1) / BK;
    const int wq_first = q0 + wave * 32;       // this wave's first / last query row
    const int wq_last = wq_first + 31;
    const int lim = CAUSAL ? min(Tkv - 1, qrow + off) : (Tkv - 1);   // last key this row may see

    // ---- per-thread constant offsets of the block loads and LDS stores ----
    uint32_t k_goff[KCH], k_soff[KCH];
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
        const int ch = tid + i * NT;
        const int row = ch >> 3, col = (ch & 7) * 8;
        k_goff[i] = (uint32_t)(row * D + col) * 2u;
        k_soff[i] = (uint32_t)(row * KPITCH + col);
    }
    uint32_t v_goff[VUN], v_soff[VUN];
#pragma unroll
    for (int u = 0; u < VUN; ++u) {
        const int un = tid + u * NT;
        const int kg = un >> 4, dg = un & 15;
        v_goff[u] = (uint32_t)((4 * kg) * D + 4 * dg) * 2u;
        v_soff[u] = (uint32_t)((4 * dg) * VPITCH + 4 * kg);
    }

    u32x4_t kreg[KCH];
    u32x2_t vreg[VUN][4];

    auto fetch = [&](int j) {
        const int kb = j * BK;
        const uint32_t bytes = (uint32_t)(Tkv - kb) * (uint32_t)(D * 2);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)kb * D, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + (size_t)kb * D, bytes);
#pragma unroll
        for (int i = 0; i < KCH; ++i) kreg[i] = buffer_load_b128(rk, k_goff[i]);
#pragma unroll
        for (int u = 0; u < VUN; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) vreg[u][i] = buffer_load_b64(rv, v_goff[u] + (uint32_t)(i * D * 2));
    };

    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) *reinterpret_cast<u32x4_t*>(&Ks[buf][k_soff[i]]) = kreg[i];
#pragma unroll
        for (int u = 0; u < VUN; ++u) {
            // vreg[u][i] holds V[4kg+i][4dg .. 4dg+3]; row 4dg+cc of V^T gets
            // the four keys 4kg .. 4kg+3 of column 4dg+cc.
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const int w = cc >> 1;
                const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
                const u32x2_t out = {__builtin_amdgcn_perm(vreg[u][1][w], vreg[u][0][w], sel),
                                     __builtin_amdgcn_perm(vreg[u][3][w], vreg[u][2][w], sel)};
                *reinterpret_cast<u32x2_t*>(&Vt[buf][v_soff[u] + cc * VPITCH]) = out;
            }
        }
    };

    f32x16_t oacc[2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m = kNegInf;   // reference max of S * c (log2 units), raised only when needed
    float l = 0.f;       // this lane's share of the running sum (relative to m)

    // One key block for this wave.  MASK applies the causal / ragged element mask.
    auto step = [&](int buf, int kb, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        f32x16_t s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8_t a =
                    *reinterpret_cast<const bf16x8_t*>(&Ks[buf][(32 * kt + ln) * KPITCH + 16 * t + 8 * hf]);
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kt], 0, 0, 0);
            }
        }
        if constexpr (MASK) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (key > lim) s[kt][r] = kNegInf;
                }
        }
        // exponentials against the current reference; packed to bf16 pairs
        uint32_t pw[16];
        float rs = 0.f;
        auto exponentiate = [&](float mref) {
            rs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kt = i >> 3, r = 2 * (i & 7);
                const float p0 = fast_exp2(__builtin_fmaf(s[kt][r], c, -mref));
                const float p1 = fast_exp2(__builtin_fmaf(s[kt][r + 1], c, -mref));
                pw[i] = pack_bf16x2(p0, p1);
                rs += p0 + p1;
            }
        };
        exponentiate(m);
        const float row = half_swap_sum(rs);
        if (__builtin_amdgcn_ballot_w64(!(row <= kSumLimit)) != 0) {
            // raise the reference to the true running max and rescale
            float mx = kNegInf;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
            mx = half_swap_max(mx);
            const float m_new = fmaxf(m, mx * c);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2(m - m_use);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            m = m_new;
            exponentiate(m_use);
        }
        l += rs;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const u32x4_t pv = {pw[4 * st], pw[4 * st + 1], pw[4 * st + 2], pw[4 * st + 3]};
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                const uint16_t* vrow = &Vt[buf][(32 * dt + ln) * VPITCH + 16 * st + 4 * hf];
                const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
                const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 8);
                const u32x4_t aw = {lo[0], lo[1], hi[0], hi[1]};
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, aw), pb, oacc[dt],
                                                                   0, 0, 0);
            }
        }
    };

    // Blocks [0, nfull) need no element mask for any row of the tile: they lie
    // inside the key range and, for causal, left of every row's diagonal.
    // Blocks [nfull, nblk) may be masked (diagonal or ragged end) or, for a
    // wave whose rows all precede them, skipped.
    const int nfull = CAUSAL ? min(Tkv / BK, (q0 + off + 1) / BK) : Tkv / BK;

    fetch(0);
    stage(0);
    __syncthreads();

    int j = 0;
    for (; j < nfull; ++j) {
        const int buf = j & 1;
        if (j + 1 < nblk) fetch(j + 1);
        step(buf, j * BK, std::false_type{});
        if (j + 1 < nblk) stage(buf ^ 1);
        __syncthreads();
    }
    for (; j < nblk; ++j) {
        const int buf = j & 1;
        if (j + 1 < nblk) fetch(j + 1);
        const int kb = j * BK;
        if (!CAUSAL || kb <= wq_last + off) step(buf, kb, std::true_type{});
        if (j + 1 < nblk) stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: divide once, write O (bf16) and LSE (fp32) ----
    const float lsum = half_swap_sum(l);
    if (qrow < Tq) {
        const float inv = 1.0f / lsum;
        uint16_t* orow = O + qbase + (size_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2_t w = {pack_bf16x2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv),
                                   pack_bf16x2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv)};
                *reinterpret_cast<u32x2_t*>(orow + 32 * dt + 8 * g + 4 * hf) = w;
            }
        if (LSE != nullptr && hf == 0)
            LSE[(size_t)bh * Tq + qrow] = (m + __builtin_log2f(lsum)) * 0.69314718055994530942f;
    }
}

template <int WAVES, bool CAUSAL>
hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
    constexpr int BQ = WAVES * 32;
    const int nqt = (a.Tq + BQ - 1) / BQ;
    const long long grid = (long long)nqt * a.B * a.H;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_bf16_d64_kernel<WAVES, CAUSAL>), dim3((unsigned)grid), dim3(WAVES * 64), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.Tq, a.Tkv,
                       a.B * a.H, nqt, a.c);
    return hipGetLastError();
}

}  // namespace

bool prefill_bf16_fits(int Tkv) {
    // buffer-load ranges are 32-bit byte counts per (batch, head)
    return (long long)Tkv * D * 2 < (1LL << 31);
}

hipError_t launch_prefill_bf16_d64(const PrefillArgs& a, hipStream_t stream, const char** name) {
    if (a.causal) {
        *name = "prefill_bf16_d64<waves=4,bq=128,bk=64,causal>";
        return launch_one<4, true>(a, stream);
    }
    *name = "prefill_bf16_d64<waves=4,bq=128,bk=64>";
    return launch_one<4, false>(a, stream);
}

}  // namespace attn
