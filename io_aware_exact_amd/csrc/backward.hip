// Exact attention backward, bf16 inputs, head width 64 or 128, gfx950.
//
// The forward pass keeps O and one log-sum-exp per query row, not the
// probabilities; they are rebuilt here block by block from Q, K, V and that
// row value ("IO-Aware Attention: Tiling the Score Matrix Without
// Materializing It", section "What has to stay in fast memory"): another
// sweep of matrix products costs less than writing the T_q x T_kv
// probabilities out and reading them back.  With c = scale * log2 e,
// lse2 = lse * log2 e and D_i = sum_d dO_id O_id:
//
//   P  = exp2(c * Q K^T - lse2)         (recomputed per block, never stored)
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D)
//   dQ = scale * dS K,   dK = scale * dS^T Q
//
// Two kernels, no atomics, dQ first:
// * bwd_dq: one workgroup per 128-query tile, the forward's layout (one query
//   per lane, key blocks of 64 at d = 64, 32 at d = 128): S^T = K Q^T,
//   dP^T = V dO^T, dQ^T += K^T dS^T with K^T read transposed from the ring.
//   It first forms its rows' (lse2, D) from LSE, O and the dO fragment it
//   holds anyway, and writes them for bwd_dkdv.
// * bwd_dkdv: one workgroup per 128-key tile (32 keys per wave, one key per
//   lane column).  K and V of the wave stay in VGPRs as MFMA B operands; Q and
//   dO blocks (64 rows at d = 64, 32 at d = 128) and their row statistics
//   stream through a 3-stage LDS ring filled by DMA.  Per block: S = Q K^T
//   and dP = dO V^T (Q, dO read as rows), then dV^T += dO^T P and
//   dK^T += Q^T dS with dO^T, Q^T read by ds_read_b64_tr_b16, so P and dS go
//   from the accumulator layout to the B operand with only a bf16 pack.
// Both kernels unroll their block loops by the ring depth, so every LDS read
// is a per-lane address fixed before the loop plus a constant offset, and
// no loop holds a branch that joins with the accumulators live (the register
// allocator copies them at such joins).
// Q and dO (in bwd_dkdv) and K (in bwd_dq) are read both as rows and
// transposed, so their LDS chunk swizzle is conflict-free for both patterns.
// Products are bf16 MFMA with fp32 accumulation; P and dS are rounded to
// bf16 (nearest even) as MFMA operands; dQ, dK, dV are written in fp32.
#include <cstdio>

#include "common.hpp"
#include "launch.hpp"

namespace attn {
namespace {

// Geometry per head width.  The chunk swizzle serves rows read both ways:
// a row read (32 rows x one 16-byte chunk pair per instruction) and a
// transposed read (8 rows x 64 bytes) both touch every LDS bank equally.
// d = 64 (128-byte rows): 16 consecutive rows map a chunk to 8 distinct chunks
// x 2 bank halves, rows r, r+1 vs r+2, r+3 land in different 64-byte halves.
// d = 128 (256-byte rows): 16 consecutive rows map a chunk to 16 distinct
// chunks, rows r..r+3 to 4 distinct 64-byte segments.  In both, rows r and
// r + 16 share a swizzle and rows r and r + 8 do not.
template <int D>
struct BwdGeo;
template <>
struct BwdGeo<64> {
    static constexpr int BQ2 = 64;   // dK/dV kernel: query rows per streamed block
    static constexpr int BK = 64;    // dQ kernel: keys per streamed block
    static constexpr int KV_MINW = 2;
    static __device__ __forceinline__ int swz(int row) { return ((row >> 1) & 7) ^ (((row >> 1) & 1) << 2); }
};
template <>
struct BwdGeo<128> {
    static constexpr int BQ2 = 32;
    static constexpr int BK = 32;
    static constexpr int KV_MINW = 1;   // K, V and both accumulators: 192 registers before any temporary
    static __device__ __forceinline__ int swz(int row) { return (row & 15) ^ ((row & 3) << 2); }
};

// Byte offset of the 8-byte piece holding columns col..col+3 of a swizzled row.
template <int D>
__device__ __forceinline__ uint32_t tr_off(int row, int col) {
    return (uint32_t)(row * D * 2 + ((((col >> 3) ^ BwdGeo<D>::swz(row)) << 4) | ((col & 4) << 1)));
}

// 16-byte LDS load at a byte address plus a constant (the instruction's
// offset field); the compiler tracks its wait.
template <int OFF>
__device__ __forceinline__ bf16x8_t lds_b128(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS instruction offset");
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>((uintptr_t)(addr + OFF));
}

// Transposed-read offsets of a lane: lane group lg = lane / 16, jj = lane % 16
// addresses row 4(lg/2) + jj/4 (and + 8), columns 32dt + 16(lg%2) + 4(jj%4).
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, uint32_t (&o)[D / 32][2]) {
    const int lg = lane >> 4, jj = lane & 15;
    const int row = 4 * (lg >> 1) + (jj >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        const int col = 32 * dt + 16 * (lg & 1) + 4 * (jj & 3);
        o[dt][0] = tr_off<D>(row, col);
        o[dt][1] = tr_off<D>(row + 8, col);
    }
}

// Transposed reads for the 16-row k-step STP of a 32-row group: every
// 32-column tile dt, rows 16 STP + (0..7) and + 8, at the lane's addresses
// a[dt][0] and a[dt][1] (ring base and tr_offsets) plus a constant OFF (ring
// stage and operand).  Rows r and r + 8 differ in their swizzle, rows r and
// r + 16 do not, so each tile keeps one address per 8-row half and the
// k-step is an immediate.
template <int D, int STP, int OFF>
__device__ __forceinline__ void tr_kstep_at(const uint32_t (&a)[D / 32][2], u32x4_t (&r)[D / 32]) {
    constexpr int F = OFF + STP * 16 * D * 2;
#pragma unroll
    for (int d2 = 0; d2 < D / 32; d2 += 2)
        lds_read_tr16_x4<F, F, F, F>(a[d2][0], a[d2][1], a[d2 + 1][0], a[d2 + 1][1], r[d2], r[d2 + 1]);
}

// Head width 64: k-steps S0 and S1 of one operand behind one wait.
template <int S0, int S1, int OFF>
__device__ __forceinline__ void tr_kstep2_d64_at(const uint32_t (&a)[2][2], u32x4_t (&r0)[2], u32x4_t (&r1)[2]) {
    constexpr int F0 = OFF + S0 * 16 * 64 * 2, F1 = OFF + S1 * 16 * 64 * 2;
    const uint32_t ad[8] = {a[0][0], a[0][1], a[1][0], a[1][1], a[0][0], a[0][1], a[1][0], a[1][1]};
    u32x4_t r[4];
    lds_read_tr16_x8<F0, F0, F0, F0, F1, F1, F1, F1>(ad, r);
    r0[0] = r[0];
    r0[1] = r[1];
    r1[0] = r[2];
    r1[1] = r[3];
}

// Head width 64: k-step STP of two operands at constants G and Q from the
// same addresses (dO and Q, one block apart in a stage) behind one wait.
template <int STP, int G, int Q>
__device__ __forceinline__ void tr_kstep2_d64_pair_at(const uint32_t (&a)[2][2], u32x4_t (&rg)[2],
                                                      u32x4_t (&rq)[2]) {
    constexpr int F0 = G + STP * 16 * 64 * 2, F1 = Q + STP * 16 * 64 * 2;
    const uint32_t ad[8] = {a[0][0], a[0][1], a[1][0], a[1][1], a[0][0], a[0][1], a[1][0], a[1][1]};
    u32x4_t r[4];
    lds_read_tr16_x8<F0, F0, F0, F0, F1, F1, F1, F1>(ad, r);
    rg[0] = r[0];
    rg[1] = r[1];
    rq[0] = r[2];
    rq[1] = r[3];
}

// 16-byte LDS load of four floats at a byte address plus a byte offset.
__device__ __forceinline__ f32x4_t lds_f32x4(uint32_t addr, int off) {
    return *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>((uintptr_t)(addr + off));
}

// ------------------------------------------------------------------ dK, dV

constexpr int KV_WAVES = 4;
constexpr int BKV = 32 * KV_WAVES;   // keys per workgroup
constexpr int NS = 3;                // ring stages

// QS = 2 (query halves, for grids with few key tiles): the waves form
// KV_WAVES/2 key groups of 32 keys, and the two waves of a group take the two
// 32-row sub-tiles of every query block; the pair sums its dK, dV partials
// through LDS at the end.  Tiles are then 64 keys and the serial query loop
// of a tile is half as long.
template <int D, bool CAUSAL, int QS = 1>
__global__ __launch_bounds__(KV_WAVES * 64, BwdGeo<D>::KV_MINW)
void bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                     const float2* __restrict__ stats, float* __restrict__ dK, float* __restrict__ dV,
                     int Tq, int Tkv, int BH, float c, float scale) {
    using G = BwdGeo<D>;
    constexpr int ROWB = D * 2;
    constexpr int TQ = D / 16;
    constexpr int DT = D / 32;
    constexpr int CPR = ROWB / 16;
    constexpr int RPG = 1024 / ROWB;
    constexpr int BQ2 = G::BQ2;
    constexpr int NSUB = BQ2 / 32;           // 32-row sub-tiles per block
    constexpr int QBLK = BQ2 * ROWB;         // 8 KiB
    constexpr int STAGE = 2 * QBLK + 1024;
    constexpr int KV_LI = QBLK / 1024 / KV_WAVES;
    static_assert(KV_LI * KV_WAVES * 1024 == QBLK, "block rows must split evenly over the waves");
    static_assert(QS == 1 || (QS == 2 && NSUB == 2), "query halves split a block's two sub-tiles");
    constexpr int KG = KV_WAVES / QS;        // key groups of 32 keys
    constexpr int BKVT = 32 * KG;            // keys per workgroup
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NS][STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 31;
    const int hf = lane >> 5;
    const int kg = wave % KG;                // key group
    const int qh = wave / KG;                // query sub-tile of every block (QS = 2)

    // causal: the first key tiles see the most query rows, so they go first
    const int bh = blockIdx.x % BH;
    const int kt = blockIdx.x / BH;
    const int k0 = kt * BKVT;
    const int off = Tkv - Tq;
    const int key = k0 + 32 * kg + ln;          // this lane's key column

    const size_t qbase = (size_t)bh * Tq * D;
    const size_t kvbase = (size_t)bh * Tkv * D;

    // K and V fragments (B operands): key `key`, d = 16t + 8hf + (0..7)
    bf16x8_t kf[TQ], vf[TQ];
    if (key < Tkv) {
        const u32x4_t* ks = reinterpret_cast<const u32x4_t*>(K + kvbase + (size_t)key * D + 8 * hf);
        const u32x4_t* vs = reinterpret_cast<const u32x4_t*>(V + kvbase + (size_t)key * D + 8 * hf);
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
            kf[t] = __builtin_bit_cast(bf16x8_t, ks[2 * t]);
            vf[t] = __builtin_bit_cast(bf16x8_t, vs[2 * t]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
            kf[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0});
            vf[t] = kf[t];
        }
    }

    // query blocks that see any key of this tile (bottom-right causal)
    const int nqb = (Tq + BQ2 - 1) / BQ2;
    const int qb_first = CAUSAL ? max(0, k0 - off) / BQ2 : 0;

    // DMA: wave w moves row groups g = w + 4i (1 KiB) of Q and dO, and every
    // wave moves the block's row statistics (BQ2 * 8 bytes)
    uint32_t voff[KV_LI];
#pragma unroll
    for (int i = 0; i < KV_LI; ++i) {
        const int g = wave + KV_WAVES * i;
        const int row = RPG * g + lane / CPR;
        voff[i] = (uint32_t)(row * ROWB + (((lane % CPR) ^ G::swz(row)) << 4));
    }
    auto issue = [&](int j) {
        const bool live = j < nqb;
        const int q0 = j * BQ2;
        const uint32_t bytes = live ? (uint32_t)(Tq - q0) * (uint32_t)ROWB : 0u;
        const size_t eoff = live ? (size_t)q0 * D : 0;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qbase + eoff, bytes);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(dO + qbase + eoff, bytes);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(stats + (size_t)bh * Tq + (live ? q0 : 0),
                                                    live ? (uint32_t)(Tq - q0) * 8u : 0u);
        uint8_t* st = &ring[(j - qb_first) % NS][0];   // block j sits in stage (j - qb_first) % NS
#pragma unroll
        for (int i = 0; i < KV_LI; ++i) {
            const int g = wave + KV_WAVES * i;
            buffer_load_lds_b128(rq, voff[i], st + g * 1024);
            buffer_load_lds_b128(rg, voff[i], st + QBLK + g * 1024);
        }
        buffer_load_lds_b128(rs, (uint32_t)lane * 16u, st + 2 * QBLK);
    };

    // row-read offsets (A operand of S = Q K^T and dP = dO V^T): row ln, chunk 2t + hf
    uint32_t r_off[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) r_off[t] = (uint32_t)(ln * ROWB + (((2 * t + hf) ^ G::swz(ln)) << 4));
    // transposed-read offsets (A operand of dV^T = dO^T P, dK^T = Q^T dS): lane group
    // lg = lane / 16, jj = lane % 16 addresses row 4(lg/2) + jj/4 (+8), columns
    // 32dt + 16(lg%2) + 4(jj%4)
    uint32_t t_off[DT][2];
    tr_offsets<D>(lane, t_off);

    f32x16_t dkt[DT], dvt[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dkt[dt][r] = 0.f;
            dvt[dt][r] = 0.f;
        }

    // Per-lane LDS addresses in ring stage 0 (query halves: of this wave's
    // sub-tile); a stage adds a constant, so the block loop below is unrolled
    // by the ring depth and blocks need no address arithmetic.
    const uint32_t ring_lds = lds_addr(&ring[0][0]);
    const uint32_t sub0 = QS == 2 ? (uint32_t)(qh * 32 * ROWB) : 0u;
    uint32_t q_ra[TQ];                   // rows of Q (dO: + QBLK)
#pragma unroll
    for (int t = 0; t < TQ; ++t) q_ra[t] = ring_lds + sub0 + r_off[t];
    uint32_t t_ra[DT][2];                // transposed reads of Q (dO: + QBLK)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        t_ra[dt][0] = ring_lds + sub0 + t_off[dt][0];
        t_ra[dt][1] = ring_lds + sub0 + t_off[dt][1];
    }
    // row statistics (lse2, D) of rows 4hf.. of the sub-tile
    const uint32_t s_ra = ring_lds + 2 * QBLK + (uint32_t)((QS == 2 ? qh * 32 : 0) * 8 + 4 * hf * 8);

    // one 32-row sub-tile of the block in ring stage S; q0 = first row of the
    // block, qs = the sub-tile, qo = its byte offset beyond the addresses above
    auto subtile = [&](auto stage_tag, int q0, int qs, uint32_t qo, uint32_t so8) {
        constexpr int SO = decltype(stage_tag)::value * STAGE;
        f32x16_t s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = 0.f;
            dp[r] = 0.f;
        }
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
            const bf16x8_t a = lds_b128<SO>(q_ra[t] + qo);
            const bf16x8_t g = lds_b128<SO + QBLK>(q_ra[t] + qo);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[t], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g, vf[t], dp, 0, 0, 0);
        }
        // element r of this lane: query row qs*32 + 8(r/4) + 4hf + r%4 of the block, key `key`
        uint32_t pw[8], dw[8];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int rb = qs * 32 + 8 * g4 + 4 * hf;           // first of 4 consecutive rows
            const f32x4_t st0 = lds_f32x4(s_ra + so8, SO + 64 * g4);       // (lse2, D) rows rb, rb+1
            const f32x4_t st1 = lds_f32x4(s_ra + so8, SO + 64 * g4 + 16);  // rows rb+2, rb+3
            float p[4], ds[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lse2 = (i < 2) ? st0[2 * i] : st1[2 * (i - 2)];
                const float dd = (i < 2) ? st0[2 * i + 1] : st1[2 * (i - 2) + 1];
                const int r = 4 * g4 + i;
                // causal: a key right of the row's diagonal gets exponent
                // -inf (exp2 gives 0, no branch).  Rows past Tq need no mask:
                // their Q, dO and statistics arrive zero-filled, so p = 1,
                // dS = p (0 - 0) = 0 and the dO^T column is 0 -- they add
                // exact zeros to dV and dK.
                float x = __builtin_fmaf(s[r], c, -lse2);
                if constexpr (CAUSAL) x = key > q0 + rb + i + off ? -__builtin_inff() : x;
                const float pe = fast_exp2(x);
                p[i] = pe;
                ds[i] = pe * (dp[r] - dd);
            }
            pw[2 * g4] = pack_bf16x2(p[0], p[1]);
            pw[2 * g4 + 1] = pack_bf16x2(p[2], p[3]);
            dw[2 * g4] = pack_bf16x2(ds[0], ds[1]);
            dw[2 * g4 + 1] = pack_bf16x2(ds[2], ds[3]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS over the sub-tile's 32 rows (two 16-row k-steps)
        uint32_t ta[DT][2];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            ta[dt][0] = t_ra[dt][0] + qo;
            ta[dt][1] = t_ra[dt][1] + qo;
        }
        auto kstep = [&](auto stp_tag) {
            constexpr int stp = decltype(stp_tag)::value;
            const u32x4_t pv = {pw[4 * stp], pw[4 * stp + 1], pw[4 * stp + 2], pw[4 * stp + 3]};
            const u32x4_t dv = {dw[4 * stp], dw[4 * stp + 1], dw[4 * stp + 2], dw[4 * stp + 3]};
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
            const bf16x8_t db = __builtin_bit_cast(bf16x8_t, dv);
            if constexpr (D == 64 && QS > 1) {
                // dO^T and Q^T operands of this k-step behind one wait (the
                // 8 extra registers would make QS = 1 spill)
                u32x4_t ag[2], aq[2];
                tr_kstep2_d64_pair_at<stp, SO + QBLK, SO>(ta, ag, aq);
#pragma unroll
                for (int dt = 0; dt < 2; ++dt)
                    dvt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ag[dt]), pb,
                                                                      dvt[dt], 0, 0, 0);
#pragma unroll
                for (int dt = 0; dt < 2; ++dt)
                    dkt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, aq[dt]), db,
                                                                      dkt[dt], 0, 0, 0);
            } else {
                u32x4_t a[DT];
                tr_kstep_at<D, stp, SO + QBLK>(ta, a);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    dvt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[dt]), pb,
                                                                      dvt[dt], 0, 0, 0);
                tr_kstep_at<D, stp, SO>(ta, a);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    dkt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[dt]), db,
                                                                      dkt[dt], 0, 0, 0);
            }
        };
        kstep(std::integral_constant<int, 0>{});
        kstep(std::integral_constant<int, 1>{});
    };

#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue(qb_first + j);
    // Every sub-tile runs the one body with the causal element mask, also
    // where no element is masked or where every element is (a wave whose
    // keys follow all of a sub-tile's rows then adds exact zeros).  A branch
    // between an unmasked and a masked body, or around the body, makes the
    // register allocator copy the four accumulators (64 VGPRs) at the join
    // in every iteration.
    auto blk = [&](int j, auto stage_tag) {
        wait_vmcnt<(2 * KV_LI + 1) * (NS - 2)>();   // this wave's part of block j has landed
        __syncthreads();                            // ... everyone's, and the previous stage is free
        issue(j + NS - 1);
        const int q0 = j * BQ2;
        __builtin_amdgcn_sched_barrier(0);          // no instruction moves between blocks
        if constexpr (QS == 2) {
            subtile(stage_tag, q0, qh, 0u, 0u);
        } else {
            // one sub-tile at a time (not unrolled: two would double the live registers)
#pragma nounroll
            for (int qs = 0; qs < NSUB; ++qs)
                subtile(stage_tag, q0, qs, (uint32_t)(qs * 32 * ROWB), (uint32_t)(qs * 32 * 8));
        }
    };
    static_assert(NS == 3, "the unrolled loop below assumes a 3-stage ring");
    int j = qb_first;
    for (; j + 2 < nqb; j += 3) {
        blk(j, std::integral_constant<int, 0>{});
        blk(j + 1, std::integral_constant<int, 1>{});
        blk(j + 2, std::integral_constant<int, 2>{});
    }
    if (j < nqb) blk(j, std::integral_constant<int, 0>{});
    if (j + 1 < nqb) blk(j + 1, std::integral_constant<int, 1>{});
    wait_vmcnt<0>();    // no DMA may still be writing LDS when the workgroup retires

    if constexpr (QS == 2) {
        // the second wave of each key group hands its partial sums to the
        // first through the ring (lane-major on both sides, conflict-free)
        constexpr int NREG = 2 * DT * 16;
        static_assert(KG * NREG * 64 * 4 <= NS * STAGE, "merge buffer must fit in the ring");
        __syncthreads();                      // every wave is done reading the ring
        float* xb = reinterpret_cast<float*>(&ring[0][0]) + kg * NREG * 64 + lane;
        if (qh == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    xb[(dt * 16 + r) * 64] = dkt[dt][r];
                    xb[((DT + dt) * 16 + r) * 64] = dvt[dt][r];
                }
        }
        __syncthreads();
        if (qh == 1) return;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dkt[dt][r] += xb[(dt * 16 + r) * 64];
                dvt[dt][r] += xb[((DT + dt) * 16 + r) * 64];
            }
    }

    // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane = key column, element r = d 32dt + 8(r/4) + 4hf + r%4
    if (key < Tkv) {
        float* dkrow = dK + kvbase + (size_t)key * D;
        float* dvrow = dV + kvbase + (size_t)key * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                float4 a, b;
                a.x = dkt[dt][4 * g4] * scale;
                a.y = dkt[dt][4 * g4 + 1] * scale;
                a.z = dkt[dt][4 * g4 + 2] * scale;
                a.w = dkt[dt][4 * g4 + 3] * scale;
                b.x = dvt[dt][4 * g4];
                b.y = dvt[dt][4 * g4 + 1];
                b.z = dvt[dt][4 * g4 + 2];
                b.w = dvt[dt][4 * g4 + 3];
                *reinterpret_cast<float4*>(dkrow + 32 * dt + 8 * g4 + 4 * hf) = a;
                *reinterpret_cast<float4*>(dvrow + 32 * dt + 8 * g4 + 4 * hf) = b;
            }
    }
}

// ----------------------------------------------------------------------- dQ

constexpr int DQ_WAVES = 4;
constexpr int BQ = 32 * DQ_WAVES;   // query rows per workgroup

// KS = 2 (key halves, d = 64, for grids with few query tiles): the waves form
// DQ_WAVES/2 row groups of 32 rows, and the two waves of a group take the two
// 32-key halves of every key block; the pair sums its dQ partials through LDS
// at the end.  Tiles are then 64 rows and the serial key loop of a tile is
// half as long.
// Three waves per SIMD at d = 64 (the one-row-group form then spills four
// registers and is still faster than at two waves).
template <int D, bool CAUSAL, int KS = 1>
__global__ __launch_bounds__(DQ_WAVES * 64, D == 64 ? 3 : 2)
void bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                   const uint16_t* __restrict__ O, const float* __restrict__ LSE,
                   float2* __restrict__ stats, float* __restrict__ dQ,
                   int Tq, int Tkv, int BH, int nqt, float c, float scale) {
    using G = BwdGeo<D>;
    constexpr int ROWB = D * 2;
    constexpr int TQ = D / 16;
    constexpr int DT = D / 32;
    constexpr int CPR = ROWB / 16;
    constexpr int RPG = 1024 / ROWB;
    constexpr int BK = G::BK;            // keys per streamed block
    constexpr int KT = BK / 32;          // 32-key tiles per block
    constexpr int KBLK = BK * ROWB;      // 8 KiB
    constexpr int DQ_LI = KBLK / 1024 / DQ_WAVES;
    static_assert(DQ_LI * DQ_WAVES * 1024 == KBLK, "block rows must split evenly over the waves");
    static_assert(KS == 1 || (KS == 2 && KT == 2), "key halves split a block's two 32-key tiles");
    constexpr int RG = DQ_WAVES / KS;        // row groups of 32 rows
    constexpr int BQT = 32 * RG;             // query rows per workgroup
    constexpr int WKT = KT / KS;             // 32-key tiles per wave per block
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NS][2][KBLK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 31;
    const int hf = lane >> 5;
    const int rg = wave % RG;                // row group
    const int kh = wave / RG;                // 32-key tile of every block (KS = 2)

    const int bh = blockIdx.x % BH;
    const int rank = blockIdx.x / BH;
    const int qt = CAUSAL ? (nqt - 1 - rank) : rank;   // heaviest tiles first
    const int q0 = qt * BQT;
    const int off = Tkv - Tq;
    const size_t qbase = (size_t)bh * Tq * D;
    const size_t kvbase = (size_t)bh * Tkv * D;
    const uint16_t* Kh = K + kvbase;
    const uint16_t* Vh = V + kvbase;

    // Q and dO fragments (B operands): row q0 + 32*rg + ln, d = 16t + 8hf + (0..7)
    const int qrow = q0 + rg * 32 + ln;
    bf16x8_t qf[TQ], gf[TQ];
    float lse2 = 0.f, dd = 0.f;
    if (qrow < Tq) {
        const u32x4_t* qs = reinterpret_cast<const u32x4_t*>(Q + qbase + (size_t)qrow * D + 8 * hf);
        const u32x4_t* gs = reinterpret_cast<const u32x4_t*>(dO + qbase + (size_t)qrow * D + 8 * hf);
        const u32x4_t* os = reinterpret_cast<const u32x4_t*>(O + qbase + (size_t)qrow * D + 8 * hf);
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
            qf[t] = __builtin_bit_cast(bf16x8_t, qs[2 * t]);
            const u32x4_t g = gs[2 * t];
            const u32x4_t o = os[2 * t];
            gf[t] = __builtin_bit_cast(bf16x8_t, g);
            // this lane's half of D = sum_d dO_d O_d (the other half is in lane ^ 32)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dd = __builtin_fmaf(bf16_lo(o[i]), bf16_lo(g[i]), dd);
                dd = __builtin_fmaf(bf16_hi(o[i]), bf16_hi(g[i]), dd);
            }
        }
        lse2 = LSE[(size_t)bh * Tq + qrow] * 1.44269504088896340736f;
    } else {
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
            qf[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0});
            gf[t] = qf[t];
        }
    }
    dd = half_swap_sum(dd);
    // the row statistics bwd_dkdv reads: one lane per row writes them
    if (qrow < Tq && hf == 0 && kh == 0) stats[(size_t)bh * Tq + qrow] = make_float2(lse2, dd);

    const int kend = CAUSAL ? min(Tkv, q0 + BQT + off) : Tkv;
    const int nblk = (kend + BK - 1) / BK;
    const int lim = CAUSAL ? min(Tkv - 1, qrow + off) : (Tkv - 1);   // last key this row sees

    uint32_t voff[DQ_LI];
#pragma unroll
    for (int i = 0; i < DQ_LI; ++i) {
        const int g = wave + DQ_WAVES * i;
        const int row = RPG * g + lane / CPR;
        voff[i] = (uint32_t)(row * ROWB + (((lane % CPR) ^ G::swz(row)) << 4));
    }
    auto issue = [&](int j) {
        const int kb = j * BK;
        const bool live = j < nblk;
        const uint32_t bytes = live ? (uint32_t)(Tkv - kb) * (uint32_t)ROWB : 0u;
        const size_t eoff = live ? (size_t)kb * D : 0;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + eoff, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + eoff, bytes);
        uint8_t* st = &ring[j % NS][0][0];
#pragma unroll
        for (int i = 0; i < DQ_LI; ++i) {
            const int g = wave + DQ_WAVES * i;
            buffer_load_lds_b128(rk, voff[i], st + g * 1024);
            buffer_load_lds_b128(rv, voff[i], st + KBLK + g * 1024);
        }
    };

    uint32_t r_off[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) r_off[t] = (uint32_t)(ln * ROWB + (((2 * t + hf) ^ G::swz(ln)) << 4));
    uint32_t t_off[DT][2];
    tr_offsets<D>(lane, t_off);

    f32x16_t dqt[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqt[dt][r] = 0.f;

    // Per-lane LDS addresses in ring stage 0 of this wave's keys (rows
    // wko.. of the stage); a stage adds a constant, so the loop below is
    // unrolled by the ring depth and blocks need no address arithmetic.
    const int wko = KS == 2 ? kh * 32 : 0;
    const uint32_t ring0 = lds_addr(&ring[0][0][0]) + (uint32_t)(wko * ROWB);
    uint32_t k_ra[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) k_ra[t] = ring0 + r_off[t];
    uint32_t t_ra[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        t_ra[dt][0] = ring0 + t_off[dt][0];
        t_ra[dt][1] = ring0 + t_off[dt][1];
    }

    // one block for this wave in ring stage S: its WKT 32-key tiles (kb = first key)
    auto step = [&](auto stage_tag, int kb, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr int SO = decltype(stage_tag)::value * 2 * KBLK;
        // S^T and dP^T for the wave's keys; lane = query column
        uint32_t dw[8 * WKT];
#pragma unroll
        for (int kt = 0; kt < WKT; ++kt) {
            f32x16_t s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = 0.f;
                dp[r] = 0.f;
            }
#pragma unroll
            for (int t = 0; t < TQ; ++t) {
                const bf16x8_t a = kt ? lds_b128<SO + 32 * ROWB>(k_ra[t]) : lds_b128<SO>(k_ra[t]);
                const bf16x8_t b = kt ? lds_b128<SO + KBLK + 32 * ROWB>(k_ra[t]) : lds_b128<SO + KBLK>(k_ra[t]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, gf[t], dp, 0, 0, 0);
            }
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = __builtin_fmaf(s[r], c, -lse2);
                if constexpr (MASK) {
                    // a masked score gets exponent -inf: exp2 gives 0, no branch
                    const int kk = kb + 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
                    x = kk > lim ? -__builtin_inff() : x;
                }
                ds[r] = fast_exp2(x) * (dp[r] - dd);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) dw[8 * kt + i] = pack_bf16x2(ds[2 * i], ds[2 * i + 1]);
        }
        // dQ^T += K^T dS^T: four 16-key k-steps
        auto kstep = [&](auto stp_tag) {
            constexpr int stp = decltype(stp_tag)::value;
            const u32x4_t dv = {dw[4 * stp], dw[4 * stp + 1], dw[4 * stp + 2], dw[4 * stp + 3]};
            const bf16x8_t db = __builtin_bit_cast(bf16x8_t, dv);
            u32x4_t a[DT];
            tr_kstep_at<D, stp, SO>(t_ra, a);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                dqt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[dt]), db, dqt[dt],
                                                                  0, 0, 0);
        };
        // head width 64: two k-steps' K^T operands behind one wait
        auto kstep_pair = [&](auto stp_tag) {
            constexpr int stp = decltype(stp_tag)::value;
            u32x4_t a0[2], a1[2];
            tr_kstep2_d64_at<stp, stp + 1, SO>(t_ra, a0, a1);
            const u32x4_t d0 = {dw[4 * stp], dw[4 * stp + 1], dw[4 * stp + 2], dw[4 * stp + 3]};
            const u32x4_t d1 = {dw[4 * stp + 4], dw[4 * stp + 5], dw[4 * stp + 6], dw[4 * stp + 7]};
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
                dqt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a0[dt]),
                                                                  __builtin_bit_cast(bf16x8_t, d0), dqt[dt], 0, 0, 0);
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
                dqt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a1[dt]),
                                                                  __builtin_bit_cast(bf16x8_t, d1), dqt[dt], 0, 0, 0);
        };
        if constexpr (D == 64) {
            kstep_pair(std::integral_constant<int, 0>{});
            if constexpr (WKT > 1) kstep_pair(std::integral_constant<int, 2>{});
        } else {
            kstep(std::integral_constant<int, 0>{});
            kstep(std::integral_constant<int, 1>{});
            if constexpr (WKT > 1) {
                kstep(std::integral_constant<int, 2>{});
                kstep(std::integral_constant<int, 3>{});
            }
        }
    };

    const int nfull = CAUSAL ? min(Tkv / BK, (q0 + off + 1) / BK) : Tkv / BK;
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue(j);
    static_assert(NS == 3, "the unrolled loop below assumes a 3-stage ring");
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // block j sits in stage j % NS
    auto blk = [&](int j, auto stage_tag, auto mask_tag) {
        wait_vmcnt<2 * DQ_LI * (NS - 2)>();
        __syncthreads();
        issue(j + NS - 1);
        step(stage_tag, j * BK + wko, mask_tag);
    };
    int j = 0;
    for (; j + 2 < nfull; j += 3) {
        blk(j, I0{}, std::false_type{});
        blk(j + 1, I1{}, std::false_type{});
        blk(j + 2, I2{}, std::false_type{});
    }
    // The rest (at most two unmasked blocks, then the diagonal and ragged
    // ones) runs the masked body, also for a block whose keys all follow this
    // wave's rows (every score masked: it adds exact zeros), three blocks at
    // a time from j = 0 mod 3, so stages stay compile-time.  A stage chosen
    // at run time, or a branch around a block, made the register allocator
    // copy the accumulator at the join on every such block.
    for (; j + 2 < nblk; j += 3) {
        blk(j, I0{}, std::true_type{});
        blk(j + 1, I1{}, std::true_type{});
        blk(j + 2, I2{}, std::true_type{});
    }
    if (j < nblk) blk(j, I0{}, std::true_type{});
    if (j + 1 < nblk) blk(j + 1, I1{}, std::true_type{});
    wait_vmcnt<0>();

    if constexpr (KS == 2) {
        // the second wave of each row group hands its dQ^T partial to the
        // first through the ring (lane-major on both sides, conflict-free)
        constexpr int NREG = DT * 16;
        static_assert(RG * NREG * 64 * 4 <= NS * 2 * KBLK, "merge buffer must fit in the ring");
        __syncthreads();                      // every wave is done reading the ring
        float* xb = reinterpret_cast<float*>(&ring[0][0][0]) + rg * NREG * 64 + lane;
        if (kh == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xb[(dt * 16 + r) * 64] = dqt[dt][r];
        }
        __syncthreads();
        if (kh == 1) return;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) dqt[dt][r] += xb[(dt * 16 + r) * 64];
    }

    // dQ = scale * (dQ^T)^T: lane = query row, element r = d 32dt + 8(r/4) + 4hf + r%4
    if (qrow < Tq) {
        float* row = dQ + qbase + (size_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                float4 a;
                a.x = dqt[dt][4 * g4] * scale;
                a.y = dqt[dt][4 * g4 + 1] * scale;
                a.z = dqt[dt][4 * g4 + 2] * scale;
                a.w = dqt[dt][4 * g4 + 3] * scale;
                *reinterpret_cast<float4*>(row + 32 * dt + 8 * g4 + 4 * hf) = a;
            }
    }
}

// d = 64 grids with fewer than three 128-wide tiles per compute unit split
// each tile's serial loop over a pair of waves (query halves for dK/dV, key
// halves for dQ).
bool bwd_kv_halves(const BackwardArgs& a) {
    return a.d == 64 && (long long)((a.Tkv + BKV - 1) / BKV) * a.B * a.H < 3LL * 256;
}
bool bwd_q_halves(const BackwardArgs& a) {
    return a.d == 64 && (long long)((a.Tq + BQ - 1) / BQ) * a.B * a.H < 3LL * 256;
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_c(const BackwardArgs& a, hipStream_t stream) {
    const int BHn = a.B * a.H;
    float2* stats = static_cast<float2*>(a.workspace);
    bool kv_halves = false, q_halves = false;
    if constexpr (D == 64) {
        kv_halves = bwd_kv_halves(a);
        q_halves = bwd_q_halves(a);
    }
    // dQ first: it writes the row statistics that dK/dV reads
    if constexpr (D == 64) {
        if (q_halves) {
            const int nqt = (a.Tq + BQ / 2 - 1) / (BQ / 2);
            hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, 2>), dim3((unsigned)(nqt * BHn)), dim3(DQ_WAVES * 64), 0,
                               stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                               static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout),
                               static_cast<const uint16_t*>(a.o), a.lse, stats, a.dq, a.Tq, a.Tkv, BHn, nqt, a.c,
                               a.scale);
        }
    }
    if (!q_halves) {
        const int nqt = (a.Tq + BQ - 1) / BQ;
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(nqt * BHn)), dim3(DQ_WAVES * 64), 0, stream,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout),
                           static_cast<const uint16_t*>(a.o), a.lse, stats, a.dq, a.Tq, a.Tkv, BHn, nqt, a.c,
                           a.scale);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (D == 64) {
        if (kv_halves) {
            const int nkt = (a.Tkv + BKV / 2 - 1) / (BKV / 2);
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, 2>), dim3((unsigned)(nkt * BHn)), dim3(KV_WAVES * 64), 0,
                               stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                               static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout), stats, a.dk,
                               a.dv, a.Tq, a.Tkv, BHn, a.c, a.scale);
        }
    }
    if (!kv_halves) {
        const int nkt = (a.Tkv + BKV - 1) / BKV;
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(nkt * BHn)), dim3(KV_WAVES * 64), 0, stream,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout), stats, a.dk,
                           a.dv, a.Tq, a.Tkv, BHn, a.c, a.scale);
    }
    return hipGetLastError();
}

thread_local char g_name[128];

}  // namespace

bool backward_supports(int d) { return d == 64 || d == 128; }

size_t backward_workspace_bytes(int B, int H, int Tq) { return (size_t)B * H * Tq * sizeof(float2); }

hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t stream, const char** name) {
    const int bq2 = a.d == 128 ? BwdGeo<128>::BQ2 : BwdGeo<64>::BQ2;
    const int bk = a.d == 128 ? BwdGeo<128>::BK : BwdGeo<64>::BK;
    const bool kvh = bwd_kv_halves(a), qh = bwd_q_halves(a);
    snprintf(g_name, sizeof g_name, "bwd_bf16_d%d<dq+stats(bq=%d,bk=%d%s)+dkdv(bk=%d,bq=%d%s)%s>", a.d,
             qh ? BQ / 2 : BQ, bk, qh ? ",key_halves=2" : "", kvh ? BKV / 2 : BKV, bq2,
             kvh ? ",query_halves=2" : "", a.causal ? ",causal" : "");
    *name = g_name;
    if (a.d == 128) {
        if (a.causal) return launch_bwd_c<128, true>(a, stream);
        return launch_bwd_c<128, false>(a, stream);
    }
    if (a.causal) return launch_bwd_c<64, true>(a, stream);
    return launch_bwd_c<64, false>(a, stream);
}

}  // namespace attn
