// Exact attention forward (prefill), bf16 inputs, head width 64 or 128, gfx950.
//
// One workgroup owns a tile of BQ = 32 * WAVES query rows of one (batch, head)
// and streams the key/value blocks of BK rows past it (BK = 64 for d = 64;
// BK = 32 for d = 128, whose rows are twice as long -- the halved block the
// head width 128 needs in "IO-Aware Attention", section "What has to stay in
// fast memory") ("IO-Aware Attention:
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
// rescaled by exp2(m_old - m_new)) whenever either half of a row's block sum
// (the keys one lane holds) exceeds 2^15 or is not finite, which bounds every
// block row sum by 2^16 and keeps fp32 far from overflow.  Blocks therefore
// cost no row max and no exchange between lanes in the common case: softmax
// work is one FMA, one exp2 and one add per score and a bf16 pack per pair --
// the VALU budget is what limits a d = 64 head on CDNA4, since each score
// carries only 4*64 MFMA flops.  (The row sum stays fp32: a sum of the bf16-rounded
// terms would cost the log-sum-exp up to 2^-9 relative on short rows.)
//
// Layout choices for CDNA4:
// * Computing the transposed products puts one query row in each lane (lane
//   l and l+32 hold the two halves of row l % 32), so row sums are lane-local
//   plus one v_permlane32_swap, the softmax rescale is a per-lane scalar, and
//   the fp32 accumulator of the first product is already the B operand of the
//   second (only a bf16 pack in between).
// * Q stays in VGPRs for the whole key loop (d/4 VGPRs per lane).
// * K and V blocks go from HBM straight into an NS-stage LDS ring with
//   buffer_load ... lds (no staging registers, no LDS store instructions;
//   the buffer range check zero-fills the ragged end).  Rows keep their
//   natural 2d-byte layout with the 16-byte chunks XOR-swizzled per row, so
//   the K operand reads (ds_read_b128) and the V operand reads are free of
//   bank conflicts.  V is read with ds_read_b64_tr_b16, which hands every
//   lane four consecutive keys of one column: exactly the operand layout of
//   the PV product, without transposing V anywhere.
// * One barrier per block: it publishes block j (waited for with vmcnt) and
//   frees the stage block j+NS-1 is then loaded into.
// * Causal: the key loop stops at the tile's diagonal block; element masks
//   are applied only on blocks that cross a wave's diagonal or the ragged end,
//   and a wave whose rows all lie above a block skips its math for that block.
// * Tiles are launched heaviest-first (last query tiles first) and the
//   linear block id keeps every tile of one (batch, head) on one XCD when the
//   number of heads is a multiple of 8 (full attention: an XCD's heads one
//   after another), else a head's tiles on as few XCDs as the count allows.
// * Grids of too few 128-row tiles (d = 64) use 64-row tiles whose key loop
//   is split over the two waves of a pair and merged through LDS at the end
//   (KS = 2 below), which halves the serial chain of the heaviest tiles.
#include <cstdio>

#include "common.hpp"
#include "launch.hpp"

namespace attn {
namespace {

// Largest share of a block row sum that one lane (half of the row's keys)
// keeps without raising m: 2^15, so the row's block sum stays within 2^16.
// Each lane tests its own half, and the test needs no exchange between the
// two halves.
constexpr float kHalfSumLimit = 32768.0f;

// A 16-byte LDS load at an LDS byte address plus a constant (the constant
// lands in the instruction's offset field); the compiler tracks its wait.
template <int OFF>
__device__ __forceinline__ bf16x8_t lds_load_b128(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>((uintptr_t)(addr + OFF));
}

// LDS DMA of 16 bytes per lane with a constant added (in the instruction's
// offset field, so inside the buffer range check) to both the global and the
// LDS address.
template <int OFF>
__device__ __forceinline__ void buffer_load_lds_b128_off(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
    static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, (int)voff, 0, OFF, 0);
}

// Tile geometry per head width.  Rows are D*2 bytes; LDS chunk swizzles
// (16-byte chunk index within a row) make the K operand reads (ds_read_b128,
// 32 rows x one chunk pair per instruction) and the V transposed reads (8
// rows x 64 bytes per instruction) free of bank conflicts.
template <int D>
struct Geo;
template <>
struct Geo<64> {
    static constexpr int BK = 64;
    // 128-byte rows: two rows share a 256-byte bank line
    static __device__ __forceinline__ int swz_k(int row) { return (row >> 1) & 7; }
    static __device__ __forceinline__ int swz_v(int row) { return ((row >> 1) & 1) << 2; }
};
template <>
struct Geo<128> {
    static constexpr int BK = 32;
    // 256-byte rows: one row per bank line; K chunks rotate over 16 rows, V's
    // 64-byte segments over 4
    static __device__ __forceinline__ int swz_k(int row) { return row & 15; }
    static __device__ __forceinline__ int swz_v(int row) { return (row & 3) << 2; }
};

// Key blocks of bk keys a query tile must visit (causal: up to its last
// row's diagonal).
__host__ __device__ __forceinline__ int tile_blocks(int qt, int bq, int bk, int Tq, int Tkv, bool causal) {
    const int kend = causal ? min(Tkv, (qt + 1) * bq + (Tkv - Tq)) : Tkv;
    return (kend + bk - 1) / bk;
}

// Slices per head in the XCD-aware tile order: 8 / gcd(BH, 8).
__host__ __device__ __forceinline__ int head_slices(int BH) {
    const int g = (BH & 1) ? 1 : (BH & 2) ? 2 : (BH & 4) ? 4 : 8;
    return 8 / g;
}

// Chunks a tile of nblk key blocks is split into when a work unit takes at
// most `chunk` blocks (chunk <= 0: never split).
__host__ __device__ __forceinline__ int tile_chunks(int nblk, int chunk) {
    return chunk > 0 ? (nblk + chunk - 1) / chunk : 1;
}

// One work unit = one query tile x one chunk of its key blocks.  Chunk cc of a
// tile split into nch chunks covers blocks [cc*nblk/nch, (cc+1)*nblk/nch).
// Units of unsplit tiles write O and LSE; units of split tiles write their
// partial result (O normalised by the chunk's own sum, and the chunk's
// base-2 log-sum-exp) to `part`, merged later by prefill_combine_kernel.
//
// KS = 2 (key halves, d = 64 only): the waves form WAVES/2 query row groups of
// 32 rows, and each row group has two waves that take the two 32-key halves of
// every 64-key stage; the pair merges its two (m, l, O) states through LDS at
// the end with the same rescaling.  Tiles are then BQ = 64 rows and the serial
// key loop of a tile is half as long, for shapes with too few 128-row tiles
// to fill the chip (no workspace, no second kernel).
template <int D, int WAVES, int NS, bool CAUSAL, int KS = 1>
__global__ __launch_bounds__(WAVES * 64, 2)
void prefill_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                         const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                         float* __restrict__ LSE, float* __restrict__ part, int Tq, int Tkv, int BH,
                         int nqt, int chunk, int nch_max, float c) {
    using G = Geo<D>;
    static_assert(KS == 1 || (KS == 2 && D == 64 && WAVES % 2 == 0), "key halves need 64-key stages");
    constexpr int BK = G::BK;                 // keys per ring stage
    constexpr int WK = BK / KS;               // keys per wave per stage
    constexpr int RG = WAVES / KS;            // query row groups of 32 rows
    constexpr int BQ = RG * 32;
    constexpr int ROWB = D * 2;               // bytes per K/V row
    constexpr int TILEB = BK * ROWB;          // bytes per K (or V) block: 8 KiB
    constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
    constexpr int RPG = 1024 / ROWB;          // rows per 1 KiB load instruction
    constexpr int TQ = D / 16;                // k-steps of the QK product
    constexpr int DT = D / 32;                // 32-column tiles of O
    constexpr int KT = WK / 32;               // 32-key tiles of S
    constexpr int ST = WK / 16;               // 16-key steps of the PV product
    static_assert((TILEB / 1024) % WAVES == 0, "row groups of a block must split evenly over the waves");
    constexpr int LI = TILEB / 1024 / WAVES;  // 1 KiB load instructions per wave per operand per block

    __shared__ __attribute__((aligned(1024))) uint8_t ring[NS][2][TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int ln = lane & 31;
    const int hf = lane >> 5;
    const int rg = wave % RG;                 // query row group
    const int kh = wave / RG;                 // key half of every stage (KS = 2)

    // unit id = (cc * nqt + rank) * BH + bh: first chunks of every tile first,
    // heaviest tiles first within a chunk index, and all units of one
    // (batch, head) on one XCD when BH is a multiple of 8.
    // Causal key halves with at least three rounds of 32 units per XCD (one
    // per compute unit per round, three resident per compute unit): the
    // second round runs light-to-heavy (a snake over the heaviest-first
    // order), so the units that share a compute unit sum to similar work.
    const int id = blockIdx.x;
    int bh, rank, cc;
    if (CAUSAL && KS == 2 && BH % 8 == 0 && nqt * (BH >> 3) >= 96) {
        const int xcd = id & 7, k = id >> 3;        // k-th unit of this XCD
        const int per = BH >> 3;                    // heads per XCD
        const int round = k / 32, pos = k % 32;
        const bool full = (round + 1) * 32 <= nqt * per;
        const int p = ((round & 1) && full) ? round * 32 + 31 - pos : k;
        rank = p / per;
        bh = (p % per) * 8 + xcd;
        cc = 0;
    } else if (!CAUSAL && KS == 1 && chunk <= 0 && (BH & 7) == 0) {
        // Full attention, B*H a multiple of 8: XCD x (block ids x, x+8, ...)
        // runs its heads x, x+8, ... one after another, every tile of a head
        // before the next head, so the few heads it streams at once keep
        // their K/V in its L2 (tiles of a head cost the same: no order by
        // weight is needed).
        const int xcd = id & 7, k = id >> 3;
        rank = k % nqt;
        bh = (k / nqt) * 8 + xcd;
        cc = 0;
    } else if (KS == 1 && chunk <= 0 && (BH & 7) != 0 && nqt % head_slices(BH) == 0) {
        // B*H not a multiple of 8: each head's tiles are split into
        // s = 8 / gcd(B*H, 8) slices by rank mod s, and XCD x (block ids
        // x, x+8, ...) owns the B*H/gcd consecutive slices starting at slice
        // x*B*H/gcd -- fewer than two heads per XCD, so their K/V stays in
        // its L2 -- taken heaviest rank first.
        const int sl_per_head = head_slices(BH);
        const int spx = BH * sl_per_head / 8;          // slices per XCD
        const int xcd = id & 7, k = id >> 3;
        const int grp = k / spx, i = k % spx;
        const int first = xcd * spx;
        int sl = first, seen = 0;
        for (int p = 0; p < sl_per_head; ++p) {        // slices of parity p, in order
            const int lo = first + ((p - first % sl_per_head) + sl_per_head) % sl_per_head;
            const int cnt = lo < first + spx ? (first + spx - 1 - lo) / sl_per_head + 1 : 0;
            if (i < seen + cnt) {
                sl = lo + (i - seen) * sl_per_head;
                break;
            }
            seen += cnt;
        }
        rank = grp * sl_per_head + sl % sl_per_head;
        bh = sl / sl_per_head;
        cc = 0;
    } else {
        bh = id % BH;
        const int rest = id / BH;
        rank = rest % nqt;
        cc = rest / nqt;
    }
    const int qt = CAUSAL ? (nqt - 1 - rank) : rank;
    const int q0 = qt * BQ;
    const int off = Tkv - Tq;                 // bottom-right causal alignment

    const int nblk = tile_blocks(qt, BQ, BK, Tq, Tkv, CAUSAL);
    const int nch = tile_chunks(nblk, chunk);
    if (cc >= nch) return;                    // this tile has fewer chunks (uniform per workgroup)
    const int jlo = (int)(((long long)cc * nblk) / nch);
    const int jhi = (int)(((long long)(cc + 1) * nblk) / nch);

    const size_t qbase = (size_t)bh * Tq * D;
    const size_t kvbase = (size_t)bh * Tkv * D;
    const uint16_t* Kh = K + kvbase;
    const uint16_t* Vh = V + kvbase;

    // ---- Q fragment: row q0 + 32*rg + ln, d = 16t + 8hf + (0..7) ----
    const int qrow = q0 + rg * 32 + ln;
    bf16x8_t qf[TQ];
    if (qrow < Tq) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(Q + qbase + (size_t)qrow * D + 8 * hf);
#pragma unroll
        for (int t = 0; t < TQ; ++t) qf[t] = __builtin_bit_cast(bf16x8_t, src[2 * t]);
    } else {
#pragma unroll
        for (int t = 0; t < TQ; ++t) qf[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0});
    }

    const int wq_first = q0 + rg * 32;         // this wave's first / last query row
    const int wq_last = wq_first + 31;
    const int lim = CAUSAL ? min(Tkv - 1, qrow + off) : (Tkv - 1);   // last key this row may see

    // ---- DMA loads (head width 128): wave w moves row groups g = w + WAVES*i
    // (RPG rows = 1 KiB each) ----
    uint32_t k_voff[LI], v_voff[LI];
#pragma unroll
    for (int i = 0; i < LI; ++i) {
        const int g = wave + WAVES * i;
        const int row = RPG * g + lane / CPR;
        const int slot = lane % CPR;          // the chunk position this lane fills in LDS
        k_voff[i] = (uint32_t)(row * ROWB + ((slot ^ G::swz_k(row)) << 4));
        v_voff[i] = (uint32_t)(row * ROWB + ((slot ^ G::swz_v(row)) << 4));
    }
    // ---- DMA loads (head width 64): wave w moves the 1 KiB row groups g0 and
    // g0 + 2, with g0 = (w mod 2) + 4 (w / 2).  The two are 16 rows apart, where
    // the K and V chunk swizzles (functions of row bits 1-3) agree, so the
    // second load is the first plus 2 KiB in the instruction's offset field
    // (applied to the global and the LDS address alike, inside the buffer
    // range check): one offset register per operand.  At head width 128 the
    // matching rows are 4 KiB apart, past the 12-bit offset field. ----
    const int g0 = (wave & 1) + 4 * (wave >> 1);
    const int row0 = RPG * g0 + lane / CPR;
    const uint32_t k_voff0 = (uint32_t)(row0 * ROWB + (((lane % CPR) ^ G::swz_k(row0)) << 4));
    const uint32_t v_voff0 = (uint32_t)(row0 * ROWB + (((lane % CPR) ^ G::swz_v(row0)) << 4));
    // (128-row tiles, head width 64) DMA of K and V block j into stage
    // S = (j - jlo) % NS.  Blocks past the unit's end still issue, with an
    // empty range (no memory traffic; the base is never dereferenced), so that
    // every wave's vmcnt count stays uniform.
    auto issue = [&](int j, auto stage_tag) {
        static_assert(D == 64 && LI == 2 && RPG == 8 && WAVES == 4, "row-group mapping of the head-width-64 DMA");
        constexpr int S = decltype(stage_tag)::value;
        const uint32_t kb = (uint32_t)j * BK;
        const uint32_t bytes = j < jhi ? (uint32_t)(Tkv - (int)kb) * (uint32_t)ROWB : 0u;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)kb * D, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + (size_t)kb * D, bytes);
        uint8_t* st = &ring[S][0][0] + g0 * 1024;
        buffer_load_lds_b128_off<0>(rk, k_voff0, st);
        buffer_load_lds_b128_off<2048>(rk, k_voff0, st);
        buffer_load_lds_b128_off<0>(rv, v_voff0, st + TILEB);
        buffer_load_lds_b128_off<2048>(rv, v_voff0, st + TILEB);
    };

    // (head width 128) the same with the stage chosen at run time: block j
    // goes to stage j % NS.
    auto issue_rt = [&](int j) {
        const int kb = j * BK;
        const bool live = j < jhi;
        const uint32_t bytes = live ? (uint32_t)(Tkv - kb) * (uint32_t)ROWB : 0u;
        const size_t eoff = live ? (size_t)kb * D : 0;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + eoff, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + eoff, bytes);
        uint8_t* st = &ring[j % NS][0][0];
#pragma unroll
        for (int i = 0; i < LI; ++i) {
            const int g = wave + WAVES * i;
            buffer_load_lds_b128(rk, k_voff[i], st + g * 1024);
            buffer_load_lds_b128(rv, v_voff[i], st + TILEB + g * 1024);
        }
    };

    // ---- per-lane LDS read offsets (within a stage) ----
    // K operand of step t: row 32kt + ln, chunk 2t + hf (kt adds 32 rows).
    uint32_t k_roff[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) k_roff[t] = (uint32_t)(ln * ROWB + (((2 * t + hf) ^ G::swz_k(ln)) << 4));
    // V operand (transposed read) of step st, d-tile dt: lane group lg = lane / 16,
    // j = lane % 16 addresses row 16st + 4(lg/2) + j/4 (+8 for the second half),
    // columns 32dt + 16(lg%2) + 4(j%4) .. +3 (st adds 16 rows).
    uint32_t v_roff[DT];
    {
        const int lg = lane >> 4, jj = lane & 15;
        const int row = 4 * (lg >> 1) + (jj >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int col = 32 * dt + 16 * (lg & 1) + 4 * (jj & 3);
            v_roff[dt] = (uint32_t)(row * ROWB + ((((col >> 3) ^ G::swz_v(row)) << 4) | ((col & 4) << 1)));
        }
    }

    f32x16_t oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m = kNegInf;   // reference max of S * c (log2 units), raised only when needed
    float l = 0.f;       // this lane's share of the running sum (relative to m)

    // One key block for this wave at a run-time stage (head width 128: its
    // compile-time-stage form below needs more VGPRs than three waves per
    // SIMD allow).  MASK applies the causal / ragged element mask.
    auto step_rt = [&](const uint8_t* kst, int kb, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const uint8_t* vst = kst + TILEB;
        f32x16_t s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
            for (int t = 0; t < TQ; ++t) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kst + k_roff[t] + kt * 32 * ROWB);
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kt], 0, 0, 0);
            }
        }
        const uint32_t vbase = lds_addr(vst);
        if constexpr (MASK) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (key > lim) s[kt][r] = kNegInf;
                }
        }
        // exponentials against the current reference; packed to bf16 pairs
        uint32_t pw[8 * KT];
        float rs = 0.f;
        auto exponentiate = [&](float mref) {
            rs = 0.f;
#pragma unroll
            for (int i = 0; i < 8 * KT; ++i) {
                const int kt = i >> 3, r = 2 * (i & 7);
                const float p0 = fast_exp2(__builtin_fmaf(s[kt][r], c, -mref));
                const float p1 = fast_exp2(__builtin_fmaf(s[kt][r + 1], c, -mref));
                pw[i] = pack_bf16x2(p0, p1);
                rs = i == 0 ? p0 + p1 : rs + (p0 + p1);   // no add of the zero start value
            }
        };
        exponentiate(m);
        if (__builtin_amdgcn_ballot_w64(!(rs <= kHalfSumLimit)) != 0) {
            // raise the reference to the true running max and rescale
            float mx = kNegInf;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
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
        auto pv_step = [&](auto st_tag) {
            constexpr int st = decltype(st_tag)::value;
            constexpr int o = st * 16 * ROWB;
            const u32x4_t pv = {pw[4 * st], pw[4 * st + 1], pw[4 * st + 2], pw[4 * st + 3]};
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
#pragma unroll
            for (int d2 = 0; d2 < DT; d2 += 2) {
                const uint32_t va = vbase + v_roff[d2], vc = vbase + v_roff[d2 + 1];
                u32x4_t a0, a1;
                lds_read_tr16_x4<o, o + 8 * ROWB, o, o + 8 * ROWB>(va, va, vc, vc, a0, a1);
                oacc[d2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a0), pb, oacc[d2],
                                                                   0, 0, 0);
                oacc[d2 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a1), pb,
                                                                       oacc[d2 + 1], 0, 0, 0);
            }
        };
        pv_step(std::integral_constant<int, 0>{});
        pv_step(std::integral_constant<int, 1>{});
        if constexpr (ST > 2) {
            pv_step(std::integral_constant<int, 2>{});
            pv_step(std::integral_constant<int, 3>{});
        }
    };

    // (KS = 1) stage S of the ring: LDS read addresses are per-lane bases in
    // stage 0 plus compile-time offsets
    const uint32_t ring_lds = lds_addr(&ring[0][0][0]);
    uint32_t k_ra1[TQ], v_ra1[DT];
#pragma unroll
    for (int t = 0; t < TQ; ++t) k_ra1[t] = ring_lds + k_roff[t];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) v_ra1[dt] = ring_lds + TILEB + v_roff[dt];
    auto step = [&](auto stage_tag, int kb, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr int SO = decltype(stage_tag)::value * 2 * TILEB;
        f32x16_t s[KT];
        auto qk_tile = [&](auto kt_tag) {
            constexpr int kt = decltype(kt_tag)::value;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
            for (int t = 0; t < TQ; ++t) {
                const bf16x8_t a = lds_load_b128<SO + kt * 32 * ROWB>(k_ra1[t]);
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kt], 0, 0, 0);
            }
        };
        qk_tile(std::integral_constant<int, 0>{});
        if constexpr (KT > 1) qk_tile(std::integral_constant<int, 1>{});
        if constexpr (MASK) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (key > lim) s[kt][r] = kNegInf;
                }
        }
        // exponentials against the current reference; packed to bf16 pairs
        uint32_t pw[8 * KT];
        float rs = 0.f;
        auto exponentiate = [&](float mref) {
            rs = 0.f;
#pragma unroll
            for (int i = 0; i < 8 * KT; ++i) {
                const int kt = i >> 3, r = 2 * (i & 7);
                const float p0 = fast_exp2(__builtin_fmaf(s[kt][r], c, -mref));
                const float p1 = fast_exp2(__builtin_fmaf(s[kt][r + 1], c, -mref));
                pw[i] = pack_bf16x2(p0, p1);
                rs = i == 0 ? p0 + p1 : rs + (p0 + p1);   // no add of the zero start value
            }
        };
        exponentiate(m);
        if (__builtin_amdgcn_ballot_w64(!(rs <= kHalfSumLimit)) != 0) {
            // raise the reference to the true running max and rescale
            float mx = kNegInf;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
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
        auto pv_step = [&](auto st_tag) {
            constexpr int st = decltype(st_tag)::value;
            constexpr int o = st * 16 * ROWB;
            const u32x4_t pv = {pw[4 * st], pw[4 * st + 1], pw[4 * st + 2], pw[4 * st + 3]};
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
#pragma unroll
            for (int d2 = 0; d2 < DT; d2 += 2) {
                u32x4_t a0, a1;
                lds_read_tr16_x4<SO + o, SO + o + 8 * ROWB, SO + o, SO + o + 8 * ROWB>(
                    v_ra1[d2], v_ra1[d2], v_ra1[d2 + 1], v_ra1[d2 + 1], a0, a1);
                oacc[d2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a0), pb, oacc[d2],
                                                                   0, 0, 0);
                oacc[d2 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a1), pb,
                                                                       oacc[d2 + 1], 0, 0, 0);
            }
        };
        pv_step(std::integral_constant<int, 0>{});
        pv_step(std::integral_constant<int, 1>{});
        if constexpr (ST > 2) {
            pv_step(std::integral_constant<int, 2>{});
            pv_step(std::integral_constant<int, 3>{});
        }
    };

    // Blocks [0, nfull) need no element mask for any row of the tile: they lie
    // inside the key range and, for causal, left of every row's diagonal.
    // Blocks [nfull, nblk) may be masked (diagonal or ragged end) or, for a
    // wave whose rows all precede them, skipped.
    const int nfull = CAUSAL ? min(Tkv / BK, (q0 + off + 1) / BK) : Tkv / BK;

    if constexpr (KS == 2) {
        // Software-pipelined key loop: iteration j runs the QK product of
        // block j+1 on the matrix cores while the VALU does the softmax of
        // block j, then the PV product of block j.  K of block b lives in
        // ring[b % NS][0] and V in ring[b % NS][1]; K runs one block ahead of
        // V, so iteration j issues K(j+NS) and V(j+NS-1), each into the stage
        // the previous iteration finished with, and every operand is still
        // requested NS-1 iterations before its use.  The interior loop is
        // unrolled by two so that stage indices are compile-time constants
        // (immediate LDS offsets) and the two score buffers alternate without
        // copies.  Units are unsplit here (jlo = 0).
        static_assert(NS == 2, "the unrolled loop below assumes a 2-stage ring");
        constexpr int HALF = WK * ROWB;
        constexpr int STAGEB = 2 * TILEB;     // bytes per ring stage (K + V)
        const uint32_t ring0 = lds_addr(&ring[0][0][0]) + (uint32_t)(kh * HALF);
        uint32_t k_ra[TQ], v_ra[DT];          // per-lane LDS read addresses in stage 0
#pragma unroll
        for (int t = 0; t < TQ; ++t) k_ra[t] = ring0 + k_roff[t];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) v_ra[dt] = ring0 + TILEB + v_roff[dt];
        // DMA of block b into stage S: the descriptor covers block b to the
        // end of the head (empty past the end: no memory traffic, and its
        // base is then never dereferenced)
        static_assert(LI == 2 && RPG == 8 && WAVES == 4, "row-group mapping of the head-width-64 DMA");
        auto issue_blk = [&](int b, auto stage_tag, auto which_tag) {
            constexpr int S = decltype(stage_tag)::value;
            constexpr int W = decltype(which_tag)::value;
            const uint32_t kb = (uint32_t)b * BK;
            const uint32_t bytes = (uint32_t)max(Tkv - (int)kb, 0) * (uint32_t)ROWB;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc((W ? Vh : Kh) + (size_t)kb * D, bytes);
            uint8_t* st = &ring[S][W][0] + g0 * 1024;
            buffer_load_lds_b128_off<0>(rs, W ? v_voff0 : k_voff0, st);
            buffer_load_lds_b128_off<2048>(rs, W ? v_voff0 : k_voff0, st);
        };
        auto qk = [&](auto stage_tag) {
            constexpr int S = decltype(stage_tag)::value;
            f32x16_t acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int t = 0; t < TQ; ++t) {
                const bf16x8_t a = lds_load_b128<S * STAGEB>(k_ra[t]);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], acc, 0, 0, 0);
            }
            return acc;
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        issue_blk(0, I0{}, I0{});             // K(0)
        issue_blk(1, I1{}, I0{});             // K(1)
        issue_blk(0, I0{}, I1{});             // V(0)
        wait_vmcnt<2 * LI * (NS - 1)>();      // K(0) has landed
        __syncthreads();
        // one block j in stage S = j % 2; sc holds S of block j, nxt receives
        // S of block j+1
        auto body = [&](int j, f32x16_t& sc, f32x16_t& nxt, auto mask_tag, auto stage_tag) {
            constexpr bool MASK = decltype(mask_tag)::value;
            constexpr int S = decltype(stage_tag)::value;
            constexpr int S1 = (S + 1) % NS, SP = (S + NS - 1) % NS;
            wait_vmcnt<2 * LI * (NS - 2)>();  // K(j+1) and V(j) have landed (this wave's part)
            __syncthreads();                  // ... everyone's; iteration j-1 is done everywhere
            issue_blk(j + NS, stage_tag, I0{});                              // K(j+2) replaces K(j)
            issue_blk(j + NS - 1, std::integral_constant<int, SP>{}, I1{});  // V(j+1) replaces V(j-1)
            if constexpr (MASK) {
                // diagonal / ragged block (a block this wave's rows all
                // precede is masked whole and adds nothing)
                const int kb = j * BK + kh * WK;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (key > lim) sc[r] = kNegInf;
                }
            }
            constexpr int VO = S * STAGEB;
            nxt = qk(std::integral_constant<int, S1>{});   // past the last block: unused
            // this block's V operands (both 16-key steps), read while the
            // matrix pipe runs the next block's QK products
            u32x4_t va[2][2];
            lds_read_tr16_x4<VO, VO + 8 * ROWB, VO, VO + 8 * ROWB>(v_ra[0], v_ra[0], v_ra[1], v_ra[1], va[0][0],
                                                                   va[0][1]);
            lds_read_tr16_x4<VO + 16 * ROWB, VO + 24 * ROWB, VO + 16 * ROWB, VO + 24 * ROWB>(
                v_ra[0], v_ra[0], v_ra[1], v_ra[1], va[1][0], va[1][1]);
            uint32_t pw[8];
            float rs = 0.f;
            auto exponentiate = [&](float mref) {
                float p0 = fast_exp2(__builtin_fmaf(sc[0], c, -mref));
                float p1 = fast_exp2(__builtin_fmaf(sc[1], c, -mref));
                pw[0] = pack_bf16x2(p0, p1);
                rs = p0 + p1;
#pragma unroll
                for (int i = 1; i < 8; ++i) {
                    p0 = fast_exp2(__builtin_fmaf(sc[2 * i], c, -mref));
                    p1 = fast_exp2(__builtin_fmaf(sc[2 * i + 1], c, -mref));
                    pw[i] = pack_bf16x2(p0, p1);
                    rs += p0 + p1;
                }
            };
            exponentiate(m);
            if (__builtin_amdgcn_ballot_w64(!(rs <= kHalfSumLimit)) != 0) {
                float mx = kNegInf;
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
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
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const u32x4_t pv = {pw[4 * st], pw[4 * st + 1], pw[4 * st + 2], pw[4 * st + 3]};
                const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
#pragma unroll
                for (int dt = 0; dt < 2; ++dt) {
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va[st][dt]), pb,
                                                                       oacc[dt], 0, 0, 0);
                }
            }
        };
        f32x16_t sa = qk(I0{}), sb;
        int j = 0;
        const int jfull = min(nfull, jhi);
        if (jfull > 0) {
            // block 0 is unmasked for every row: start the reference at this
            // wave's row max over it, so the first block takes the plain path
            // instead of the rescale pass (a masked block 0 keeps m = -inf)
            float mx = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[r]);
            m = half_swap_max(mx) * c;
        }
        for (; j + 1 < jfull; j += 2) {
            body(j, sa, sb, std::false_type{}, I0{});
            body(j + 1, sb, sa, std::false_type{}, I1{});
        }
        // The rest (at most one unmasked block, then the diagonal and ragged
        // ones) runs the masked body, whose tests are false on an unmasked
        // block, also two blocks at a time: j is even here, so both stages
        // stay compile-time and the score buffers alternate without copies.
        // (One block at a time, with the stage chosen at run time and the
        // scores copied back, made the register allocator copy the
        // accumulators on every such block.)
        for (; j + 1 < jhi; j += 2) {
            body(j, sa, sb, std::true_type{}, I0{});
            body(j + 1, sb, sa, std::true_type{}, I1{});
        }
        if (j < jhi) body(j, sa, sb, std::true_type{}, I0{});
    } else if constexpr (D == 64) {
        // Block j sits in stage (j - jlo) % NS; the interior loop is unrolled
        // by NS so that stages are compile-time (immediate LDS offsets).
        static_assert(NS == 3, "the unrolled loop below assumes a 3-stage ring");
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        issue(jlo, I0{});
        issue(jlo + 1, I1{});
        auto blk = [&](int j, auto stage_tag, auto mask_tag) {
            constexpr int S = decltype(stage_tag)::value;
            wait_vmcnt<2 * LI * (NS - 2)>();  // this wave's part of block j has landed
            __syncthreads();                  // ... everyone's, and the stage of block j-1 is free
            issue(j + NS - 1, std::integral_constant<int, (S + NS - 1) % NS>{});
            const int kb = j * BK;
            // masked blocks: no instruction moves between them (interleaving
            // the unrolled masked blocks costs registers)
            if constexpr (decltype(mask_tag)::value) __builtin_amdgcn_sched_barrier(0);
            if (!decltype(mask_tag)::value || !CAUSAL || kb <= wq_last + off) step(stage_tag, kb, mask_tag);
        };
        int j = jlo;
        const int jfull = min(nfull, jhi);
        for (; j + 2 < jfull; j += 3) {
            blk(j, I0{}, std::false_type{});
            blk(j + 1, I1{}, std::false_type{});
            blk(j + 2, I2{}, std::false_type{});
        }
        // The rest (at most two unmasked blocks, then the diagonal and ragged
        // ones) runs the masked body, three blocks at a time from
        // j - jlo = 0 mod 3, so stages stay compile-time.  (A stage chosen at
        // run time made the register allocator copy the accumulators at the
        // join on every such block.)
        for (; j + 2 < jhi; j += 3) {
            blk(j, I0{}, std::true_type{});
            blk(j + 1, I1{}, std::true_type{});
            blk(j + 2, I2{}, std::true_type{});
        }
        if (j < jhi) blk(j, I0{}, std::true_type{});
        if (j + 1 < jhi) blk(j + 1, I1{}, std::true_type{});
    } else {
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue_rt(jlo + j);

    int j = jlo;
    const int jfull = min(nfull, jhi);
    for (; j < jfull; ++j) {
        wait_vmcnt<2 * LI * (NS - 2)>();      // this wave's part of block j has landed
        __syncthreads();                      // ... everyone's, and stage (j-1) % NS is free
        issue_rt(j + NS - 1);
        step_rt(&ring[j % NS][0][0], j * BK, std::false_type{});
    }
    for (; j < jhi; ++j) {
        wait_vmcnt<2 * LI * (NS - 2)>();
        __syncthreads();
        issue_rt(j + NS - 1);
        const int kb = j * BK;
        if (!CAUSAL || kb <= wq_last + off) step_rt(&ring[j % NS][0][0], kb, std::true_type{});
    }
    }
    wait_vmcnt<0>();    // no DMA may still be writing LDS when the workgroup retires

    if constexpr (KS == 2) {
        // The second wave of each row group hands (O, m, l) to the first
        // through the ring (same lane layout on both sides: lane-major,
        // conflict-free); the first merges with the rescaling merge:
        // M = max(m_a, m_b), O = 2^(m_a-M) O_a + 2^(m_b-M) O_b, likewise l.
        constexpr int NREG = DT * 16 + 2;
        static_assert(RG * NREG * 64 * 4 <= NS * 2 * TILEB, "merge buffer must fit in the ring");
        __syncthreads();                      // every wave is done reading the ring
        float* xb = reinterpret_cast<float*>(&ring[0][0][0]) + rg * NREG * 64 + lane;
        if (kh == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xb[(dt * 16 + r) * 64] = oacc[dt][r];
            xb[DT * 16 * 64] = m;
            xb[(DT * 16 + 1) * 64] = l;
        }
        __syncthreads();
        if (kh == 1) return;
        const float mb = xb[DT * 16 * 64];
        const float lb = xb[(DT * 16 + 1) * 64];
        const float mm = fmaxf(m, mb);
        const float mu = (mm == kNegInf) ? 0.f : mm;
        const float wa = fast_exp2(m - mu), wb = fast_exp2(mb - mu);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] = wa * oacc[dt][r] + wb * xb[(dt * 16 + r) * 64];
        l = wa * l + wb * lb;
        m = mm;
    }

    // ---- epilogue: divide once, write O (bf16) and LSE (fp32) ----
    const float lsum = half_swap_sum(l);
    if (nch > 1) {
        // partial of a split tile; a row may see no key of a later chunk
        // (causal), then its weight is zero: o = 0, lse2 = -inf
        if (qrow < Tq) {
            const size_t rec = ((size_t)bh * nqt + qt) * nch_max + cc;
            float* prow = part + (rec * BQ + (qrow - q0)) * D;
            const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float4 w;
                    w.x = oacc[dt][4 * g] * inv;
                    w.y = oacc[dt][4 * g + 1] * inv;
                    w.z = oacc[dt][4 * g + 2] * inv;
                    w.w = oacc[dt][4 * g + 3] * inv;
                    *reinterpret_cast<float4*>(prow + 32 * dt + 8 * g + 4 * hf) = w;
                }
            if (hf == 0) {
                float* plse = part + (size_t)BH * nqt * nch_max * BQ * D;
                plse[rec * BQ + (qrow - q0)] = lsum > 0.f ? m + __builtin_log2f(lsum) : kNegInf;
            }
        }
        return;
    }
    if (qrow < Tq) {
        const float inv = 1.0f / lsum;
        uint16_t* orow = O + qbase + (size_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
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

// Head width 64, full attention, 256-row tiles.  Each of the 4 waves owns 64
// query rows as two 32-row sub-tiles u = 0, 1 (rows 64w + 32u + ln) and all 64
// keys of every stage, so every K and V operand it reads from LDS feeds both
// sub-tiles: a query row pulls half the LDS operand bytes of
// prefill_bf16_kernel, a wave's work per stage doubles (32 MFMAs, 2 x 32
// scores per lane), and two waves fit per SIMD -- 512 resident tiles where the
// 128-row kernel has 768.  Grids whose 128-row tiles would need a partly
// filled last round use it.  Ring (3 stages), DMA mapping, swizzles, the lazy
// reference max and the head-major tile order are prefill_bf16_kernel's; the
// only element mask is the ragged end of the key axis.
__global__ __launch_bounds__(256, 2)
void prefill_bf16_d64_r256_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                  const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                  float* __restrict__ LSE, int Tq, int Tkv, int BH, int nqt, float c) {
    using G = Geo<64>;
    constexpr int D = 64, BK = 64, ROWB = 2 * D, TILEB = BK * ROWB, CPR = ROWB / 16, RPG = 1024 / ROWB;
    constexpr int TQ = D / 16, DT = D / 32, KT = BK / 32, NS = 3, BQ = 256;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NS][2][TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 31;
    const int hf = lane >> 5;

    const int id = blockIdx.x;
    int bh, qt;
    if ((BH & 7) == 0) {
        // XCD x (block ids x, x+8, ...) runs its heads x, x+8, ... one after
        // another, every tile of a head before the next head
        const int xcd = id & 7, k = id >> 3;
        qt = k % nqt;
        bh = (k / nqt) * 8 + xcd;
    } else {
        bh = id % BH;
        qt = id / BH;
    }
    const int q0 = qt * BQ;
    const int nblk = (Tkv + BK - 1) / BK;
    const int nfull = Tkv / BK;               // blocks with no key past the end

    const size_t qbase = (size_t)bh * Tq * D;
    const size_t kvbase = (size_t)bh * Tkv * D;
    const uint16_t* Kh = K + kvbase;
    const uint16_t* Vh = V + kvbase;

    // Q fragments of the two sub-tiles: row q0 + 64w + 32u + ln, d = 16t + 8hf + (0..7)
    bf16x8_t qf[2][TQ];
    int qrow[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        qrow[u] = q0 + 64 * wave + 32 * u + ln;
        if (qrow[u] < Tq) {
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(Q + qbase + (size_t)qrow[u] * D + 8 * hf);
#pragma unroll
            for (int t = 0; t < TQ; ++t) qf[u][t] = __builtin_bit_cast(bf16x8_t, src[2 * t]);
        } else {
#pragma unroll
            for (int t = 0; t < TQ; ++t) qf[u][t] = __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0});
        }
    }

    // DMA: wave w moves the 1 KiB row groups g0 and g0 + 2 of K and V, as in
    // prefill_bf16_kernel (the second load is the first plus 2 KiB in the
    // instruction's offset field)
    const int g0 = (wave & 1) + 4 * (wave >> 1);
    const int row0 = RPG * g0 + lane / CPR;
    const uint32_t k_voff0 = (uint32_t)(row0 * ROWB + (((lane % CPR) ^ G::swz_k(row0)) << 4));
    const uint32_t v_voff0 = (uint32_t)(row0 * ROWB + (((lane % CPR) ^ G::swz_v(row0)) << 4));
    auto issue = [&](int j, auto stage_tag) {
        constexpr int S = decltype(stage_tag)::value;
        const uint32_t kb = (uint32_t)j * BK;
        const uint32_t bytes = j < nblk ? (uint32_t)(Tkv - (int)kb) * (uint32_t)ROWB : 0u;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)kb * D, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + (size_t)kb * D, bytes);
        uint8_t* st = &ring[S][0][0] + g0 * 1024;
        buffer_load_lds_b128_off<0>(rk, k_voff0, st);
        buffer_load_lds_b128_off<2048>(rk, k_voff0, st);
        buffer_load_lds_b128_off<0>(rv, v_voff0, st + TILEB);
        buffer_load_lds_b128_off<2048>(rv, v_voff0, st + TILEB);
    };

    // per-lane LDS read addresses in stage 0: K operand of step t (row ln,
    // chunk 2t + hf; kt adds 32 rows), V operand of d-tile dt (transposed read)
    const uint32_t ring_lds = lds_addr(&ring[0][0][0]);
    uint32_t k_ra[TQ], v_ra[DT];
#pragma unroll
    for (int t = 0; t < TQ; ++t) k_ra[t] = ring_lds + (uint32_t)(ln * ROWB + (((2 * t + hf) ^ G::swz_k(ln)) << 4));
    {
        const int lg = lane >> 4, jj = lane & 15;
        const int row = 4 * (lg >> 1) + (jj >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int col = 32 * dt + 16 * (lg & 1) + 4 * (jj & 3);
            v_ra[dt] = ring_lds + TILEB +
                       (uint32_t)(row * ROWB + ((((col >> 3) ^ G::swz_v(row)) << 4) | ((col & 4) << 1)));
        }
    }

    f32x16_t oacc[2][DT];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[u][dt][r] = 0.f;
    float m[2] = {kNegInf, kNegInf};
    float l[2] = {0.f, 0.f};

    // One 64-key stage as two 32-key halves kt, each QK -> softmax -> PV for
    // both sub-tiles (two live score tiles instead of four; the lazy
    // reference is checked per half, which any grouping of keys allows).
    // One 64-key stage: QK for both sub-tiles (each K operand read feeds two
    // MFMAs), the softmax of each, then PV (each V operand read feeds two).
    auto step = [&](uint32_t so, int kb, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        f32x16_t s[2][KT];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[u][kt][r] = 0.f;
        auto qk_tile = [&](auto kt_tag) {
            constexpr int kt = decltype(kt_tag)::value;
#pragma unroll
            for (int t = 0; t < TQ; ++t) {
                const bf16x8_t a = lds_load_b128<kt * 32 * ROWB>(k_ra[t] + so);
                s[0][kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0][t], s[0][kt], 0, 0, 0);
                s[1][kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[1][t], s[1][kt], 0, 0, 0);
            }
        };
        qk_tile(std::integral_constant<int, 0>{});
        qk_tile(std::integral_constant<int, 1>{});
        if constexpr (MASK) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (key >= Tkv) {
                        s[0][kt][r] = kNegInf;
                        s[1][kt][r] = kNegInf;
                    }
                }
        }
        uint32_t pw[2][8 * KT];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float rs = 0.f;
            auto exponentiate = [&](float mref) {
                rs = 0.f;
#pragma unroll
                for (int i = 0; i < 8 * KT; ++i) {
                    const int kt = i >> 3, r = 2 * (i & 7);
                    const float p0 = fast_exp2(__builtin_fmaf(s[u][kt][r], c, -mref));
                    const float p1 = fast_exp2(__builtin_fmaf(s[u][kt][r + 1], c, -mref));
                    pw[u][i] = pack_bf16x2(p0, p1);
                    rs = i == 0 ? p0 + p1 : rs + (p0 + p1);   // no add of the zero start value
                }
            };
            exponentiate(m[u]);
            if (__builtin_amdgcn_ballot_w64(!(rs <= kHalfSumLimit)) != 0) {
                // raise the reference to the true running max and rescale
                float mx = kNegInf;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[u][kt][r]);
                mx = half_swap_max(mx);
                const float m_new = fmaxf(m[u], mx * c);
                const float m_use = (m_new == kNegInf) ? 0.f : m_new;
                const float alpha = fast_exp2(m[u] - m_use);
                l[u] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[u][dt][r] *= alpha;
                m[u] = m_new;
                exponentiate(m_use);
            }
            l[u] += rs;
        }
        // O^T += V^T bf16(P)^T over four 16-key steps; each V operand serves both sub-tiles
        auto pv_step = [&](auto st_tag) {
            constexpr int st = decltype(st_tag)::value;
            constexpr int o = st * 16 * ROWB;
            const uint32_t va = v_ra[0] + so, vc = v_ra[1] + so;
            u32x4_t a0, a1;
            lds_read_tr16_x4<o, o + 8 * ROWB, o, o + 8 * ROWB>(va, va, vc, vc, a0, a1);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const u32x4_t pv = {pw[u][4 * st], pw[u][4 * st + 1], pw[u][4 * st + 2], pw[u][4 * st + 3]};
                const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
                oacc[u][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a0), pb,
                                                                     oacc[u][0], 0, 0, 0);
                oacc[u][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a1), pb,
                                                                     oacc[u][1], 0, 0, 0);
            }
        };
        pv_step(std::integral_constant<int, 0>{});
        pv_step(std::integral_constant<int, 1>{});
        pv_step(std::integral_constant<int, 2>{});
        pv_step(std::integral_constant<int, 3>{});
    };

    // block j in stage j % 3: wait for it, free stage (j - 1) % 3 with the
    // barrier, refill that stage with block j + 2
    auto issue_rt = [&](int j) {
        switch (j % 3) {
            case 0: issue(j, std::integral_constant<int, 0>{}); break;
            case 1: issue(j, std::integral_constant<int, 1>{}); break;
            default: issue(j, std::integral_constant<int, 2>{}); break;
        }
    };
    issue_rt(0);
    issue_rt(1);
    auto blk = [&](int j, auto mask_tag) {
        wait_vmcnt<4 * (NS - 2)>();           // this wave's part of block j has landed
        __syncthreads();                      // ... everyone's, and stage (j-1) % 3 is free
        issue_rt(j + NS - 1);
        step((uint32_t)(j % 3) * (2 * TILEB), j * BK, mask_tag);
    };
    int j = 0;
    for (; j < nfull; ++j) blk(j, std::false_type{});
    for (; j < nblk; ++j) blk(j, std::true_type{});
    wait_vmcnt<0>();    // no DMA may still be writing LDS when the workgroup retires

    // epilogue: divide once, write O (bf16) and LSE (fp32)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float lsum = half_swap_sum(l[u]);
        if (qrow[u] < Tq) {
            const float inv = 1.0f / lsum;
            uint16_t* orow = O + qbase + (size_t)qrow[u] * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x2_t w = {pack_bf16x2(oacc[u][dt][4 * g] * inv, oacc[u][dt][4 * g + 1] * inv),
                                       pack_bf16x2(oacc[u][dt][4 * g + 2] * inv, oacc[u][dt][4 * g + 3] * inv)};
                    *reinterpret_cast<u32x2_t*>(orow + 32 * dt + 8 * g + 4 * hf) = w;
                }
            if (LSE != nullptr && hf == 0)
                LSE[(size_t)bh * Tq + qrow[u]] = (m[u] + __builtin_log2f(lsum)) * 0.69314718055994530942f;
        }
    }
}

// Merge the chunk partials of each split tile: for row r with chunk results
// (O_c, lse2_c), M = max_c lse2_c, w_c = 2^(lse2_c - M),
// O = sum_c w_c O_c / sum_c w_c and LSE = (M + log2 sum_c w_c) ln 2 -- the
// rescaling merge of "IO-Aware Attention", section "Parallelism and the cost
// of the split", applied online over groups of CG chunks so that every load
// of a group is in flight at once.  blockIdx.x = tile (qt * BH + bh, the XCD
// of the tile's units), blockIdx.y = a slice of 256 / (D/4) rows; each thread
// owns 4 columns of one row.
constexpr int CG = 4;

template <int D, int BQ>
__global__ __launch_bounds__(256)
void prefill_combine_kernel(const float* __restrict__ part, uint16_t* __restrict__ O, float* __restrict__ LSE,
                            int Tq, int Tkv, int BH, int nqt, int chunk, int nch_max, int causal) {
    constexpr int TPR = D / 4;                // threads per row
    constexpr int RPW = 256 / TPR;            // rows per workgroup
    const int bh = blockIdx.x % BH;
    const int qt = blockIdx.x / BH;
    const int nch = tile_chunks(tile_blocks(qt, BQ, Geo<D>::BK, Tq, Tkv, causal != 0), chunk);
    if (nch <= 1) return;
    const int r = blockIdx.y * RPW + (int)threadIdx.x / TPR;
    const int col = 4 * ((int)threadIdx.x % TPR);
    const int qrow = qt * BQ + r;
    if (qrow >= Tq) return;
    const size_t rec0 = ((size_t)bh * nqt + qt) * nch_max;
    const float* plse = part + (size_t)BH * nqt * nch_max * BQ * D;
    float M = kNegInf, L = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < nch; k0 += CG) {
        float lk[CG];
        float4 x[CG];
#pragma unroll
        for (int i = 0; i < CG; ++i) {
            const int k = min(k0 + i, nch - 1);   // repeats of the last chunk get weight 0 below
            lk[i] = plse[(rec0 + k) * BQ + r];
            x[i] = *reinterpret_cast<const float4*>(part + ((rec0 + k) * BQ + r) * D + col);
        }
        float mg = M;
#pragma unroll
        for (int i = 0; i < CG; ++i)
            if (k0 + i < nch) mg = fmaxf(mg, lk[i]);
        const float alpha = fast_exp2(M - mg);   // M = -inf on the first group: alpha = 0
        L *= alpha;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] *= alpha;
#pragma unroll
        for (int i = 0; i < CG; ++i) {
            const float w = (k0 + i < nch) ? fast_exp2(lk[i] - mg) : 0.f;
            L += w;
            acc[0] = __builtin_fmaf(w, x[i].x, acc[0]);
            acc[1] = __builtin_fmaf(w, x[i].y, acc[1]);
            acc[2] = __builtin_fmaf(w, x[i].z, acc[2]);
            acc[3] = __builtin_fmaf(w, x[i].w, acc[3]);
        }
        M = mg;
    }
    const float inv = 1.0f / L;
    const u32x2_t w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    *reinterpret_cast<u32x2_t*>(O + ((size_t)bh * Tq + qrow) * D + col) = w;
    if (LSE != nullptr && col == 0)
        LSE[(size_t)bh * Tq + qrow] = (M + __builtin_log2f(L)) * 0.69314718055994530942f;
}

constexpr int kWaves = 4;
constexpr int kStages = 3;
constexpr int kBQ = kWaves * 32;
constexpr int kBQHalves = kWaves / 2 * 32;   // tile rows of the key-halves variant
constexpr int kStagesHalves = 2;             // its ring: K one block ahead of V, 32 KiB

// The key-halves variant (d = 64, unsplit) takes over when the 128-row tiles
// would leave the chip short of work: fewer than three resident tiles per
// compute unit.
bool use_key_halves(const PrefillArgs& a, int nch_max) {
    if (a.d != 64 || nch_max > 1) return false;
    const long long tiles = (long long)((a.Tq + kBQ - 1) / kBQ) * a.B * a.H;
    return tiles < 3LL * 256;
}

// The 256-row full-attention kernel (d = 64, unsplit, not key halves) where
// its 512 resident tiles need fewer rounds than the 128-row kernel's 768:
// there the 128-row grid ends in a partly filled round.
bool use_rows256(const PrefillArgs& a, int nch_max) {
    if (a.d != 64 || a.causal || nch_max > 1 || use_key_halves(a, nch_max)) return false;
    const long long bh = (long long)a.B * a.H;
    const long long rounds128 = ((a.Tq + kBQ - 1) / kBQ * bh + 3 * 256 - 1) / (3 * 256);
    const long long rounds256 = ((a.Tq + 255) / 256 * bh + 2 * 256 - 1) / (2 * 256);
    return rounds256 < rounds128;
}

hipError_t launch_rows256(const PrefillArgs& a, hipStream_t stream) {
    const int nqt = (a.Tq + 255) / 256;
    const long long grid = (long long)nqt * a.B * a.H;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(prefill_bf16_d64_r256_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.Tq, a.Tkv,
                       a.B * a.H, nqt, a.c);
    return hipGetLastError();
}

template <bool CAUSAL>
hipError_t launch_halves(const PrefillArgs& a, hipStream_t stream) {
    const int nqt = (a.Tq + kBQHalves - 1) / kBQHalves;
    const long long grid = (long long)nqt * a.B * a.H;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_bf16_kernel<64, kWaves, kStagesHalves, CAUSAL, 2>), dim3((unsigned)grid),
                       dim3(kWaves * 64), 0, stream, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                       static_cast<uint16_t*>(a.o), a.lse, static_cast<float*>(nullptr), a.Tq, a.Tkv, a.B * a.H,
                       nqt, 0, 1, a.c);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_one(const PrefillArgs& a, int chunk, int nch_max, hipStream_t stream) {
    const int nqt = (a.Tq + kBQ - 1) / kBQ;
    const long long tiles = (long long)nqt * a.B * a.H;
    const long long grid = tiles * nch_max;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, kWaves, kStages, CAUSAL>), dim3((unsigned)grid), dim3(kWaves * 64),
                       0, stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                       static_cast<float*>(a.workspace), a.Tq, a.Tkv, a.B * a.H, nqt, chunk, nch_max, a.c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nch_max <= 1) return e;
    constexpr int RPW = 256 / (D / 4);
    hipLaunchKernelGGL((prefill_combine_kernel<D, kBQ>), dim3((unsigned)tiles, kBQ / RPW), dim3(256), 0, stream,
                       static_cast<const float*>(a.workspace), static_cast<uint16_t*>(a.o), a.lse, a.Tq, a.Tkv,
                       a.B * a.H, nqt, chunk, nch_max, a.causal ? 1 : 0);
    return hipGetLastError();
}

int block_keys(int d) { return d == 128 ? Geo<128>::BK : Geo<64>::BK; }

thread_local char g_name[128];

}  // namespace

bool prefill_bf16_supports(int d) { return d == 64 || d == 128; }

bool prefill_bf16_fits(int Tkv, int d) {
    // buffer-load ranges are 32-bit byte counts per (batch, head)
    return (long long)Tkv * d * 2 < (1LL << 31);
}

PrefillSplit prefill_bf16_split_plan(int B, int H, int Tq, int Tkv, int d, bool causal, int kv_chunk) {
    PrefillSplit p{0, 1, 0};
    if (!prefill_bf16_supports(d)) return p;
    const int bk = block_keys(d);
    const int nqt = (Tq + kBQ - 1) / kBQ;
    int maxb = 0;
    long long total = 0;
    for (int qt = 0; qt < nqt; ++qt) {
        const int nb = tile_blocks(qt, kBQ, bk, Tq, Tkv, causal);
        maxb = nb > maxb ? nb : maxb;
        total += nb;
    }
    int chunk = 0;
    if (kv_chunk > 0) {
        chunk = (kv_chunk + bk - 1) / bk;
    } else {
        // automatic: split only when the query tiles alone leave the chip
        // short of work -- at d = 64, when even the 64-row key-halves tiles
        // number at most one per compute unit (above that the key-halves
        // kernel is faster than any split, measured on 1-16 heads of 1K-16K
        // keys); at d = 128, fewer than 3 resident 128-row tiles per compute
        // unit -- with units of an even share of all key blocks over 768
        // slots but never under 1024 keys: a unit pays a few microseconds of
        // start-up latency plus its partial's round trip, which shorter
        // units do not earn back.
        const long long slots = 3LL * 256;
        const long long tiles = (long long)nqt * B * H;
        const bool short_of_work = d == 64 ? (long long)((Tq + kBQHalves - 1) / kBQHalves) * B * H <= 256
                                           : tiles < slots;
        if (short_of_work) {
            const long long share = (total * B * H + slots - 1) / slots;
            const int min_blocks = 1024 / bk;
            chunk = (int)(share < min_blocks ? min_blocks : share);
        }
    }
    if (chunk <= 0 || chunk >= maxb) return p;
    p.chunk = chunk;
    p.nch_max = tile_chunks(maxb, chunk);
    p.workspace_bytes = (size_t)B * H * nqt * p.nch_max * kBQ * (d + 1) * sizeof(float);
    return p;
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, const PrefillSplit& sp, hipStream_t stream,
                               const char** name) {
    const int bk = block_keys(a.d);
    if (use_key_halves(a, sp.nch_max)) {
        snprintf(g_name, sizeof g_name, "prefill_bf16_d64<waves=4,bq=%d,bk=64,key_halves=2,stages=%d%s>", kBQHalves, kStagesHalves,
                 a.causal ? ",causal" : "");
        *name = g_name;
        return a.causal ? launch_halves<true>(a, stream) : launch_halves<false>(a, stream);
    }
    if (use_rows256(a, sp.nch_max)) {
        snprintf(g_name, sizeof g_name, "prefill_bf16_d64<waves=4,bq=256,bk=64,stages=3,rows_per_wave=64>");
        *name = g_name;
        return launch_rows256(a, stream);
    }
    if (sp.nch_max > 1)
        snprintf(g_name, sizeof g_name, "prefill_bf16_d%d<waves=4,bq=128,bk=%d,stages=3%s,kv_chunk=%d>+combine",
                 a.d, bk, a.causal ? ",causal" : "", sp.chunk * bk);
    else
        snprintf(g_name, sizeof g_name, "prefill_bf16_d%d<waves=4,bq=128,bk=%d,stages=3%s>", a.d, bk,
                 a.causal ? ",causal" : "");
    *name = g_name;
    const int chunk = sp.nch_max > 1 ? sp.chunk : 0;
    if (a.d == 128) {
        if (a.causal) return launch_one<128, true>(a, chunk, sp.nch_max, stream);
        return launch_one<128, false>(a, chunk, sp.nch_max, stream);
    }
    if (a.causal) return launch_one<64, true>(a, chunk, sp.nch_max, stream);
    return launch_one<64, false>(a, chunk, sp.nch_max, stream);
}

}  // namespace attn
