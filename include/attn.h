/*
 * Exact IO-aware attention forward for AMD MI355X (gfx950) -- C ABI.
 *
 * Every entry point computes, for each (batch b, head h),
 *
 *     S = scale * Q K^T          (T_q x T_kv; never written to memory)
 *     S[i, j] = -inf  where causal and j > i + (T_kv - T_q)
 *     O = softmax_rows(S) V,     LSE_i = ln sum_j exp(S[i, j])
 *
 * i.e. the definition of "FlashAttention IO-aware tiling lab" (S = QK^T /
 * sqrt(d), P = softmax(S), O = PV) and of "Attention and Its Computational
 * Cost", section "What is being computed", evaluated block by block with the
 * running-max / running-sum recurrence of "IO-Aware Attention: Tiling the
 * Score Matrix Without Materializing It", section "Softmax over blocks,
 * exactly".  The causal rule is aligned to the bottom-right corner, so for
 * self-attention (T_q == T_kv) row i sees keys 0..i, and a single new query
 * sees every cached key.  LSE is the natural-log normaliser of each row in
 * units of the scaled score, kept for a backward pass ("IO-Aware Attention",
 * section "What has to stay in fast memory").
 *
 * Layout: Q and O are [B, H, T_q, d], K and V are [B, H, T_kv, d] (H_kv key/value
 * heads for attn_decode_gqa), all contiguous row-major with d innermost; LSE is
 * [B, H, T_q] fp32.  bf16 data
 * is passed as 16-bit words (the upper half of the IEEE fp32 bit pattern).
 *
 * Ownership: every pointer is caller-owned device memory.  The library never
 * allocates, frees or retains a pointer past the call.  Inputs must not alias
 * outputs or the workspace.
 *
 * Execution: calls are asynchronous on `stream` (NULL = the null stream) and
 * return once the kernels are enqueued; results are valid after the stream is
 * synchronised.  There is no internal synchronisation, no host<->device
 * copy and no memset, so a call can be captured into a HIP graph (stream
 * capture) and replayed; the kernels are deterministic, so a replay gives the
 * same bits as a direct call.
 *
 * Errors: arguments are validated before any HIP call; a failing call
 * enqueues nothing and returns one of the negative codes below, with a
 * thread-local description in attn_status_string().  No call aborts.
 */
#ifndef IO_AWARE_EXACT_ATTN_H
#define IO_AWARE_EXACT_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ATTN_OK = 0,
    ATTN_EINVAL = -1,       /* null pointer, size < 1, scale not finite or <= 0, causal with T_q > T_kv,
                               pointer not 16-byte aligned, num_splits < 0, aliasing output, sizes overflow */
    ATTN_EUNSUPPORTED = -2, /* head width d not built for this path, or one head's K/V (or Q) past
                               2^31 bytes, the reach of a 32-bit buffer range */
    ATTN_EHIP = -3,         /* the HIP runtime reported an error while enqueueing */
    ATTN_EWORKSPACE = -4    /* workspace missing or smaller than the call's *_workspace_bytes() */
};

/*
 * attn_fwd -- bf16 attention forward (prefill, or decode when T_q == 1).
 *
 *   q, k, v  device pointers to bf16 Q [B,H,Tq,d], K and V [B,H,Tkv,d]
 *   o        device pointer to bf16 O [B,H,Tq,d] (written)
 *   lse      device pointer to fp32 LSE [B,H,Tq] (written), or NULL to skip it
 *   causal   0 or 1 (bottom-right aligned mask; needs Tq <= Tkv)
 *   scale    multiplier of q.k, finite and > 0 (the pages use 1/sqrt(d))
 *
 * Products use bf16 MFMA with fp32 accumulation; the softmax statistics and
 * the output accumulator are fp32 ("IO-Aware Attention", section "Where the
 * approach stops helping": 32-bit accumulation and rescaling); P is rounded to
 * bf16 (nearest even) before the PV product and O is rounded once at the end.
 * Those two roundings, each at most 2^-8 relative, bound every element:
 * |O - O_exact| <= 2^-8 (|O_exact| + A) plus fp32 rounding, where A is the
 * attention output with |V| as values (so at most 2^-7 max|V| for a row).
 * Supported: d in {64, 128} (64- and 32-key blocks), Tkv*d*2 < 2^31 bytes per
 * head; for T_q == 1 the decode kernel runs unsplit (no workspace).  T_q and
 * T_kv need not be multiples of any tile.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Tq, int Tkv, int d, int causal, float scale, hipStream_t stream);

/*
 * attn_fwd_split_workspace_bytes -- bytes of workspace attn_fwd_split needs for
 * this shape and kv_chunk; 0 when that call would not split (then it needs no
 * workspace) or when the arguments are invalid.  The workspace holds, per
 * chunk of a split tile, the partial output and partial normaliser that
 * "IO-Aware Attention", section "Parallelism and the cost of the split", has
 * each key partition produce before the merge.  Caller-owned device memory.
 */
size_t attn_fwd_split_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int causal, int kv_chunk);

/*
 * attn_fwd_split -- attn_fwd with the key axis of long query tiles split
 * across workgroups ("IO-Aware Attention", section "Parallelism and the cost
 * of the split": when the query blocks alone do not fill the device, key
 * partitions each produce a partial output and normaliser, merged with the
 * same rescaling).  The result equals attn_fwd's up to fp32 rounding order.
 *
 *   kv_chunk   keys per work unit, rounded up to a multiple of 64; a query tile
 *              (128 rows) whose key range is longer is split into
 *              ceil(range / kv_chunk) near-equal chunks.  0 = the library
 *              picks: it splits only when the chip is short of work -- at
 *              d = 64 when there are at most 256 query tiles of 64 rows (one
 *              per compute unit), at d = 128 when there are fewer than 768
 *              tiles of 128 rows (3 per compute unit) -- into chunks of an
 *              even share of all key blocks over 768 units but at least 1024
 *              keys, and only tiles longer than that.  A call that does not
 *              split runs exactly as attn_fwd.
 *   workspace  device memory of at least attn_fwd_split_workspace_bytes(...)
 *              bytes (may be NULL when that is 0); contents on entry are
 *              ignored.  Partials of split tiles: per (batch, head, tile,
 *              chunk) 128 x d fp32 values and 128 fp32 log-sum-exps.
 *   other arguments as attn_fwd.
 *
 * When split, a second kernel (the merge) follows on the same stream.
 * Errors: as attn_fwd; ATTN_EINVAL for kv_chunk < 0; ATTN_EWORKSPACE when a
 * split is planned and the workspace is NULL or too small.
 */
int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Tq, int Tkv, int d, int causal, float scale, int kv_chunk,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_fwd_f32 -- the exact path: fp32 inputs, fp32 products, fp32 output.
 * Same arguments and semantics as attn_fwd with every tensor fp32: the same
 * definition ("FlashAttention IO-aware tiling lab"; "Attention and Its
 * Computational Cost", section "What is being computed") with the same
 * blockwise recurrence, and no reduced-precision step anywhere, the 32-bit
 * arithmetic "IO-Aware Attention", section "Where the approach stops
 * helping", asks of the accumulation and rescaling.  Errors as attn_fwd.
 * Supported: d in {16, 32, 64, 128}, any T_q >= 1, T_kv >= 1.
 */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int H, int Tq, int Tkv, int d, int causal, float scale, hipStream_t stream);

/*
 * attn_decode_workspace_bytes -- bytes of workspace attn_decode needs:
 * B*H*num_splits*(d+2)*4 (one fp32 partial output of d values plus its
 * running max and running sum per partition, the per-partition state of
 * "IO-Aware Attention", section "Parallelism and the cost of the split"),
 * 0 when num_splits <= 1 or any size is < 1.  Caller-owned device memory.
 */
size_t attn_decode_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * attn_decode_splits -- the number of key partitions the library picks for a
 * decode step (num_splits = 0): enough for about 512 workgroups (at most 16
 * partitions; 64 for groups of 4 or more query heads, whose kernel runs one
 * wave per workgroup; grids of fewer than 16 head tiles take one workgroup
 * per compute unit, 256 / tiles partitions, at most 64), and none holding
 * less than 64 KiB of K and V (16384/d keys).  A single sequence offers only H
 * independent heads, too few to occupy the chip; splitting the key axis is
 * the remedy "Attention and Its Computational Cost" proposes for its batch-1
 * decode measurement ("The other shape: one query, many keys").  Returns 0
 * for invalid or unsupported arguments (d not in {64, 128}, Hq % Hkv != 0).
 */
int attn_decode_splits(int B, int Hq, int Hkv, int Tkv, int d);

/*
 * attn_decode -- one query per (batch, head) against T_kv cached keys, with
 * the key axis split into num_splits partitions ("IO-Aware Attention",
 * section "Parallelism and the cost of the split": each partition produces a
 * partial output and normaliser, merged with the same rescaling in a second
 * kernel on the same stream).
 *
 *   q, o       bf16 [B,H,1,d];  k, v bf16 [B,H,Tkv,d];  lse fp32 [B,H] or NULL
 *   scale      finite and > 0
 *   num_splits >= 1, or 0 for attn_decode_splits(B,H,H,Tkv,d); values above
 *              Tkv are clamped to Tkv.  Partition p covers keys
 *              [floor(p*Tkv/P), floor((p+1)*Tkv/P)).
 *   workspace  device memory of at least attn_decode_workspace_bytes(B,H,d,num_splits)
 *              bytes (may be NULL when num_splits == 1); contents on entry are ignored.
 *
 * Supported: d in {64, 128}.
 */
int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int Tkv, int d, float scale, int num_splits,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_gqa -- attn_decode with grouped-query attention: Hq query heads
 * share Hkv key/value heads, query head h reading key/value head
 * h / (Hq / Hkv) ("Attention and Its Computational Cost", section "The other
 * shape: one query, many keys": keeping fewer key and value heads than query
 * heads shrinks the cache that every decode step streams).  Each K/V byte is
 * read from memory once for all the query heads of its group.
 *
 *   q, o       bf16 [B,Hq,1,d];  k, v bf16 [B,Hkv,Tkv,d];  lse fp32 [B,Hq] or NULL
 *   Hkv        >= 1 and dividing Hq (Hkv == Hq is attn_decode; Hkv == 1 is
 *              multi-query attention)
 *   workspace  at least attn_decode_workspace_bytes(B,Hq,d,num_splits) bytes
 *   other arguments as attn_decode.
 *
 * Groups of 4 or more query heads run on the matrix cores (the heads of a
 * group are the columns of an MFMA tile); smaller groups on the vector ALUs.
 * Errors: ATTN_EINVAL also when Hkv < 1 or Hq % Hkv != 0.  Supported: d in
 * {64, 128}, Tkv*d*2 < 2^31 bytes per head (also for attn_decode).
 */
int attn_decode_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int Tkv, int d, float scale, int num_splits,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_noalloc -- attn_decode_gqa for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the partition partials go to a scratch array the
 * library holds on each device (one per device, kept until the process ends)
 * instead of a caller workspace.  The call allocates and frees nothing.
 *
 *   arguments  as attn_decode_gqa, without the workspace
 *
 * Limit: the partials, attn_decode_workspace_bytes(B,Hq,d,P) for the
 * partition count P actually used (after num_splits == 0 is resolved and
 * clamped to Tkv), must fit in attn_decode_noalloc_max_bytes() (32 MiB);
 * a larger call returns ATTN_EWORKSPACE before any launch.  P == 1 uses no
 * scratch.  The scratch's address on a device is looked up on the first
 * call made with that device current.
 * Every call on one device shares its scratch: two calls that may run at
 * the same time on one device (different streams, or host threads without an
 * order between them) race on it and give wrong results; order them on one
 * stream.  Each call overwrites every record it later reads, so nothing needs
 * clearing between calls.  Errors: as attn_decode_gqa, plus ATTN_EHIP when the
 * scratch address cannot be obtained.
 */
int attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Tkv, int d, float scale, int num_splits,
                        hipStream_t stream);

/* attn_decode_noalloc_max_bytes -- size of that per-device scratch (32 MiB). */
size_t attn_decode_noalloc_max_bytes(void);

/*
 * attn_bwd_workspace_bytes -- bytes of workspace attn_bwd needs: B*H*Tq*8
 * (per query row its log-sum-exp in base 2 and D = sum_d dO*O, fp32: the O(n)
 * row constants "IO-Aware Attention", section "What has to stay in fast
 * memory", keeps beside the inputs).  0 when any size is < 1.  Caller-owned
 * device memory.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int Tq);

/*
 * attn_bwd -- backward pass of attn_fwd: gradients of sum(O * dO) with
 * respect to Q, K and V, recomputing the softmax from Q, K, V and the saved
 * per-row log-sum-exp instead of storing it ("IO-Aware Attention", section
 * "What has to stay in fast memory": the saved state is O(n d) plus O(n) row
 * constants).  With P = exp(scale*Q K^T - lse) (masked entries 0) and
 * D_i = sum_d dO_id O_id:
 *
 *     dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q
 *
 *   q, k, v    the forward's bf16 inputs [B,H,Tq,d], [B,H,Tkv,d] (x2)
 *   o, lse     the forward's bf16 output [B,H,Tq,d] and fp32 LSE [B,H,Tq]
 *              (natural log, as attn_fwd writes it; required)
 *   dout       bf16 upstream gradient dO [B,H,Tq,d]
 *   dq, dk, dv fp32 outputs [B,H,Tq,d], [B,H,Tkv,d] (x2), fully written
 *   causal, scale   as in the forward call
 *   workspace  at least attn_bwd_workspace_bytes(B,H,Tq) bytes; contents on
 *              entry are ignored
 *
 * Two kernels on `stream`: dQ per query tile, which also writes each row's
 * statistics (lse * log2 e and D = sum dO * O) to the workspace, then dK/dV per
 * key tile, which reads them; no atomics, so results are deterministic.  Products are bf16 MFMA with
 * fp32 accumulation; P and dS are rounded to bf16 as MFMA operands.
 * Errors: as attn_fwd, plus ATTN_EINVAL for NULL dout/lse/dq/dk/dv or
 * overlapping buffers, ATTN_EWORKSPACE for a missing or small workspace.
 * Supported: d in {64, 128}, Tq*d*2 and Tkv*d*2 < 2^31 bytes per head.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             float* dq, float* dk, float* dv, int B, int H, int Tq, int Tkv, int d, int causal, float scale,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_last_kernel -- name and tile configuration of the kernel(s) enqueued by
 * this thread's last successful call, e.g.
 * "prefill_bf16_d64<waves=4,bq=128,bk=64,stages=3,causal>" ("Attention and Its
 * Computational Cost", section "Which kernel ran": a measurement of attention
 * names the kernel that ran).  Empty before the first call.  The string is
 * thread-local and valid until this thread's next call.
 */
const char* attn_last_kernel(void);

/*
 * attn_status_string -- description of `status`; for the calling thread's most
 * recent failure with that code it carries the detail (which argument, or the
 * HIP error text).  Thread-local storage, valid until the next call.  This is
 * the C form of the argument errors of "E8.1 IO-aware attention", "Do it in
 * code" (a block size below 1 is refused with an error that says why): every
 * entry point checks its arguments before touching the device and reports a
 * refusal as a status code whose text names the argument.
 */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_EXACT_ATTN_H */
