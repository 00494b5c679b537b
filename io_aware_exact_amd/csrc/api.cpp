// C ABI of the attention library: argument validation, shape-based kernel
// choice and error reporting.  Validation happens before any HIP call, so a
// rejected call touches neither the device nor the runtime.
#include "attn.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "launch.hpp"

namespace {

thread_local std::string g_detail;
thread_local int g_detail_code = 0;
thread_local std::string g_last_kernel;

constexpr double kLog2e = 1.4426950408889634074;

int fail(int code, const std::string& what) {
    g_detail_code = code;
    g_detail = what;
    return code;
}

const char* generic(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_EINVAL: return "invalid argument";
        case ATTN_EUNSUPPORTED: return "unsupported configuration";
        case ATTN_EHIP: return "HIP runtime error";
        case ATTN_EWORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;
    const char* name;
};

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// Checks shared by every entry point.  `es` is the element size of q/k/v/o.
// Q/O have H query heads, K/V have Hkv key/value heads.
int check_common(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
                 int Hkv, int Tq, int Tkv, int d, int causal, float scale, size_t es) {
    if (!q) return fail(ATTN_EINVAL, "q is NULL");
    if (!k) return fail(ATTN_EINVAL, "k is NULL");
    if (!v) return fail(ATTN_EINVAL, "v is NULL");
    if (!o) return fail(ATTN_EINVAL, "o is NULL");
    if (B < 1) return fail(ATTN_EINVAL, "B must be >= 1");
    if (H < 1) return fail(ATTN_EINVAL, "H must be >= 1");
    if (Hkv < 1) return fail(ATTN_EINVAL, "Hkv must be >= 1");
    if (H % Hkv != 0) return fail(ATTN_EINVAL, "the number of query heads must be a multiple of Hkv");
    if (Tq < 1) return fail(ATTN_EINVAL, "Tq must be >= 1");
    if (Tkv < 1) return fail(ATTN_EINVAL, "Tkv must be >= 1");
    if (d < 1) return fail(ATTN_EINVAL, "d must be >= 1");
    if (causal != 0 && causal != 1) return fail(ATTN_EINVAL, "causal must be 0 or 1");
    if (!std::isfinite(scale) || !(scale > 0.f)) return fail(ATTN_EINVAL, "scale must be finite and > 0");
    if (causal && Tq > Tkv) return fail(ATTN_EINVAL, "causal attention needs Tq <= Tkv");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return fail(ATTN_EINVAL, "q, k, v and o must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(ATTN_EINVAL, "lse must be 4-byte aligned");
    // sizes: B*H*T*d*es must fit comfortably in 63 bits
    const double qbytes = double(B) * H * Tq * d * es;
    const double kbytes = double(B) * Hkv * Tkv * d * es;
    if (qbytes > 4.0e18 || kbytes > 4.0e18) return fail(ATTN_EINVAL, "tensor sizes overflow");
    const uint64_t BH = uint64_t(B) * uint64_t(H);
    if (BH > 0x7fffffffull) return fail(ATTN_EINVAL, "B*H must fit in 31 bits");
    const Range rq{reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(q) + uint64_t(qbytes), "q"};
    const Range rk{reinterpret_cast<uintptr_t>(k), reinterpret_cast<uintptr_t>(k) + uint64_t(kbytes), "k"};
    const Range rv{reinterpret_cast<uintptr_t>(v), reinterpret_cast<uintptr_t>(v) + uint64_t(kbytes), "v"};
    const Range ro{reinterpret_cast<uintptr_t>(o), reinterpret_cast<uintptr_t>(o) + uint64_t(qbytes), "o"};
    for (const Range* in : {&rq, &rk, &rv})
        if (overlap(ro, *in)) return fail(ATTN_EINVAL, std::string("o overlaps ") + in->name);
    if (lse) {
        const Range rl{reinterpret_cast<uintptr_t>(lse), reinterpret_cast<uintptr_t>(lse) + BH * uint64_t(Tq) * 4,
                       "lse"};
        for (const Range* other : {&rq, &rk, &rv, &ro})
            if (overlap(rl, *other)) return fail(ATTN_EINVAL, std::string("lse overlaps ") + other->name);
    }
    return ATTN_OK;
}

int finish(hipError_t e, const char* name) {
    if (e != hipSuccess) return fail(ATTN_EHIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    g_last_kernel = name ? name : "";
    return ATTN_OK;
}

int run_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int Tkv,
               int d, float scale, int splits, void* ws, hipStream_t stream) {
    attn::DecodeArgs a{q, k, v, o, lse, B, H, Hkv, Tkv, d, splits, float(double(scale) * kLog2e), ws};
    const char* name = nullptr;
    (void)hipGetLastError();   // clear any stale error so the launch status is ours
    return finish(attn::launch_decode_bf16(a, stream, &name), name);
}

// Checks of a decode call (one query per (batch, query head)) and the
// partition count it will use: num_splits, or the automatic count for 0,
// clamped to Tkv.
int check_decode(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int Hq,
                 int Hkv, int Tkv, int d, float scale, int num_splits, int* splits) {
    int st = check_common(q, k, v, o, lse, B, Hq, Hkv, 1, Tkv, d, 0, scale, 2);
    if (st != ATTN_OK) return st;
    if (num_splits < 0) return fail(ATTN_EINVAL, "num_splits must be >= 0");
    if (d != 64 && d != 128) return fail(ATTN_EUNSUPPORTED, "decode supports d in {64, 128}");
    // buffer-load ranges are 32-bit byte counts per (batch, kv head)
    if (double(Tkv) * d * 2 >= 2147483648.0)
        return fail(ATTN_EUNSUPPORTED, "decode supports Tkv*d*2 < 2^31 bytes per head");
    if (num_splits == 0) num_splits = attn::decode_auto_splits(B, Hq, Hkv, Tkv, d);
    *splits = num_splits > Tkv ? Tkv : num_splits;
    if (*splits > 65535) return fail(ATTN_EUNSUPPORTED, "decode supports at most 65535 partitions");
    return ATTN_OK;
}

// The workspace must be 16-byte aligned and overlap none of the tensors.
int check_workspace(const void* ws, size_t need, const void* q, const void* k, const void* v, const void* o,
                    const float* lse, uint64_t qbytes, uint64_t kvbytes, uint64_t lsebytes) {
    if (!aligned(ws, 16)) return fail(ATTN_EINVAL, "workspace must be 16-byte aligned");
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(ws), w1 = w0 + need;
    const uintptr_t ptrs[4] = {reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(k),
                               reinterpret_cast<uintptr_t>(v), reinterpret_cast<uintptr_t>(o)};
    const uint64_t lens[4] = {qbytes, kvbytes, kvbytes, qbytes};
    for (int i = 0; i < 4; ++i)
        if (w0 < ptrs[i] + lens[i] && ptrs[i] < w1) return fail(ATTN_EINVAL, "workspace overlaps a tensor");
    if (lse) {
        const uintptr_t l0 = reinterpret_cast<uintptr_t>(lse), l1 = l0 + lsebytes;
        if (w0 < l1 && l0 < w1) return fail(ATTN_EINVAL, "workspace overlaps lse");
    }
    return ATTN_OK;
}

// bf16 forward; `split` selects the work-unit plan (no split for attn_fwd).
int run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Tq, int Tkv,
            int d, int causal, float scale, const attn::PrefillSplit& split, void* ws, hipStream_t stream) {
    if (Tq == 1) {
        // a single query row: the decode kernel, unsplit (bottom-right causal
        // alignment lets the one row see every key, so causal changes nothing)
        return run_decode(q, k, v, o, lse, B, H, H, Tkv, d, scale, 1, nullptr, stream);
    }
    attn::PrefillArgs a{q, k, v, o, lse, B, H, Tq, Tkv, d, causal != 0, float(double(scale) * kLog2e), ws};
    const char* name = nullptr;
    (void)hipGetLastError();
    return finish(attn::launch_prefill_bf16(a, split, stream, &name), name);
}

// Shape checks of the bf16 forward beyond check_common.
int check_fwd_shape(int B, int H, int Tq, int Tkv, int d) {
    if (Tq == 1) {
        if (d != 64 && d != 128) return fail(ATTN_EUNSUPPORTED, "bf16 single-query path supports d in {64, 128}");
        // the decode kernel it runs on has the same 32-bit buffer ranges per head
        if (double(Tkv) * d * 2 >= 2147483648.0)
            return fail(ATTN_EUNSUPPORTED, "bf16 single-query path supports Tkv*d*2 < 2^31 bytes per head");
        return ATTN_OK;
    }
    if (!attn::prefill_bf16_supports(d)) return fail(ATTN_EUNSUPPORTED, "bf16 prefill supports d in {64, 128}");
    if (!attn::prefill_bf16_fits(Tkv, d))
        return fail(ATTN_EUNSUPPORTED, "bf16 prefill supports Tkv*d*2 < 2^31 bytes per head");
    if (double(B) * H * ((Tq + 127) / 128) > 2147483647.0) return fail(ATTN_EINVAL, "grid too large");
    return ATTN_OK;
}

// The split plan of attn_fwd_split, or no split when the shape has none.
attn::PrefillSplit fwd_split_plan(int B, int H, int Tq, int Tkv, int d, int causal, int kv_chunk) {
    if (Tq == 1 || !attn::prefill_bf16_supports(d)) return attn::PrefillSplit{0, 1, 0};
    attn::PrefillSplit p = attn::prefill_bf16_split_plan(B, H, Tq, Tkv, d, causal != 0, kv_chunk);
    if (double(B) * H * ((Tq + 127) / 128) * p.nch_max > 2147483647.0) return attn::PrefillSplit{0, 1, 0};
    return p;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Tq, int Tkv,
             int d, int causal, float scale, hipStream_t stream) {
    int st = check_common(q, k, v, o, lse, B, H, H, Tq, Tkv, d, causal, scale, 2);
    if (st != ATTN_OK) return st;
    if ((st = check_fwd_shape(B, H, Tq, Tkv, d)) != ATTN_OK) return st;
    return run_fwd(q, k, v, o, lse, B, H, Tq, Tkv, d, causal, scale, attn::PrefillSplit{0, 1, 0}, nullptr, stream);
}

size_t attn_fwd_split_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int causal, int kv_chunk) {
    if (B < 1 || H < 1 || Tq < 1 || Tkv < 1 || d < 1 || (causal != 0 && causal != 1) || kv_chunk < 0) return 0;
    if (causal && Tq > Tkv) return 0;
    return fwd_split_plan(B, H, Tq, Tkv, d, causal, kv_chunk).workspace_bytes;
}

int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Tq, int Tkv,
                   int d, int causal, float scale, int kv_chunk, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    int st = check_common(q, k, v, o, lse, B, H, H, Tq, Tkv, d, causal, scale, 2);
    if (st != ATTN_OK) return st;
    if (kv_chunk < 0) return fail(ATTN_EINVAL, "kv_chunk must be >= 0");
    if ((st = check_fwd_shape(B, H, Tq, Tkv, d)) != ATTN_OK) return st;
    const attn::PrefillSplit plan = fwd_split_plan(B, H, Tq, Tkv, d, causal, kv_chunk);
    if (plan.nch_max > 1) {
        if (!workspace) return fail(ATTN_EWORKSPACE, "workspace is NULL");
        if (workspace_bytes < plan.workspace_bytes)
            return fail(ATTN_EWORKSPACE, "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                                             std::to_string(plan.workspace_bytes));
        const uint64_t qb = uint64_t(B) * H * Tq * d * 2, kvb = uint64_t(B) * H * Tkv * d * 2;
        if ((st = check_workspace(workspace, plan.workspace_bytes, q, k, v, o, lse, qb, kvb,
                                  uint64_t(B) * H * Tq * 4)) != ATTN_OK)
            return st;
    }
    return run_fwd(q, k, v, o, lse, B, H, Tq, Tkv, d, causal, scale, plan, workspace, stream);
}


int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int Tq,
                 int Tkv, int d, int causal, float scale, hipStream_t stream) {
    int st = check_common(q, k, v, o, lse, B, H, H, Tq, Tkv, d, causal, scale, 4);
    if (st != ATTN_OK) return st;
    if (!attn::prefill_f32_supports(d)) return fail(ATTN_EUNSUPPORTED, "fp32 path supports d in {16, 32, 64, 128}");
    if (double(B) * H * Tq > 2147483647.0) return fail(ATTN_EINVAL, "grid too large");
    attn::PrefillArgs a{q, k, v, o, lse, B, H, Tq, Tkv, d, causal != 0, float(double(scale) * kLog2e), nullptr};
    const char* name = nullptr;
    (void)hipGetLastError();
    return finish(attn::launch_prefill_f32(a, stream, &name), name);
}

size_t attn_decode_workspace_bytes(int B, int H, int d, int num_splits) {
    if (B < 1 || H < 1 || d < 1 || num_splits <= 1) return 0;
    return size_t(B) * size_t(H) * size_t(num_splits) * size_t(d + 2) * sizeof(float);
}

int attn_decode_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                    int Tkv, int d, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
    int splits = 0;
    int st = check_decode(q, k, v, o, lse, B, Hq, Hkv, Tkv, d, scale, num_splits, &splits);
    if (st != ATTN_OK) return st;
    if (splits > 1) {
        const size_t need = attn_decode_workspace_bytes(B, Hq, d, splits);
        if (!workspace) return fail(ATTN_EWORKSPACE, "workspace is NULL");
        if (workspace_bytes < need)
            return fail(ATTN_EWORKSPACE, "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                                             std::to_string(need));
        const uint64_t kvb = uint64_t(B) * Hkv * Tkv * d * 2, qb = uint64_t(B) * Hq * d * 2;
        if ((st = check_workspace(workspace, need, q, k, v, o, lse, qb, kvb, uint64_t(B) * Hq * 4)) != ATTN_OK)
            return st;
    }
    return run_decode(q, k, v, o, lse, B, Hq, Hkv, Tkv, d, scale, splits, workspace, stream);
}

int attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                        int Tkv, int d, float scale, int num_splits, hipStream_t stream) {
    int splits = 0;
    int st = check_decode(q, k, v, o, lse, B, Hq, Hkv, Tkv, d, scale, num_splits, &splits);
    if (st != ATTN_OK) return st;
    void* scratch = nullptr;
    if (splits > 1) {
        const size_t need = attn_decode_workspace_bytes(B, Hq, d, splits);
        if (need > attn::kDecodeScratchBytes)
            return fail(ATTN_EWORKSPACE, "the partials need " + std::to_string(need) +
                                             " bytes; the library's scratch holds " +
                                             std::to_string(attn::kDecodeScratchBytes) +
                                             " (use fewer splits, or attn_decode_gqa with a workspace)");
        const hipError_t e = attn::decode_scratch(&scratch);
        if (e != hipSuccess)
            return fail(ATTN_EHIP, std::string("scratch lookup failed: ") + hipGetErrorString(e));
    }
    return run_decode(q, k, v, o, lse, B, Hq, Hkv, Tkv, d, scale, splits, scratch, stream);
}

size_t attn_decode_noalloc_max_bytes(void) { return attn::kDecodeScratchBytes; }

int attn_decode_splits(int B, int Hq, int Hkv, int Tkv, int d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Tkv < 1 || (d != 64 && d != 128)) return 0;
    return attn::decode_auto_splits(B, Hq, Hkv, Tkv, d);
}

int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Tkv, int d,
                float scale, int num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return attn_decode_gqa(q, k, v, o, lse, B, H, H, Tkv, d, scale, num_splits, workspace, workspace_bytes, stream);
}

size_t attn_bwd_workspace_bytes(int B, int H, int Tq) {
    if (B < 1 || H < 1 || Tq < 1) return 0;
    return attn::backward_workspace_bytes(B, H, Tq);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             float* dq, float* dk, float* dv, int B, int H, int Tq, int Tkv, int d, int causal, float scale,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int st = check_common(q, k, v, o, nullptr, B, H, H, Tq, Tkv, d, causal, scale, 2);
    if (st != ATTN_OK) return st;
    if (!dout) return fail(ATTN_EINVAL, "dout is NULL");
    if (!lse) return fail(ATTN_EINVAL, "lse is NULL (the backward pass recomputes P from it)");
    if (!dq || !dk || !dv) return fail(ATTN_EINVAL, "dq, dk and dv must not be NULL");
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return fail(ATTN_EINVAL, "dout, dq, dk and dv must be 16-byte aligned");
    if (!aligned(lse, 4)) return fail(ATTN_EINVAL, "lse must be 4-byte aligned");
    if (!attn::backward_supports(d)) return fail(ATTN_EUNSUPPORTED, "backward supports d in {64, 128}");
    if (double(Tkv) * d * 2 >= 2147483648.0 || double(Tq) * d * 2 >= 2147483648.0)
        return fail(ATTN_EUNSUPPORTED, "backward supports T*d*2 < 2^31 bytes per head");
    if (double(B) * H * ((std::max(Tq, Tkv) + 127) / 128) > 2147483647.0) return fail(ATTN_EINVAL, "grid too large");
    const size_t need = attn::backward_workspace_bytes(B, H, Tq);
    if (!workspace) return fail(ATTN_EWORKSPACE, "workspace is NULL");
    if (workspace_bytes < need)
        return fail(ATTN_EWORKSPACE, "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                                         std::to_string(need));
    // every input, output and the workspace must be disjoint
    const uint64_t qb = uint64_t(B) * H * Tq * d * 2, kvb = uint64_t(B) * H * Tkv * d * 2;
    const Range ins[6] = {{reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(q) + qb, "q"},
                          {reinterpret_cast<uintptr_t>(k), reinterpret_cast<uintptr_t>(k) + kvb, "k"},
                          {reinterpret_cast<uintptr_t>(v), reinterpret_cast<uintptr_t>(v) + kvb, "v"},
                          {reinterpret_cast<uintptr_t>(o), reinterpret_cast<uintptr_t>(o) + qb, "o"},
                          {reinterpret_cast<uintptr_t>(dout), reinterpret_cast<uintptr_t>(dout) + qb, "dout"},
                          {reinterpret_cast<uintptr_t>(lse), reinterpret_cast<uintptr_t>(lse) + uint64_t(B) * H * Tq * 4,
                           "lse"}};
    const Range outs[4] = {{reinterpret_cast<uintptr_t>(dq), reinterpret_cast<uintptr_t>(dq) + 2 * qb, "dq"},
                           {reinterpret_cast<uintptr_t>(dk), reinterpret_cast<uintptr_t>(dk) + 2 * kvb, "dk"},
                           {reinterpret_cast<uintptr_t>(dv), reinterpret_cast<uintptr_t>(dv) + 2 * kvb, "dv"},
                           {reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need,
                            "workspace"}};
    for (int i = 0; i < 4; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return fail(ATTN_EINVAL, std::string(outs[i].name) + " overlaps " + r.name);
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j]))
                return fail(ATTN_EINVAL, std::string(outs[i].name) + " overlaps " + outs[j].name);
    }
    if (!aligned(workspace, 16)) return fail(ATTN_EINVAL, "workspace must be 16-byte aligned");
    attn::BackwardArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, H, Tq, Tkv, d, causal != 0,
                         float(double(scale) * kLog2e), scale, workspace};
    const char* name = nullptr;
    (void)hipGetLastError();
    return finish(attn::launch_backward_bf16(a, stream, &name), name);
}

const char* attn_last_kernel(void) { return g_last_kernel.c_str(); }

const char* attn_status_string(int status) {
    if (status != ATTN_OK && status == g_detail_code && !g_detail.empty()) return g_detail.c_str();
    return generic(status);
}

}  // extern "C"
