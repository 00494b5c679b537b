// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace attn {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, Tq, Tkv, d;
    bool causal;
    float c;          // scale * log2(e)
    void* workspace;  // split partials (prefill_bf16 with a split plan), else unused
};

// How a bf16 prefill is divided into work units: tiles whose key range is
// longer than `chunk` key blocks are split into near-equal chunks.
struct PrefillSplit {
    int chunk;               // blocks per unit (0 = no split)
    int nch_max;             // chunks of the longest tile (1 = no split)
    size_t workspace_bytes;  // partials: B*H*tiles*nch_max*128*(d+1) floats
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, Hkv, Tkv, d;   // H query heads, Hkv key/value heads (H % Hkv == 0)
    int num_splits;   // already clamped to [1, Tkv]
    float c;          // scale * log2(e)
    void* workspace;  // B*H*num_splits*(d+2) floats, unused when num_splits == 1
};

bool prefill_bf16_supports(int d);
bool prefill_bf16_fits(int Tkv, int d);
PrefillSplit prefill_bf16_split_plan(int B, int H, int Tq, int Tkv, int d, bool causal, int kv_chunk);
hipError_t launch_prefill_bf16(const PrefillArgs& a, const PrefillSplit& split, hipStream_t stream,
                               const char** name);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream, const char** name);
bool prefill_f32_supports(int d);
struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    float* dq;
    float* dk;
    float* dv;
    int B, H, Tq, Tkv, d;
    bool causal;
    float c;          // scale * log2(e)
    float scale;
    void* workspace;  // per query row (lse * log2 e, D) as float2
};

bool backward_supports(int d);
size_t backward_workspace_bytes(int B, int H, int Tq);
hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t stream, const char** name);

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream, const char** name);
// (decode_mfma.hip) grouped-query decode on the matrix cores, groups of 4 and more
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream, const char** name);
// (decode.hip) the merge of a.num_splits partial records per query head
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream);
int decode_auto_splits(int B, int Hq, int Hkv, int Tkv, int d);

// Size of the library's own per-device decode partials (32 MiB), and its
// device address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace attn
