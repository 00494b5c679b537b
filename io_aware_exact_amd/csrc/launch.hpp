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
    float c;   // scale * log2(e)
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

hipError_t launch_prefill_bf16_d64(const PrefillArgs& a, hipStream_t stream, const char** name);
bool prefill_bf16_fits(int Tkv);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream, const char** name);
bool prefill_f32_supports(int d);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream, const char** name);

}  // namespace attn
