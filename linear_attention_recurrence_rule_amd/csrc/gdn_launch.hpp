// Host-side launch interface between the C ABI layer (gdn_api.hip) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const float* initial_state;  // may be null (zero state)
    float* final_state;          // may be null (not written); may alias initial_state
    float* y;
    int B, T, H, dk, dv;
    bool bf16;
    float scale;
    void* workspace;             // bf16 path: per-chunk T' blocks (prefill_bf16_workspace_bytes)
    hipStream_t stream;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    float* state;
    float* y;
    int N, H, dk, dv;
    bool bf16;
    float scale;
    hipStream_t stream;
};

struct NormArgs {
    const float* y;
    const void* z;
    const float* weight;  // may be null
    float eps;
    void* out;
    long rows;
    int dv;
    bool bf16;
    hipStream_t stream;
};

hipError_t launch_prefill(const PrefillArgs& a);
hipError_t launch_prefill_bf16(const PrefillArgs& a);
size_t prefill_bf16_workspace_bytes(int B, int T, int H);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_gated_rmsnorm(const NormArgs& a);

}  // namespace gdn
