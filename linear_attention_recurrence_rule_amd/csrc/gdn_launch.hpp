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
    void* workspace;             // bf16 path: status word + per-chunk T' blocks (prefill_bf16_workspace_bytes)
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

struct FrontendArgs {
    const void* q_proj;
    const void* k_proj;
    const void* v_proj;
    const float* conv_q;        // [H, d_k, width]
    const float* conv_k;
    const float* conv_v;        // [H, d_v, width]
    const float* a_logit;       // [B, T, H]
    const float* b_logit;
    const float* A;             // [H]
    const float* b_alpha;       // [H]
    const void* q_hist;         // [B, width-1, H, d] or null (zeros)
    const void* k_hist;
    const void* v_hist;
    void* q;
    void* k;
    void* v;
    float* alpha;
    float* beta;
    int B, T, H, dk, dv, width;
    bool bf16;
    float eps;
    hipStream_t stream;
};

struct MtpArgs {
    bool commit;                // false: verify a draft block; true: commit the accepted prefix
    const void* q;              // [N, K, H, d_k] (verify only)
    const void* k;              // [N, K, H, d_k]
    const void* v;              // [N, K, H, d_v] (verify only)
    const float* alpha;         // [N, K, H]
    const float* beta;
    float* state;               // [N, H, d_k, d_v]; read only when verifying
    float* y;                   // [N, K, H, d_v] (verify)
    float* e;                   // [N, K, H, d_v] misses: written by verify (may be null), read by commit
    float* prefix;              // [N, K, H, d_k, d_v] or null (verify)
    const int* accepted;        // [N] (commit)
    int N, K, H, dk, dv;
    bool bf16;
    float scale;
    hipStream_t stream;
    // verify after committing a previous block (all null for a plain verify)
    const void* pend_k = nullptr;        // [N, Kp, H, d_k]
    const float* pend_alpha = nullptr;   // [N, Kp, H]
    const float* pend_beta = nullptr;
    const float* pend_e = nullptr;       // [N, Kp, H, d_v]
    const int* pend_accepted = nullptr;  // [N]
    int Kp = 0;
};

struct PrefillBwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const float* initial_state;  // may be null (zero state)
    const float* dy;             // [B, T, H, d_v]
    const float* d_final_state;  // may be null (zero)
    float* dq;
    float* dk;
    float* dv;
    float* dalpha;
    float* dbeta;
    float* d_initial_state;      // may be null (not written)
    int B, T, H, dk_, dv_;
    bool bf16;
    float scale;
    void* workspace;             // prefill_bwd_workspace_bytes
    hipStream_t stream;
};

struct QsaPrepArgs {
    const void* q_proj;         // [B, n, H, D]
    const void* k_proj;         // [B, n, D]
    const float* q_weight;      // [D] or null (1)
    const float* k_weight;      // [D] or null (1)
    void* q_out;                // [B, n, H, D]
    void* kbar_out;             // [B, n / r, D]
    int B, n, H, D, r, rope_dims;
    float rope_base, eps;
    bool bf16;
    hipStream_t stream;
};

struct QsaSelectArgs {
    const void* q;              // [B, n, H, D]
    const void* kbar;           // [B, n / r, D]
    int* idx;                   // [B, n, KB]
    int B, n, H, D, r, KB;
    bool bf16;
    void* workspace;            // qsa_select_workspace_bytes bytes
    hipStream_t stream;
};

hipError_t launch_prefill(const PrefillArgs& a);
hipError_t launch_prefill_bf16(const PrefillArgs& a);
// Chunk-start states S_c ([B H nchunks][d][d]) and E_c ([B H nchunks][64][d]),
// as fp16 at the start of the given fp32-sized buffers, from the bf16 chunked
// walk without y; d_k = d_v in {64, 128}; the workspace as for
// launch_prefill_bf16.
hipError_t launch_prefill_bf16_states(const PrefillArgs& a, float* S, float* E);

// The backward's reverse walk for bf16 inputs (d_k = d_v = d in {64, 128}):
// dS' per chunk and dR per chunk (as fp16, laid out as their fp32 slots,
// at the slots' start), dv and d_initial_state (fp32), from the backward
// workspace's g (fp32, [B H nchunks] x 64) and T slots ([B H nchunks] x 16 KB,
// holding fp16 T then fp16 P, 64 x 64 each).
struct RevWalkArgs {
    const void* q;
    const void* k;
    const float* beta;
    const float* dy;
    const float* dST;            // may be null
    const float* g;
    const float* Tm;
    float* dS;
    float* dR;
    float* dv;
    float* dS0;                  // may be null
    int B, T, H, d;
    float scale;
    hipStream_t stream;
};
hipError_t launch_bwd_reverse_walk(const RevWalkArgs& a);
size_t prefill_bf16_workspace_bytes(int B, int T, int H);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_gated_rmsnorm(const NormArgs& a);
hipError_t launch_frontend(const FrontendArgs& a);
hipError_t launch_mtp(const MtpArgs& a);
hipError_t launch_prefill_bwd(const PrefillBwdArgs& a);
size_t prefill_bwd_workspace_bytes(int B, int T, int H, int dk, int dv);
hipError_t launch_qsa_prep(const QsaPrepArgs& a);
hipError_t launch_qsa_select(const QsaSelectArgs& a);
hipError_t launch_qsa_select4(const QsaSelectArgs& a);
size_t qsa_select_workspace_bytes(int B, int n, int H, int r, int KB);
size_t qsa_select4_workspace_bytes(int B, int n, int r, int KB);

}  // namespace gdn
