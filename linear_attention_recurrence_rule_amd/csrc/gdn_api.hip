// C ABI of libgdn: argument validation and dispatch.  Every check runs on the
// host before anything is launched; nothing here allocates, synchronises or
// keeps state between calls.
#include <stdint.h>

#include <climits>
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_launch.hpp"

namespace {

bool head_size_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(gdn_dtype t) { return t == GDN_F32 || t == GDN_BF16; }

// Element counts must stay well inside 64-bit indexing and the grid limit.
bool fits(long long a, long long b, long long c, long long d) {
    const long long lim = 1LL << 46;
    long long n = a;
    for (long long f : {b, c, d}) {
        if (f != 0 && n > lim / f) return false;
        n *= f;
    }
    return true;
}

gdn_status from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

}  // namespace

extern "C" {

namespace {

gdn_status prefill_check(int B, int T, int H, int d_k, int d_v, gdn_dtype qkv_dtype) {
    if (!dtype_ok(qkv_dtype)) return GDN_ERR_DTYPE;
    if (B <= 0 || H <= 0 || T < 0) return GDN_ERR_SHAPE;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    if (!fits(B, T, H, 128) || static_cast<long long>(B) * H > 65535) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

size_t workspace_needed(int B, int T, int H, gdn_dtype qkv_dtype) {
    return (qkv_dtype == GDN_BF16 && T > 0) ? gdn::prefill_bf16_workspace_bytes(B, T, H) : 0;
}

}  // namespace

size_t gdn_prefill_workspace_bytes(int B, int T, int H, int d_k, int d_v, gdn_dtype qkv_dtype) {
    if (prefill_check(B, T, H, d_k, d_v, qkv_dtype) != GDN_OK) return 0;
    return workspace_needed(B, T, H, qkv_dtype);
}

namespace {

// Every argument check of gdn_prefill_fwd except the workspace's.
gdn_status prefill_args_check(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                              const float* initial_state, const float* final_state, const float* y, int B, int T,
                              int H, int d_k, int d_v, gdn_dtype qkv_dtype) {
    const gdn_status st = prefill_check(B, T, H, d_k, d_v, qkv_dtype);
    if (st != GDN_OK) return st;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !y)) return GDN_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(alpha), static_cast<const void*>(beta),
                          static_cast<const void*>(initial_state), static_cast<const void*>(final_state),
                          static_cast<const void*>(y)})
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    return GDN_OK;
}

}  // namespace

gdn_status gdn_prefill_fwd(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* initial_state, float* final_state, float* y,
                           int B, int T, int H, int d_k, int d_v, gdn_dtype qkv_dtype, float scale,
                           void* workspace, size_t workspace_bytes, void* hip_stream) {
    const gdn_status st = prefill_args_check(q, k, v, alpha, beta, initial_state, final_state, y, B, T, H, d_k, d_v,
                                             qkv_dtype);
    if (st != GDN_OK) return st;
    if (workspace && !aligned16(workspace)) return GDN_ERR_ALIGN;
    const size_t need = workspace_needed(B, T, H, qkv_dtype);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
    if (!final_state && T == 0) return GDN_OK;
    gdn::PrefillArgs a{q, k, v, alpha, beta, initial_state, final_state, y,
                       B, T, H, d_k, d_v, qkv_dtype == GDN_BF16, scale, workspace,
                       static_cast<hipStream_t>(hip_stream)};
    return from_hip(gdn::launch_prefill(a));
}

// ---------------------------------------------------------------------------
// gdn_prefill_fwd_noalloc: the same call with its scratch in a static device
// array, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).  Nothing
// here allocates or frees.
// ---------------------------------------------------------------------------
namespace {

// One array per GPU, held from module load until the process ends.
static __device__ __align__(256) unsigned char scratch[GDN_PREFILL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void* g_scratch[kMaxDevices];   // the array's device address on each GPU

// The device address of `scratch` on the current GPU.  In host code the
// array's name is only a stand-in, so its address is looked up once per device,
// with that device current, and kept; kernels only ever receive that address.
hipError_t scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_scratch_lock);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

gdn_status gdn_prefill_fwd_noalloc(const void* q, const void* k, const void* v, const float* alpha,
                                   const float* beta, const float* initial_state, float* final_state, float* y,
                                   int B, int T, int H, int d_k, int d_v, gdn_dtype qkv_dtype, float scale,
                                   void* hip_stream) {
    const gdn_status st = prefill_args_check(q, k, v, alpha, beta, initial_state, final_state, y, B, T, H, d_k, d_v,
                                             qkv_dtype);
    if (st != GDN_OK) return st;
    const size_t need = workspace_needed(B, T, H, qkv_dtype);
    if (need > GDN_PREFILL_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
    if (!final_state && T == 0) return GDN_OK;
    void* ws = nullptr;
    if (need > 0 && scratch_on_current_device(&ws) != hipSuccess) return GDN_ERR_LAUNCH;
    return gdn_prefill_fwd(q, k, v, alpha, beta, initial_state, final_state, y, B, T, H, d_k, d_v, qkv_dtype, scale,
                           ws, need, hip_stream);
}

gdn_status gdn_prefill_status(const void* workspace, void* hip_stream) {
    if (!workspace) return GDN_ERR_NULL;
    if (!aligned16(workspace)) return GDN_ERR_ALIGN;
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    unsigned word = 0;
    if (hipStreamSynchronize(s) != hipSuccess) return GDN_ERR_LAUNCH;
    if (hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return GDN_ERR_LAUNCH;
    return word == 0 ? GDN_OK : GDN_ERR_DEVICE;
}

gdn_status gdn_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, float* state, float* y, int N, int H, int d_k, int d_v,
                           gdn_dtype qkv_dtype, float scale, void* hip_stream) {
    if (!dtype_ok(qkv_dtype)) return GDN_ERR_DTYPE;
    if (N < 0 || H <= 0) return GDN_ERR_SHAPE;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    if (!fits(N, H, d_k, d_v) || static_cast<long long>(N) * H > INT_MAX) return GDN_ERR_UNSUPPORTED;
    if (N == 0) return GDN_OK;
    if (!q || !k || !v || !alpha || !beta || !state || !y) return GDN_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(alpha), static_cast<const void*>(beta),
                          static_cast<const void*>(state), static_cast<const void*>(y)})
        if (!aligned16(p)) return GDN_ERR_ALIGN;
    gdn::DecodeArgs a{q, k, v, alpha, beta, state, y, N, H, d_k, d_v, qkv_dtype == GDN_BF16, scale,
                      static_cast<hipStream_t>(hip_stream)};
    return from_hip(gdn::launch_decode(a));
}

gdn_status gdn_gated_rmsnorm(const float* y, const void* z, const float* weight, float eps, void* out,
                             long rows, int d_v, gdn_dtype io_dtype, void* hip_stream) {
    if (!dtype_ok(io_dtype)) return GDN_ERR_DTYPE;
    if (rows < 0) return GDN_ERR_SHAPE;
    if (!head_size_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    if (!fits(rows, d_v, 1, 1) || rows / (256 / (d_v / 4)) >= INT_MAX) return GDN_ERR_UNSUPPORTED;
    if (rows == 0) return GDN_OK;
    if (!y || !z || !out) return GDN_ERR_NULL;
    for (const void* p : {static_cast<const void*>(y), z, static_cast<const void*>(weight),
                          static_cast<const void*>(out)})
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    gdn::NormArgs a{y, z, weight, eps, out, rows, d_v, io_dtype == GDN_BF16,
                    static_cast<hipStream_t>(hip_stream)};
    return from_hip(gdn::launch_gated_rmsnorm(a));
}

gdn_status gdn_frontend_fwd(const void* q_proj, const void* k_proj, const void* v_proj, const float* conv_q,
                            const float* conv_k, const float* conv_v, const float* a_logit, const float* b_logit,
                            const float* A, const float* b_alpha, const void* q_hist, const void* k_hist,
                            const void* v_hist, void* q, void* k, void* v, float* alpha, float* beta, int B, int T,
                            int H, int d_k, int d_v, int conv_width, gdn_dtype io_dtype, float norm_eps,
                            void* hip_stream) {
    if (!dtype_ok(io_dtype)) return GDN_ERR_DTYPE;
    if (B <= 0 || H <= 0 || T < 0 || conv_width < 1 || !(norm_eps >= 0.f)) return GDN_ERR_SHAPE;
    if (conv_width > 4 || !head_size_ok(d_k) || !head_size_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    if (!fits(B, T, H, 128) || static_cast<long long>(B) * H * ((T + 31) / 32) / 2 >= INT_MAX)
        return GDN_ERR_UNSUPPORTED;
    if (T == 0) return GDN_OK;
    for (const void* p : {q_proj, k_proj, v_proj, static_cast<const void*>(conv_q), static_cast<const void*>(conv_k),
                          static_cast<const void*>(conv_v), static_cast<const void*>(a_logit),
                          static_cast<const void*>(b_logit), static_cast<const void*>(A),
                          static_cast<const void*>(b_alpha), static_cast<const void*>(q), static_cast<const void*>(k),
                          static_cast<const void*>(v), static_cast<const void*>(alpha), static_cast<const void*>(beta)})
        if (!p) return GDN_ERR_NULL;
    for (const void* p : {q_proj, k_proj, v_proj, q_hist, k_hist, v_hist, static_cast<const void*>(q),
                          static_cast<const void*>(k), static_cast<const void*>(v)})
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    gdn::FrontendArgs a{q_proj, k_proj, v_proj, conv_q, conv_k, conv_v, a_logit, b_logit, A, b_alpha,
                        q_hist, k_hist, v_hist, q, k, v, alpha, beta, B, T, H, d_k, d_v, conv_width,
                        io_dtype == GDN_BF16, norm_eps, static_cast<hipStream_t>(hip_stream)};
    return from_hip(gdn::launch_frontend(a));
}

namespace {

gdn_status bwd_check(int B, int T, int H, int d_k, int d_v, gdn_dtype qkv_dtype) {
    if (!dtype_ok(qkv_dtype)) return GDN_ERR_DTYPE;
    if (B <= 0 || H <= 0 || T < 0) return GDN_ERR_SHAPE;
    if (!head_size_ok(d_k) || d_k != d_v) return GDN_ERR_UNSUPPORTED;
    if (!fits(B, T, H, 128) || static_cast<long long>(B) * H > 65535 || (T + 63) / 64 > 65535)
        return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

}  // namespace

size_t gdn_prefill_bwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, gdn_dtype qkv_dtype) {
    if (bwd_check(B, T, H, d_k, d_v, qkv_dtype) != GDN_OK || T == 0) return 0;
    return gdn::prefill_bwd_workspace_bytes(B, T, H, d_k, d_v);
}

gdn_status gdn_prefill_bwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                           const float* initial_state, const float* dy, const float* d_final_state, float* dq,
                           float* dk, float* dv, float* dalpha, float* dbeta, float* d_initial_state, int B, int T,
                           int H, int d_k, int d_v, gdn_dtype qkv_dtype, float scale, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
    const gdn_status st = bwd_check(B, T, H, d_k, d_v, qkv_dtype);
    if (st != GDN_OK) return st;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !dy || !dq || !dk || !dv || !dalpha || !dbeta))
        return GDN_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(alpha), static_cast<const void*>(beta),
                          static_cast<const void*>(initial_state), static_cast<const void*>(dy),
                          static_cast<const void*>(d_final_state), static_cast<const void*>(dq),
                          static_cast<const void*>(dk), static_cast<const void*>(dv),
                          static_cast<const void*>(dalpha), static_cast<const void*>(dbeta),
                          static_cast<const void*>(d_initial_state)})
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    const size_t need = T == 0 ? 0 : gdn::prefill_bwd_workspace_bytes(B, T, H, d_k, d_v);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return GDN_ERR_ALIGN;
    gdn::PrefillBwdArgs a{q, k, v, alpha, beta, initial_state, dy, d_final_state, dq, dk, dv, dalpha, dbeta,
                          d_initial_state, B, T, H, d_k, d_v, qkv_dtype == GDN_BF16, scale, workspace,
                          static_cast<hipStream_t>(hip_stream)};
    return from_hip(gdn::launch_prefill_bwd(a));
}

namespace {

gdn_status mtp_check(int N, int K, int H, int d_k, int d_v, gdn_dtype qkv_dtype) {
    if (!dtype_ok(qkv_dtype)) return GDN_ERR_DTYPE;
    if (N < 0 || K < 0 || H <= 0) return GDN_ERR_SHAPE;
    if (K > 8 || !head_size_ok(d_k) || !head_size_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    if (!fits(N, K, H, static_cast<long long>(d_k) * d_v) || static_cast<long long>(N) * K * H > INT_MAX)
        return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

}  // namespace

gdn_status gdn_decode_mtp_verify(const void* q, const void* k, const void* v, const float* alpha,
                                 const float* beta, const float* state, float* y, float* e,
                                 float* prefix_states, int N, int K, int H, int d_k, int d_v,
                                 gdn_dtype qkv_dtype, float scale, void* hip_stream) {
    const gdn_status st = mtp_check(N, K, H, d_k, d_v, qkv_dtype);
    if (st != GDN_OK) return st;
    if (N == 0 || K == 0) return GDN_OK;
    if (!q || !k || !v || !alpha || !beta || !state || !y) return GDN_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(alpha), static_cast<const void*>(beta),
                          static_cast<const void*>(state), static_cast<const void*>(y),
                          static_cast<const void*>(e), static_cast<const void*>(prefix_states)})
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    gdn::MtpArgs a{false, q, k, v, alpha, beta, const_cast<float*>(state), y, e, prefix_states, nullptr,
                   N, K, H, d_k, d_v, qkv_dtype == GDN_BF16, scale, static_cast<hipStream_t>(hip_stream)};
    return from_hip(gdn::launch_mtp(a));
}

gdn_status gdn_decode_mtp_commit(const void* k, const float* alpha, const float* beta, const float* e,
                                 const int* accepted, float* state, int N, int K, int H, int d_k, int d_v,
                                 gdn_dtype qkv_dtype, void* hip_stream) {
    const gdn_status st = mtp_check(N, K, H, d_k, d_v, qkv_dtype);
    if (st != GDN_OK) return st;
    if (N == 0 || K == 0) return GDN_OK;
    if (!k || !alpha || !beta || !e || !accepted || !state) return GDN_ERR_NULL;
    for (const void* p : {k, static_cast<const void*>(alpha), static_cast<const void*>(beta),
                          static_cast<const void*>(e), static_cast<const void*>(accepted),
                          static_cast<const void*>(state)})
        if (!aligned16(p)) return GDN_ERR_ALIGN;
    gdn::MtpArgs a{true, nullptr, k, nullptr, alpha, beta, state, nullptr, const_cast<float*>(e), nullptr,
                   accepted, N, K, H, d_k, d_v, qkv_dtype == GDN_BF16, 1.f, static_cast<hipStream_t>(hip_stream)};
    return from_hip(gdn::launch_mtp(a));
}

namespace {

bool qsa_dim_ok(int D) { return D == 32 || D == 64 || D == 128; }

gdn_status qsa_select_check(int B, int n, int H, int D, int r, int K, gdn_dtype dtype) {
    if (!dtype_ok(dtype)) return GDN_ERR_DTYPE;
    if (B <= 0 || n < 0 || H <= 0 || r < 1 || K < 1) return GDN_ERR_SHAPE;
    if (!qsa_dim_ok(D) || B > 65535) return GDN_ERR_UNSUPPORTED;
    const long long nb = n / r;
    if (!fits(B, n, H, D) || !fits(B, n, (nb + 63) / 64 * 64, 4) || !fits(B, n, (K + r - 1) / r, 4) ||
        static_cast<long long>(B) * n > INT_MAX)
        return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

}  // namespace

gdn_status gdn_qsa_prep(const void* q_proj, const void* k_proj, const float* q_weight, const float* k_weight,
                        void* q_out, void* kbar_out, int B, int n, int H, int D, int r, int rope_dims,
                        float rope_base, float eps, gdn_dtype io_dtype, void* hip_stream) {
    if (!dtype_ok(io_dtype)) return GDN_ERR_DTYPE;
    if (B <= 0 || n < 0 || H <= 0 || r < 1 || rope_dims < 0 || (rope_dims & 1) || !(eps >= 0.f) ||
        !(rope_base > 0.f))
        return GDN_ERR_SHAPE;
    if (!qsa_dim_ok(D) || rope_dims > D) return GDN_ERR_UNSUPPORTED;
    if (!fits(B, n, H, D) || (static_cast<long long>(B) * n * (H + 1) + 3) / 4 > INT_MAX) return GDN_ERR_UNSUPPORTED;
    if (n == 0) return GDN_OK;
    if (!q_proj || !k_proj || !q_out || !kbar_out) return GDN_ERR_NULL;
    for (const void* p : {q_proj, k_proj, static_cast<const void*>(q_weight), static_cast<const void*>(k_weight),
                          static_cast<const void*>(q_out), static_cast<const void*>(kbar_out)})
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    gdn::QsaPrepArgs a{q_proj, k_proj, q_weight, k_weight, q_out, kbar_out, B, n, H, D, r, rope_dims, rope_base,
                       eps, io_dtype == GDN_BF16, static_cast<hipStream_t>(hip_stream)};
    return from_hip(gdn::launch_qsa_prep(a));
}

size_t gdn_qsa_select_workspace_bytes(int B, int n, int H, int D, int r, int K, gdn_dtype dtype) {
    if (qsa_select_check(B, n, H, D, r, K, dtype) != GDN_OK) return 0;
    return gdn::qsa_select_workspace_bytes(B, n, H, r, (K + r - 1) / r);
}

gdn_status gdn_qsa_select(const void* q, const void* kbar, int* block_idx, int B, int n, int H, int D, int r, int K,
                          gdn_dtype dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
    const gdn_status st = qsa_select_check(B, n, H, D, r, K, dtype);
    if (st != GDN_OK) return st;
    if (n == 0) return GDN_OK;
    if (!q || !block_idx || (n / r > 0 && !kbar)) return GDN_ERR_NULL;
    for (const void* p : {q, kbar, static_cast<const void*>(block_idx)})
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    const size_t need = gdn::qsa_select_workspace_bytes(B, n, H, r, (K + r - 1) / r);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return GDN_ERR_ALIGN;
    gdn::QsaSelectArgs a{q, kbar, block_idx, B, n, H, D, r, (K + r - 1) / r, dtype == GDN_BF16, workspace,
                         static_cast<hipStream_t>(hip_stream)};
    return from_hip(gdn::launch_qsa_select(a));
}

gdn_status gdn_decode_mtp_commit_verify(const void* q, const void* k, const void* v, const float* alpha,
                                        const float* beta, float* state, float* y, float* e, const void* prev_k,
                                        const float* prev_alpha, const float* prev_beta, const float* prev_e,
                                        const int* prev_accepted, int N, int K, int K_prev, int H, int d_k, int d_v,
                                        gdn_dtype qkv_dtype, float scale, void* hip_stream) {
    gdn_status st = mtp_check(N, K, H, d_k, d_v, qkv_dtype);
    if (st == GDN_OK) st = mtp_check(N, K_prev, H, d_k, d_v, qkv_dtype);
    if (st != GDN_OK) return st;
    if (K < 1 || K_prev < 1) return GDN_ERR_SHAPE;
    if (N == 0) return GDN_OK;
    if (!q || !k || !v || !alpha || !beta || !state || !y || !prev_k || !prev_alpha || !prev_beta || !prev_e ||
        !prev_accepted)
        return GDN_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(alpha), static_cast<const void*>(beta),
                          static_cast<const void*>(state), static_cast<const void*>(y), static_cast<const void*>(e),
                          prev_k, static_cast<const void*>(prev_alpha), static_cast<const void*>(prev_beta),
                          static_cast<const void*>(prev_e), static_cast<const void*>(prev_accepted)})
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    // e may share prev_e's buffer only when both blocks have the same length:
    // then each workgroup reads its own rows of prev_e before it writes the
    // same rows of e.  With K != K_prev the rows belong to other workgroups.
    if (e && e == prev_e && K != K_prev) return GDN_ERR_SHAPE;
    gdn::MtpArgs a{false, q, k, v, alpha, beta, state, y, e, nullptr, nullptr, N, K, H, d_k, d_v,
                   qkv_dtype == GDN_BF16, scale, static_cast<hipStream_t>(hip_stream)};
    a.pend_k = prev_k;
    a.pend_alpha = prev_alpha;
    a.pend_beta = prev_beta;
    a.pend_e = prev_e;
    a.pend_accepted = prev_accepted;
    a.Kp = K_prev;
    return from_hip(gdn::launch_mtp(a));
}

const char* gdn_status_string(gdn_status status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "invalid size argument";
        case GDN_ERR_DTYPE: return "unknown dtype code";
        case GDN_ERR_ALIGN: return "pointer is not 16-byte aligned";
        case GDN_ERR_UNSUPPORTED: return "unsupported head size or problem size";
        case GDN_ERR_LAUNCH: return "HIP kernel launch failed";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_DEVICE: return "the call wrote non-finite y or state (inputs outside the fp16 operand range?)";
    }
    return "unknown status";
}

}  // extern "C"
