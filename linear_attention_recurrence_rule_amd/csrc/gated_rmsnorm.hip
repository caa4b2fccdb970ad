// Output epilogue of the GDN mixer (slinene ai-papers-daily page on
// Qwen3.8-Next, Module A): a sigmoid gate times a zero-centred RMSNorm of the
// mixer output, per (token, head) row of d_v values:
//     out = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + w)
// A pure stream (read y and z, write out once), bound by HBM bandwidth.
// Each row is handled by d_v/4 lanes holding one float4 each; the row's sum of
// squares is reduced with cross-lane shuffles, so no LDS is used.  A thread
// covers kNormPasses rows and loads all of them before reducing any.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kNormPasses = 2;   // rows per thread, loaded before any is reduced

template <int DV, bool kBf16>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const float* __restrict__ y,
                                                            const void* __restrict__ z,
                                                            const float* __restrict__ weight, float eps,
                                                            void* __restrict__ out, long rows) {
    constexpr int kLanesPerRow = DV / 4;
    constexpr int kRowsPerPass = 256 / kLanesPerRow;
    const int tid = threadIdx.x;
    const int sub = tid % kLanesPerRow;
    const long row0 = static_cast<long>(blockIdx.x) * kRowsPerPass * kNormPasses + tid / kLanesPerRow;

    // all loads first, so that each thread has several requests in flight
    float4 yv[kNormPasses];
    float zv[kNormPasses][4];
#pragma unroll
    for (int p = 0; p < kNormPasses; ++p) {
        const long row = row0 + p * kRowsPerPass;
        const long base = (row < rows ? row : rows - 1) * DV + sub * 4;   // clamped; not stored
        yv[p] = *reinterpret_cast<const float4*>(y + base);
        if constexpr (kBf16) {
            const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(z) + base);
            zv[p][0] = bf16_to_f32(static_cast<uint16_t>(raw.x & 0xffffu));
            zv[p][1] = bf16_to_f32(static_cast<uint16_t>(raw.x >> 16));
            zv[p][2] = bf16_to_f32(static_cast<uint16_t>(raw.y & 0xffffu));
            zv[p][3] = bf16_to_f32(static_cast<uint16_t>(raw.y >> 16));
        } else {
            const float4 zz = *reinterpret_cast<const float4*>(static_cast<const float*>(z) + base);
            zv[p][0] = zz.x; zv[p][1] = zz.y; zv[p][2] = zz.z; zv[p][3] = zz.w;
        }
    }
    float w[4] = {0.f, 0.f, 0.f, 0.f};
    if (weight) {
        const float4 ww = reinterpret_cast<const float4*>(weight)[sub];
        w[0] = ww.x; w[1] = ww.y; w[2] = ww.z; w[3] = ww.w;
    }
#pragma unroll
    for (int p = 0; p < kNormPasses; ++p) {
        const long row = row0 + p * kRowsPerPass;
        float ss = yv[p].x * yv[p].x + yv[p].y * yv[p].y + yv[p].z * yv[p].z + yv[p].w * yv[p].w;
#pragma unroll
        for (int off = 1; off < kLanesPerRow; off <<= 1) ss += __shfl_xor(ss, off);
        if (row >= rows) continue;
        // hardware reciprocal square root and reciprocal (about 1 ulp each)
        const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / DV) + eps);
        const float yy[4] = {yv[p].x, yv[p].y, yv[p].z, yv[p].w};
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float gate = __builtin_amdgcn_rcpf(1.0f + __expf(-zv[p][i]));
            o[i] = gate * (yy[i] * inv) * (1.0f + w[i]);
        }
        const long base = row * DV + sub * 4;
        // streaming stores: the output is not read again here
        if constexpr (kBf16) {
            const uint32_t lo = pack_bf16x2(o[0], o[1]);
            const uint32_t hi = pack_bf16x2(o[2], o[3]);
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + base));
        } else {
            __builtin_nontemporal_store(float4v{o[0], o[1], o[2], o[3]},
                                        reinterpret_cast<float4v*>(static_cast<float*>(out) + base));
        }
    }
}

template <int DV, bool kBf16>
static hipError_t launch_norm_t(const NormArgs& a) {
    constexpr int kRowsPerBlock = 256 / (DV / 4) * kNormPasses;
    const long blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL((gated_rmsnorm_kernel<DV, kBf16>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, a.stream, a.y, a.z, a.weight, a.eps, a.out, a.rows);
    return hipGetLastError();
}

template <bool kBf16>
static hipError_t launch_norm_dt(const NormArgs& a) {
    switch (a.dv) {
        case 16: return launch_norm_t<16, kBf16>(a);
        case 32: return launch_norm_t<32, kBf16>(a);
        case 64: return launch_norm_t<64, kBf16>(a);
        case 128: return launch_norm_t<128, kBf16>(a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gated_rmsnorm(const NormArgs& a) {
    if (a.rows == 0) return hipSuccess;
    return a.bf16 ? launch_norm_dt<true>(a) : launch_norm_dt<false>(a);
}

}  // namespace gdn
