// Output epilogue of the GDN mixer (slinene ai-papers-daily page on
// Qwen3.8-Next, Module A): a sigmoid gate times a zero-centred RMSNorm of the
// mixer output, per (token, head) row of d_v values:
//     out = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + w)
// A pure stream (read y and z, write out once), bound by HBM bandwidth.
// Each row is handled by d_v/8 lanes holding 8 values each: lane `sub` takes
// columns 4 sub .. 4 sub + 3 of each half of the row, so that every load and
// store instruction covers whole contiguous lines of y, z and out.  The row's
// sum of squares is reduced with DPP lane moves inside the lane group, so no
// LDS is used.  A thread covers kNormPasses rows and loads all of them before
// reducing any.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kNormPasses = 2;   // rows per thread, loaded before any is reduced

// Sum over aligned groups of L lanes (L = 2, 4, 8, 16), every lane getting
// the group's sum: quad swaps, then the half-row and row mirrors.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
    auto mv = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
    };
    x += mv(x, std::integral_constant<int, 0xB1>{});           // quad_perm [1, 0, 3, 2]
    if constexpr (L >= 4) x += mv(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2, 3, 0, 1]
    if constexpr (L >= 8) x += mv(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
    if constexpr (L >= 16) x += mv(x, std::integral_constant<int, 0x140>{});  // row_mirror
    return x;
}

template <int DV, bool kBf16>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const float* __restrict__ y,
                                                            const void* __restrict__ z,
                                                            const float* __restrict__ weight, float eps,
                                                            void* __restrict__ out, long rows) {
    constexpr int kLanesPerRow = DV / 8;
    constexpr int kRowsPerPass = 256 / kLanesPerRow;
    static_assert(kLanesPerRow >= 2 && kLanesPerRow <= 16, "d_v in 16 .. 128");
    const int tid = threadIdx.x;
    const int sub = tid % kLanesPerRow;
    const long row0 = static_cast<long>(blockIdx.x) * kRowsPerPass * kNormPasses + tid / kLanesPerRow;

    // all loads first, so that each thread has several requests in flight
    float yv[kNormPasses][8];
    float zv[kNormPasses][8];
#pragma unroll
    for (int p = 0; p < kNormPasses; ++p) {
        const long row = row0 + p * kRowsPerPass;
        // columns 4 sub .. 4 sub + 3 (values 0..3) and DV / 2 + 4 sub .. (values 4..7)
        const long base = (row < rows ? row : rows - 1) * DV + sub * 4;   // clamped; not stored
        // streaming loads: y and z are read once (about 8% faster than
        // cached loads at 32K tokens x 32 heads)
        const float4v y0 = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(y + base));
        const float4v y1 = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(y + base + DV / 2));
        yv[p][0] = y0[0]; yv[p][1] = y0[1]; yv[p][2] = y0[2]; yv[p][3] = y0[3];
        yv[p][4] = y1[0]; yv[p][5] = y1[1]; yv[p][6] = y1[2]; yv[p][7] = y1[3];
        if constexpr (kBf16) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 r0 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(z) + base));
            const u32x2 r1 =
                __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(z) + base + DV / 2));
            const uint32_t wds[4] = {r0[0], r0[1], r1[0], r1[1]};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                zv[p][2 * i] = bf16_to_f32(static_cast<uint16_t>(wds[i] & 0xffffu));
                zv[p][2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(wds[i] >> 16));
            }
        } else {
            const float4v z0 = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(static_cast<const float*>(z) + base));
            const float4v z1 =
                __builtin_nontemporal_load(reinterpret_cast<const float4v*>(static_cast<const float*>(z) + base + DV / 2));
            zv[p][0] = z0[0]; zv[p][1] = z0[1]; zv[p][2] = z0[2]; zv[p][3] = z0[3];
            zv[p][4] = z1[0]; zv[p][5] = z1[1]; zv[p][6] = z1[2]; zv[p][7] = z1[3];
        }
    }
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0.f;
    if (weight) {
        const float4 w0 = reinterpret_cast<const float4*>(weight)[sub];
        const float4 w1 = reinterpret_cast<const float4*>(weight + DV / 2)[sub];
        w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
        w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
    }
#pragma unroll
    for (int p = 0; p < kNormPasses; ++p) {
        const long row = row0 + p * kRowsPerPass;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += yv[p][i] * yv[p][i];
        ss = group_sum<kLanesPerRow>(ss);
        if (row >= rows) continue;
        // hardware reciprocal square root and reciprocal (about 1 ulp each)
        const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / DV) + eps);
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float gate = __builtin_amdgcn_rcpf(1.0f + __expf(-zv[p][i]));
            o[i] = gate * (yv[p][i] * inv) * (1.0f + w[i]);
        }
        const long base = row * DV + sub * 4;
        // streaming stores: the output is not read again here
        if constexpr (kBf16) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])},
                                        reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + base));
            __builtin_nontemporal_store(u32x2{pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])},
                                        reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + base + DV / 2));
        } else {
            __builtin_nontemporal_store(float4v{o[0], o[1], o[2], o[3]},
                                        reinterpret_cast<float4v*>(static_cast<float*>(out) + base));
            __builtin_nontemporal_store(float4v{o[4], o[5], o[6], o[7]},
                                        reinterpret_cast<float4v*>(static_cast<float*>(out) + base + DV / 2));
        }
    }
}

template <int DV, bool kBf16>
static hipError_t launch_norm_t(const NormArgs& a) {
    constexpr int kRowsPerBlock = 256 / (DV / 8) * kNormPasses;
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
