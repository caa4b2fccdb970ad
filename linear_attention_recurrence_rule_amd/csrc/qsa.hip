// QSA (Qwen Sparse Attention) indexer on gfx950.
//
// Module B of the slinene ai-papers-daily page on "On the Design of
// Qwen3.8-Next Architecture": an MQA indexer (H query heads, one shared key
// head) scores the context at block granularity and picks, per query, the
// K_B = ceil(K / r) best complete blocks.
//
//   prep:    q_i^h  = PRoPE(RMSNorm(q_proj_i^h), i)
//            kbar_b = PRoPE(RMSNorm(mean_{j<r} k_{b r + j}), b r)     (pool first, rotate after)
//   scores:  I_ib = sum_h ReLU(<q_i^h, kbar_b>) for complete blocks, b r + r - 1 <= i
//   select:  the K_B largest I_ib per query (ties: the later block), reported
//            as ascending block indices, -1 padded.
//
// The partial rotary embedding turns the first rope_dims entries in
// rotate-half pairs (j, j + rope_dims/2) by pos * base^(-2 j / rope_dims).
//
// Kernels:
//   qsa_prep_kernel   eight rows per wave (query heads or pooled keys), two
//                     dimensions per lane; the rotation angle is formed and
//                     reduced modulo 2 pi in double precision, so that long
//                     positions keep their phase.
//   qsa_score_kernel  (head counts other than four; four heads select
//                     without storing the scores, in qsa_topk.hip)
//                     64 queries x 64 blocks per workgroup, one head at a
//                     time through LDS: bf16 MFMA 16x16x32 (exact products,
//                     fp32 sums) or fp32 MFMA 16x16x4 for fp32 operands; ReLU
//                     per head, summed, written for complete blocks only.
//   qsa_select_kernel one wave per query on the stored scores: select_row
//                     (qsa_wave.hpp).
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include "qsa_wave.hpp"

namespace gdn {
namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// prep: grid (rows / (4 kPrepRows)), 256 threads; each wave takes kPrepRows
// consecutive rows.  Rows [0, B n H) are query heads, rows [B n H, B n H +
// B nb) pooled keys.  A lane's rotary frequencies (double precision, one
// exp2 per dimension) are formed once and serve all of the wave's rows.
// ---------------------------------------------------------------------------
constexpr int kPrepRows = 8;

// Sum over the wave with DPP lane moves (row shifts, then the row broadcasts
// of lanes 15 and 31), read from lane 63.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    auto mv = [](float x, auto ctrl, auto rmask, auto bc) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                          decltype(rmask)::value, 0xf, decltype(bc)::value));
    };
    v += mv(v, std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xf>{}, std::true_type{});
    v += mv(v, std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xf>{}, std::true_type{});
    v += mv(v, std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xf>{}, std::true_type{});
    v += mv(v, std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xf>{}, std::true_type{});
    v += mv(v, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{}, std::false_type{});
    v += mv(v, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{}, std::false_type{});
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
template <bool kBf16>
__device__ __forceinline__ void store_out(void* p, long i, float x) {
    if constexpr (kBf16) static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
    else static_cast<float*>(p)[i] = x;
}

template <bool kBf16>
__global__ __launch_bounds__(256) void qsa_prep_kernel(const void* __restrict__ q_proj, const void* __restrict__ k_proj,
                                                       const float* __restrict__ q_weight,
                                                       const float* __restrict__ k_weight, void* __restrict__ q_out,
                                                       void* __restrict__ kbar_out, int B, int n, int H, int D, int r,
                                                       int rope_dims, double log2_base, float eps) {
    const int lane = threadIdx.x & 63;
    const long row0 = (static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kPrepRows;
    const long nq = static_cast<long>(B) * n * H;
    const int nb = n / r;
    const long nk = static_cast<long>(B) * nb;
    // this lane's dimensions d = lane + 64 e, their rotary partners and frequencies
    const int half = rope_dims / 2;
    int pl[2], pe[2];
    double freq[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int d = lane + 64 * e;
        // the partner value lives in lane (d +- half) mod 64, slot (d +- half) / 64
        const int pd = d < half ? d + half : d - half;
        pl[e] = (pd >= 0 ? pd : 0) & 63;
        pe[e] = (pd >= 0 ? pd : 0) >> 6;
        const int j = d < half ? d : d - half;
        freq[e] = d < rope_dims ? exp2(-2.0 * j / rope_dims * log2_base) : 0.0;
    }
    for (int i = 0; i < kPrepRows; ++i) {
        const long row = row0 + i;
        if (row >= nq + nk) return;                  // whole waves drop out together
        const bool is_q = row < nq;
        float x[2];
        long pos;
        const float* w = is_q ? q_weight : k_weight;
        if (is_q) {
            pos = (row / H) % n;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int d = lane + 64 * e;
                x[e] = d < D ? load_in<kBf16>(q_proj, row * D + d) : 0.f;
            }
        } else {
            const long kr = row - nq, b = kr / nb, blk = kr - b * nb;
            pos = blk * r;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int d = lane + 64 * e;
                float s = 0.f;
                if (d < D)
                    for (int j = 0; j < r; ++j) s += load_in<kBf16>(k_proj, (b * n + blk * r + j) * D + d);
                x[e] = s / static_cast<float>(r);
            }
        }
        // RMSNorm
        const float ss = wave_sum_dpp(x[0] * x[0] + x[1] * x[1]);
        const float inv = 1.f / sqrtf(ss / static_cast<float>(D) + eps);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int d = lane + 64 * e;
            x[e] *= inv;
            if (w && d < D) x[e] *= w[d];
        }
        // partial rotary embedding: dimension d < rope_dims pairs with d +- half
        float y[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int d = lane + 64 * e;
            const float p0 = __shfl(x[0], pl[e]), p1 = __shfl(x[1], pl[e]);
            const float partner = pe[e] ? p1 : p0;
            y[e] = x[e];
            if (d < rope_dims) {
                const double ang = static_cast<double>(pos) * freq[e];
                const double red = ang - 6.283185307179586 * floor(ang * 0.15915494309189535);
                float s, c;
                sincosf(static_cast<float>(red), &s, &c);
                y[e] = d < half ? x[e] * c - partner * s : x[e] * c + partner * s;
            }
        }
        void* out = is_q ? q_out : kbar_out;
        const long base = (is_q ? row : row - nq) * D;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int d = lane + 64 * e;
            if (d < D) store_out<kBf16>(out, base + d, y[e]);
        }
    }
}

// ---------------------------------------------------------------------------
// scores: grid (ceil(n / 64), ceil(nb / 64), B), 256 threads.
// ---------------------------------------------------------------------------
template <int D, bool kBf16>
__global__ __launch_bounds__(256) void qsa_score_kernel(const void* __restrict__ q, const void* __restrict__ kbar,
                                                        float* __restrict__ scores, int n, int H, int r, int nb,
                                                        long ldS) {
    constexpr int TQ = 64, TB = 64;
    constexpr int ES = kBf16 ? 2 : 4;                // element size
    constexpr int LD = D + (kBf16 ? 8 : 4);          // padded row, in elements
    const int qt = blockIdx.x, bt = blockIdx.y, b = blockIdx.z;
    const int i0 = qt * TQ, b0 = bt * TB;
    const int ilast = min(i0 + TQ, n) - 1;
    if (b0 >= (ilast + 1) / r) return;               // no complete block of this tile is visible
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;

    __shared__ __align__(16) unsigned char smem[(TQ + TB) * LD * ES];
    auto* sQ = smem;
    auto* sK = smem + TQ * LD * ES;

    // key tile (rows past nb are zero)
    constexpr int kVec = 16 / ES;                    // elements per 16-byte load
    for (int idx = tid; idx < TB * D / kVec; idx += 256) {
        const int rr = idx / (D / kVec), cc = idx - rr * (D / kVec);
        const int blk = b0 + rr;
        float4v v = {0.f, 0.f, 0.f, 0.f};
        if (blk < nb)
            v = *reinterpret_cast<const float4v*>(static_cast<const unsigned char*>(kbar) +
                                                  ((static_cast<long>(b) * nb + blk) * D + cc * kVec) * ES);
        *reinterpret_cast<float4v*>(sK + (rr * LD + cc * kVec) * ES) = v;
    }
    float4v tot[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) tot[t] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int h = 0; h < H; ++h) {
        if (h) __syncthreads();                      // previous head's reads are done
        for (int idx = tid; idx < TQ * D / kVec; idx += 256) {
            const int rr = idx / (D / kVec), cc = idx - rr * (D / kVec);
            const int i = i0 + rr;
            float4v v = {0.f, 0.f, 0.f, 0.f};
            if (i < n)
                v = *reinterpret_cast<const float4v*>(static_cast<const unsigned char*>(q) +
                                                      (((static_cast<long>(b) * n + i) * H + h) * D + cc * kVec) * ES);
            *reinterpret_cast<float4v*>(sQ + (rr * LD + cc * kVec) * ES) = v;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float4v acc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (kBf16) {
                const __bf16* A = reinterpret_cast<const __bf16*>(sQ) + (16 * wave + (l & 15)) * LD + 8 * (l >> 4);
                const __bf16* Bt = reinterpret_cast<const __bf16*>(sK) + (16 * t + (l & 15)) * LD + 8 * (l >> 4);
#pragma unroll
                for (int k = 0; k < D; k += 32)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(A + k),
                                                                  *reinterpret_cast<const bf16x8*>(Bt + k), acc, 0, 0, 0);
            } else {
                // split-K lanes: lane group l / 16 owns the run [(l/16) D/4, (l/16 + 1) D/4)
                const float* A = reinterpret_cast<const float*>(sQ) + (16 * wave + (l & 15)) * LD + (l >> 4) * (D / 4);
                const float* Bt = reinterpret_cast<const float*>(sK) + (16 * t + (l & 15)) * LD + (l >> 4) * (D / 4);
#pragma unroll
                for (int k = 0; k < D / 4; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[k], Bt[k], acc, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) tot[t][j] += fmaxf(acc[j], 0.f);
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int blk = b0 + 16 * t + (l & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = i0 + 16 * wave + 4 * (l >> 4) + j;
            if (i < n && blk < (i + 1) / r) scores[(static_cast<long>(b) * n + i) * ldS + blk] = tot[t][j];
        }
    }
}

// One wave per query row; four rows per workgroup (materialised scores, any
// number of query heads).
__global__ __launch_bounds__(256) void qsa_select_kernel(const float* __restrict__ scores, int* __restrict__ idx,
                                                         int n, int r, int KB, long ldS) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i = blockIdx.x * 4 + w, b = blockIdx.y;
    if (i >= n) return;                              // whole waves drop out
    const int m = (i + 1) / r;                       // complete blocks visible to query i
    int* out = idx + (static_cast<long>(b) * n + i) * KB;
    if (m <= KB) {                                   // every candidate is selected
        for (int j = lane; j < KB; j += 64) out[j] = j < m ? j : -1;
        return;
    }
    __shared__ unsigned shist[4][kBins];
    __shared__ unsigned sck[4][64];
    __shared__ int sci[4][64];
    select_row(scores + (static_cast<long>(b) * n + i) * ldS, m, KB, -1.f, out, shist[w], sck[w], sci[w]);
}

}  // namespace qsa

// Workspace: four query heads select without storing the scores (see
// qsa_topk.hip); other head counts store the fp32 scores, rows padded to 64
// blocks.
size_t qsa_select_workspace_bytes(int B, int n, int H, int r, int KB) {
    if (H == 4) return qsa_select4_workspace_bytes(B, n, r, KB);
    const long nb = n / r;
    const long ld = (nb + 63) / 64 * 64;
    return static_cast<size_t>(B) * n * ld * 4;
}

template <bool kBf16>
static hipError_t launch_qsa_prep_t(const QsaPrepArgs& a) {
    const long rows = static_cast<long>(a.B) * a.n * a.H + static_cast<long>(a.B) * (a.n / a.r);
    hipLaunchKernelGGL((qsa::qsa_prep_kernel<kBf16>), dim3(static_cast<unsigned>((rows + 4 * qsa::kPrepRows - 1) / (4 * qsa::kPrepRows))), dim3(256), 0,
                       a.stream, a.q_proj, a.k_proj, a.q_weight, a.k_weight, a.q_out, a.kbar_out, a.B, a.n, a.H, a.D,
                       a.r, a.rope_dims, std::log2(static_cast<double>(a.rope_base)), a.eps);
    return hipGetLastError();
}

hipError_t launch_qsa_prep(const QsaPrepArgs& a) {
    return a.bf16 ? launch_qsa_prep_t<true>(a) : launch_qsa_prep_t<false>(a);
}

template <int D, bool kBf16>
static hipError_t launch_qsa_select_t(const QsaSelectArgs& a) {
    const int nb = a.n / a.r;
    const long ld = (nb + 63) / 64 * 64;
    float* scores = static_cast<float*>(a.workspace);
    if (nb > 0)
        hipLaunchKernelGGL((qsa::qsa_score_kernel<D, kBf16>), dim3((a.n + 63) / 64, (nb + 63) / 64, a.B), dim3(256), 0,
                           a.stream, a.q, a.kbar, scores, a.n, a.H, a.r, nb, ld);
    hipLaunchKernelGGL(qsa::qsa_select_kernel, dim3((a.n + 3) / 4, a.B), dim3(256), 0, a.stream, scores, a.idx, a.n,
                       a.r, a.KB, ld);
    return hipGetLastError();
}

template <bool kBf16>
static hipError_t launch_qsa_select_dt(const QsaSelectArgs& a) {
    switch (a.D) {
        case 32: return launch_qsa_select_t<32, kBf16>(a);
        case 64: return launch_qsa_select_t<64, kBf16>(a);
        case 128: return launch_qsa_select_t<128, kBf16>(a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_qsa_select(const QsaSelectArgs& a) {
    if (a.H == 4) return launch_qsa_select4(a);
    return a.bf16 ? launch_qsa_select_dt<true>(a) : launch_qsa_select_dt<false>(a);
}

}  // namespace gdn
