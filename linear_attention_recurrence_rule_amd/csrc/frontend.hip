// Front end of the Gated DeltaNet mixer (slinene ai-papers-daily page on
// Qwen3.8-Next, Module A, parameterisation block; the mixer figure of the
// paper.rainbus.top digest): from the projected streams to the recurrence
// inputs,
//     q = L2Norm(SiLU(ShortConv(q_proj)))      k likewise
//     v = SiLU(ShortConv(v_proj))
//     beta = sigmoid(b_logit),  alpha = exp(-exp(A_h) softplus(a_logit + b_alpha_h))
// ShortConv is a causal depthwise convolution over time of width W (1..4),
// one filter per (head, channel), no bias; the W-1 rows before the first
// token come from the caller's history or are zero.  L2Norm divides by
// sqrt(sum(x^2) + eps) over the head dimension.
//
// One pass per stream (q, k, v), each a pure stream over its input and output
// (HBM-bound); with d_k = d_v the three passes run as one launch.  A row group of lanes owns one (sequence, head) and a run of
// kRun consecutive tokens; each lane owns 16 bytes of a row (8 bf16 or 4
// fp32 channels), keeps its filter
// taps and the last W-1 input rows in registers and slides along the run
// kStep tokens at a time (their norms reduce together), loading the next
// step's rows while the current ones are processed.  The L2 norm is a
// DPP / swizzle reduction inside the row group.  Row groups of a wave
// take consecutive heads, so a wave's loads and stores cover adjacent rows.
// The v pass also writes alpha and beta (one lane per row group).
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace frontend {

constexpr int kRun = 32;   // tokens per row group
constexpr int kStep = 4;   // tokens processed together (kRun is a multiple)

// Each lane moves 16 bytes of a row: 8 bf16 or 4 fp32 channels.
template <bool kBf16>
struct Lane {
    static constexpr int N = kBf16 ? 8 : 4;
    typedef float Vec __attribute__((ext_vector_type(N)));
};

// A lane's 16 bytes as loaded, and converted to floats.  Prefetched rows stay
// raw until the step that uses them, so that the conversion does not wait
// for a load just issued.
template <bool kBf16>
using Raw = typename std::conditional<kBf16, uint4, float4v>::type;
template <bool kBf16>
__device__ __forceinline__ Raw<kBf16> loadr(const void* p, long i) {
    if constexpr (kBf16) return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    else return *reinterpret_cast<const float4v*>(static_cast<const float*>(p) + i);
}
template <bool kBf16>
__device__ __forceinline__ typename Lane<kBf16>::Vec cvt(const Raw<kBf16>& r) {
    if constexpr (kBf16) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
        typename Lane<kBf16>::Vec v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(w[e] << 16);
            v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
        return v;
    } else {
        return r;
    }
}
template <bool kBf16>
__device__ __forceinline__ typename Lane<kBf16>::Vec loadv(const void* p, long i) {
    return cvt<kBf16>(loadr<kBf16>(p, i));
}

template <bool kBf16>
__device__ __forceinline__ void storev(void* p, long i, typename Lane<kBf16>::Vec x) {
    if constexpr (kBf16) {
        uint4 r;
        r.x = pack_bf16x2(x[0], x[1]);
        r.y = pack_bf16x2(x[2], x[3]);
        r.z = pack_bf16x2(x[4], x[5]);
        r.w = pack_bf16x2(x[6], x[7]);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + i) = r;
    } else {
        *reinterpret_cast<float4v*>(static_cast<float*>(p) + i) = x;
    }
}

// hardware reciprocal (about 1 ulp): the outputs are rounded to bf16 or
// compared at float32 tolerance, and x -> -inf still gives x * 0 = -0
__device__ __forceinline__ float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float silu(float x) { return x * sigmoid(x); }
__device__ __forceinline__ float softplus(float x) { return x > 20.f ? x : log1pf(__expf(x)); }

// Sum over aligned groups of N lanes (N a power of two up to 32), every lane
// getting the group's total: DPP quad permutations and row mirrors inside a
// row of 16, then a 32-lane swizzle that swaps the two rows.
template <int N>
__device__ __forceinline__ float row_sum(float x) {
    auto dpp = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
    };
    if constexpr (N > 1) x += dpp(x, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
    if constexpr (N > 2) x += dpp(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
    if constexpr (N > 4) x += dpp(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
    if constexpr (N > 8) x += dpp(x, std::integral_constant<int, 0x140>{});   // row_mirror
    if constexpr (N > 16) x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));   // lane ^ 16
    return x;
}

// One block of a stream pass: row groups blk * RPB .. of the stream.
template <int D, int W, bool kNorm, bool kGates, bool kBf16>
__device__ __forceinline__ void stream_block(const void* __restrict__ x, const float* __restrict__ w,
                                             const void* __restrict__ hist, void* __restrict__ out,
                                             const float* __restrict__ a_logit, const float* __restrict__ b_logit,
                                             const float* __restrict__ A, const float* __restrict__ b_alpha,
                                             float* __restrict__ alpha, float* __restrict__ beta, int B, int T, int H,
                                             float eps, long blk) {
    using Vec = typename Lane<kBf16>::Vec;
    constexpr int NC = Lane<kBf16>::N;      // channels per lane
    constexpr int LPR = D / NC;             // lanes per row
    constexpr int RPB = 256 / LPR;          // row groups per block
    const int tid = threadIdx.x;
    const int sub = tid % LPR;
    const long task = blk * RPB + tid / LPR;
    const int nruns = (T + kRun - 1) / kRun;
    const int h = static_cast<int>(task % H);
    const long rest = task / H;
    const int run = static_cast<int>(rest % nruns);
    const int b = static_cast<int>(rest / nruns);
    if (b >= B) return;                      // whole row groups drop out together
    const int t0 = run * kRun, t1 = min(t0 + kRun, T);
    const long row_stride = static_cast<long>(H) * D;
    const long base = (static_cast<long>(b) * T * H + h) * D + NC * sub;   // element (b, t = 0, h, NC sub)

    // filter taps of this lane's channels: wt[j][c] = w[h][NC sub + c][j]
    Vec wt[W];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < W; ++j) wt[j][c] = w[(static_cast<long>(h) * D + NC * sub + c) * W + j];

    // kStep tokens per step, independent of each other given the inputs, so
    // their reductions overlap; the next step's rows are loaded meanwhile.
    // Offsets inside the run are 32-bit (a run spans kRun rows).
    const int last = t1 - 1 - t0;
    const int rs = static_cast<int>(row_stride);
    const long run_base = base + t0 * row_stride;
    using R = Raw<kBf16>;
    auto load_rows = [&](R (&r)[kStep], int r0) {
#pragma unroll
        for (int u = 0; u < kStep; ++u) r[u] = loadr<kBf16>(x, run_base + min(r0 + u, last) * rs);
    };
    // the run's first rows go out first, ahead of the window rows
    R ra[kStep], rb[kStep];
    load_rows(ra, 0);

    // the W-1 rows before t0: from the sequence, the caller's history, or
    // zero.  Both loads are issued with clamped indices and the choice made
    // afterwards, so that the loads overlap instead of each waiting in a branch.
    Vec win[W > 1 ? W - 1 : 1];
    {
        Raw<kBf16> rx[W > 1 ? W - 1 : 1], rh[W > 1 ? W - 1 : 1];
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int t = t0 - (W - 1) + j;
            rx[j] = loadr<kBf16>(x, base + (t >= 0 ? t : 0) * row_stride);
            if (hist) {
                const int slot = t < 0 ? W - 1 + t : 0;
                rh[j] = loadr<kBf16>(hist, ((static_cast<long>(b) * (W - 1) + slot) * H + h) * D + NC * sub);
            }
        }
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int t = t0 - (W - 1) + j;
            win[j] = t >= 0 ? cvt<kBf16>(rx[j]) : (hist ? cvt<kBf16>(rh[j]) : Vec{});
        }
    }

    // the gate logits of the run, one token per lane (several when the row
    // group has fewer lanes than the run has tokens), loaded up front
    constexpr int kGPer = kGates ? (kRun + LPR - 1) / LPR : 1;
    float al[kGPer], bl[kGPer];
    if constexpr (kGates) {
#pragma unroll
        for (int u = 0; u < kGPer; ++u) {
            const int t = min(t0 + sub + u * LPR, t1 - 1);
            const long g = (static_cast<long>(b) * T + t) * H + h;
            al[u] = a_logit[g];
            bl[u] = b_logit[g];
        }
    }

    // every step loads the next one's rows (clamped to the run's last row, so
    // the loads are unconditional and the wait counts exact)
    auto step = [&](const R (&cur_raw)[kStep], R (&nxt)[kStep], int r0) {
        load_rows(nxt, r0 + kStep);
        Vec cur[kStep];
#pragma unroll
        for (int u = 0; u < kStep; ++u) cur[u] = cvt<kBf16>(cur_raw[u]);
        Vec s[kStep];
#pragma unroll
        for (int u = 0; u < kStep; ++u) {
            // conv over rows r0+u-(W-1) .. r0+u: the window holds the W-1 rows
            // before r0, cur the rows r0 .. r0+kStep-1
            Vec c = wt[W - 1] * cur[u];
#pragma unroll
            for (int j = 0; j < W - 1; ++j) {
                const int src = u - (W - 1) + j;   // row r0 + src
                c += wt[j] * (src >= 0 ? cur[src >= 0 ? src : 0] : win[(W - 1) + src >= 0 ? (W - 1) + src : 0]);
            }
#pragma unroll
            for (int e = 0; e < NC; ++e) s[u][e] = silu(c[e]);
        }
        if constexpr (kNorm) {
            float ss[kStep];
#pragma unroll
            for (int u = 0; u < kStep; ++u) {
                ss[u] = 0.f;
#pragma unroll
                for (int e = 0; e < NC; ++e) ss[u] += s[u][e] * s[u][e];
            }
#pragma unroll
            for (int u = 0; u < kStep; ++u) ss[u] = row_sum<LPR>(ss[u]);
#pragma unroll
            for (int u = 0; u < kStep; ++u) s[u] *= __builtin_amdgcn_rsqf(ss[u] + eps);
        }
#pragma unroll
        for (int u = 0; u < kStep; ++u)
            if (r0 + u <= last) storev<kBf16>(out, run_base + (r0 + u) * rs, s[u]);
        // the window moves to the last W-1 rows of this step
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int src = kStep - (W - 1) + j;   // row r0 + src
            win[j] = src >= 0 ? cur[src >= 0 ? src : 0] : win[j + kStep < W - 1 ? j + kStep : 0];
        }
    };
    // the run's steps unrolled over two register sets, so that no copies are
    // needed (steps past a short run's last row compute on clamped rows and
    // store nothing)
#pragma unroll
    for (int k = 0; k < kRun / kStep; ++k) {
        if (k % 2 == 0) step(ra, rb, k * kStep);
        else step(rb, ra, k * kStep);
    }
    if constexpr (kGates) {
        const float ea = __expf(A[h]), ba = b_alpha[h];
#pragma unroll
        for (int u = 0; u < kGPer; ++u) {
            const int t = t0 + sub + u * LPR;
            if (t < t1) {
                const long g = (static_cast<long>(b) * T + t) * H + h;
                beta[g] = sigmoid(bl[u]);
                alpha[g] = __expf(-ea * softplus(al[u] + ba));
            }
        }
    }
}

template <int D, int W, bool kNorm, bool kGates, bool kBf16>
__global__ __launch_bounds__(256) void stream_kernel(const void* __restrict__ x, const float* __restrict__ w,
                                                     const void* __restrict__ hist, void* __restrict__ out,
                                                     const float* __restrict__ a_logit,
                                                     const float* __restrict__ b_logit,
                                                     const float* __restrict__ A, const float* __restrict__ b_alpha,
                                                     float* __restrict__ alpha, float* __restrict__ beta, int B,
                                                     int T, int H, float eps) {
    stream_block<D, W, kNorm, kGates, kBf16>(x, w, hist, out, a_logit, b_logit, A, b_alpha, alpha, beta, B, T, H,
                                             eps, blockIdx.x);
}

// All three passes in one launch when d_k = d_v: blocks [0, nb) are q's,
// [nb, 2 nb) k's and [2 nb, 3 nb) v's, so the passes share one grid and
// one tail instead of three.
template <int D, int W, bool kBf16>
__global__ __launch_bounds__(256) void qkv_kernel(const FrontendArgs a, long nb) {
    const long bx = blockIdx.x;
    if (bx < 2 * nb) {                               // block-uniform
        const bool isq = bx < nb;
        stream_block<D, W, true, false, kBf16>(isq ? a.q_proj : a.k_proj, isq ? a.conv_q : a.conv_k,
                                               isq ? a.q_hist : a.k_hist, isq ? a.q : a.k, nullptr, nullptr,
                                               nullptr, nullptr, nullptr, nullptr, a.B, a.T, a.H, a.eps,
                                               isq ? bx : bx - nb);
    } else {
        stream_block<D, W, false, true, kBf16>(a.v_proj, a.conv_v, a.v_hist, a.v, a.a_logit, a.b_logit, a.A,
                                               a.b_alpha, a.alpha, a.beta, a.B, a.T, a.H, a.eps, bx - 2 * nb);
    }
}

template <int D>
static long blocks_of(const FrontendArgs& a, int nc) {
    const long tasks = static_cast<long>(a.B) * a.H * ((a.T + kRun - 1) / kRun);
    const int rpb = 256 / (D / nc);
    return (tasks + rpb - 1) / rpb;
}

template <int D, int W, bool kBf16>
static hipError_t launch_qkv(const FrontendArgs& a) {
    const long nb = blocks_of<D>(a, Lane<kBf16>::N);
    hipLaunchKernelGGL((qkv_kernel<D, W, kBf16>), dim3(static_cast<unsigned>(3 * nb)), dim3(256), 0, a.stream, a, nb);
    return hipGetLastError();
}

template <int D, int W, bool kNorm, bool kGates, bool kBf16>
static hipError_t launch_stream(const void* x, const float* w, const void* hist, void* out, const FrontendArgs& a) {
    const long blocks = blocks_of<D>(a, Lane<kBf16>::N);
    hipLaunchKernelGGL((stream_kernel<D, W, kNorm, kGates, kBf16>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, a.stream, x, w, hist, out, a.a_logit, a.b_logit, a.A, a.b_alpha, a.alpha, a.beta, a.B, a.T,
                       a.H, a.eps);
    return hipGetLastError();
}

template <int W, bool kNorm, bool kGates, bool kBf16>
static hipError_t launch_d(int d, const void* x, const float* w, const void* hist, void* out, const FrontendArgs& a) {
    switch (d) {
        case 16: return launch_stream<16, W, kNorm, kGates, kBf16>(x, w, hist, out, a);
        case 32: return launch_stream<32, W, kNorm, kGates, kBf16>(x, w, hist, out, a);
        case 64: return launch_stream<64, W, kNorm, kGates, kBf16>(x, w, hist, out, a);
        case 128: return launch_stream<128, W, kNorm, kGates, kBf16>(x, w, hist, out, a);
        default: return hipErrorInvalidValue;
    }
}

template <int W, bool kBf16>
static hipError_t launch_all(const FrontendArgs& a) {
    if (a.dk == a.dv) {
        switch (a.dk) {
            case 16: return launch_qkv<16, W, kBf16>(a);
            case 32: return launch_qkv<32, W, kBf16>(a);
            case 64: return launch_qkv<64, W, kBf16>(a);
            case 128: return launch_qkv<128, W, kBf16>(a);
            default: return hipErrorInvalidValue;
        }
    }
    hipError_t e = launch_d<W, true, false, kBf16>(a.dk, a.q_proj, a.conv_q, a.q_hist, a.q, a);
    if (e != hipSuccess) return e;
    e = launch_d<W, true, false, kBf16>(a.dk, a.k_proj, a.conv_k, a.k_hist, a.k, a);
    if (e != hipSuccess) return e;
    return launch_d<W, false, true, kBf16>(a.dv, a.v_proj, a.conv_v, a.v_hist, a.v, a);
}

template <bool kBf16>
static hipError_t launch_w(const FrontendArgs& a) {
    switch (a.width) {
        case 1: return launch_all<1, kBf16>(a);
        case 2: return launch_all<2, kBf16>(a);
        case 3: return launch_all<3, kBf16>(a);
        case 4: return launch_all<4, kBf16>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace frontend

hipError_t launch_frontend(const FrontendArgs& a) {
    if (a.T == 0) return hipSuccess;
    return a.bf16 ? frontend::launch_w<true>(a) : frontend::launch_w<false>(a);
}

}  // namespace gdn
