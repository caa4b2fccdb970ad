// Chunked backward of the gated delta rule on gfx950.
//
// The forward is the delta form of the slinene ai-papers-daily page on
// "On the Design of Qwen3.8-Next Architecture" (Module A), evaluated in
// chunks of C = 64 tokens (UT form):
//     g = in-chunk cumsum of log alpha,  gamma = exp(g),  lam_t = exp(g_n - g_t)
//     T = (I + A)^-1,  A_ti = beta_t Gamma_ti k_t.k_i (i < t) = beta_t M_ti
//     E = T diag(beta) (V - diag(gamma) K S)
//     Y = scale (diag(gamma) Q S + P E),  P_ti = Gamma_ti q_t.k_i (i <= t)
//     S' = gamma_n S + K^T diag(lam) E
// The backward applies the chain rule to these chunk equations in four
// passes (the pages only mention a backward kernel as part of the FlashQLA
// library; this is the plain reverse-mode derivation):
//   1. prep (chunk-parallel): g, T, P and M per chunk.
//   2. states (sequential over chunks, per 16-column slice of the state):
//      the chunk-start states S_c and the chunk products E_c.
//   3. reverse states (sequential, reverse order, per slice): the gradient of
//      each chunk's end state dS'_c, and with it
//          dE = scale P^T dY + diag(lam) K dS',   dR = T^T dE,   dV = diag(beta) dR
//          dS = gamma_n dS' + scale Q^T diag(gamma) dY - K^T diag(beta gamma) dR
//   4. gradients (chunk-parallel): with X1 = dY S^T, X2 = dR S^T, X3 = E dS'^T,
//      X4 = dY E^T, X5 = dR E^T,  dP = scale X4 (i <= t),  dA = -X5 (i < t):
//          dq = scale gamma X1 + (dP o Gamma) K
//          dk = lam X3 - beta gamma X2 + (Dm + Dm^T) K + (dP o Gamma)^T Q,
//               Dm_ti = beta_t dA_ti Gamma_ti
//          dbeta_t = dR_t.v_t - gamma_t k_t.X2_t + sum_i dA_ti M_ti
//          dg_t = gamma_t (scale q_t.X1_t - beta_t k_t.X2_t) + rows/cols of dP o P
//                 and dA o A - lam_t k_t.X3_t  (+ the chunk-end terms at t = n)
//          dalpha_s = (sum_{t >= s} dg_t) / alpha_s.
// Every contraction is an fp32 MFMA (16x16x4) on LDS tiles, except the
// prep pass's Gram tiles of bf16 inputs, which are bf16 MFMAs (exact products,
// fp32 sums) on fragments loaded straight from HBM; the workspace holds the
// per-chunk matrices and states in fp32.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace bwd {

constexpr int C = 64;
constexpr float kLogFloor = -30.f;   // same floor of log(alpha) as the forward

// acc += A B for one 16x16 tile over k in [k0, k0 + N), fp32 MFMA 16x16x4.
//   kAt = false: A row-major (A[r][k] at A[r * lda + k], A at the tile's first row)
//   kAt = true:  A stored transposed (A[r][k] at A[k * lda + r], A at the tile's first row index)
//   kBr = false: B given transposed (B[k][n] at B[n * ldb + k], B at the tile's first column)
//   kBr = true:  B row-major (B[k][n] at B[k * ldb + n], B at the tile's first column)
// so a tile stored row-major serves both as an operand and as its transpose.
// Split-K lane layout: lane group l / 16 owns the contiguous run
// [k0 + (l/16) N/4, ... + N/4) and step s takes element s of every run (the
// four partial sums of one MFMA cover different k, and their total is the
// same contraction).  All operand values are read from LDS before the first
// MFMA, so the dependent MFMA chain never waits on LDS latency; row-major
// runs are read as float4.
template <bool kAt, bool kBr, int N>
__device__ __forceinline__ float4v mma_n(const float* A, int lda, const float* B, int ldb, int k0, float4v acc) {
    constexpr int S = N / 4;
    static_assert(S % 4 == 0, "contraction length must be a multiple of 16");
    const int l = threadIdx.x & 63, r = l & 15, kb = k0 + (l >> 4) * S;
    float a[S], b[S];
#pragma unroll
    for (int s = 0; s < S; s += 4) {
        if constexpr (kAt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) a[s + e] = A[(kb + s + e) * lda + r];
        } else {
            const float4v x = *reinterpret_cast<const float4v*>(&A[r * lda + kb + s]);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[s + e] = x[e];
        }
        if constexpr (kBr) {
#pragma unroll
            for (int e = 0; e < 4; ++e) b[s + e] = B[(kb + s + e) * ldb + r];
        } else {
            const float4v x = *reinterpret_cast<const float4v*>(&B[r * ldb + kb + s]);
#pragma unroll
            for (int e = 0; e < 4; ++e) b[s + e] = x[e];
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    return acc;
}
// acc += (A + A^T) B over k in [k0, k0 + N): A row-major and square (leading
// dimension lda), rows r0 .. r0 + 15 of the sum; B row-major at the tile's
// first column.  Split-K lane layout of mma_n, operands read first.
template <int N>
__device__ __forceinline__ float4v mma_sym_n(const float* A, int lda, int r0, const float* B, int ldb, int k0,
                                             float4v acc) {
    constexpr int S = N / 4;
    const int l = threadIdx.x & 63, r = r0 + (l & 15), kb = k0 + (l >> 4) * S;
    float a[S], b[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        a[s] = A[r * lda + kb + s] + A[(kb + s) * lda + r];
        b[s] = B[(kb + s) * ldb + (l & 15)];
    }
#pragma unroll
    for (int s = 0; s < S; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    return acc;
}

// The same contractions on fp16 MFMAs, for bf16 inputs: each lane reads the
// operand values of mma_n's split-K layout from the fp32 LDS tiles, rounds
// them to fp16, and feeds eight at a time to 16x16x32 MFMAs (a remainder of
// four padded with zeros); the k grouping differs from mma_n's but is the
// same for both operands, so the sum is the same contraction, with fp32
// accumulation.  One MFMA then covers 32 values of k instead of 4.  Only the
// 16x16x32 shape touches these accumulators: on gfx950 a 16x16x16 f16 MFMA
// that reads an accumulator just written by a 16x16x32 one has given wrong
// sums.
template <int N>
__device__ __forceinline__ float4v mma_h8(const float* a, const float* b, float4v acc) {
    half8 x = {}, y = {};
#pragma unroll
    for (int e = 0; e < N; ++e) {
        x[e] = static_cast<_Float16>(a[e]);
        y[e] = static_cast<_Float16>(b[e]);
    }
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, acc, 0, 0, 0);
}
template <int S>
__device__ __forceinline__ float4v mma_h_run(const float (&a)[S], const float (&b)[S], float4v acc) {
#pragma unroll
    for (int s = 0; s + 8 <= S; s += 8) acc = mma_h8<8>(a + s, b + s, acc);
    if constexpr (S % 8 == 4) acc = mma_h8<4>(a + S - 4, b + S - 4, acc);
    return acc;
}
template <bool kAt, bool kBr, int N>
__device__ __forceinline__ float4v mma_n_h(const float* A, int lda, const float* B, int ldb, int k0, float4v acc) {
    constexpr int S = N / 4;
    const int l = threadIdx.x & 63, r = l & 15, kb = k0 + (l >> 4) * S;
    float a[S], b[S];
#pragma unroll
    for (int s = 0; s < S; s += 4) {
        if constexpr (kAt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) a[s + e] = A[(kb + s + e) * lda + r];
        } else {
            const float4v x = *reinterpret_cast<const float4v*>(&A[r * lda + kb + s]);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[s + e] = x[e];
        }
        if constexpr (kBr) {
#pragma unroll
            for (int e = 0; e < 4; ++e) b[s + e] = B[(kb + s + e) * ldb + r];
        } else {
            const float4v x = *reinterpret_cast<const float4v*>(&B[r * ldb + kb + s]);
#pragma unroll
            for (int e = 0; e < 4; ++e) b[s + e] = x[e];
        }
    }
    return mma_h_run<S>(a, b, acc);
}
template <int N>
__device__ __forceinline__ float4v mma_sym_n_h(const float* A, int lda, int r0, const float* B, int ldb, int k0,
                                               float4v acc) {
    constexpr int S = N / 4;
    const int l = threadIdx.x & 63, r = r0 + (l & 15), kb = k0 + (l >> 4) * S;
    float a[S], b[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        a[s] = A[r * lda + kb + s] + A[(kb + s) * lda + r];
        b[s] = B[(kb + s) * ldb + (l & 15)];
    }
    return mma_h_run<S>(a, b, acc);
}
// Contraction in the precision of the inputs: fp16 operands for bf16 inputs,
// fp32 for fp32 inputs.
template <bool kHalf, bool kAt, bool kBr, int N>
__device__ __forceinline__ float4v mma_x(const float* A, int lda, const float* B, int ldb, int k0, float4v acc) {
    if constexpr (kHalf) return mma_n_h<kAt, kBr, N>(A, lda, B, ldb, k0, acc);
    else return mma_n<kAt, kBr, N>(A, lda, B, ldb, k0, acc);
}
template <bool kHalf, int N>
__device__ __forceinline__ float4v mma_sym_x(const float* A, int lda, int r0, const float* B, int ldb, int k0,
                                             float4v acc) {
    if constexpr (kHalf) return mma_sym_n_h<N>(A, lda, r0, B, ldb, k0, acc);
    else return mma_sym_n<N>(A, lda, r0, B, ldb, k0, acc);
}

// acc += A B^T over the 32 values of k of two fp16 tiles held row-major in
// LDS (16 rows each, k along the row, leading dimension ld): lane group g
// takes k = 8 g .. 8 g + 7 of both operands, one 16-byte read each.
__device__ __forceinline__ half8 frag_h(const _Float16* A, int ld) {
    const int l = threadIdx.x & 63;
    return *reinterpret_cast<const half8*>(A + (l & 15) * ld + 8 * (l >> 4));
}
__device__ __forceinline__ float4v mma_hh(half8 a, half8 b, float4v acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ half4 to_h4(float4v x) {
    return half4{static_cast<_Float16>(x[0]), static_cast<_Float16>(x[1]), static_cast<_Float16>(x[2]),
                 static_cast<_Float16>(x[3])};
}

__device__ __forceinline__ float dpp_sum4(float x) {          // sum over a quad
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));
    return x;
}
// Inclusive prefix sum over the 64 lanes with DPP moves: shifts by 1, 2, 4
// and 8 within each row of 16 lanes (zeros shifted in), then the last lane of
// rows 0 and 2 added into rows 1 and 3, then lane 31 into rows 2 and 3.
template <int kCtrl, int kRowMask, bool kZeroFill>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xf, kZeroFill));
}
__device__ __forceinline__ float dpp_scan64(float v) {
    v += dpp_move<0x111, 0xf, true>(v);
    v += dpp_move<0x112, 0xf, true>(v);
    v += dpp_move<0x114, 0xf, true>(v);
    v += dpp_move<0x118, 0xf, true>(v);
    v += dpp_move<0x142, 0xa, false>(v);
    v += dpp_move<0x143, 0xc, false>(v);
    return v;
}
// bf16 MFMA on fragments (exact products, fp32 sums): 16x16x32 on 8-element
// fragments, 16x16x16 on 4-element ones.
__device__ __forceinline__ float4v mma_bf16(uint4 a, uint4 b, float4v c) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ float4v mma_bf16(uint2 a, uint2 b, float4v c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                    0, 0, 0);
}
__device__ __forceinline__ float dpp_sum8(float x) {          // sum over 8 consecutive lanes
    x = dpp_sum4(x);
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_sum16(float x) {         // sum over a row of 16 lanes
    x = dpp_sum8(x);
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false));
}

// The sequential walks run one workgroup per (head, 16-column slice).  All
// slices of a head read the same chunk tiles, so they are placed on the same
// XCD (consecutive workgroup ids go to the 8 XCDs in turn) to share its L2:
// block L -> XCD L % 8, and XCD x walks the heads x, x + 8, ...  gridDim.x is
// kSlices * 8 * ceil(BH / 8); ids past the last head return at once.
template <int kSlices>
__device__ __forceinline__ bool slice_of_block(int BH, int& slice, int& bh) {
    const int L = blockIdx.x, xcd = L & 7, r = L >> 3;
    slice = r % kSlices;
    bh = (r / kSlices) * 8 + xcd;
    return bh < BH;
}

// Four consecutive input elements as loaded (bf16: 8 bytes, fp32: 16 bytes).
template <bool kBf16> struct Raw4Of { typedef float4v type; };
template <> struct Raw4Of<true> { typedef uint2 type; };
template <bool kBf16> using Raw4 = typename Raw4Of<kBf16>::type;

template <bool kBf16>
__device__ __forceinline__ Raw4<kBf16> raw_load(const void* p, long i) {
    if constexpr (kBf16) return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    else return *reinterpret_cast<const float4v*>(static_cast<const float*>(p) + i);
}
template <bool kBf16>
__device__ __forceinline__ float4v raw_cvt(Raw4<kBf16> u) {
    if constexpr (kBf16)
        return float4v{bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xffffu),
                       bf16_to_f32(u.y >> 16)};
    else return u;
}
template <bool kBf16>
__device__ __forceinline__ float4v load4(const void* p, long i) { return raw_cvt<kBf16>(raw_load<kBf16>(p, i)); }

// The C x D rows of chunk c of a [B, T, H, D] input (head h), held in
// registers between an early load and a later store into a row-major LDS
// tile.  Every load is unconditional (clamped rows), so that a prefetch of
// the next chunk never makes the compiler wait inside the current one.
template <int D, int NT, bool kBf16>
struct RowTile {
    static constexpr int kItems = C * D / 4;
    static constexpr int kPer = (kItems + NT - 1) / NT;
    Raw4<kBf16> r[kPer];
    __device__ __forceinline__ void load(const void* p, int b, int c, int T, int H, int h) {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            int i = threadIdx.x + NT * m;
            i = i < kItems ? i : kItems - 1;
            const int t = i / (D / 4), c4 = i - t * (D / 4);
            const int tg = c * C + t, tc = tg < T ? tg : T - 1;
            r[m] = raw_load<kBf16>(p, ((static_cast<long>(b) * T + tc) * H + h) * D + 4 * c4);
        }
    }
    __device__ __forceinline__ void store(float* s, int ld, int c, int T) const {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int i = threadIdx.x + NT * m;
            if (i < kItems) {
                const int t = i / (D / 4), c4 = i - t * (D / 4);
                const float4v x = c * C + t < T ? raw_cvt<kBf16>(r[m]) : float4v{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<float4v*>(&s[t * ld + 4 * c4]) = x;
            }
        }
    }
    // The transpose as fp16, [d][token] with leading dimension ld.  Rows
    // past T (clamped copies of the last row, so finite) are zeroed by a
    // factor rather than a select, which the compiler may turn into a branch
    // with the prefetched load sunk into it.
    __device__ __forceinline__ void store_t(_Float16* s, int ld, int c, int T) const {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int i = threadIdx.x + NT * m;
            // (no run-time check where the items divide evenly: a branch here
            // would also take the prefetched load into it)
            if (kItems % NT == 0 || i < kItems) {
                const int t = i / (D / 4), c4 = i - t * (D / 4);
                const float live = c * C + t < T ? 1.f : 0.f;
                const float4v x = raw_cvt<kBf16>(r[m]) * live;
#pragma unroll
                for (int e = 0; e < 4; ++e) s[(4 * c4 + e) * ld + t] = static_cast<_Float16>(x[e]);
            }
        }
    }
};

// A C x C float32 chunk matrix of the workspace, register-staged the same way.
template <int NT>
struct MatTile {
    static constexpr int kPer = C * C / 4 / NT;
    float4v r[kPer];
    __device__ __forceinline__ void load(const float* g) {
#pragma unroll
        for (int m = 0; m < kPer; ++m) r[m] = reinterpret_cast<const float4v*>(g)[threadIdx.x + NT * m];
    }
    __device__ __forceinline__ void store(float* s, int ld) const {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int i = threadIdx.x + NT * m, t = i / (C / 4), c4 = i - t * (C / 4);
            *reinterpret_cast<float4v*>(&s[t * ld + 4 * c4]) = r[m];
        }
    }
};

// ---------------------------------------------------------------------------
// Pass 1: gates, T, P and M of one chunk.  grid (nch, B*H), 256 threads.
// ---------------------------------------------------------------------------
template <int DK, bool kBf16>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                       const float* __restrict__ alpha,
                                                       const float* __restrict__ beta, float* __restrict__ ws_g,
                                                       float* __restrict__ ws_T, float* __restrict__ ws_P,
                                                       float* __restrict__ ws_M, int T, int H, int nch) {
    constexpr int LDK = DK + 4, LDA = C + 4, LDT = C + 4;
    // bf16 inputs go straight from HBM into MFMA fragments, so LDS holds only A and T
    constexpr int kQA = !kBf16 && C * LDK > C * LDA ? C * LDK : C * LDA;
    constexpr int kKT = !kBf16 && C * LDK > C * LDT + 4 * 256 ? C * LDK : C * LDT + 4 * 256;   // K, later T + 4 tiles
    const int c = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh - b * H;
    const long bhn = static_cast<long>(bh) * nch + c;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;

    __shared__ __align__(16) float sK[kKT];
    __shared__ __align__(16) float sQA[kQA];          // Q, then A = diag(beta) M
    __shared__ float sg[C], sb[C];

    // bf16: lane (r + 16 g) of fragment [I][s] holds row 16 I + r, columns
    // 32 s + 8 g .. + 8 (4-column fragments at d_k = 16); rows past T are zero.
    using Frag = typename std::conditional<(DK >= 32), uint4, uint2>::type;
    constexpr int KS = DK >= 32 ? DK / 32 : 1, FW = DK >= 32 ? 8 : 4;
    // (wave w's own block, the A operand of its four tiles, is loaded apart so
    // that no fragment array is indexed by the wave number)
    Frag kf[kBf16 ? 4 : 1][KS], ka[KS], qf[KS];
    if constexpr (kBf16) {
        const int lr = l & 15, lg = l >> 4;
        auto at = [&](int I) {
            const int tg = c * C + 16 * I + lr;
            return ((static_cast<long>(b) * T + (tg < T ? tg : T - 1)) * H + h) * DK + FW * lg;
        };
        auto live = [&](int I) { return c * C + 16 * I + lr < T; };
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const Frag kv = *reinterpret_cast<const Frag*>(static_cast<const uint16_t*>(k) + at(I) + 32 * st);
                kf[I][st] = live(I) ? kv : Frag{};
            }
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const Frag kv = *reinterpret_cast<const Frag*>(static_cast<const uint16_t*>(k) + at(wave) + 32 * st);
            const Frag qv = *reinterpret_cast<const Frag*>(static_cast<const uint16_t*>(q) + at(wave) + 32 * st);
            ka[st] = live(wave) ? kv : Frag{};
            qf[st] = live(wave) ? qv : Frag{};
        }
    } else {
        RowTile<DK, 256, kBf16> tq, tk;
        tq.load(q, b, c, T, H, h);
        tk.load(k, b, c, T, H, h);
        tq.store(sQA, LDK, c, T);
        tk.store(sK, LDK, c, T);
    }
    if (wave == 0) {
        const int tg = c * C + l;
        const long gi = (static_cast<long>(b) * T + (tg < T ? tg : T - 1)) * H + h;
        const float a = alpha[gi], be = beta[gi];
        const float x = dpp_scan64(tg < T ? fmaxf(__logf(a), kLogFloor) : 0.f);   // prefix sum over the chunk
        sg[l] = x;
        sb[l] = tg < T ? be : 0.f;
        ws_g[bhn * C + l] = x;
    }
    __syncthreads();

    // Gram tiles: 16 of K K^T and 16 of Q K^T; the ones above the diagonal are zero
    float4v kk[4], qk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int p = wave * 4 + u, ti = p >> 2, tj = p & 3;
        kk[u] = qk[u] = float4v{0.f, 0.f, 0.f, 0.f};
        if (tj <= ti) {
            if constexpr (kBf16) {
#pragma unroll
                for (int st = 0; st < KS; ++st) {
                    kk[u] = mma_bf16(ka[st], kf[u][st], kk[u]);
                    qk[u] = mma_bf16(qf[st], kf[u][st], qk[u]);
                }
            } else {
                kk[u] = mma_x<kBf16, false, false, DK>(&sK[16 * ti * LDK], LDK, &sK[16 * tj * LDK], LDK, 0, kk[u]);
                qk[u] = mma_x<kBf16, false, false, DK>(&sQA[16 * ti * LDK], LDK, &sK[16 * tj * LDK], LDK, 0, qk[u]);
            }
        }
    }
    __syncthreads();                                   // Q is no longer read: its space takes A
    float* gP = ws_P + bhn * C * C;
    float* gM = ws_M + bhn * C * C;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int p = wave * 4 + u, ti = p >> 2, tj = p & 3;
        const int col = 16 * tj + (l & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * ti + 4 * (l >> 4) + j;
            const float gam = row >= col ? __expf(sg[row] - sg[col]) : 0.f;
            const float m = row > col ? gam * kk[u][j] : 0.f;
            const float pv = row >= col ? gam * qk[u][j] : 0.f;
            gM[row * C + col] = m;
            gP[row * C + col] = pv;
            // bf16 inputs, d >= 64: the reverse walk reads fp16 P from the
            // second half of the chunk's T slot
            if constexpr (kBf16 && DK >= 64) reinterpret_cast<_Float16*>(ws_T + bhn * C * C)[C * C + row * C + col] = pv;
            sQA[row * LDA + col] = sb[row] * m;
        }
    }
    __syncthreads();

    // T = (I + A)^-1 in 16x16 blocks, assembled in sK (K is no longer read):
    // wave w inverts diagonal block w by forward substitution (a quad of lanes
    // per column, lane & 3 holding the rows i = part (mod 4)), then one block
    // sub-diagonal per step on MFMA,
    //     T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ,
    // whose terms all lie on earlier sub-diagonals.
    float* sT = sK;
    float* sY = sK + C * LDT + 256 * wave;             // this wave's 16x16 scratch tile
    {
        const int bd = wave, c = l >> 2, part = l & 3;
        const float* Ab = sQA + 16 * bd * LDA + 16 * bd;
        float tc[4] = {0.f, 0.f, 0.f, 0.f};            // rows part, part + 4, ... of column c
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int i = 4 * m + part;
                if (i < t) s += Ab[t * LDA + i] * tc[m];
            }
            s = dpp_sum4(s);
            const float v = (t == c ? 1.f : 0.f) - s;
            if (part == (t & 3)) tc[t >> 2] = v;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) sT[(16 * bd + 4 * m + part) * LDT + 16 * bd + c] = tc[m];
    }
    __syncthreads();
    const int lr = l & 15, lg = l >> 4;
#pragma unroll
    for (int lev = 1; lev < 4; ++lev) {
        if (wave + lev < 4) {
            const int J = wave, I = J + lev;
            float4v y = float4v{0.f, 0.f, 0.f, 0.f};
            const float* Ai = sQA + 16 * I * LDA;
            const float* Bj = sT + 16 * J;
            if (lev == 1) y = mma_x<kBf16, false, true, 16>(Ai, LDA, Bj, LDT, 16 * J, y);
            else if (lev == 2) y = mma_x<kBf16, false, true, 32>(Ai, LDA, Bj, LDT, 16 * J, y);
            else y = mma_x<kBf16, false, true, 48>(Ai, LDA, Bj, LDT, 16 * J, y);
#pragma unroll
            for (int e = 0; e < 4; ++e) sY[(4 * lg + e) * 16 + lr] = y[e];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const float4v t =
                mma_x<kBf16, false, true, 16>(sT + 16 * I * LDT + 16 * I, LDT, sY, 16, 0, float4v{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * I + 4 * lg + e) * LDT + 16 * J + lr] = -t[e];
        }
        __syncthreads();
    }
    // T out, zero above the diagonal blocks (fp16 in the first half of the
    // slot for bf16 inputs with d >= 64, where only the reverse walk reads it)
    float* gT = ws_T + bhn * C * C;
#pragma unroll
    for (int it = 0; it < C * C / 4 / 256; ++it) {
        const int idx = tid + 256 * it, row = idx / (C / 4), c4 = 4 * (idx % (C / 4));
        float4v v = *reinterpret_cast<const float4v*>(&sT[row * LDT + c4]);
        if (c4 / 16 > row / 16) v = float4v{0.f, 0.f, 0.f, 0.f};
        if constexpr (kBf16 && DK >= 64)
            *reinterpret_cast<half4*>(reinterpret_cast<_Float16*>(gT) + row * C + c4) = to_h4(v);
        else
            *reinterpret_cast<float4v*>(&gT[row * C + c4]) = v;
    }
}

// ---------------------------------------------------------------------------
// Pass 2: chunk-start states and E, walking the chunks forward.
// grid (DV / 16 slices x 8 x ceil(B*H / 8)), 512 threads (8 waves); state
// row block m of the slice lives in wave m's accumulators.  Per chunk:
//   1. K S for row block w % 4, its d_k columns split between waves w and
//      w + 4 as two partial sums, added in LDS into R = diag(beta) (V -
//      diag(gamma) K S).
//   2. E = T R (waves 0..3, one row block each), written out, (lam E)^T kept.
//   3. S' = gamma_n S + K^T (lam E), one state block per wave.
// The next chunk's inputs are loaded into registers while the current chunk
// is computed.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool kBf16>
__global__ __launch_bounds__(512) void bwd_states_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                         const float* __restrict__ beta,
                                                         const float* __restrict__ S0,
                                                         const float* __restrict__ ws_g,
                                                         const float* __restrict__ ws_T, float* __restrict__ ws_S,
                                                         float* __restrict__ ws_E, int T, int H, int nch, int BH) {
    constexpr int SV = 16, LDK = DK + 4, LDT = C + 4, LDS_ = DK + 4, LDR = C + 4;
    constexpr int NST = DK / 16;                       // state row blocks, one per wave
    constexpr int NT = 512;
    constexpr int KH = DK >= 32 ? DK / 2 : DK;         // d_k columns of K S in the first partial sum
    int slice, bh;
    if (!slice_of_block<DV / 16>(BH, slice, bh)) return;
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
    const int rb = wave & 3, half = wave >> 2;
    const int col0 = slice * SV;
    const bool owns = wave < NST;

    __shared__ __align__(16) float sK[C * LDK];
    __shared__ __align__(16) float sT[C * LDT];
    __shared__ __align__(16) float sSt[SV * LDS_];     // S^T (the slice)
    __shared__ __align__(16) float sKSp[2][SV * LDR];  // the two partial sums of (K S)^T
    __shared__ __align__(16) float sRt[SV * LDR];      // R^T
    __shared__ __align__(16) float sEt[SV * LDR];      // (lam E)^T
    __shared__ float sV[C][SV + 1];
    __shared__ float sg[C], sb[C];

    RowTile<DK, NT, kBf16> pk;
    MatTile<NT> pt;
    Raw4<kBf16> pv;
    float pg = 0.f, pb = 0.f;
    const int vt = (tid >> 2) & 63, vc = tid & 3;
    auto fetch = [&](int cc) {
        const long bhn = static_cast<long>(bh) * nch + cc;
        pk.load(k, b, cc, T, H, h);
        pt.load(ws_T + bhn * C * C);
        const int tg = cc * C + vt, tc = tg < T ? tg : T - 1;
        pv = raw_load<kBf16>(v, ((static_cast<long>(b) * T + tc) * H + h) * DV + col0 + 4 * vc);
        const int tl = tid & 63, tgl = cc * C + tl;
        pg = ws_g[bhn * C + tl];
        pb = beta[(static_cast<long>(b) * T + (tgl < T ? tgl : T - 1)) * H + h];
    };
    auto publish = [&](int cc) {
        pk.store(sK, LDK, cc, T);
        pt.store(sT, LDT);
        if (tid < 256) {
            const float4v x = cc * C + vt < T ? raw_cvt<kBf16>(pv) : float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) sV[vt][4 * vc + e] = x[e];
        }
        if (tid < C) {
            sg[tid] = pg;
            sb[tid] = cc * C + tid < T ? pb : 0.f;
        }
    };

    float4v st = {0.f, 0.f, 0.f, 0.f};
    if (owns) {
        if (S0) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                st[j] = S0[(static_cast<long>(bh) * DK + 16 * wave + 4 * (l >> 4) + j) * DV + col0 + (l & 15)];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sSt[(l & 15) * LDS_ + 16 * wave + 4 * (l >> 4) + j] = st[j];
    }
    fetch(0);
    publish(0);
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        const long bhn = static_cast<long>(bh) * nch + c;
        fetch(c + 1 < nch ? c + 1 : c);
        // chunk-start state out
        if (owns) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ws_S[(bhn * DK + 16 * wave + 4 * (l >> 4) + j) * DV + col0 + (l & 15)] = st[j];
        }
        // 1. K S for row block rb, d_k columns [0, KH) or [KH, DK)
        if (half == 0 || KH < DK) {
            float4v ks = {0.f, 0.f, 0.f, 0.f};
            if (half == 0) ks = mma_x<kBf16, false, false, KH>(&sK[16 * rb * LDK], LDK, sSt, LDS_, 0, ks);
            else if constexpr (KH < DK) ks = mma_x<kBf16, false, false, DK - KH>(&sK[16 * rb * LDK], LDK, sSt, LDS_, KH, ks);
#pragma unroll
            for (int j = 0; j < 4; ++j) sKSp[half][(l & 15) * LDR + 16 * rb + 4 * (l >> 4) + j] = ks[j];
        }
        __syncthreads();
        for (int i = tid; i < SV * C; i += NT) {
            const int cc = i / C, r = i - cc * C;
            const float ks = KH < DK ? sKSp[0][cc * LDR + r] + sKSp[1][cc * LDR + r] : sKSp[0][cc * LDR + r];
            sRt[cc * LDR + r] = sb[r] * (sV[r][cc] - __expf(sg[r]) * ks);
        }
        __syncthreads();
        // 2. E = T R (T lower triangular), written out; (lam E)^T kept for the update
        if (wave < 4) {
            float4v e = {0.f, 0.f, 0.f, 0.f};
            e = mma_x<kBf16, false, false, C>(&sT[16 * wave * LDT], LDT, sRt, LDR, 0, e);   // T is zero above the diagonal
            const float gn = sg[C - 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * wave + 4 * (l >> 4) + j;
                ws_E[(bhn * C + r) * DV + col0 + (l & 15)] = e[j];
                sEt[(l & 15) * LDR + r] = __expf(gn - sg[r]) * e[j];
            }
        }
        __syncthreads();
        // 3. S' = gamma_n S + K^T (lam E)
        if (owns) {
            const float gam_n = __expf(sg[C - 1]);
            st = mma_x<kBf16, true, false, C>(&sK[16 * wave], LDK, sEt, LDR, 0, gam_n * st);
#pragma unroll
            for (int j = 0; j < 4; ++j) sSt[(l & 15) * LDS_ + 16 * wave + 4 * (l >> 4) + j] = st[j];
        }
        __syncthreads();
        publish(c + 1 < nch ? c + 1 : c);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Pass 3: state gradients, walking the chunks backward.  grid as pass 2,
// 512 threads (8 waves).  State row block m of the slice lives in wave m's
// accumulators.  Per chunk:
//   1. dE = scale P^T dY + diag(lam) K dS': row block w % 4; wave w / 4 = 0
//      takes P^T dY and the first ka columns of K dS', wave w / 4 = 1 the
//      rest, as two partial sums added in LDS.  scale gamma dY is formed.
//   2. dR = T^T dE (waves 0..3, one row block each; dV = beta dR) while every
//      wave m < DK / 16 starts its block of dS with gamma_n dS' + Q^T (scale
//      gamma dY).
//   3. dS += K^T (-beta gamma dR).
// ---------------------------------------------------------------------------
template <int DK, int DV, bool kBf16>
__global__ __launch_bounds__(512) void bwd_dstates_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const float* __restrict__ beta,
    const float* __restrict__ dy, const float* __restrict__ dST, const float* __restrict__ ws_g,
    const float* __restrict__ ws_T, const float* __restrict__ ws_P, float* __restrict__ ws_dS,
    float* __restrict__ ws_dR, float* __restrict__ dv_out, float* __restrict__ dS0, int T, int H, int nch,
    int BH, float scale) {
    constexpr int SV = 16, LDK = DK + 4, LDX = C + 4, LDS_ = DK + 4;
    constexpr int NST = DK / 16;                       // state row blocks, one per wave
    constexpr int NT = 512;
    constexpr int KA = DK == 128 ? 32 : 0;             // columns of K dS' taken with P^T dY
    int slice, bh;
    if (!slice_of_block<DV / 16>(BH, slice, bh)) return;
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
    const int rb = wave & 3, half = wave >> 2;
    const int col0 = slice * SV;
    const bool owns = wave < NST;

    __shared__ __align__(16) float sQ[C * LDK];
    __shared__ __align__(16) float sK[C * LDK];
    __shared__ __align__(16) float sT[C * LDX];
    __shared__ __align__(16) float sP[C * LDX];
    __shared__ __align__(16) float sdYt[SV * LDX];     // dY^T
    __shared__ __align__(16) float sB1t[SV * LDX];     // (scale gamma dY)^T
    __shared__ __align__(16) float sB2t[SV * LDX];     // (-beta gamma dR)^T
    __shared__ __align__(16) float sdEp[2][SV * LDX];  // the two partial sums of dE^T
    __shared__ __align__(16) float sdEt[SV * LDX];     // dE^T
    __shared__ __align__(16) float sdSt[SV * LDS_];    // dS'^T
    __shared__ float sg[C], sb[C];

    RowTile<DK, NT, kBf16> pq, pk;
    MatTile<NT> pt, pp;
    float4v pdy = {0.f, 0.f, 0.f, 0.f};
    float pg = 0.f, pb = 0.f;
    const int yt = (tid >> 2) & 63, yc = tid & 3;
    auto fetch = [&](int cc) {
        const long bhn = static_cast<long>(bh) * nch + cc;
        pq.load(q, b, cc, T, H, h);
        pk.load(k, b, cc, T, H, h);
        pt.load(ws_T + bhn * C * C);
        pp.load(ws_P + bhn * C * C);
        const int tg = cc * C + yt, tc = tg < T ? tg : T - 1;
        pdy = *reinterpret_cast<const float4v*>(&dy[((static_cast<long>(b) * T + tc) * H + h) * DV + col0 + 4 * yc]);
        const int tl = tid & 63, tgl = cc * C + tl;
        pg = ws_g[bhn * C + tl];
        pb = beta[(static_cast<long>(b) * T + (tgl < T ? tgl : T - 1)) * H + h];
    };
    auto publish = [&](int cc) {
        pq.store(sQ, LDK, cc, T);
        pk.store(sK, LDK, cc, T);
        pt.store(sT, LDX);
        pp.store(sP, LDX);
        if (tid < 256) {
            const float4v x = cc * C + yt < T ? pdy : float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) sdYt[(4 * yc + e) * LDX + yt] = x[e];
        }
        if (tid < C) {
            sg[tid] = pg;
            sb[tid] = cc * C + tid < T ? pb : 0.f;
        }
    };

    float4v ds = {0.f, 0.f, 0.f, 0.f};
    if (owns) {
        if (dST) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ds[j] = dST[(static_cast<long>(bh) * DK + 16 * wave + 4 * (l >> 4) + j) * DV + col0 + (l & 15)];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sdSt[(l & 15) * LDS_ + 16 * wave + 4 * (l >> 4) + j] = ds[j];
    }
    fetch(nch - 1);
    publish(nch - 1);
    __syncthreads();

    for (int c = nch - 1; c >= 0; --c) {
        const long bhn = static_cast<long>(bh) * nch + c;
        fetch(c > 0 ? c - 1 : 0);
        if (owns) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ws_dS[(bhn * DK + 16 * wave + 4 * (l >> 4) + j) * DV + col0 + (l & 15)] = ds[j];
        }
        // 1. the two partial sums of dE for row block rb
        {
            const float gn = sg[C - 1];
            float4v acc = {0.f, 0.f, 0.f, 0.f};
            float4v kd = {0.f, 0.f, 0.f, 0.f};
            if (half == 0) {
                acc = mma_x<kBf16, true, false, C>(&sP[16 * rb], LDX, sdYt, LDX, 0, acc);   // P^T is zero below the diagonal
                if constexpr (KA > 0) kd = mma_x<kBf16, false, false, KA>(&sK[16 * rb * LDK], LDK, sdSt, LDS_, 0, kd);
            } else {
                kd = mma_x<kBf16, false, false, DK - KA>(&sK[16 * rb * LDK], LDK, sdSt, LDS_, KA, kd);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rb + 4 * (l >> 4) + j;
                sdEp[half][(l & 15) * LDX + r] = scale * acc[j] + __expf(gn - sg[r]) * kd[j];
            }
        }
        for (int i = tid; i < SV * C; i += NT) {
            const int cc = i / C, t = i - cc * C;
            sB1t[cc * LDX + t] = scale * __expf(sg[t]) * sdYt[cc * LDX + t];
        }
        __syncthreads();
        for (int i = tid; i < SV * C; i += NT) {
            const int cc = i / C, t = i - cc * C;
            sdEt[cc * LDX + t] = sdEp[0][cc * LDX + t] + sdEp[1][cc * LDX + t];
        }
        __syncthreads();
        // 2. dR = T^T dE, dV = diag(beta) dR (waves 0..3); dS starts with gamma_n dS' + Q^T (scale gamma dY)
        if (wave < 4) {
            float4v r = {0.f, 0.f, 0.f, 0.f};
            r = mma_x<kBf16, true, false, C>(&sT[16 * wave], LDX, sdEt, LDX, 0, r);   // T^T is zero below the diagonal
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * wave + 4 * (l >> 4) + j, tg = c * C + t;
                ws_dR[(bhn * C + t) * DV + col0 + (l & 15)] = r[j];
                if (tg < T) dv_out[((static_cast<long>(b) * T + tg) * H + h) * DV + col0 + (l & 15)] = sb[t] * r[j];
                sB2t[(l & 15) * LDX + t] = -sb[t] * __expf(sg[t]) * r[j];
            }
        }
        const float gam_n = __expf(sg[C - 1]);
        if (owns) ds = mma_x<kBf16, true, false, C>(&sQ[16 * wave], LDK, sB1t, LDX, 0, gam_n * ds);
        __syncthreads();
        // 3. dS += K^T (-beta gamma dR)
        if (owns) ds = mma_x<kBf16, true, false, C>(&sK[16 * wave], LDK, sB2t, LDX, 0, ds);
        __syncthreads();                       // every read of this chunk's tiles is done
        if (owns) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sdSt[(l & 15) * LDS_ + 16 * wave + 4 * (l >> 4) + j] = ds[j];
        }
        publish(c > 0 ? c - 1 : 0);
        __syncthreads();
    }
    if (dS0 && owns) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            dS0[(static_cast<long>(bh) * DK + 16 * wave + 4 * (l >> 4) + j) * DV + col0 + (l & 15)] = ds[j];
    }
}

// ---------------------------------------------------------------------------
// Pass 4: per-chunk gradients dq, dk, dbeta, dalpha.  grid (nch, B*H), 512
// threads.  d_k = d_v = D.
// ---------------------------------------------------------------------------
template <int D, bool kBf16>
__global__ __launch_bounds__(512) void bwd_grads_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ dy,
    const float* __restrict__ ws_g, const float* __restrict__ ws_P, const float* __restrict__ ws_M,
    const float* __restrict__ ws_S, const float* __restrict__ ws_dS, const float* __restrict__ ws_E,
    const float* __restrict__ ws_dR, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dalpha, float* __restrict__ dbeta, int T, int H, int nch, float scale) {
    constexpr int SL = 16, LDL = SL + 4, LDX = C + 4, LDK = D + 4;
    constexpr int NB = D / 16;                      // column blocks of X1..X3
    constexpr int NP = 4 * NB;                      // (row block, column block) pairs
    constexpr int PPW = (NP + 7) / 8;               // pairs per wave
    const int c = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh - b * H;
    const long bhn = static_cast<long>(bh) * nch + c;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;

    // phase-1 slabs and phase-2 P, M share one region
    constexpr int kSlabFloats = 4 * C * LDL + 2 * D * LDL;
    constexpr int kPMFloats = 2 * C * LDX;
    constexpr int kRegion = kSlabFloats > kPMFloats ? kSlabFloats : kPMFloats;
    __shared__ __align__(16) float sR[kRegion];
    // q and k: fp32 row-major for the fp32-operand path; for bf16 inputs
    // with d >= 64, their fp16 transposes [d][token] (leading dimension LDT)
    constexpr bool kH = kBf16 && D >= 64;
    constexpr int LDT = C + 8;
    __shared__ __align__(16) float sQ[kH ? 4 : C * LDK];
    __shared__ __align__(16) float sK[kH ? 4 : C * LDK];
    __shared__ __align__(16) _Float16 hQt[kH ? D * LDT : 8];
    __shared__ __align__(16) _Float16 hKt[kH ? D * LDT : 8];
    __shared__ __align__(16) float sX4[C * LDX];    // X4, then dP o Gamma
    __shared__ __align__(16) float sX5[C * LDX];    // X5, then Dm
    __shared__ float sg[C], sb[C], sa[C];
    __shared__ float sQX1[C], sKX2[C], sKX3[C], sDRv[C], sColPP[C], sColAA[C], sRowPP[C], sRowAA[C], sRowAM[C];
    __shared__ float sSdS;

    float* sdY = sR;
    float* sdR = sR + C * LDL;
    float* sE = sR + 2 * C * LDL;
    float* sV = sR + 3 * C * LDL;
    float* sS = sR + 4 * C * LDL;
    float* sdS = sS + D * LDL;

    float4v x1[PPW], x2[PPW], x3[PPW], x4[2], x5[2];
#pragma unroll
    for (int u = 0; u < PPW; ++u) x1[u] = x2[u] = x3[u] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 2; ++u) x4[u] = x5[u] = float4v{0.f, 0.f, 0.f, 0.f};
    float drv = 0.f, sds = 0.f;

    // per-token values and phase-2 operands are loaded into registers first
    float pre_a = 1.f, pre_b = 0.f, pre_g = 0.f;
    if (tid < C) {
        const int tg = c * C + tid;
        const long gi = (static_cast<long>(b) * T + (tg < T ? tg : T - 1)) * H + h;
        pre_a = alpha[gi];
        pre_b = beta[gi];
        pre_g = ws_g[bhn * C + tid];
    }
    RowTile<D, 512, kBf16> tq, tk;
    MatTile<512> tp, tm;
    tq.load(q, b, c, T, H, h);
    tk.load(k, b, c, T, H, h);
    tp.load(ws_P + bhn * C * C);
    tm.load(ws_M + bhn * C * C);
    const int rt = (tid & 255) >> 2, rc = tid & 3;                 // row item: row rt, columns 4 rc..
    const int si = tid % (D * SL / 4), sr = si >> 2, sc = si & 3;  // state item: row sr, columns 4 sc..
    const int tg0 = c * C + rt, tc0 = tg0 < T ? tg0 : T - 1;
    const long row0 = (static_cast<long>(b) * T + tc0) * H + h;
    if constexpr (kBf16 && D >= 64) {
        // bf16 inputs: 32-column d_v slabs (whole 128-byte lines of the fp32
        // rows, one load item per thread and row array), rounded to fp16 once
        // when stored, so that each MFMA operand is one 16-byte LDS read and
        // each MFMA covers 32 values of d_v.  Row stride 40 halfs (80 bytes)
        // keeps the 16-byte operand reads free of bank conflicts.
        constexpr int SH = 32, LDH = SH + 8, NSH = D / SH, NSI = D / 64;
        constexpr int kDepthH = NSH < 3 ? NSH : 3;
        static_assert((3 * C + 2 * D) * LDH * 2 <= kRegion * 4, "fp16 slabs fit the slab region");
        _Float16* hY = reinterpret_cast<_Float16*>(sR);   // dY slab, C x LDH
        _Float16* hR = hY + C * LDH;                      // dR slab
        _Float16* hE = hR + C * LDH;                      // E slab
        _Float16* hS = hE + C * LDH;                      // S slab, D x LDH
        _Float16* hD = hS + D * LDH;                      // dS slab
        const int hr = tid >> 3, hc = tid & 7;            // row item: row hr, columns 4 hc ..
        const int tgh = c * C + hr, tch = tgh < T ? tgh : T - 1;
        const long rowh = (static_cast<long>(b) * T + tch) * H + h;
        // S, dS, E and dR come as fp16 (the walks for bf16 inputs store them
        // rounded, at the start of their fp32-sized slots)
        const _Float16* S16 = reinterpret_cast<const _Float16*>(ws_S);
        const _Float16* dS16 = reinterpret_cast<const _Float16*>(ws_dS);
        const _Float16* E16 = reinterpret_cast<const _Float16*>(ws_E);
        const _Float16* dR16 = reinterpret_cast<const _Float16*>(ws_dR);
        struct SlabH {
            float4v dy;
            half4 dr, e, s[NSI], ds[NSI];
            Raw4<true> v;
        };
        SlabH f[kDepthH];
        auto fetch = [&](SlabH& x, int v0) {
            x.dy = *reinterpret_cast<const float4v*>(&dy[rowh * D + v0 + 4 * hc]);
            x.v = raw_load<true>(v, rowh * D + v0 + 4 * hc);
            x.dr = *reinterpret_cast<const half4*>(&dR16[(bhn * C + hr) * D + v0 + 4 * hc]);
            x.e = *reinterpret_cast<const half4*>(&E16[(bhn * C + hr) * D + v0 + 4 * hc]);
#pragma unroll
            for (int i = 0; i < NSI; ++i) {
                x.s[i] = *reinterpret_cast<const half4*>(&S16[(bhn * D + hr + 64 * i) * D + v0 + 4 * hc]);
                x.ds[i] = *reinterpret_cast<const half4*>(&dS16[(bhn * D + hr + 64 * i) * D + v0 + 4 * hc]);
            }
        };
        auto f32 = [](half4 hv) {
            return float4v{static_cast<float>(hv[0]), static_cast<float>(hv[1]), static_cast<float>(hv[2]),
                           static_cast<float>(hv[3])};
        };
#pragma unroll
        for (int s = 0; s < kDepthH; ++s) fetch(f[s], s * SH);
#pragma unroll
        for (int s = 0; s < NSH; ++s) {
            SlabH& x = f[s % kDepthH];
            {
                // rows past T (clamped copies of the last row) zeroed by a
                // factor: a select may become a branch with the load sunk into it
                const float live = tgh < T ? 1.f : 0.f;
                const float4v xdy = x.dy * live, xv = raw_cvt<true>(x.v) * live;
                *reinterpret_cast<half4*>(&hY[hr * LDH + 4 * hc]) = to_h4(xdy);
                *reinterpret_cast<half4*>(&hR[hr * LDH + 4 * hc]) = x.dr;
                *reinterpret_cast<half4*>(&hE[hr * LDH + 4 * hc]) = x.e;
                const float4v dr = f32(x.dr);
                drv += dr.x * xv.x + dr.y * xv.y + dr.z * xv.z + dr.w * xv.w;
#pragma unroll
                for (int i = 0; i < NSI; ++i) {
                    *reinterpret_cast<half4*>(&hS[(hr + 64 * i) * LDH + 4 * hc]) = x.s[i];
                    *reinterpret_cast<half4*>(&hD[(hr + 64 * i) * LDH + 4 * hc]) = x.ds[i];
                    const float4v sv = f32(x.s[i]), dsv = f32(x.ds[i]);
                    sds += sv.x * dsv.x + sv.y * dsv.y + sv.z * dsv.z + sv.w * dsv.w;
                }
            }
            if (s == 0) {
                tq.store_t(hQt, LDT, c, T);
                tk.store_t(hKt, LDT, c, T);
            }
            __syncthreads();
            if (s + kDepthH < NSH) fetch(x, (s + kDepthH) * SH);
            // the same pairs as the fp32 path; repeated fragment reads of one
            // tile (the B tiles of a wave's pairs, E as both operands) are the
            // same loads and are read once
#pragma unroll
            for (int u = 0; u < PPW; ++u) {
                const int p = wave + 8 * u;
                if (p < NP) {
                    const int ti = p / NB, tj = p - ti * NB;
                    const half8 bS = frag_h(&hS[16 * tj * LDH], LDH), bD = frag_h(&hD[16 * tj * LDH], LDH);
                    x1[u] = mma_hh(frag_h(&hY[16 * ti * LDH], LDH), bS, x1[u]);
                    x2[u] = mma_hh(frag_h(&hR[16 * ti * LDH], LDH), bS, x2[u]);
                    x3[u] = mma_hh(frag_h(&hE[16 * ti * LDH], LDH), bD, x3[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int p = wave + 8 * u, ti = p >> 2, tj = p & 3;
                if (tj <= ti) {
                    const half8 bE = frag_h(&hE[16 * tj * LDH], LDH);
                    x4[u] = mma_hh(frag_h(&hY[16 * ti * LDH], LDH), bE, x4[u]);
                    x5[u] = mma_hh(frag_h(&hR[16 * ti * LDH], LDH), bE, x5[u]);
                }
            }
            __syncthreads();
        }
    } else {
        // d_v slabs in flight: slab s is loaded kDepth slabs before its use, into
        // register set s % kDepth (the slab loop is unrolled, so the sets are
        // fixed registers and every load is unconditional)
        constexpr int NS = D / SL;
        constexpr int kDepth = NS < 4 ? NS : 4;
        struct Slab {
            float4v dy, dr, e, s, ds;
            Raw4<kBf16> v;
        };
        Slab f[kDepth];
        auto fetch = [&](Slab& x, int v0) {
            x.dy = *reinterpret_cast<const float4v*>(&dy[row0 * D + v0 + 4 * rc]);
            x.v = raw_load<kBf16>(v, row0 * D + v0 + 4 * rc);
            x.dr = *reinterpret_cast<const float4v*>(&ws_dR[(bhn * C + rt) * D + v0 + 4 * rc]);
            x.e = *reinterpret_cast<const float4v*>(&ws_E[(bhn * C + rt) * D + v0 + 4 * rc]);
            x.s = *reinterpret_cast<const float4v*>(&ws_S[(bhn * D + sr) * D + v0 + 4 * sc]);
            x.ds = *reinterpret_cast<const float4v*>(&ws_dS[(bhn * D + sr) * D + v0 + 4 * sc]);
        };
    #pragma unroll
        for (int s = 0; s < kDepth; ++s) fetch(f[s], s * SL);
    #pragma unroll
        for (int s = 0; s < NS; ++s) {
            Slab& x = f[s % kDepth];
            if (tid < C * SL / 4) {
                float4v xdy = x.dy, xv = raw_cvt<kBf16>(x.v);
                if (tg0 >= T) xdy = xv = float4v{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<float4v*>(&sdY[rt * LDL + 4 * rc]) = xdy;
                *reinterpret_cast<float4v*>(&sdR[rt * LDL + 4 * rc]) = x.dr;
                *reinterpret_cast<float4v*>(&sE[rt * LDL + 4 * rc]) = x.e;
                *reinterpret_cast<float4v*>(&sV[rt * LDL + 4 * rc]) = xv;
                drv += x.dr.x * xv.x + x.dr.y * xv.y + x.dr.z * xv.z + x.dr.w * xv.w;
            }
            if (tid < D * SL / 4) {
                *reinterpret_cast<float4v*>(&sS[sr * LDL + 4 * sc]) = x.s;
                *reinterpret_cast<float4v*>(&sdS[sr * LDL + 4 * sc]) = x.ds;
                sds += x.s.x * x.ds.x + x.s.y * x.ds.y + x.s.z * x.ds.z + x.s.w * x.ds.w;
            }
            if (s == 0) {
                tq.store(sQ, LDK, c, T);
                tk.store(sK, LDK, c, T);
            }
            __syncthreads();
            if (s + kDepth < NS) fetch(x, (s + kDepth) * SL);
    #pragma unroll
            for (int u = 0; u < PPW; ++u) {
                const int p = wave + 8 * u;
                if (p < NP) {
                    const int ti = p / NB, tj = p - ti * NB;
                    x1[u] = mma_x<kBf16, false, false, SL>(&sdY[16 * ti * LDL], LDL, &sS[16 * tj * LDL], LDL, 0, x1[u]);
                    x2[u] = mma_x<kBf16, false, false, SL>(&sdR[16 * ti * LDL], LDL, &sS[16 * tj * LDL], LDL, 0, x2[u]);
                    x3[u] = mma_x<kBf16, false, false, SL>(&sE[16 * ti * LDL], LDL, &sdS[16 * tj * LDL], LDL, 0, x3[u]);
                }
            }
    #pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int p = wave + 8 * u, ti = p >> 2, tj = p & 3;
                if (tj <= ti) {
                    x4[u] = mma_x<kBf16, false, false, SL>(&sdY[16 * ti * LDL], LDL, &sE[16 * tj * LDL], LDL, 0, x4[u]);
                    x5[u] = mma_x<kBf16, false, false, SL>(&sdR[16 * ti * LDL], LDL, &sE[16 * tj * LDL], LDL, 0, x5[u]);
                }
            }
            __syncthreads();
        }
    }

    // ---- phase 2 ----
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int p = wave + 8 * u, ti = p >> 2, tj = p & 3;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * ti + 4 * (l >> 4) + j, col = 16 * tj + (l & 15);
            sX4[row * LDX + col] = x4[u][j];
            sX5[row * LDX + col] = x5[u][j];
        }
    }
    float* sP = sR;
    float* sM = sR + C * LDX;
    tp.store(sP, LDX);
    tm.store(sM, LDX);
    if (tid < C) {
        const int tg = c * C + tid;
        sg[tid] = pre_g;
        sb[tid] = tg < T ? pre_b : 0.f;
        sa[tid] = tg < T ? pre_a : 1.f;
        sQX1[tid] = sKX2[tid] = sKX3[tid] = 0.f;
    }
    if (tid == 0) sSdS = 0.f;
    // dR . v per row: the partial sums sit in the lanes of the row's load
    // items (8 lanes per row with 32-column fp16 slabs, 4 with 16-column ones)
    if constexpr (kBf16 && D >= 64) {
        const float s = dpp_sum8(drv);
        if ((tid & 7) == 0) sDRv[tid >> 3] = s;
    } else {
        const float s = dpp_sum4(drv);
        if (tid < C * SL / 4 && (tid & 3) == 0) sDRv[tid >> 2] = s;
    }
    __syncthreads();
    // <dS', S> over the whole block
    {
        float s = sds;
        s = dpp_sum16(s);
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (l == 0) atomicAdd(&sSdS, s);
    }
    // row scalars from X1..X3: q.X1, k.X2, k.X3
#pragma unroll
    for (int u = 0; u < PPW; ++u) {
        const int p = wave + 8 * u;
        if (p < NP) {
            const int ti = p / NB, tj = p - ti * NB, col = 16 * tj + (l & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * ti + 4 * (l >> 4) + j;
                float qv, kv;
                if constexpr (kH) {
                    qv = static_cast<float>(hQt[col * LDT + row]);
                    kv = static_cast<float>(hKt[col * LDT + row]);
                } else {
                    qv = sQ[row * LDK + col];
                    kv = sK[row * LDK + col];
                }
                const float a1 = dpp_sum16(qv * x1[u][j]);
                const float a2 = dpp_sum16(kv * x2[u][j]);
                const float a3 = dpp_sum16(kv * x3[u][j]);
                if ((l & 15) == 0) {
                    atomicAdd(&sQX1[row], a1);
                    atomicAdd(&sKX2[row], a2);
                    atomicAdd(&sKX3[row], a3);
                }
            }
        }
    }
    // column sums of dP o P and dA o A: lane group of 8 per column
    {
        const int i = tid >> 3, part = tid & 7;
        float pp = 0.f, aa = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int t = 8 * part + m;
            const float dP = i <= t ? scale * sX4[t * LDX + i] : 0.f;
            const float dA = i < t ? -sX5[t * LDX + i] : 0.f;
            pp += dP * sP[t * LDX + i];
            aa += dA * sb[t] * sM[t * LDX + i];
        }
        pp = dpp_sum8(pp);
        aa = dpp_sum8(aa);
        if (part == 0) {
            sColPP[i] = pp;
            sColAA[i] = aa;
        }
    }
    __syncthreads();
    // row sums, and X4 -> dP o Gamma, X5 -> Dm in place
    {
        const int t = tid >> 3, part = tid & 7;
        float pp = 0.f, aa = 0.f, am = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int i = 8 * part + m;
            const float dP = i <= t ? scale * sX4[t * LDX + i] : 0.f;
            const float dA = i < t ? -sX5[t * LDX + i] : 0.f;
            const float gam = i <= t ? __expf(sg[t] - sg[i]) : 0.f;
            const float mv = sM[t * LDX + i];
            pp += dP * sP[t * LDX + i];
            aa += dA * sb[t] * mv;
            am += dA * mv;
            sX4[t * LDX + i] = dP * gam;
            sX5[t * LDX + i] = sb[t] * dA * gam;
        }
        pp = dpp_sum8(pp);
        aa = dpp_sum8(aa);
        am = dpp_sum8(am);
        if (part == 0) {
            sRowPP[t] = pp;
            sRowAA[t] = aa;
            sRowAM[t] = am;
        }
    }
    __syncthreads();
    // per-token scalars: dbeta, dg, then dlog(alpha) as a reverse cumsum
    if (wave == 0) {
        const int t = l, tg = c * C + t;
        const float gam = __expf(sg[t]), lam = __expf(sg[C - 1] - sg[t]);
        const float dgam = scale * sQX1[t] - sb[t] * sKX2[t];
        const float dlam = sKX3[t];
        const float db = sDRv[t] - gam * sKX2[t] + sRowAM[t];
        float dg = gam * dgam + sRowPP[t] - sColPP[t] + sRowAA[t] - sColAA[t] - lam * dlam;
        const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dpp_scan64(lam * dlam)), 63));
        if (t == C - 1) dg += tot + gam * sSdS;
        // reverse inclusive scan dl_s = sum_{t >= s} dg_t: a prefix scan of the
        // lane-reversed values, reversed back
        const float x = __shfl(dpp_scan64(__shfl(dg, C - 1 - t)), C - 1 - t);
        if (tg < T) {
            const long gi = (static_cast<long>(b) * T + tg) * H + h;
            dbeta[gi] = db;
            const float a = sa[t];
            dalpha[gi] = __logf(a) >= kLogFloor ? x / a : 0.f;
        }
    }
    // bf16 inputs, d >= 64: G = dP o Gamma, its transpose and Dm + Dm^T as
    // fp16 tiles (in the slab region: P and M are no longer read), so that
    // every operand of the dq and dk contractions is one 16-byte LDS read
    _Float16* hG = reinterpret_cast<_Float16*>(sR);
    _Float16* hGt = hG + C * LDT;
    _Float16* hDs = hGt + C * LDT;
    if constexpr (kH) {
        static_assert(3 * C * LDT * 2 <= kRegion * 4, "fp16 G tiles fit the slab region");
        __syncthreads();                                   // every read of P and M is done
        for (int idx = tid; idx < C * C; idx += 512) {
            const int t = idx / C, i = idx - t * C;
            const float gv = sX4[t * LDX + i];
            hG[t * LDT + i] = static_cast<_Float16>(gv);
            hGt[i * LDT + t] = static_cast<_Float16>(gv);
            hDs[t * LDT + i] = static_cast<_Float16>(sX5[t * LDX + i] + sX5[i * LDX + t]);
        }
        __syncthreads();
    }
    // dq and dk tiles
#pragma unroll
    for (int u = 0; u < PPW; ++u) {
        const int p = wave + 8 * u;
        if (p < NP) {
            const int ti = p / NB, tj = p - ti * NB, col = 16 * tj + (l & 15);
            float4v aq, ak;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * ti + 4 * (l >> 4) + j;
                const float gam = __expf(sg[row]), lam = __expf(sg[C - 1] - sg[row]);
                aq[j] = scale * gam * x1[u][j];
                ak[j] = lam * x3[u][j] - sb[row] * gam * x2[u][j];
            }
            if constexpr (kH) {
#pragma unroll
                for (int ks = 0; ks < C / 32; ++ks) {
                    const half8 bK = frag_h(&hKt[16 * tj * LDT + 32 * ks], LDT);
                    aq = mma_hh(frag_h(&hG[16 * ti * LDT + 32 * ks], LDT), bK, aq);
                    ak = mma_hh(frag_h(&hDs[16 * ti * LDT + 32 * ks], LDT), bK, ak);
                    ak = mma_hh(frag_h(&hGt[16 * ti * LDT + 32 * ks], LDT), frag_h(&hQt[16 * tj * LDT + 32 * ks], LDT), ak);
                }
            } else {
                aq = mma_x<kBf16, false, true, C>(&sX4[16 * ti * LDX], LDX, &sK[16 * tj], LDK, 0, aq);   // dP o Gamma: lower
                ak = mma_sym_x<kBf16, C>(sX5, LDX, 16 * ti, &sK[16 * tj], LDK, 0, ak);
                ak = mma_x<kBf16, true, true, C>(&sX4[16 * ti], LDX, &sQ[16 * tj], LDK, 0, ak);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * ti + 4 * (l >> 4) + j, tg = c * C + row;
                if (tg < T) {
                    const long o = ((static_cast<long>(b) * T + tg) * H + h) * D + col;
                    dq[o] = aq[j];
                    dk[o] = ak[j];
                }
            }
        }
    }
}

// T == 0: the initial-state gradient is the final-state gradient (or zero).
__global__ __launch_bounds__(256) void bwd_copy_state_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                             long n) {
    const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace bwd

size_t prefill_bwd_workspace_bytes(int B, int T, int H, int dk, int dv) {
    const size_t nch = (static_cast<size_t>(T) + bwd::C - 1) / bwd::C;
    const size_t bhn = static_cast<size_t>(B) * H * nch;
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    return up(bhn * bwd::C * 4) + 3 * up(bhn * bwd::C * bwd::C * 4) + 2 * up(bhn * dk * dv * 4) +
           2 * up(bhn * bwd::C * dv * 4);
}

template <int D, bool kBf16>
static hipError_t launch_bwd_t(const PrefillBwdArgs& a) {
    const int nch = (a.T + bwd::C - 1) / bwd::C;
    const size_t bhn = static_cast<size_t>(a.B) * a.H * nch;
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    char* w = static_cast<char*>(a.workspace);
    float* g = reinterpret_cast<float*>(w);            w += up(bhn * bwd::C * 4);
    float* Tm = reinterpret_cast<float*>(w);           w += up(bhn * bwd::C * bwd::C * 4);
    float* P = reinterpret_cast<float*>(w);            w += up(bhn * bwd::C * bwd::C * 4);
    float* M = reinterpret_cast<float*>(w);            w += up(bhn * bwd::C * bwd::C * 4);
    float* S = reinterpret_cast<float*>(w);            w += up(bhn * D * D * 4);
    float* dS = reinterpret_cast<float*>(w);           w += up(bhn * D * D * 4);
    float* E = reinterpret_cast<float*>(w);            w += up(bhn * bwd::C * D * 4);
    float* dR = reinterpret_cast<float*>(w);
    const int BH = a.B * a.H;
    const dim3 gc(nch, BH), gs((D / 16) * 8 * ((BH + 7) / 8), 1);
    hipLaunchKernelGGL((bwd::bwd_prep_kernel<D, kBf16>), gc, dim3(256), 0, a.stream, a.q, a.k, a.alpha, a.beta,
                       g, Tm, P, M, a.T, a.H, nch);
    if constexpr (kBf16 && D >= 64) {
        // S_c and E_c from the forward's chunked walk (the same chain, with its
        // own T' and base-2 gates); its workspace sits in the dS region, which
        // the reverse walk fills only afterwards
        static_assert(sizeof(float) * D * D >= 7168, "the forward's per-chunk workspace fits the dS slot");
        PrefillArgs pa{};
        pa.q = a.q;
        pa.k = a.k;
        pa.v = a.v;
        pa.alpha = a.alpha;
        pa.beta = a.beta;
        pa.initial_state = a.initial_state;
        pa.final_state = nullptr;
        pa.y = nullptr;
        pa.B = a.B;
        pa.T = a.T;
        pa.H = a.H;
        pa.dk = D;
        pa.dv = D;
        pa.bf16 = true;
        pa.scale = a.scale;
        pa.workspace = dS;
        pa.stream = a.stream;
        const hipError_t e = launch_prefill_bf16_states(pa, S, E);
        if (e != hipSuccess) return e;
    } else {
        hipLaunchKernelGGL((bwd::bwd_states_kernel<D, D, kBf16>), gs, dim3(512), 0, a.stream, a.k, a.v, a.beta,
                           a.initial_state, g, Tm, S, E, a.T, a.H, nch, BH);
    }
    if constexpr (kBf16 && D >= 64) {
        // the reverse walk with the dS chain in one wave's registers
        RevWalkArgs ra{};
        ra.q = a.q;
        ra.k = a.k;
        ra.beta = a.beta;
        ra.dy = a.dy;
        ra.dST = a.d_final_state;
        ra.g = g;
        ra.Tm = Tm;
        ra.dS = dS;
        ra.dR = dR;
        ra.dv = a.dv;
        ra.dS0 = a.d_initial_state;
        ra.B = a.B;
        ra.T = a.T;
        ra.H = a.H;
        ra.d = D;
        ra.scale = a.scale;
        ra.stream = a.stream;
        const hipError_t e = launch_bwd_reverse_walk(ra);
        if (e != hipSuccess) return e;
    } else {
        hipLaunchKernelGGL((bwd::bwd_dstates_kernel<D, D, kBf16>), gs, dim3(512), 0, a.stream, a.q, a.k, a.beta,
                           a.dy, a.d_final_state, g, Tm, P, dS, dR, a.dv, a.d_initial_state, a.T, a.H, nch, BH,
                           a.scale);
    }
    hipLaunchKernelGGL((bwd::bwd_grads_kernel<D, kBf16>), gc, dim3(512), 0, a.stream, a.q, a.k, a.v, a.alpha,
                       a.beta, a.dy, g, P, M, S, dS, E, dR, a.dq, a.dk, a.dalpha, a.dbeta, a.T, a.H, nch, a.scale);
    return hipGetLastError();
}

template <bool kBf16>
static hipError_t launch_bwd_dt(const PrefillBwdArgs& a) {
    if (a.dk_ != a.dv_) return hipErrorInvalidValue;
    switch (a.dk_) {
        case 16: return launch_bwd_t<16, kBf16>(a);
        case 32: return launch_bwd_t<32, kBf16>(a);
        case 64: return launch_bwd_t<64, kBf16>(a);
        case 128: return launch_bwd_t<128, kBf16>(a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill_bwd(const PrefillBwdArgs& a) {
    if (a.T == 0) {
        if (!a.d_initial_state) return hipSuccess;
        const long n = static_cast<long>(a.B) * a.H * a.dk_ * a.dv_;
        hipLaunchKernelGGL(bwd::bwd_copy_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                           a.stream, a.d_final_state, a.d_initial_state, n);
        return hipGetLastError();
    }
    return a.bf16 ? launch_bwd_dt<true>(a) : launch_bwd_dt<false>(a);
}

}  // namespace gdn
