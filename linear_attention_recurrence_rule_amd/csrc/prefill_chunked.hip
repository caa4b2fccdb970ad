// bf16 chunked prefill of the gated delta rule on gfx950 (slinene
// ai-papers-daily page on Qwen3.8-Next, Module A: the delta-form recurrence,
// evaluated 64 tokens at a time in its chunkwise WY / UT-transform form).
//
// Per chunk of C = 64 tokens with start state S (g = in-chunk prefix sum of
// log alpha, gamma = exp(g), Gamma_ti = exp(g_t - g_i), d_t = exp(g_last - g_t)):
//   A  = strictLower(diag(beta) (Gamma o K K^T)),   T' = (I + A)^-1 diag(beta)
//   E  = T' (V - diag(gamma) K S)          (rows: beta_t times token t's miss)
//   Y  = diag(gamma) Q S + P E,            P = lower(Gamma o Q K^T)
//   S' = gamma_last S + K^T diag(d) E
// T' and the gates depend only on k, alpha and beta, so a chunk-parallel
// kernel (prep_kernel) computes them once per (head, chunk) into a workspace; the
// sequential kernel (main_kernel) then runs the chunks of one (head,
// 16-column value slice) in order.
//
// main_kernel: 8 waves with fixed roles, one workgroup barrier per chunk.
//   wave 0      state wave: K S, R = V - gamma K S, E = T' R, S += K^T D E.
//               The float32 state slice never leaves registers; every MFMA
//               operand it produces (S, R, E) is fed to the next MFMA straight
//               from the accumulator registers (split-K operand layout below),
//               so the chain has no LDS round trip.
//   waves 1, 2  output waves (token blocks {0,3} and {1,2}): Q S and P (built
//               transposed so it feeds the MFMA from registers), then, once
//               the state wave has published E, Y += P E -> y.
//   waves 3..7  loader waves (q and k on waves 3, 5, 6, 7; v, T' and the
//               gates on wave 4, which shares the state wave's SIMD): chunk
//               c+1 goes to the other LDS buffer from registers loaded during
//               the previous chunk.
// Loads run one chunk ahead in two register sets; they are unconditional
// (addresses clamped to the last token, whose copies past the end of the
// sequence are harmless: beta = 0 there) so that the compiler's wait counts
// stay exact across the chunk loop.
// Split-K operand layout: for a 16x16x32 MFMA, slot s of lane (m + 16 g) holds
// K-index 16*(s/4) + 4 g + s%4 of its row/column.  Two 16x16 accumulator tiles
// (lane (n + 16 g) holds rows 4 g .. 4 g + 3 of column n) stacked along K are
// exactly such a B operand, and A operands are read from LDS in the same order.
// LDS tiles are fp16 row-major with 16-byte chunks XOR-swizzled by row; the
// operands that need a tile transposed (K^T, and V in accumulator order) are
// read with gfx950's transposing LDS load instead of a second, transposed copy.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace chunked {

constexpr int C = 64;                    // tokens per chunk
constexpr int NB = C / 16;               // 16-token blocks per chunk
constexpr int NTB = NB * (NB + 1) / 2;   // lower 16x16 blocks of a chunk matrix
constexpr int TBLK = 256;                // halfs per 16x16 block
constexpr int NGATE = 3 * C;             // per-chunk gate floats: g, gamma, d
constexpr int WS_CHUNK = NTB * TBLK + 2 * NGATE;   // workspace halfs per (head, chunk)
constexpr float kLogDecayFloor = -30.0f; // exp(-30) ~ 9e-14: alpha = 0 stays finite
constexpr int kXcds = 8;
constexpr int kStatusBytes = 256;        // workspace header holding the call's device status word

// Row I of lower block number b in the order (0,0),(1,0),(1,1),(2,0),(2,1),
// (2,2),(3,0),...; its column is b - I (I + 1) / 2.
__device__ __forceinline__ int lower_block_row(int b) { return b >= 6 ? 3 : b >= 3 ? 2 : b >= 1 ? 1 : 0; }

typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4v mma(half8 a, half8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half4 to_h4(float a, float b, float c, float d) {
    return half4{static_cast<_Float16>(a), static_cast<_Float16>(b), static_cast<_Float16>(c),
                 static_cast<_Float16>(d)};
}
__device__ __forceinline__ half4 to_h4(float4v v) { return to_h4(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ half8 cat(half4 lo, half4 hi) {
    return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Offset (in halfs) of element (row, col) of a row-major fp16 tile with LD
// halfs per row whose 16-byte chunks are XOR-swizzled by the row index.
template <int LD>
__device__ __forceinline__ int swz(int row, int col) {
    constexpr int kMask = LD / 8 - 1;   // LD / 8 chunks per row, a power of two
    return row * LD + (((col >> 3) ^ row) & kMask) * 8 + (col & 7);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4 a + b receives, in slot j, element b of the 4-element run addressed
// by lane 4 j + a of the same group.
typedef __fp16 fp16x4_tr __attribute__((__vector_size__(8)));
__device__ __forceinline__ half4 ld_tr4(const _Float16* p) {
    const fp16x4_tr r = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
        (__attribute__((address_space(3))) fp16x4_tr*)(const_cast<_Float16*>(p)));
    return __builtin_bit_cast(half4, r);
}
template <int LD>
__device__ __forceinline__ half4 ld4(const _Float16* base, int row, int col) {
    return *reinterpret_cast<const half4*>(base + swz<LD>(row, col));
}
template <int LD>
__device__ __forceinline__ half8 ld8(const _Float16* base, int row, int col) {
    return *reinterpret_cast<const half8*>(base + swz<LD>(row, col));
}
// Split-K operand of row `row` for the 32-wide K step starting at k0.
template <int LD>
__device__ __forceinline__ half8 ld_split(const _Float16* base, int row, int k0, int g) {
    return cat(ld4<LD>(base, row, k0 + 4 * g), ld4<LD>(base, row, k0 + 16 + 4 * g));
}
// Same for a 16-wide K (only the lower four slots carry data).
template <int LD>
__device__ __forceinline__ half8 ld_split_lo(const _Float16* base, int row, int k0, int g) {
    return cat(ld4<LD>(base, row, k0 + 4 * g), half4{});
}
// Split-K operand of the transpose of a row-major (swz<LD>) tile X: lane
// (m + 16 g) gets X[k0 + 16 (s / 4) + 4 g + s % 4][m0 + m] in slot s, so the
// operand's rows are columns m0 .. m0 + 15 of X and its K index runs over rows
// k0 .. k0 + 31 of X.  Lane (4 j + a) of group g addresses the run
// X[k0 + 4 g + j][m0 + 4 a .. + 4] (and 16 rows further for slots 4 .. 7).
template <int LD>
__device__ __forceinline__ half8 ld_split_tr(const _Float16* base, int m0, int k0, int lane) {
    const int g = lane >> 4, x = lane & 15;
    const int row = k0 + 4 * g + (x >> 2), col = m0 + 4 * (x & 3);
    return cat(ld_tr4(base + swz<LD>(row, col)), ld_tr4(base + swz<LD>(row + 16, col)));
}

// ===========================================================================
// prep_kernel: T' = (I + A)^-1 diag(beta) for one (head, chunk), one wave per
// chunk.  Every product runs from registers, so the waves never wait for one
// another:
//   * the Gram tiles K_J K_I^T come from bf16 MFMAs on k fragments loaded
//     straight from HBM (lane (r + 16 g) of the fragment of token block I
//     holds row 16 I + r, columns 8 g .. + 8 of each 32-wide step; the same
//     fragment serves as the A operand of one tile and the B operand of
//     another);
//   * each lane then holds 4 consecutive columns of one row of A, which is
//     exactly the A operand of a 16x16x16 MFMA, so A's sub-diagonal blocks stay
//     in registers;
//   * the 16x16 diagonal blocks of T are inverted by forward substitution in
//     float32 (lane = (block, column)), then one block sub-diagonal per step,
//         T'_IJ = -T_II * sum_{K=J}^{I-1} A_IK T'_KJ,   T'_JJ = T_JJ diag(beta_J),
//     (the column scaling by beta commutes with the sum, so T' is built
//     directly), whose accumulator layout is again the B operand of the next
//     step.
// The k fragments of the wave's next chunk reuse the registers of the
// current one once its Gram tiles are formed.  Per-wave LDS only stages the
// diagonal blocks and the output.
// ===========================================================================
constexpr int kPrepWaves = 4;        // waves (chunks in flight) per workgroup
constexpr int kPrepResidentWGs = 768; // three workgroups per CU

template <int DK>
struct PrepCfg {
    static constexpr int KSTEP = DK >= 32 ? DK / 32 : 1;   // MFMA K steps over d_k
    static constexpr int LDA = 16 + 4;                     // float row stride of a diagonal block
    static constexpr int ABLK = 16 * LDA + 8;              // float stride between blocks (bank offset)
};

// One wave's staging area.  The diagonal blocks of A are dead once the
// substitution has read them, so the diagonal blocks of T reuse their space
// (one wave's LDS reads and writes execute in program order).
struct alignas(16) PrepWaveSmem {
    union {
        float Ad[NB * (16 * (16 + 4) + 8)];   // diagonal blocks of A, float32 row-major
        struct {
            _Float16 Tc[NB * TBLK];           // diagonal blocks of T', column-major
            _Float16 Tu[NB * TBLK];           // diagonal blocks of T (unscaled), row-major
        } t;
    };
    _Float16 Tr[NTB * TBLK];                  // T', lower blocks row-major (the output)
    float g[C], beta[C];
};

template <int DK>
struct PrepFrag {
    static constexpr bool kWide = DK >= 32;
    using type = typename std::conditional<kWide, uint4, uint2>::type;
};

__device__ __forceinline__ float4v mma_gram(uint4 a, uint4 b, float4v c) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ float4v mma_gram(uint2 a, uint2 b, float4v c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                    0, 0, 0);
}
__device__ __forceinline__ float4v mma16(half4 a, half4 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void prep_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__host__ __device__ constexpr int lower_tile(int I, int J) { return I * (I + 1) / 2 + J; }

// Inclusive prefix sum over the 64 lanes with DPP moves: shifts by 1, 2, 4, 8
// within each row of 16 lanes (zeros shifted in), then the last lane of row 0
// added to row 1 and of row 2 to row 3, then lane 31 added to rows 2 and 3.
template <int kCtrl, int kRowMask, bool kZeroFill>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xf, kZeroFill));
}
__device__ __forceinline__ float wave_scan_incl(float v) {
    v += dpp_move<0x111, 0xf, true>(v);   // row_shr:1
    v += dpp_move<0x112, 0xf, true>(v);   // row_shr:2
    v += dpp_move<0x114, 0xf, true>(v);   // row_shr:4
    v += dpp_move<0x118, 0xf, true>(v);   // row_shr:8
    v += dpp_move<0x142, 0xa, false>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_move<0x143, 0xc, false>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Workspace layout: a kStatusBytes header whose first word is the call's
// device status (cleared by prep_kernel, set by a wait in main_kernel that
// gave up), then for each (b*H + h, chunk), WS_CHUNK halfs: the NTB lower
// 16x16 blocks of T' in the order (0,0),(1,0),(1,1),(2,0),...,(3,3), each
// row-major fp16, then the float32 gates g[C], gamma[C], d[C].
//
// Grid (ceil(B*H / kPrepWaves), ceil(chunks / cpw)): wave w of workgroup
// (x, y) takes head bh = kPrepWaves x + w and its chunks y cpw + j, j < cpw.
// Neighbouring workgroups run the same chunks of neighbouring heads, so the k
// rows in flight at one time are whole token rows of the (token, head, d_k)
// tensor rather than scattered 256-byte pieces.  cpw is chosen so that the
// grid is about one round of resident workgroups: each wave then pays the
// latency of its first k load once and hides the others behind its work.
// Rows past the end of the sequence load the last row (their beta is 0, so A
// has zero rows there and they never matter).
template <int DK>
__global__ __launch_bounds__(256, 3) void prep_kernel(const uint16_t* __restrict__ k,
                                                   const float* __restrict__ alpha,
                                                   const float* __restrict__ beta,
                                                   _Float16* __restrict__ ws, unsigned* __restrict__ status,
                                                   int T, int H, int BH, int nchunks, int cpw) {
    using Cfg = PrepCfg<DK>;
    using Frag = typename PrepFrag<DK>::type;
    constexpr int KS = Cfg::KSTEP, LDA = Cfg::LDA, ABLK = Cfg::ABLK;
    constexpr int FW = PrepFrag<DK>::kWide ? 8 : 4;   // bf16 elements per lane and K step
    __shared__ PrepWaveSmem smem[kPrepWaves];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int lr = l & 15, lq = l >> 4;
    PrepWaveSmem& sm = smem[w];
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *status = 0u;   // this call's status
    const int bh = static_cast<int>(blockIdx.x) * kPrepWaves + w;
    if (bh >= BH) return;   // no workgroup barriers below
    const int b = bh / H, h = bh % H;
    const long tok0 = static_cast<long>(b) * T;
    auto chunk_of = [&](int j) { return static_cast<int>(blockIdx.y) * cpw + j; };

    // lane (r + 16 g) of fragment [I][kk]: k row 16 I + r, columns kk * 32 + FW g .. + FW
    Frag kf[NB][KS];
    float ar = 1.f, br = 0.f;
    auto load = [&](int chunk) {
        const int t0 = chunk * C;
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            const uint16_t* p = k + ((tok0 + min(t0 + 16 * I + lr, T - 1)) * H + h) * DK + FW * lq;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) kf[I][kk] = *reinterpret_cast<const Frag*>(p + 32 * kk);
        }
        const long off = (tok0 + min(t0 + l, T - 1)) * H + h;
        ar = alpha[off];
        br = beta[off];
    };
    if (chunk_of(0) < nchunks) load(chunk_of(0));

    for (int j = 0; j < cpw; ++j) {
        const int chunk = chunk_of(j);
        if (chunk >= nchunks) break;
        const int t0 = chunk * C;
        // gates: in-chunk prefix sum of log alpha (identity steps past the end)
        float lg;
        {
            const float a = (t0 + l < T) ? ar : 1.f, be = (t0 + l < T) ? br : 0.f;
            lg = wave_scan_incl(fmaxf(logf(a), kLogDecayFloor));
            sm.g[l] = lg;
            sm.beta[l] = be;
        }
        prep_wave_sync();
        // Gram tiles K_J K_I^T (I >= J) in two groups of five independent
        // chains, each masked into A = strictLower(diag(beta) (Gamma o K K^T))
        // at once.  Lane (r + 16 g) of tile (I, J) holds row 16 I + r, columns
        // 16 J + 4 g .. + 4.
        half4 ah[NTB];
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
            float4v acc[5];
#pragma unroll
            for (int u = 0; u < 5; ++u) acc[u] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int u = 0; u < 5; ++u) {
                    const int t = grp * 5 + u, I = lower_block_row(t), J = t - I * (I + 1) / 2;
                    acc[u] = mma_gram(kf[J][kk], kf[I][kk], acc[u]);
                }
            // The fragments are dead after the second group, so the next
            // chunk's loads may go out from here on.  (The compiler moves
            // them to the loop's back edge; forcing them here, unconditional
            // and behind a scheduling barrier, measured no faster.)
            if (grp == 1 && j + 1 < cpw && chunk_of(j + 1) < nchunks) load(chunk_of(j + 1));
#pragma unroll
            for (int u = 0; u < 5; ++u) {
                const int t = grp * 5 + u, I = lower_block_row(t), J = t - I * (I + 1) / 2;
                const int row = I * 16 + lr, col0 = J * 16 + 4 * lq;
                const float gt = sm.g[row], bt = sm.beta[row];
                const float4v gi = *reinterpret_cast<const float4v*>(&sm.g[col0]);
                float a[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = bt * __expf(gt - gi[e]) * acc[u][e];   // inf above the diagonal: not selected
                    a[e] = (I > J || col0 + e < row) ? v : 0.f;
                }
                if (I == J)
                    *reinterpret_cast<float4v*>(&sm.Ad[I * ABLK + lr * LDA + 4 * lq]) = float4v{a[0], a[1], a[2], a[3]};
                else
                    ah[t] = to_h4(a[0], a[1], a[2], a[3]);
            }
        }
        prep_wave_sync();

        // diagonal blocks of T = (I + A)^-1: lane (c + 16 bd) solves column c of
        // block bd, whose beta (token 16 bd + c) is the lane's own
        {
            const int bd = lq, c = lr;
            const float* Ab = sm.Ad + bd * ABLK;
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float s0 = (t == c) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
                for (int i4 = 0; i4 < (t + 3) / 4; ++i4) {
                    const float4v a4 = *reinterpret_cast<const float4v*>(&Ab[t * LDA + 4 * i4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * i4 + e;
                        if (i < t) {
                            if (e & 1) s1 -= a4[e] * x[i];
                            else s0 -= a4[e] * x[i];
                        }
                    }
                }
                x[t] = s0 + s1;
            }
            const float bc = sm.beta[l];
            half8 lo, hi;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                lo[t] = static_cast<_Float16>(x[t] * bc);
                hi[t] = static_cast<_Float16>(x[t + 8] * bc);
            }
            *reinterpret_cast<half8*>(&sm.t.Tc[bd * TBLK + c * 16]) = lo;
            *reinterpret_cast<half8*>(&sm.t.Tc[bd * TBLK + c * 16 + 8]) = hi;
            _Float16* Td = sm.Tr + lower_tile(bd, bd) * TBLK;
            _Float16* Tud = sm.t.Tu + bd * TBLK;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                Td[t * 16 + c] = lo[t];
                Td[(t + 8) * 16 + c] = hi[t];
                Tud[t * 16 + c] = static_cast<_Float16>(x[t]);
                Tud[(t + 8) * 16 + c] = static_cast<_Float16>(x[t + 8]);
            }
        }
        prep_wave_sync();

        // off-diagonal blocks, one sub-diagonal per step, in accumulator layout
        // (lane (n + 16 g): rows 4 g .. + 4 of column n), which is the B operand
        // layout of the next step's products
        half4 tcl[NB], trl[NB], th[NTB];
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            tcl[I] = *reinterpret_cast<const half4*>(&sm.t.Tc[I * TBLK + lr * 16 + 4 * lq]);   // T'_II, B layout
            trl[I] = *reinterpret_cast<const half4*>(&sm.t.Tu[I * TBLK + lr * 16 + 4 * lq]);   // T_II, A layout
        }
#pragma unroll
        for (int lev = 1; lev < NB; ++lev) {
#pragma unroll
            for (int J = 0; J + lev < NB; ++J) {
                const int I = J + lev;
                float4v y = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int Kb = J; Kb < I; ++Kb) y = mma16(ah[lower_tile(I, Kb)], Kb == J ? tcl[J] : th[lower_tile(Kb, J)], y);
                const float4v t = mma16(trl[I], to_h4(y), float4v{0.f, 0.f, 0.f, 0.f});
                const half4 tn = to_h4(-t[0], -t[1], -t[2], -t[3]);
                th[lower_tile(I, J)] = tn;
                _Float16* To = sm.Tr + lower_tile(I, J) * TBLK;
#pragma unroll
                for (int e = 0; e < 4; ++e) To[(4 * lq + e) * 16 + lr] = tn[e];
            }
        }
        prep_wave_sync();

        // T' out, in 16-byte pieces
        _Float16* dst = ws + (static_cast<long>(bh) * nchunks + chunk) * WS_CHUNK;
#pragma unroll
        for (int it = 0; it < NTB * TBLK / 8 / 64; ++it) {
            const int idx = l + it * 64;
            *reinterpret_cast<half8*>(dst + 8 * idx) = *reinterpret_cast<const half8*>(&sm.Tr[8 * idx]);
        }
        // gates for the chunk walk: g, gamma = exp(g), d = exp(g_last - g)
        {
            const float glast = __shfl(lg, 63, 64);
            float* gate = reinterpret_cast<float*>(dst + NTB * TBLK);
            gate[l] = lg;
            gate[C + l] = expf(lg);
            gate[2 * C + l] = expf(glast - lg);
        }
        prep_wave_sync();   // the staging area is rewritten by the next chunk
    }
}

// ===========================================================================
// main_kernel: the sequential chunk walk for one (head, 16-column slice).
// ===========================================================================
template <int DK>
struct MainCfg {
    static constexpr int SV = 16;                  // value columns per workgroup
    static constexpr int NT = 512;                 // 8 waves
    // Waves w and w + 4 share a SIMD.  The state wave (0) shares its SIMD with
    // the lightest role, the misc loader (4); the q/k loaders are waves 3, 5,
    // 6 and 7.
    static constexpr int W_STATE = 0, W_OUT0 = 1;  // state wave, output waves 1 and 2
    static constexpr int W_MISC = 4;               // v, T' and gates loader
    static constexpr int NQKW = 4;                 // q and k loader waves
    static constexpr int LQK = NQKW * 64;          // q/k loader threads
    static constexpr int QC = DK / 8;              // 16-byte pieces per q/k row
    static constexpr int NQ = (64 * QC + LQK - 1) / LQK;   // k (and q) pieces per thread
    static constexpr int NVI = 64 * (SV / 8) / 64;         // v pieces per misc lane
    static constexpr int NTI = NTB * TBLK / 8 / 64;        // T' pieces per misc lane
    static constexpr int NGI = (NGATE / 4 + 63) / 64;      // gate pieces per misc lane
    static constexpr int NMI = NVI + NTI + NGI;            // misc pieces per lane
    static constexpr int NA = 2 * NQ > NMI ? 2 * NQ : NMI;
    static constexpr int KSTEP = DK >= 32 ? DK / 32 : 1; // 32-wide K steps over d_k
    static constexpr int NST = DK / 16;            // 16-row state tiles
    static_assert(NTB * TBLK / 8 == NTI * 64, "T' pieces fill the misc wave");
    static_assert(NGATE / 4 <= 64 * NGI, "gate pieces fit the misc wave");
};

template <int DK>
struct alignas(16) MainSmem {
    using Cfg = MainCfg<DK>;
    _Float16 K[2][C * DK];
    _Float16 Q[2][C * DK];
    _Float16 Tp[2][C * C];
    _Float16 V[2][C * Cfg::SV];     // v slice, row-major (token, column)
    _Float16 ST[2][Cfg::SV * DK];   // f16 state slice transposed, by chunk parity
    _Float16 ET[Cfg::SV * C];       // E of the current chunk, transposed
    float gate[2][NGATE];           // g, gamma, d of each buffered chunk
    int flagE;
};

__device__ __forceinline__ half8 bf16x8_to_h8(const uint4& r) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    half8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = static_cast<_Float16>(__uint_as_float(w[i] << 16));
        o[2 * i + 1] = static_cast<_Float16>(__uint_as_float(w[i] & 0xffff0000u));
    }
    return o;
}

template <int DK>
struct Prefetch {
    uint4 a[MainCfg<DK>::NA];
    int chunk;
};

// Loader pieces are 16 bytes.  q/k waves (MISC = false): a[i] holds k and
// a[NQ + i] q at (token t, piece cq), with consecutive pieces of one row on
// consecutive lanes, so a wave's load covers whole rows.  Misc wave: a[0 .. NVI) hold v (token, piece of the
// slice), then NTI pieces of T' (its 10 lower blocks, in order), then the
// gate pieces.  Loads are unconditional: tokens past the end read the last
// token's row and pieces past the gates re-read the last one (always in
// bounds), so no load sits behind a branch.
template <int DK, bool MISC>
__device__ __forceinline__ void loader_load(Prefetch<DK>& pf, int chunk, int lt, int lane, const uint16_t* q,
                                            const uint16_t* k, const uint16_t* v, const _Float16* ws, long tok0,
                                            int T, int H, int DV, int col0, int h, long wsbase) {
    using Cfg = MainCfg<DK>;
    const int t0 = chunk * C;
    pf.chunk = chunk;
    auto row = [&](int t) { return (tok0 + min(t0 + t, T - 1)) * H + h; };
    if constexpr (!MISC) {
#pragma unroll
        for (int i = 0; i < Cfg::NQ; ++i) {
            const int idx = min(lt + i * Cfg::LQK, 64 * Cfg::QC - 1);
            const int t = idx / Cfg::QC, cq = idx % Cfg::QC;
            pf.a[i] = *reinterpret_cast<const uint4*>(k + row(t) * DK + cq * 8);
            pf.a[Cfg::NQ + i] = *reinterpret_cast<const uint4*>(q + row(t) * DK + cq * 8);
        }
    } else {
#pragma unroll
        for (int i = 0; i < Cfg::NVI; ++i) {
            const int idx = lane + i * 64;
            const int t = idx / (Cfg::SV / 8), cv = idx % (Cfg::SV / 8);
            pf.a[i] = *reinterpret_cast<const uint4*>(v + row(t) * DV + col0 + cv * 8);
        }
        const uint4* src = reinterpret_cast<const uint4*>(ws + wsbase + static_cast<long>(chunk) * WS_CHUNK);
#pragma unroll
        for (int i = 0; i < Cfg::NTI + Cfg::NGI; ++i)
            pf.a[Cfg::NVI + i] = src[min(lane + i * 64, WS_CHUNK / 8 - 1)];
    }
}

// bf16 pieces (q, k, v) -> fp16 pieces in place; T' and gate pieces are
// stored as they are.  Rows past the end of the sequence hold a copy of the
// last row and need no zeroing: there beta = 0 and alpha = 1 (set by
// prep_kernel), so T' has zero rows and columns for them and they reach
// neither E nor the state, and their y rows are never stored.
// The empty asm pins every converted piece to this point, so that the
// conversion is not sunk next to the stores.
template <int DK, bool MISC>
__device__ __forceinline__ void loader_convert(Prefetch<DK>& pf) {
    using Cfg = MainCfg<DK>;
    constexpr int N = MISC ? Cfg::NVI : 2 * Cfg::NQ;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const half8 hv = bf16x8_to_h8(pf.a[i]);
        pf.a[i] = *reinterpret_cast<const uint4*>(&hv);
        asm volatile("" : "+v"(pf.a[i].x), "+v"(pf.a[i].y), "+v"(pf.a[i].z), "+v"(pf.a[i].w));
    }
}

// 16-byte LDS store (half8 carries the 16-byte alignment that the uint4 type
// lacks, so this is one ds_write_b128 rather than two 8-byte writes).
__device__ __forceinline__ void st16(void* dst, const uint4& v) {
    *reinterpret_cast<half8*>(dst) = *reinterpret_cast<const half8*>(&v);
}

template <int DK, bool MISC, int buf>
__device__ __forceinline__ void loader_store(const Prefetch<DK>& pf, MainSmem<DK>& sm, int lt, int lane) {
    using Cfg = MainCfg<DK>;
    if constexpr (!MISC) {
#pragma unroll
        for (int i = 0; i < Cfg::NQ; ++i) {
            const int idx = lt + i * Cfg::LQK;
            if (idx < 64 * Cfg::QC) {
                const int t = idx / Cfg::QC, cq = idx % Cfg::QC;
                st16(&sm.K[buf][swz<DK>(t, cq * 8)], pf.a[i]);
                st16(&sm.Q[buf][swz<DK>(t, cq * 8)], pf.a[Cfg::NQ + i]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < Cfg::NVI; ++i) {
            const int idx = lane + i * 64;
            const int t = idx / (Cfg::SV / 8), cv = idx % (Cfg::SV / 8);
            st16(&sm.V[buf][t * Cfg::SV + cv * 8], pf.a[i]);
        }
#pragma unroll
        for (int i = 0; i < Cfg::NTI; ++i) {
            const int idx = lane + i * 64;
            const int blk = idx / 32, r = (idx % 32) / 2, hh = idx % 2;
            const int I = lower_block_row(blk), J = blk - I * (I + 1) / 2;
            st16(&sm.Tp[buf][swz<C>(I * 16 + r, J * 16 + 8 * hh)], pf.a[Cfg::NVI + i]);
        }
#pragma unroll
        for (int i = 0; i < Cfg::NGI; ++i) {
            const int idx = lane + i * 64;
            if (idx < NGATE / 4)
                st16(&sm.gate[buf][4 * idx], pf.a[Cfg::NVI + Cfg::NTI + i]);
        }
    }
}

// Wait until the state wave has published E of `chunk`.  Bounded by `spin`
// sleeps, so that a missing flag ends the wait instead of hanging the device;
// returns false when it gave up (the caller then reports it, see DevStatus).
template <int DK>
__device__ __forceinline__ bool wait_published(MainSmem<DK>& sm, int chunk, int spin) {
    if (spin <= 0) return false;   // a bound of 0 gives up at once (tests of the failure path)
    for (int it = 0; __hip_atomic_load(&sm.flagE, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <= chunk; ++it) {
        if (it >= spin) return false;
        __builtin_amdgcn_s_sleep(1);
    }
    return true;
}

// A wait that gave up sets bit 0 of the call's status word (read back by
// gdn_prefill_status) and poisons the rows it would have written with NaN.
struct DevStatus {
    unsigned* word;
    int spin;
    __device__ __forceinline__ void fail() const {
        if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
};

// Loader role: during chunk c the loads of chunk c+2 are issued into one
// register set and chunk c+1 (loaded during chunk c-1, in the other set) is
// converted and stored to the other LDS buffer.  One barrier after the
// prologue and one per chunk, as in the other roles.
template <int DK, bool MISC>
__device__ __forceinline__ void loader_role(MainSmem<DK>& sm, int nchunks, int lt, int lane, const uint16_t* q,
                                            const uint16_t* k,
                                            const uint16_t* v, const _Float16* ws, long tok0, int T, int H,
                                            int DV, int col0, int h, long wsbase) {
    Prefetch<DK> pa, pb;
    auto ld = [&](Prefetch<DK>& pf, int c) {
        loader_load<DK, MISC>(pf, min(c, nchunks - 1), lt, lane, q, k, v, ws, tok0, T, H, DV, col0, h, wsbase);
    };
    // chunk c goes to LDS buffer c & 1 (a compile-time constant at each call)
    auto put = [&](Prefetch<DK>& pf, auto buf) { loader_store<DK, MISC, decltype(buf)::value>(pf, sm, lt, lane); };
    const std::integral_constant<int, 0> even{};
    const std::integral_constant<int, 1> odd{};
    if (nchunks > 0) {
        ld(pa, 0);
        loader_convert<DK, MISC>(pa);
        put(pa, even);
        ld(pa, 1);
    }
    __syncthreads();
    // Chunk pairs in an unconditional body (exact wait counts), odd tail after.
    // Loads past the last chunk re-read it (clamped).  When c + 2 == nchunks
    // the second store writes that copy into the buffer of chunk c, which
    // nothing reads any more (chunk c + 1 is the last).
    int c = 0;
    for (; c + 1 < nchunks; c += 2) {
        ld(pb, c + 2);
        loader_convert<DK, MISC>(pa);
        put(pa, odd);    // chunk c + 1
        __syncthreads();
        ld(pa, c + 3);
        loader_convert<DK, MISC>(pb);
        put(pb, even);   // chunk c + 2
        __syncthreads();
    }
    if (c < nchunks) __syncthreads();
}

template <int DK>
struct StateRegs {
    float4v S[MainCfg<DK>::NST];     // float32 state slice, accumulator layout
    half8 Sb[MainCfg<DK>::KSTEP];    // its fp16 split-K B operand
};

template <int DK>
__device__ __forceinline__ void state_refresh_operand(StateRegs<DK>& st) {
#pragma unroll
    for (int kk = 0; kk < MainCfg<DK>::KSTEP; ++kk) {
        if constexpr (DK >= 32) st.Sb[kk] = cat(to_h4(st.S[2 * kk]), to_h4(st.S[2 * kk + 1]));
        else st.Sb[kk] = cat(to_h4(st.S[0]), half4{});
    }
}

// One chunk of the state chain (state wave), software-pipelined by hand: each
// group of MFMAs finds its operand fragments already in registers because
// their LDS reads were issued one group earlier.  Scheduling barriers keep the
// compiler from sinking the reads back next to their uses (it would otherwise
// wait on every read).
template <int DK, int buf>
__device__ __forceinline__ void state_chunk(MainSmem<DK>& sm, StateRegs<DK>& st, int chunk, int lane) {
    using Cfg = MainCfg<DK>;
    constexpr int KS = Cfg::KSTEP;
    constexpr int NST = Cfg::NST;
    constexpr int NH = NST / 2 > 0 ? NST / 2 : 1;   // state tiles per half of the update
    const int lr = lane & 15, lq = lane >> 4;
    const _Float16* Kb = sm.K[buf];
    const _Float16* Tb = sm.Tp[buf];
    auto kfrag = [&](int I, int kk) {
        return DK >= 32 ? ld_split<DK>(Kb, I * 16 + lr, kk * 32, lq) : ld_split_lo<DK>(Kb, I * 16 + lr, 0, lq);
    };
    // K S, one 32-wide K step at a time, the next step's fragments in flight
    half8 ka[2][NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) ka[0][I] = kfrag(I, 0);
    half4 vv[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I)
        vv[I] = ld_tr4(&sm.V[buf][(I * 16 + 4 * lq + (lr >> 2)) * Cfg::SV + 4 * (lr & 3)]);
    float4v ks[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) ks[I] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        if (kk + 1 < KS) {
#pragma unroll
            for (int I = 0; I < NB; ++I) ka[(kk + 1) & 1][I] = kfrag(I, kk + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int I = 0; I < NB; ++I) ks[I] = mma(ka[kk & 1][I], st.Sb[kk], ks[I]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // T' and the first half of K^T, read while K S finishes
    half8 ta[NB][2];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        ta[I][0] = ld_split<C>(Tb, I * 16 + lr, 0, lq);
        ta[I][1] = I >= 2 ? ld_split<C>(Tb, I * 16 + lr, 32, lq) : half8{};
    }
    half8 kt0[NH][2];
#pragma unroll
    for (int r = 0; r < NH; ++r) {
        kt0[r][0] = ld_split_tr<DK>(Kb, r * 16, 0, lane);
        kt0[r][1] = ld_split_tr<DK>(Kb, r * 16, 32, lane);
    }
    float4v gm[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) gm[I] = *reinterpret_cast<const float4v*>(&sm.gate[buf][C + I * 16 + 4 * lq]);
    const float gl = sm.gate[buf][C + C - 1];
    __builtin_amdgcn_sched_barrier(0);
    // R = V - gamma K S, as the split-K B operand of T' R
    half4 rh[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I)
        rh[I] = to_h4(static_cast<float>(vv[I][0]) - gm[I][0] * ks[I][0], static_cast<float>(vv[I][1]) - gm[I][1] * ks[I][1],
                      static_cast<float>(vv[I][2]) - gm[I][2] * ks[I][2], static_cast<float>(vv[I][3]) - gm[I][3] * ks[I][3]);
    const half8 Rb0 = cat(rh[0], rh[1]), Rb1 = cat(rh[2], rh[3]);
    // E = T' R (T' is zero above the diagonal blocks)
    float4v e[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        e[I] = mma(ta[I][0], Rb0, float4v{0.f, 0.f, 0.f, 0.f});
        if (I >= 2) e[I] = mma(ta[I][1], Rb1, e[I]);
    }
    // gamma_last S, the accumulator input of the update (computed while T' R runs)
#pragma unroll
    for (int r = 0; r < NST; ++r) st.S[r] *= gl;
    __builtin_amdgcn_sched_barrier(0);
    // publish E for the output waves before the state update
#pragma unroll
    for (int I = 0; I < NB; ++I) *reinterpret_cast<half4*>(&sm.ET[swz<C>(lr, I * 16 + 4 * lq)]) = to_h4(e[I]);
    __hip_atomic_store(&sm.flagE, chunk + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    // second half of K^T and the decay-to-chunk-end factors, read while T' R runs
    half8 kt1[NH][2];
#pragma unroll
    for (int r = 0; r < NH; ++r) {
        if (NH + r < NST) {
            kt1[r][0] = ld_split_tr<DK>(Kb, (NH + r) * 16, 0, lane);
            kt1[r][1] = ld_split_tr<DK>(Kb, (NH + r) * 16, 32, lane);
        }
    }
    float4v dc[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) dc[I] = *reinterpret_cast<const float4v*>(&sm.gate[buf][2 * C + I * 16 + 4 * lq]);
    __builtin_amdgcn_sched_barrier(0);
    // D E as the B operand of K^T (D E)
    half4 eh[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I)
        eh[I] = to_h4(dc[I][0] * e[I][0], dc[I][1] * e[I][1], dc[I][2] * e[I][2], dc[I][3] * e[I][3]);
    const half8 Eb0 = cat(eh[0], eh[1]), Eb1 = cat(eh[2], eh[3]);
    // S = gamma_last S + K^T D E, accumulated onto the scaled state
#pragma unroll
    for (int r = 0; r < NH; ++r) {
        st.S[r] = mma(kt0[r][0], Eb0, st.S[r]);
        st.S[r] = mma(kt0[r][1], Eb1, st.S[r]);
    }
#pragma unroll
    for (int r = 0; r < NH; ++r) {
        if (NH + r < NST) {
            st.S[NH + r] = mma(kt1[r][0], Eb0, st.S[NH + r]);
            st.S[NH + r] = mma(kt1[r][1], Eb1, st.S[NH + r]);
        }
    }
    _Float16* STn = sm.ST[buf ^ 1];
#pragma unroll
    for (int r = 0; r < NST; ++r) *reinterpret_cast<half4*>(&STn[swz<DK>(lr, r * 16 + 4 * lq)]) = to_h4(st.S[r]);
    state_refresh_operand(st);
}

// One chunk of output for output wave RP, which owns token blocks I0 = RP and
// I1 = 3 - RP (so both waves build five of the ten lower P tiles).  Its q
// rows, the k rows and the fp16 state slice come from LDS.  Everything is
// computed transposed (K_J Q_I^T for P, S^T Q^T, E^T P^T), so that each lane
// holds one token row: P feeds the last MFMA straight from registers in the
// split-K order, and y leaves as one 16-byte store per lane and block.
template <int DK, int buf, int RP>
__device__ __forceinline__ void output_chunk(MainSmem<DK>& sm, int chunk, int lane, float* ylane, long ytok,
                                             int T, float scale, const DevStatus& ds) {
    using Cfg = MainCfg<DK>;
    constexpr int KS = Cfg::KSTEP;
    constexpr int Irow[2] = {RP, 3 - RP};
    constexpr int Jmax = 3 - RP;   // highest k block either q block needs
    const int lr = lane & 15, lq = lane >> 4;
    const _Float16* Kb = sm.K[buf];
    const _Float16* Qb = sm.Q[buf];
    const _Float16* STb = sm.ST[buf];
    // contiguous K-slices: lane (r + 16 g) holds K-index 8 g .. 8 g + 7 of step
    // kk (for d_k = 16 only g < 2 carry data; the rest are zero)
    auto frag = [&](const _Float16* base, int row, int kk) {
        return (DK >= 32 || lq < 2) ? ld8<DK>(base, row, kk * 32 + 8 * lq) : half8{};
    };
    half8 sf[KS], qf[2][KS], kf[2][KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        sf[kk] = frag(STb, lr, kk);
        qf[0][kk] = frag(Qb, Irow[0] * 16 + lr, kk);
        qf[1][kk] = frag(Qb, Irow[1] * 16 + lr, kk);
        kf[0][kk] = frag(Kb, lr, kk);
    }
    __builtin_amdgcn_sched_barrier(0);
    // (Q S)^T = S^T Q^T for both blocks: lane (t + 16 g) gets columns 4 g .. 4 g + 3 of row t
    float4v qs[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        qs[0] = mma(sf[kk], qf[0][kk], qs[0]);
        qs[1] = mma(sf[kk], qf[1][kk], qs[1]);
    }
    // (Q K^T)^T tiles J <= I: k block J is read once, one block ahead of its MFMAs
    float4v pacc[2][NB];
#pragma unroll
    for (int J = 0; J <= Jmax; ++J) {
        if (J + 1 <= Jmax) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) kf[(J + 1) & 1][kk] = frag(Kb, (J + 1) * 16 + lr, kk);
        }
        __builtin_amdgcn_sched_barrier(0);
        pacc[0][J] = pacc[1][J] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if (J <= Irow[0]) pacc[0][J] = mma(kf[J & 1][kk], qf[0][kk], pacc[0][J]);
            pacc[1][J] = mma(kf[J & 1][kk], qf[1][kk], pacc[1][J]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // P = Gamma o (Q K^T) on the lower tiles, lane row t = 16 I + lr, columns
    // i = 16 J + 4 lq + j; only the diagonal tile needs the i <= t mask (the
    // exponentials of its masked entries may overflow; the select drops them).
    float4v gi4[NB];
#pragma unroll
    for (int J = 0; J <= Jmax; ++J) gi4[J] = *reinterpret_cast<const float4v*>(&sm.gate[buf][J * 16 + 4 * lq]);
    half8 Pb[2][2];
    float gam_t[2];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int I = Irow[ii];
        const int t = I * 16 + lr;
        const float gt = sm.gate[buf][t];
        gam_t[ii] = sm.gate[buf][C + t];
        half4 ph[NB];
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            if (J > I) {
                ph[J] = half4{};
                continue;
            }
            float p[4] = {__expf(gt - gi4[J][0]) * pacc[ii][J][0], __expf(gt - gi4[J][1]) * pacc[ii][J][1],
                          __expf(gt - gi4[J][2]) * pacc[ii][J][2], __expf(gt - gi4[J][3]) * pacc[ii][J][3]};
            if (J == I) {
#pragma unroll
                for (int j = 0; j < 4; ++j) p[j] = (4 * lq + j <= lr) ? p[j] : 0.f;
            }
            ph[J] = to_h4(p[0], p[1], p[2], p[3]);
        }
        Pb[ii][0] = cat(ph[0], ph[1]);
        Pb[ii][1] = cat(ph[2], ph[3]);
    }
    const bool published = wait_published(sm, chunk, ds.spin);
    if (!published) ds.fail();
    const float ysc = published ? scale : __builtin_nanf("");
    // Y^T = E^T P^T + gamma (Q S)^T: lane (t + 16 g) holds row t, columns 4 g .. 4 g + 3
    const half8 Ea0 = ld_split<C>(sm.ET, lr, 0, lq), Ea1 = ld_split<C>(sm.ET, lr, 32, lq);
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int I = Irow[ii];
        float4v yv = {gam_t[ii] * qs[ii][0], gam_t[ii] * qs[ii][1], gam_t[ii] * qs[ii][2], gam_t[ii] * qs[ii][3]};
        yv = mma(Ea0, Pb[ii][0], yv);
        if (I >= 2) yv = mma(Ea1, Pb[ii][1], yv);
        const int t = chunk * C + I * 16 + lr;
        // a plain store: the slices of a head write 64-byte pieces of each y
        // row, which merge in L2 (streaming stores measured 28% more HBM writes)
        if (t < T)
            *reinterpret_cast<float4v*>(ylane + t * ytok) =
                float4v{ysc * yv[0], ysc * yv[1], ysc * yv[2], ysc * yv[3]};
    }
}

// Output role: one barrier after the prologue and one per chunk.  ylane
// points at this lane's four y columns of token 0; ytok is the token stride.
template <int DK, int RP>
__device__ __forceinline__ void output_role(MainSmem<DK>& sm, int nchunks, int lane, float* ylane, long ytok, int T,
                                            float scale, const DevStatus& ds) {
    __syncthreads();
    for (int c = 0; c < nchunks; c += 2) {
        output_chunk<DK, 0, RP>(sm, c, lane, ylane, ytok, T, scale, ds);
        __syncthreads();
        if (c + 1 < nchunks) {
            output_chunk<DK, 1, RP>(sm, c + 1, lane, ylane, ytok, T, scale, ds);
            __syncthreads();
        }
    }
}

template <int DK>
__global__ __launch_bounds__(512) void main_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, const _Float16* __restrict__ ws,
                                                   const float* __restrict__ S0, float* __restrict__ S_out,
                                                   float* __restrict__ y, int B, int T, int H, int DV, int nsl,
                                                   float scale, DevStatus ds) {
    using Cfg = MainCfg<DK>;
    __shared__ MainSmem<DK> sm;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;
    // block -> (head, slice): the slices of a head share block ids modulo kXcds
    const int xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
    const int bh = (jx / nsl) * kXcds + xcd;
    const int slice = jx % nsl;
    if (bh >= B * H) return;
    const int b = bh / H, h = bh % H;
    const int col0 = slice * Cfg::SV;
    const long tok0 = static_cast<long>(b) * T;
    const int nchunks = (T + C - 1) / C;
    const long wsbase = static_cast<long>(bh) * nchunks * WS_CHUNK;

    const bool is_state = (w == Cfg::W_STATE);
    const bool is_out = (w >= Cfg::W_OUT0 && w < Cfg::W_OUT0 + 2);
    const bool misc = (w == Cfg::W_MISC);
    const int lt = (w == 3 ? 0 : w - 4) * 64 + lane;   // q/k loader thread index (waves 3, 5, 6, 7)

    // T' is zero above its diagonal blocks; those halves of both buffers are never written again
    for (int idx = tid; idx < 2 * C * C; idx += Cfg::NT) (&sm.Tp[0][0])[idx] = static_cast<_Float16>(0.f);
    if (tid == 0) sm.flagE = 0;
    __syncthreads();

    // Each role runs its own loop with the same barrier sequence: one barrier
    // after the prologue and one after every chunk.  Keeping the roles in
    // separate loops keeps their registers from being live at the same time.
    if (is_state) {
        StateRegs<DK> st;
#pragma unroll
        for (int r = 0; r < Cfg::NST; ++r) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                st.S[r][j] = S0 ? S0[(static_cast<long>(bh) * DK + r * 16 + 4 * lq + j) * DV + col0 + lr] : 0.f;
            *reinterpret_cast<half4*>(&sm.ST[0][swz<DK>(lr, r * 16 + 4 * lq)]) = to_h4(st.S[r]);
        }
        state_refresh_operand(st);
        __syncthreads();
        // chunk pairs, so that each chunk's LDS buffer is a compile-time constant
        for (int c = 0; c < nchunks; c += 2) {
            state_chunk<DK, 0>(sm, st, c, lane);
            __syncthreads();
            if (c + 1 < nchunks) {
                state_chunk<DK, 1>(sm, st, c + 1, lane);
                __syncthreads();
            }
        }
        if (S_out) {
#pragma unroll
            for (int r = 0; r < Cfg::NST; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    S_out[(static_cast<long>(bh) * DK + r * 16 + 4 * lq + j) * DV + col0 + lr] = st.S[r][j];
        }
    } else if (is_out) {
        float* ylane = y + (tok0 * H + h) * static_cast<long>(DV) + col0 + 4 * lq;
        const long ytok = static_cast<long>(H) * DV;
        if (w == Cfg::W_OUT0) output_role<DK, 0>(sm, nchunks, lane, ylane, ytok, T, scale, ds);
        else output_role<DK, 1>(sm, nchunks, lane, ylane, ytok, T, scale, ds);
    } else if (misc) {
        loader_role<DK, true>(sm, nchunks, lt, lane, q, k, v, ws, tok0, T, H, DV, col0, h, wsbase);
    } else {
        loader_role<DK, false>(sm, nchunks, lt, lane, q, k, v, ws, tok0, T, H, DV, col0, h, wsbase);
    }
}

template <int DK>
static hipError_t launch_t(const PrefillArgs& a) {
    using Cfg = MainCfg<DK>;
    const int nchunks = (a.T + C - 1) / C;
    unsigned* status = static_cast<unsigned*>(a.workspace);
    _Float16* ws = reinterpret_cast<_Float16*>(static_cast<char*>(a.workspace) + kStatusBytes);
    if (nchunks > 0) {
        // chunks per wave: about one round of resident workgroups, at most 16
        const int BH = a.B * a.H;
        const long gx = (BH + kPrepWaves - 1) / kPrepWaves;
        const int cpw = static_cast<int>(
            std::min<long>(16, std::max<long>(1, (gx * nchunks + kPrepResidentWGs - 1) / kPrepResidentWGs)));
        const int gy = (nchunks + cpw - 1) / cpw;
        hipLaunchKernelGGL((prep_kernel<DK>), dim3(static_cast<unsigned>(gx), gy), dim3(256), 0, a.stream,
                           static_cast<const uint16_t*>(a.k), a.alpha, a.beta, ws, status, a.T, a.H, BH, nchunks,
                           cpw);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nsl = a.dv / Cfg::SV;
    const int groups = (a.B * a.H + kXcds - 1) / kXcds;
    hipLaunchKernelGGL((main_kernel<DK>), dim3(groups * kXcds * nsl), dim3(Cfg::NT), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), ws, a.initial_state, a.final_state, a.y,
                       a.B, a.T, a.H, a.dv, nsl, a.scale, DevStatus{status, a.spin_limit});
    return hipGetLastError();
}

}  // namespace chunked

size_t prefill_bf16_workspace_bytes(int B, int T, int H) {
    const long nchunks = (T + chunked::C - 1) / chunked::C;
    return chunked::kStatusBytes + static_cast<size_t>(B) * H * nchunks * chunked::WS_CHUNK * sizeof(_Float16);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a) {
    switch (a.dk) {
        case 16: return chunked::launch_t<16>(a);
        case 32: return chunked::launch_t<32>(a);
        case 64: return chunked::launch_t<64>(a);
        case 128: return chunked::launch_t<128>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
