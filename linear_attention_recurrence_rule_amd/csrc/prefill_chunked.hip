// bf16 chunked prefill of the gated delta rule on gfx950 (slinene
// ai-papers-daily page on Qwen3.8-Next, Module A: the delta-form recurrence,
// evaluated 64 tokens at a time in its chunkwise WY / UT-transform form).
//
// Per chunk of C = 64 tokens with start state S (g = in-chunk prefix sum of
// log alpha, gamma = exp(g), Gamma_ti = exp(g_t - g_i), d_t = exp(g_last - g_t);
// the kernels keep g in base-2 units, g2 = g / ln 2, so that every decay
// factor is one native 2^x):
//   A  = strictLower(diag(beta) (Gamma o K K^T)),   T' = (I + A)^-1 diag(beta)
//   E  = T' (V - diag(gamma) K S)          (rows: beta_t times token t's miss)
//   Y  = diag(gamma) Q S + P E,            P = lower(Gamma o Q K^T)
//   S' = gamma_last S + K^T diag(d) E
// T' and the gates depend only on k, alpha and beta, so a chunk-parallel
// kernel (prep_kernel) computes them once per (head, chunk) into a workspace; the
// sequential kernel (main_kernel) then runs the chunks of one (head,
// 16-column value slice) in order.
//
// main_kernel's roles and periods are described where it is defined below.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace chunked {

constexpr int C = 64;                    // tokens per chunk
constexpr int NB = C / 16;               // 16-token blocks per chunk
constexpr int NTB = NB * (NB + 1) / 2;   // lower 16x16 blocks of a chunk matrix
constexpr int TBLK = 256;                // halfs per 16x16 block
constexpr int NGATE = 4 * C;             // per-chunk gate floats: g2, gamma, d, w
constexpr int NTT = 6;                   // 16 x 32 tiles of T' in the workspace
constexpr int TTILE = 16 * 32;           // halfs per such tile
constexpr int WS_CHUNK = NTT * TTILE + 2 * NGATE;   // workspace halfs per (head, chunk)
constexpr float kLog2DecayFloor = -43.280851f;   // log2 of e^-30 ~ 9e-14: alpha = 0 stays finite
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
constexpr int kPrepGridWGs = 6144;    // workgroups per launch (eight rounds of three per CU) before a wave takes several chunks

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
// device status (cleared by prep_kernel; main_kernel sets bit 0 when it wrote
// a non-finite y and bit 1 for a non-finite final state), then for each
// (b*H + h, chunk), WS_CHUNK halfs: T' as the NTT tiles (I, h) of its rows
// 16 I .. 16 I + 15 and columns 32 h .. 32 h + 31 that are not all zero, in
// the order (0,0),(1,0),(2,0),(2,1),(3,0),(3,1), each row-major fp16 with its
// columns in split-K order (position 8 g + s holds column
// 32 h + 16 (s / 4) + 4 g + s % 4), so that the A operand of one 32-token K
// step of T' R is one 16-byte piece; then the float32 gates g2[C], gamma[C],
// d[C], w[C].
//
// Grid gx x gy = (ceil(B*H / kPrepWaves), ceil(chunks / cpw)), launched as
// one dimension: wave w of workgroup (x, y) takes head bh = kPrepWaves x + w
// and its chunks y cpw + j, j < cpw.  Each XCD runs every head group of one
// chunk group before the next, so the k rows in flight on it are whole token
// rows of the (token, head, d_k) tensor and the alpha / beta lines of a chunk
// are fetched once.  cpw is 1 unless the grid
// would exceed kPrepGridWGs workgroups: the resident waves of one round then
// hide the k-load latency of the next (measured 79.5 us at 32 heads x 512
// chunks, against 89.6 us with six chunks per wave and one round); a wave
// with several chunks loads the next one while it works on the current.
// Rows past the end of the sequence load the last row (their beta is 0, so A
// has zero rows there and they never matter).
template <int DK>
__global__ __launch_bounds__(256, 3) void prep_kernel(const uint16_t* __restrict__ k,
                                                   const float* __restrict__ alpha,
                                                   const float* __restrict__ beta,
                                                   _Float16* __restrict__ ws, unsigned* __restrict__ status,
                                                   int T, int H, int BH, int nchunks, int cpw, int gx, int gy) {
    using Cfg = PrepCfg<DK>;
    using Frag = typename PrepFrag<DK>::type;
    constexpr int KS = Cfg::KSTEP, LDA = Cfg::LDA, ABLK = Cfg::ABLK;
    constexpr int FW = PrepFrag<DK>::kWide ? 8 : 4;   // bf16 elements per lane and K step
    __shared__ PrepWaveSmem smem[kPrepWaves];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int lr = l & 15, lq = l >> 4;
    PrepWaveSmem& sm = smem[w];
    if (blockIdx.x == 0 && threadIdx.x == 0) *status = 0u;   // this call's status
    // workgroup (bx, by) of the gx x gy grid: consecutive workgroup ids go to
    // the XCDs in turn, and each XCD takes every head group of one chunk group
    // before the next, so the alpha and beta lines of a chunk (one 128-byte
    // line holds 32 heads of a token) are fetched into one L2 only
    const int xcd = static_cast<int>(blockIdx.x) % kXcds, jx = static_cast<int>(blockIdx.x) / kXcds;
    const int bx = jx % gx, by = (jx / gx) * kXcds + xcd;
    const int bh = bx * kPrepWaves + w;
    if (by >= gy || bh >= BH) return;   // no workgroup barriers below
    const int b = bh / H, h = bh % H;
    const long tok0 = static_cast<long>(b) * T;
    auto chunk_of = [&](int j) { return by * cpw + j; };

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
            lg = wave_scan_incl(fmaxf(__log2f(a), kLog2DecayFloor));
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
                    const float v = bt * __builtin_amdgcn_exp2f(gt - gi[e]) * acc[u][e];   // inf above the diagonal: not selected
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
            // x[t] = 0 for t < c and x[c] = 1 exactly (every earlier x is 0);
            // the selection below keeps the loop-invariant identity column out of
            // registers (as 16 constants it had pushed the kernel into a spill)
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float s0 = 0.f, s1 = 0.f;
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
                x[t] = (t == c) ? 1.f : s0 + s1;
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

        // T' out, one 16-byte piece per lane and tile: lane (4 r + g) of tile
        // (I, h) writes row r, split-K positions 8 g .. 8 g + 7, which are
        // columns 4 g .. 4 g + 3 of blocks (I, 2 h) and (I, 2 h + 1)
        _Float16* dst = ws + (static_cast<long>(bh) * nchunks + chunk) * WS_CHUNK;
#pragma unroll
        for (int it = 0; it < NTT; ++it) {
            const int I = it >= 4 ? 3 : (it >= 2 ? 2 : it), hh = (it == 3 || it == 5) ? 1 : 0;
            const int r = l >> 2, g = l & 3;
            const half4 lo = *reinterpret_cast<const half4*>(&sm.Tr[lower_tile(I, 2 * hh) * TBLK + r * 16 + 4 * g]);
            const half4 hi = 2 * hh + 1 <= I
                                 ? *reinterpret_cast<const half4*>(&sm.Tr[lower_tile(I, 2 * hh + 1) * TBLK + r * 16 + 4 * g])
                                 : half4{};
            *reinterpret_cast<half8*>(dst + it * TTILE + 8 * l) = cat(lo, hi);
        }
        // gates for the chunk walk, all in base 2: g2, gamma = 2^g2,
        // d = 2^(g2_last - g2) and w = 2^(g2_b - g2), where g2_b is the value
        // at the end of the token's 16-token block (the column factor of the
        // off-diagonal decay blocks of P, which are then u_t w_i with
        // u_t = 2^(g2_t - g2_b) <= 1 and w_i <= 1)
        {
            const float glast = __shfl(lg, 63, 64);
            const float gblk = __shfl(lg, l | 15, 64);
            float* gate = reinterpret_cast<float*>(dst + NTT * TTILE);
            gate[l] = lg;
            gate[C + l] = __builtin_amdgcn_exp2f(lg);
            gate[2 * C + l] = __builtin_amdgcn_exp2f(glast - lg);
            gate[3 * C + l] = __builtin_amdgcn_exp2f(gblk - lg);
        }
        prep_wave_sync();   // the staging area is rewritten by the next chunk
    }
}

// ===========================================================================
// main_kernel: the sequential chunk walk for one (head, 16-column slice).
// ===========================================================================
//
// One workgroup of 8 waves per (sequence b, head h, 16 value columns); wave w
// runs on SIMD w % 4.  The walk is cut into periods that end at a workgroup
// barrier.  In period p:
//   wave 0 (state)      chunk p: K S, R = V - gamma K S, E = T' R (written to
//                       ET[p & 1]), S <- gamma_last S + K^T D E, and the fp16
//                       copy of the new state to ST[(p + 1) & 1];
//   waves 1, 5, 2, 6    (output, one per 16-token block 3, 0, 2, 1): gamma (Q S)
//                       and P of chunk p from S_p (ST[p & 1]), K_p and their own
//                       q rows, which they load from memory two periods ahead;
//                       then y of chunk p - 1 = gamma (Q S) + P E from the
//                       gamma Q S and P of chunk p - 1 kept in registers and
//                       E_{p-1} from ET[(p - 1) & 1];
//   wave 3 (misc)       v slice, T' and gates of chunk p + 1 into LDS;
//   waves 4 and 7 (k)   k of chunk p + 1 into LDS (bf16 -> fp16).
// Nothing a period reads is written in the same period, so no role waits on
// another between barriers.  Loaders and the output waves' q loads run two
// chunks ahead in two register sets (chunk c in set c & 1).
//
// Memory access goes through buffer descriptors whose base moves by whole
// chunks in scalar registers: each lane's offsets are computed once, and
// rows past the end of the sequence read as zeros and are not written (the
// descriptor's size ends at token T).  Zero rows past the end are harmless:
// there beta = 0 and alpha = 1 (prep_kernel), so T' has zero rows and columns
// for them, they reach neither E nor the state, and their y is not stored.
//
// Split-K operand layout: for a 16x16x32 MFMA, slot s of lane (m + 16 g) holds
// K-index 16*(s/4) + 4 g + s%4 of its row/column.  Two 16x16 accumulator tiles
// (lane (n + 16 g) holds rows 4 g .. 4 g + 3 of column n) stacked along K are
// exactly such a B operand, and A operands are read from LDS in the same order.
// LDS tiles are fp16 row-major with 16-byte chunks XOR-swizzled by row; the
// operands that need a tile transposed (K^T, and V in accumulator order) are
// read with gfx950's transposing LDS load instead of a second, transposed copy.

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + bytes) (raw, stride 0): loads past the
// end return zeros, stores past the end are dropped.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long bytes) {
    const long b = bytes < 0 ? 0 : (bytes > 0x7fffffffL ? 0x7fffffffL : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(b),
                                             0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, int voff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
    return uint4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void bstore16(rsrc_t r, int voff, float4v v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, 0, 0);
}

template <int DK>
struct MainCfg {
    static constexpr int SV = 16;                  // value columns per workgroup
    static constexpr int NT = 512;                 // 8 waves
    // roles: state 0; output waves 1, 5 (blocks 3, 0; SIMD 1) and 2, 6 (blocks 2, 1; SIMD 2)
    static constexpr int W_STATE = 0, W_MISC = 3, W_K0 = 4, W_K1 = 7;
    static constexpr int QC = DK / 8;              // 16-byte pieces per q/k row
    static constexpr int KPL = C * QC / 64;        // k pieces per lane-slot and chunk
    static constexpr int NK0 = KPL * 3 / 8;        // ... on wave 4 (SIMD 0, with the state wave)
    static constexpr int NK1 = KPL - NK0;          // ... on wave 7 (SIMD 3, with the misc wave)
    static constexpr int NVI = C * (SV / 8) / 64;  // v pieces per misc lane
    static constexpr int NTI = NTT;                        // T' pieces per misc lane (one per tile)
    static constexpr int NGI = (NGATE / 4 + 63) / 64;      // gate pieces per misc lane
    static constexpr int NMI = NVI + NTI + NGI;            // misc pieces per lane
    static constexpr int KSTEP = DK >= 32 ? DK / 32 : 1;   // 32-wide K steps over d_k
    static constexpr int NST = DK / 16;            // 16-row state tiles
    static_assert(TTILE / 8 == 64, "a T' tile is one piece per lane");
    static_assert(NGATE / 4 <= 64 * NGI, "gate pieces fit the misc wave");
    static_assert(NK0 + NK1 == KPL && NK1 >= 1, "k pieces split over two waves");
};

template <int DK>
struct alignas(16) MainSmem {
    using Cfg = MainCfg<DK>;
    _Float16 K[2][C * DK];
    _Float16 Tp[2][C * C];
    _Float16 V[2][C * Cfg::SV];     // v slice, row-major (token, column)
    _Float16 ST[2][Cfg::SV * DK];   // fp16 state slice transposed: S_p in ST[p & 1]
    _Float16 ET[2][Cfg::SV * C];    // E of chunk p, transposed, in ET[p & 1]
    float gate[2][NGATE];           // g2, gamma, d, w of each buffered chunk
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

// 16-byte LDS store (half8 carries the 16-byte alignment that the uint4 type
// lacks, so this is one ds_write_b128 rather than two 8-byte writes).
__device__ __forceinline__ void st16(void* dst, const half8& v) { *reinterpret_cast<half8*>(dst) = v; }
__device__ __forceinline__ void st16(void* dst, const uint4& v) {
    *reinterpret_cast<half8*>(dst) = *reinterpret_cast<const half8*>(&v);
}

// Per-walk constants every role needs.  The q, k, v and y pointers are those
// of token 0, head 0 of this sequence: a chunk's descriptor starts at its first
// token and ends at token T of the sequence, and the lane offsets add the head
// (and slice) column, so no access leaves the sequence's rows.
struct Walk {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const _Float16* ws;  // this head's first chunk in the workspace
    float* y;
    long rowq;           // elements between consecutive tokens of q / k (H * DK)
    long rowv;           // ... of v and y (H * DV)
    unsigned hq;         // element offset of this head in a q / k row (h * DK)
    unsigned hv;         // ... of this head's slice in a v / y row (h * DV + col0)
    int T, nchunks;
    float scale;
    unsigned* status;    // the call's status word (null without a workspace: T = 0)
};

// Sets `bit` of the call's status word when any lane of the wave saw a
// non-finite value (an input or intermediate outside the fp16 operand range,
// or non-finite inputs).
__device__ __forceinline__ void report_nonfinite(unsigned* status, bool bad, unsigned bit) {
    if (status && __any(bad) && (threadIdx.x & 63) == 0)
        __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool nonfinite(float4v v) {
    return !(__builtin_isfinite(v[0]) && __builtin_isfinite(v[1]) && __builtin_isfinite(v[2]) &&
             __builtin_isfinite(v[3]));
}

// End of a period.  The scheduling barriers keep the compiler from moving
// work across it: left alone it hoists the next period's bf16 -> fp16
// conversions above the barrier, which makes the loaders wait for their
// newest loads as well.
__device__ __forceinline__ void period_end() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// Loader roles.  Chunk c's pieces live in register set c & 1.
// ---------------------------------------------------------------------------
template <int DK, int N>
struct Pieces {
    uint4 a[2][N];
};

// k loader: lane-slot ls (0 .. 63) of wave with `first` piece index; pieces
// i = first + j * 64 + ls cover whole rows (16 consecutive pieces per row at
// d_k = 128), so a wave's load is a run of contiguous rows.
template <int DK, int N>
struct KLoader {
    int voff[N];     // byte offset of each piece from the chunk's first k row
    int loff[N];     // its swizzled LDS offset (halfs)
    __device__ void init(int first, int ls, const Walk& w) {
        using Cfg = MainCfg<DK>;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int i = first + j * 64 + ls;
            const int t = i / Cfg::QC, cq = i % Cfg::QC;
            voff[j] = static_cast<int>((static_cast<unsigned>(t) * static_cast<unsigned>(w.rowq) + w.hq + cq * 8u) * 2u);
            loff[j] = swz<DK>(t, cq * 8);
        }
    }
    template <int set>
    __device__ void load(Pieces<DK, N>& p, const Walk& w, int chunk) const {
        const long t0 = static_cast<long>(chunk) * C;
        const rsrc_t r = make_rsrc(w.k + t0 * w.rowq, (w.T - t0) * w.rowq * 2);
#pragma unroll
        for (int j = 0; j < N; ++j) p.a[set][j] = bload16(r, voff[j]);
    }
    template <int set, int buf>
    __device__ void store(const Pieces<DK, N>& p, MainSmem<DK>& sm) const {
#pragma unroll
        for (int j = 0; j < N; ++j) st16(&sm.K[buf][loff[j]], bf16x8_to_h8(p.a[set][j]));
    }
};

// misc loader: v slice (converted), T' blocks and gates (fp16 / fp32 as stored).
template <int DK>
struct MiscLoader {
    using Cfg = MainCfg<DK>;
    int voff[Cfg::NVI], loff_v[Cfg::NVI], loff_t[Cfg::NTI];
    int lane;
    __device__ void init(int l, const Walk& w) {
        lane = l;
#pragma unroll
        for (int j = 0; j < Cfg::NVI; ++j) {
            const int i = l + j * 64, t = i / (Cfg::SV / 8), cv = i % (Cfg::SV / 8);
            voff[j] = static_cast<int>((static_cast<unsigned>(t) * static_cast<unsigned>(w.rowv) + w.hv + cv * 8u) * 2u);
            loff_v[j] = t * Cfg::SV + cv * 8;
        }
#pragma unroll
        for (int j = 0; j < Cfg::NTI; ++j) {
            // tile j of the workspace layout: (I, h) = (0,0),(1,0),(2,0),(2,1),(3,0),(3,1)
            const int I = j >= 4 ? 3 : (j >= 2 ? 2 : j), hh = (j == 3 || j == 5) ? 1 : 0;
            loff_t[j] = swz<C>(I * 16 + (l >> 2), 32 * hh + 8 * (l & 3));
        }
    }
    template <int set>
    __device__ void load(Pieces<DK, Cfg::NMI>& p, const Walk& w, int chunk) const {
        const long t0 = static_cast<long>(chunk) * C;
        const rsrc_t rv = make_rsrc(w.v + t0 * w.rowv, (w.T - t0) * w.rowv * 2);
#pragma unroll
        for (int j = 0; j < Cfg::NVI; ++j) p.a[set][j] = bload16(rv, voff[j]);
        const bool live = chunk < w.nchunks;
        const rsrc_t rw = make_rsrc(w.ws + static_cast<long>(chunk) * WS_CHUNK, live ? WS_CHUNK * 2 : 0);
#pragma unroll
        for (int j = 0; j < Cfg::NTI + Cfg::NGI; ++j) p.a[set][Cfg::NVI + j] = bload16(rw, (lane + j * 64) * 16);
    }
    template <int set, int buf>
    __device__ void store(const Pieces<DK, Cfg::NMI>& p, MainSmem<DK>& sm) const {
#pragma unroll
        for (int j = 0; j < Cfg::NVI; ++j) st16(&sm.V[buf][loff_v[j]], bf16x8_to_h8(p.a[set][j]));
#pragma unroll
        for (int j = 0; j < Cfg::NTI; ++j) st16(&sm.Tp[buf][loff_t[j]], p.a[set][Cfg::NVI + j]);
#pragma unroll
        for (int j = 0; j < Cfg::NGI; ++j) {
            const int i = lane + j * 64;
            if (i < NGATE / 4) st16(&sm.gate[buf][4 * i], p.a[set][Cfg::NVI + Cfg::NTI + j]);
        }
    }
};

// Loader role: prologue stores chunk 0 and has chunks 1 and 2 in flight; in
// period p it stores chunk p + 1 (buffer (p + 1) & 1, register set
// (p + 1) & 1) and then loads chunk p + 3 into the set it just emptied.
// The period bodies are unconditional, so that the compiler's wait counts
// stay exact across the loop (a load skipped on some path would make it wait
// for the newest loads too, exposing their latency every period): loads past
// the last chunk read zeros (the descriptors' sizes end at T) and the stores
// past it fill a buffer that nothing reads any more.
template <int DK, class L, class P>
__device__ __forceinline__ void loader_role(const L& ld, P& pcs, MainSmem<DK>& sm, const Walk& w) {
    const int n = w.nchunks;
    ld.template load<0>(pcs, w, 0);
    ld.template load<1>(pcs, w, 1);
    ld.template store<0, 0>(pcs, sm);
    ld.template load<0>(pcs, w, 2);
    period_end();
    // n + 1 periods, in pairs: p even stores set 1 -> buffer 1, p odd set 0 -> buffer 0
    int p = 0;
    for (; p + 1 <= n; p += 2) {
        ld.template store<1, 1>(pcs, sm);
        ld.template load<1>(pcs, w, p + 3);
        period_end();
        ld.template store<0, 0>(pcs, sm);
        ld.template load<0>(pcs, w, p + 4);
        period_end();
    }
    if (p <= n) period_end();
}

// ---------------------------------------------------------------------------
// State role.
//
// The state slice lives in NST accumulator tiles.  Their rows are the d_k
// rows of the state in an order chosen for the LDS reads (for d_k >= 32):
// the fp16 copy Sb[kk] = (tile 2 kk, tile 2 kk + 1) is the B operand of K
// step kk of K S, and there lane group g must hold 8 consecutive d_k rows, so
// that the matching A operand (K) is one 16-byte read.  Tile 2 kk + h, lane
// group g, element j therefore holds d_k row 8 ks_chunk(kk, g) + 4 h + j.
// ks_chunk picks the 16-byte chunk of each lane group so that the transposed
// reads of K^T for the update (runs of 4 rows of one tile) spread over all
// LDS banks.  For d_k = 16 the tile is in natural order.
// ---------------------------------------------------------------------------
template <int DK>
__device__ __forceinline__ int ks_chunk(int kk, int g) {
    return DK >= 64 ? 8 * (kk >> 1) + 2 * (kk & 1) + 4 * (g & 1) + (g >> 1) : g;
}
template <int DK>
__device__ __forceinline__ int state_row(int r, int g, int j) {
    return DK >= 32 ? 8 * ks_chunk<DK>(r >> 1, g) + 4 * (r & 1) + j : 4 * g + j;
}

template <int DK>
struct StateRegs {
    float4v S[MainCfg<DK>::NST];     // float32 state slice, accumulator layout
    half8 Sb[MainCfg<DK>::KSTEP];    // its fp16 B operand of K S
};

// State-saving walk (for the backward pass): the state wave leaves S_p (the
// fp32 state slice at the start of chunk p) and E_p in these buffers during
// period p, and the copy waves write them out in period p + 1.
template <int DK>
struct SaveBufs {
    float S[2][16][DK + 4];   // [slice column][d_k row]
    float E[2][16][C + 4];    // [slice column][token of the chunk]
};
struct NoSaveBufs {};

template <int DK>
__device__ __forceinline__ void state_refresh_operand(StateRegs<DK>& st) {
#pragma unroll
    for (int kk = 0; kk < MainCfg<DK>::KSTEP; ++kk) {
        if constexpr (DK >= 32) st.Sb[kk] = cat(to_h4(st.S[2 * kk]), to_h4(st.S[2 * kk + 1]));
        else st.Sb[kk] = cat(to_h4(st.S[0]), half4{});
    }
}

// The fp16 state slice, transposed and in natural d_k order, for the output
// waves: ST[column][d_k row].
template <int DK>
__device__ __forceinline__ void state_publish(const StateRegs<DK>& st, _Float16* STb, int lane) {
    const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int r = 0; r < MainCfg<DK>::NST; ++r)
        *reinterpret_cast<half4*>(&STb[swz<DK>(lr, state_row<DK>(r, lq, 0))]) = to_h4(st.S[r]);
}

// A operand of K step `ks` (32 tokens) of K^T D E for state tile r: lane
// (m + 16 g) gets K[k0 + 16 (s / 4) + 4 g + s % 4][row m of tile r] in slot s
// (tokens in the split-K order of the accumulator tiles of E).  Lane (4 j + a)
// of group g addresses the run of tile rows 4 a .. 4 a + 3 (consecutive d_k
// columns of K) in token row k0 + 4 g + j, and 16 rows further; k0 and the
// 16-row step are multiples of 16 rows, which the swizzle does not see.
template <int DK>
__device__ __forceinline__ half8 ld_kt(const _Float16* Kb, int r, int ks, int lane) {
    const int g = lane >> 4, x = lane & 15;
    const int o = swz<DK>(4 * g + (x >> 2), state_row<DK>(r, x & 3, 0));
    return cat(ld_tr4(Kb + ks * 32 * DK + o), ld_tr4(Kb + (ks * 32 + 16) * DK + o));
}

// One chunk of the state chain.  A wave issues in order, so the chunk is
// laid out by hand as a pipeline of MFMA groups with the VALU work that
// depends on an earlier group, and the LDS reads for a later one, placed
// between their MFMAs (scheduling barriers keep that order):
//   A  K S for row blocks 0, 1 (two interleaved accumulation chains)
//   B  K S for row blocks 2, 3; R of blocks 0, 1
//   C  T' R: E blocks 0, 1 (one MFMA each) and the first K step of blocks 2,
//      3; R of blocks 2, 3; then their second K step
//   D  K^T D E over tokens 0 .. 31 (E blocks 0, 1); D E of blocks 2, 3 and E
//      to the output waves
//   E  K^T D E over tokens 32 .. 63; the fp16 copies of the new state
// LDS reads are issued one phase ahead and in bursts of at most about 15
// behind the oldest one still needed (the LDS wait counter's range).
template <int DK, int buf, bool kSave = false>
__device__ __forceinline__ void state_chunk(MainSmem<DK>& sm, StateRegs<DK>& st, int lane,
                                            SaveBufs<DK>* sv = nullptr) {
    using Cfg = MainCfg<DK>;
    constexpr int KS = Cfg::KSTEP;
    constexpr int NST = Cfg::NST;
    const int lr = lane & 15, lq = lane >> 4;
    if constexpr (kSave) {
        // S_p before the update (tile r, lane group lq holds 4 consecutive rows)
#pragma unroll
        for (int r = 0; r < NST; ++r)
            *reinterpret_cast<float4v*>(&sv->S[buf][lr][state_row<DK>(r, lq, 0)]) = st.S[r];
    }
    const _Float16* Kb = sm.K[buf];
    const _Float16* Tb = sm.Tp[buf];
    const float* gate = sm.gate[buf];
    // K rows of row block I (the block enters as a pointer offset: the
    // swizzle only sees the row within the block)
    auto kfrag = [&](int I, int kk) {
        if constexpr (DK >= 32) return ld8<DK>(Kb + I * 16 * DK, lr, 8 * ks_chunk<DK>(kk, lq));
        else return ld_split_lo<DK>(Kb + I * 16 * DK, lr, 0, lq);
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    auto resid = [&](const half4& v, const float4v& g, const float4v& k) {
        return to_h4(static_cast<float>(v[0]) - g[0] * k[0], static_cast<float>(v[1]) - g[1] * k[1],
                     static_cast<float>(v[2]) - g[2] * k[2], static_cast<float>(v[3]) - g[3] * k[3]);
    };
    auto dscale = [](const float4v& d, const float4v& e) {
        return to_h4(d[0] * e[0], d[1] * e[1], d[2] * e[2], d[3] * e[3]);
    };
    const float gl = gate[C + C - 1];
    half8 kA[KS][2], kB[KS][2];   // K fragments of row blocks 0, 1 and 2, 3
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int i = 0; i < 2; ++i) kA[kk][i] = kfrag(i, kk);
    half4 vv[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I)
        vv[I] = ld_tr4(&sm.V[buf][(I * 16 + 4 * lq + (lr >> 2)) * Cfg::SV + 4 * (lr & 3)]);
    float4v gm[NB], dc[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) gm[I] = *reinterpret_cast<const float4v*>(&gate[C + I * 16 + 4 * lq]);
    fence();
    // A: K S for blocks 0, 1; K fragments of blocks 2, 3 in flight; the state
    // scaled by gamma_last alongside (the accumulator input of the update)
    float4v ks[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) ks[I] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
        for (int i = 0; i < 2; ++i) kB[kk][i] = kfrag(2 + i, kk);
        fence();
#pragma unroll
        for (int i = 0; i < 2; ++i) ks[i] = mma(kA[kk][i], st.Sb[kk], ks[i]);
#pragma unroll
        for (int r = kk * NST / KS; r < (kk + 1) * NST / KS; ++r) st.S[r] *= gl;
        fence();
    }
    // B: K S for blocks 2, 3; T' and d in flight; R of blocks 0, 1 once
    // their chains are done (after the first step here)
    half8 ta[NB][2];
    half4 rh[NB];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        if (kk == 0) {
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                ta[I][0] = ld8<C>(Tb + I * 16 * C, lr, 8 * lq);
                ta[I][1] = I >= 2 ? ld8<C>(Tb + I * 16 * C, lr, 32 + 8 * lq) : half8{};
            }
        }
        if (kk == (KS >= 2 ? 1 : 0)) {
#pragma unroll
            for (int I = 0; I < NB; ++I) dc[I] = *reinterpret_cast<const float4v*>(&gate[2 * C + I * 16 + 4 * lq]);
        }
        fence();
#pragma unroll
        for (int i = 0; i < 2; ++i) ks[2 + i] = mma(kB[kk][i], st.Sb[kk], ks[2 + i]);
        if (kk == 0) {
            fence();
            rh[0] = resid(vv[0], gm[0], ks[0]);
            rh[1] = resid(vv[1], gm[1], ks[1]);
        }
        fence();
    }
    const half8 Rb0 = cat(rh[0], rh[1]);
    // C: T' R; the first K step of K^T in flight
    half8 kt[2][NST];   // [K step over the chunk's tokens][state tile]
#pragma unroll
    for (int r = 0; r < NST; ++r) kt[0][r] = ld_kt<DK>(Kb, r, 0, lane);
    fence();
    float4v e[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) e[I] = mma(ta[I][0], Rb0, float4v{0.f, 0.f, 0.f, 0.f});
    fence();
    rh[2] = resid(vv[2], gm[2], ks[2]);
    rh[3] = resid(vv[3], gm[3], ks[3]);
    const half8 Rb1 = cat(rh[2], rh[3]);
    fence();
#pragma unroll
    for (int I = 2; I < NB; ++I) e[I] = mma(ta[I][1], Rb1, e[I]);
    fence();
    if constexpr (kSave) {
#pragma unroll
        for (int I = 0; I < NB; ++I) *reinterpret_cast<float4v*>(&sv->E[buf][lr][I * 16 + 4 * lq]) = e[I];
        fence();
    }
    // D: K^T D E over tokens 0 .. 31; the second K step of K^T in flight
    const half8 Eb0 = cat(dscale(dc[0], e[0]), dscale(dc[1], e[1]));
#pragma unroll
    for (int r = 0; r < NST; ++r) kt[1][r] = ld_kt<DK>(Kb, r, 1, lane);
    fence();
#pragma unroll
    for (int r = 0; r < NST; ++r) {
        st.S[r] = mma(kt[0][r], Eb0, st.S[r]);
        if (r == NST / 2 && !kSave) {
            fence();
#pragma unroll
            for (int I = 0; I < NB; ++I)
                *reinterpret_cast<half4*>(&sm.ET[buf][swz<C>(lr, I * 16 + 4 * lq)]) = to_h4(e[I]);
            fence();
        }
    }
    const half8 Eb1 = cat(dscale(dc[2], e[2]), dscale(dc[3], e[3]));
    fence();
    // E: K^T D E over tokens 32 .. 63, then the fp16 copies of the new state
#pragma unroll
    for (int r = 0; r < NST; ++r) st.S[r] = mma(kt[1][r], Eb1, st.S[r]);
    fence();
    state_refresh_operand(st);
    if constexpr (!kSave) state_publish<DK>(st, sm.ST[buf ^ 1], lane);
}

template <int DK, bool kSave = false>
__device__ __forceinline__ void state_role(MainSmem<DK>& sm, const Walk& w, const float* S0, float* S_out,
                                           long sbase, int DV, int lane, SaveBufs<DK>* sv = nullptr) {
    using Cfg = MainCfg<DK>;
    const int lr = lane & 15, lq = lane >> 4;
    StateRegs<DK> st;
#pragma unroll
    for (int r = 0; r < Cfg::NST; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) st.S[r][j] = S0 ? S0[sbase + static_cast<long>(state_row<DK>(r, lq, j)) * DV + lr] : 0.f;
    state_refresh_operand(st);
    state_publish<DK>(st, sm.ST[0], lane);
    period_end();
    const int n = w.nchunks;
    int p = 0;
    for (; p + 1 < n; p += 2) {
        state_chunk<DK, 0, kSave>(sm, st, lane, sv);
        period_end();
        state_chunk<DK, 1, kSave>(sm, st, lane, sv);
        period_end();
    }
    if (p < n) {
        state_chunk<DK, 0, kSave>(sm, st, lane, sv);
        period_end();
        ++p;
    }
    period_end();   // the output waves' last period
    bool bad = false;
#pragma unroll
    for (int r = 0; r < Cfg::NST; ++r) bad |= nonfinite(st.S[r]);
    report_nonfinite(w.status, bad, 2u);
    if (S_out) {
#pragma unroll
        for (int r = 0; r < Cfg::NST; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) S_out[sbase + static_cast<long>(state_row<DK>(r, lq, j)) * DV + lr] = st.S[r][j];
    }
}

// ---------------------------------------------------------------------------
// Output role.  Four waves, one per 16-token block I of the chunk: blocks 3
// and 0 share SIMD 1, blocks 2 and 1 SIMD 2, so that each SIMD interleaves two
// independent instruction streams.  Everything is computed transposed
// (K_J Q_I^T for P, S^T Q^T, E^T P^T), so that each lane holds one token row:
// P feeds the last MFMA straight from registers in the split-K order, and y
// leaves as one 16-byte store per lane.
// ---------------------------------------------------------------------------
template <int DK>
struct OutRegs {
    static constexpr int KS = MainCfg<DK>::KSTEP;
    uint4 qraw[2][KS];      // bf16 q of chunk c in set c & 1 (this wave's block)
    half8 qh[KS];           // fp16 q of the current chunk
    half8 Pb[2][2];         // P of chunk c in set c & 1, B operand of E^T P^T
    float4v qsg[2];         // gamma (Q S)^T of chunk c in set c & 1
    int qoff;               // byte offset of the lane's q piece in a chunk
    int yoff;               // byte offset of the lane's y piece in a chunk
    float ysum;             // sum of every y the lane wrote (non-finite once one is)
};

// fp16 q of the chunk in register set `set` (d_k = 16: only lane groups 0
// and 1 carry data).
template <int DK, int set>
__device__ __forceinline__ void out_convert_q(OutRegs<DK>& o, int lq) {
#pragma unroll
    for (int kk = 0; kk < OutRegs<DK>::KS; ++kk)
        o.qh[kk] = (DK >= 32 || lq < 2) ? bf16x8_to_h8(o.qraw[set][kk]) : half8{};
}

template <int DK, int set>
__device__ __forceinline__ void out_load_q(OutRegs<DK>& o, const Walk& w, int chunk) {
    constexpr int KS = MainCfg<DK>::KSTEP;
    const long t0 = static_cast<long>(chunk) * C;
    const rsrc_t r = make_rsrc(w.q + t0 * w.rowq, (w.T - t0) * w.rowq * 2);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) o.qraw[set][kk] = bload16(r, o.qoff + kk * 64);
}

// Period work of the output wave of block I.  Everything runs unconditionally
// (exact wait counts across the loop).  Order: gamma Q S and P of chunk c (in
// the last period, c = nchunks, of stale buffers and zero q: computed and
// never used), then y of chunk c - 1 from the P and gamma Q S kept in the
// other set, then the q loads of chunk c + 2 and the conversion of chunk
// c + 1's q (loaded a period ago), which thus sits behind this period's work
// instead of in front of the next period's MFMAs.
template <int DK, int I, int buf>
__device__ __forceinline__ void output_period(MainSmem<DK>& sm, OutRegs<DK>& o, const Walk& w, int c, int lane) {
    using Cfg = MainCfg<DK>;
    constexpr int KS = Cfg::KSTEP;
    const int lr = lane & 15, lq = lane >> 4;
    constexpr int cs = buf;   // chunk c lives in set c & 1 == buf
    const _Float16* Kb = sm.K[buf];
    const _Float16* STb = sm.ST[buf];
    const float* gate = sm.gate[buf];
    // contiguous K-slices: lane (r + 16 g) holds K-index 8 g .. 8 g + 7 of step
    // kk (for d_k = 16 only g < 2 carry data; the rest are zero)
    auto frag = [&](const _Float16* base, int row, int kk) {
        return (DK >= 32 || lq < 2) ? ld8<DK>(base, row, kk * 32 + 8 * lq) : half8{};
    };
    half8 sf[KS], kf[2][KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        sf[kk] = frag(STb, lr, kk);
        kf[0][kk] = frag(Kb, lr, kk);
    }
    __builtin_amdgcn_sched_barrier(0);
    // (Q S)^T = S^T Q^T, interleaved with the first P tile: lane (t + 16 g)
    // gets columns 4 g .. 4 g + 3 of row t
    float4v qs = {0.f, 0.f, 0.f, 0.f};
    // (Q K^T)^T tiles J <= I: k block J is read once, one block ahead of its MFMAs
    float4v pacc[NB];
#pragma unroll
    for (int J = 0; J <= I; ++J) {
        if (J + 1 <= I) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) kf[(J + 1) & 1][kk] = frag(Kb + (J + 1) * 16 * DK, lr, kk);
        }
        __builtin_amdgcn_sched_barrier(0);
        pacc[J] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if (J == 0) qs = mma(sf[kk], o.qh[kk], qs);
            pacc[J] = mma(kf[J & 1][kk], o.qh[kk], pacc[J]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // P = Gamma o (Q K^T) on the lower tiles, lane row t = 16 I + lr, columns
    // i = 16 J + 4 lq + j.  Below the diagonal block the decay factors as
    // 2^(g2_t - g2_b) w_i (g2_b: end of block J), one power per lane and tile;
    // the diagonal tile takes 2^(g2_t - g2_i) per entry with i <= t (the
    // powers of masked entries may overflow; the select drops them).
    {
        const int t = I * 16 + lr;
        const float gt = gate[t];
        o.qsg[cs] = qs * gate[C + t];
        half4 ph[NB];
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            if (J > I) {
                ph[J] = half4{};
            } else if (J < I) {
                const float4v wi = *reinterpret_cast<const float4v*>(&gate[3 * C + J * 16 + 4 * lq]);
                const float u = __builtin_amdgcn_exp2f(gt - gate[J * 16 + 15]);
                ph[J] = to_h4((u * wi) * pacc[J]);
            } else {
                const float4v gi = *reinterpret_cast<const float4v*>(&gate[J * 16 + 4 * lq]);
                float pe[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v = __builtin_amdgcn_exp2f(gt - gi[j]) * pacc[J][j];
                    pe[j] = (4 * lq + j <= lr) ? v : 0.f;
                }
                ph[J] = to_h4(pe[0], pe[1], pe[2], pe[3]);
            }
        }
        o.Pb[cs][0] = cat(ph[0], ph[1]);
        o.Pb[cs][1] = cat(ph[2], ph[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // y of chunk c - 1:  Y^T = E^T P^T + gamma (Q S)^T.  At c = 0 the
    // descriptor has size 0 and the stores are dropped.
    {
        constexpr int ps = cs ^ 1;
        const _Float16* ETp = sm.ET[buf ^ 1];
        const long t0 = static_cast<long>(c - 1) * C;
        const rsrc_t ry = make_rsrc(w.y + t0 * w.rowv, c > 0 ? (w.T - t0) * w.rowv * 4 : 0);
        float4v yv = mma(ld_split<C>(ETp, lr, 0, lq), o.Pb[ps][0], o.qsg[ps]);
        if constexpr (I >= 2) yv = mma(ld_split<C>(ETp, lr, 32, lq), o.Pb[ps][1], yv);
        yv = yv * w.scale;
        // (rows past T are zero, and so is the c = 0 result: zero P and Q S
        // from the prologue, zeroed E buffers).  The running sum stays finite
        // for any finite y below about 1e30 in magnitude.
        o.ysum += (yv[0] + yv[1]) + (yv[2] + yv[3]);
        // a plain store: the slices of a head write 64-byte pieces of each y
        // row, which merge in L2
        bstore16(ry, o.yoff, yv);
    }
    // q of chunk c + 2 into the set chunk c used; q of chunk c + 1 to fp16
    out_load_q<DK, cs>(o, w, c + 2);
    out_convert_q<DK, cs ^ 1>(o, lq);
}

template <int DK, int I>
__device__ __forceinline__ void output_role(MainSmem<DK>& sm, const Walk& w, int lane) {
    const int lr = lane & 15, lq = lane >> 4;
    OutRegs<DK> o;
    const unsigned t = I * 16 + lr;
    o.qoff = static_cast<int>((t * static_cast<unsigned>(w.rowq) + w.hq + 8u * lq) * 2u);
    o.yoff = static_cast<int>((t * static_cast<unsigned>(w.rowv) + w.hv + 4u * lq) * 4u);
    o.ysum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        o.Pb[st][0] = o.Pb[st][1] = half8{};
        o.qsg[st] = float4v{0.f, 0.f, 0.f, 0.f};
    }
    out_load_q<DK, 0>(o, w, 0);
    out_load_q<DK, 1>(o, w, 1);
    out_convert_q<DK, 0>(o, lq);
    period_end();
    const int n = w.nchunks;
    int p = 0;
    for (; p + 1 <= n; p += 2) {
        output_period<DK, I, 0>(sm, o, w, p, lane);
        period_end();
        output_period<DK, I, 1>(sm, o, w, p + 1, lane);
        period_end();
    }
    if (p <= n) {
        output_period<DK, I, 0>(sm, o, w, p, lane);
        period_end();
    }
    report_nonfinite(w.status, !__builtin_isfinite(o.ysum), 1u);
}

// Copy role of the state-saving walk: wave I writes rows I DK / 4 .. of S_p
// and tokens 16 I .. 16 I + 15 of E_p (rounded to fp16, row-major
// [row][column] as the backward pass reads them) in period p + 1, from the
// buffers the state wave filled in period p.
template <int DK>
__device__ __forceinline__ void copy_role(const SaveBufs<DK>* sv, const Walk& w, _Float16* ws_S, _Float16* ws_E,
                                          long bhn0, int DV, int col0, int I, int lane) {
    constexpr int RW = DK / 4;                 // state rows per copy wave
    const int c4 = lane & 3, lrow = lane >> 2;
    period_end();
    const int n = w.nchunks;
    for (int p = 0; p <= n; ++p) {
        if (p >= 1) {
            const int c = p - 1, buf = c & 1;
            const long bhn = bhn0 + c;
#pragma unroll
            for (int hh = 0; hh < RW / 16; ++hh) {
                const int row = I * RW + 16 * hh + lrow;
                float4v x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = sv->S[buf][4 * c4 + e][row];
                *reinterpret_cast<half4*>(&ws_S[(bhn * DK + row) * DV + col0 + 4 * c4]) = to_h4(x);
            }
            const int tok = I * 16 + lrow;
            float4v x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = sv->E[buf][4 * c4 + e][tok];
            *reinterpret_cast<half4*>(&ws_E[(bhn * C + tok) * DV + col0 + 4 * c4]) = to_h4(x);
        }
        period_end();
    }
}

template <int DK, bool kSave = false>
__global__ __launch_bounds__(512) void main_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, const _Float16* __restrict__ ws,
                                                   const float* __restrict__ S0, float* __restrict__ S_out,
                                                   float* __restrict__ y, int B, int T, int H, int DV, int nsl,
                                                   float scale, unsigned* status, float* __restrict__ ws_S,
                                                   float* __restrict__ ws_E) {
    using Cfg = MainCfg<DK>;
    __shared__ MainSmem<DK> sm;
    __shared__ typename std::conditional<kSave, SaveBufs<DK>, NoSaveBufs>::type sv;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    // block -> (head, slice): the slices of a head share block ids modulo kXcds
    const int xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
    const int bh = (jx / nsl) * kXcds + xcd;
    const int slice = jx % nsl;
    if (bh >= B * H) return;
    const int b = bh / H, h = bh % H;
    const int col0 = slice * Cfg::SV;
    const long tok0 = static_cast<long>(b) * T;
    Walk w;
    w.rowq = static_cast<long>(H) * DK;
    w.rowv = static_cast<long>(H) * DV;
    w.q = q + tok0 * w.rowq;
    w.k = k + tok0 * w.rowq;
    w.v = v + tok0 * w.rowv;
    w.y = y ? y + tok0 * w.rowv : nullptr;
    w.hq = static_cast<unsigned>(h * DK);
    w.hv = static_cast<unsigned>(h * DV + col0);
    w.T = T;
    w.nchunks = (T + C - 1) / C;
    w.ws = ws + static_cast<long>(bh) * w.nchunks * WS_CHUNK;
    w.scale = scale;
    w.status = status;

    // T' is zero above its diagonal blocks; those halves of both buffers are
    // never written again.  The E buffers start at zero: the first period's
    // (dropped) y reads one of them.
    for (int idx = tid; idx < 2 * C * C; idx += Cfg::NT) (&sm.Tp[0][0])[idx] = static_cast<_Float16>(0.f);
    for (int idx = tid; idx < 2 * Cfg::SV * C; idx += Cfg::NT) (&sm.ET[0][0])[idx] = static_cast<_Float16>(0.f);
    __syncthreads();

    // Each role runs its own loop with the same barrier sequence: one barrier
    // after the prologue and one after every period (nchunks + 1 periods).
    // (state-saving walk: the state wave and the loaders as usual, the four
    // output waves copy S_p and E_p out instead of forming y)
    if (wv == Cfg::W_STATE) {
        if constexpr (kSave)
            state_role<DK, true>(sm, w, S0, S_out, static_cast<long>(bh) * DK * DV + col0, DV, lane, &sv);
        else
            state_role<DK>(sm, w, S0, S_out, static_cast<long>(bh) * DK * DV + col0, DV, lane);
    } else if (wv == 1 || wv == 2 || wv == 5 || wv == 6) {
        const int blk = wv == 1 ? 3 : (wv == 5 ? 0 : (wv == 2 ? 2 : 1));
        if constexpr (kSave) {
            copy_role<DK>(&sv, w, reinterpret_cast<_Float16*>(ws_S), reinterpret_cast<_Float16*>(ws_E),
                          static_cast<long>(bh) * w.nchunks, DV, col0, blk, lane);
        } else {
            if (blk == 3) output_role<DK, 3>(sm, w, lane);
            else if (blk == 0) output_role<DK, 0>(sm, w, lane);
            else if (blk == 2) output_role<DK, 2>(sm, w, lane);
            else output_role<DK, 1>(sm, w, lane);
        }
    } else if (wv == Cfg::W_MISC) {
        MiscLoader<DK> ld;
        ld.init(lane, w);
        Pieces<DK, Cfg::NMI> pcs;
        loader_role<DK>(ld, pcs, sm, w);
    } else if (wv == Cfg::W_K0 && Cfg::NK0 > 0) {
        KLoader<DK, (Cfg::NK0 > 0 ? Cfg::NK0 : 1)> ld;
        ld.init(0, lane, w);
        Pieces<DK, (Cfg::NK0 > 0 ? Cfg::NK0 : 1)> pcs;
        loader_role<DK>(ld, pcs, sm, w);
    } else if (wv == Cfg::W_K1) {
        KLoader<DK, Cfg::NK1> ld;
        ld.init(Cfg::NK0 * 64, lane, w);
        Pieces<DK, Cfg::NK1> pcs;
        loader_role<DK>(ld, pcs, sm, w);
    } else {
        // idle waves: the same barrier sequence
        period_end();
        for (int p = 0; p <= w.nchunks; ++p) period_end();
    }
}

// ===========================================================================
// Reverse walk of the backward pass (bf16 inputs, d_k = d_v = DK in {64,
// 128}): the adjoint of the chunk chain above.  Per (head, 16-column value
// slice) the chunks c = n - 1 .. 0 are walked with the state gradient dS
// (d_k x 16, fp32) held in the accumulator registers of one wave, in the
// forward state wave's row order.  With g the chunk's cumulative log decay,
// gamma = exp(g), lam = exp(g_last - g), T = (I + A)^-1 and the masked gated
// Gram P = Gamma o (Q K^T) (the backward's chunk-parallel pass stores g, and
// T and P as fp16 in each chunk's T slot), chunk c turns dS' (the gradient of
// the state after the chunk) into
//     dE = scale P^T dY + diag(lam) K dS'
//     dR = T^T dE                              (dV = diag(beta) dR)
//     dS = gamma_last dS' + Q^T (scale diag(gamma) dY) - K^T (diag(beta gamma) dR)
// (the chunkwise form of the delta rule differentiated, slinene page, Module
// A).  Roles, wave w on SIMD w % 4:
//   0     the dS chain: K dS', dE, dR and the update, as the forward's state
//         wave runs K S, R, E and its update
//   1, 2  helpers: scale P^T dY and Q^T (scale gamma dY) of the next chunk
//         (neither depends on dS), left in LDS as accumulator tiles
//   3     copy: dS' (the gradient workspace), dR and dV of the previous chunk
//   7, 5  loaders of the next chunk's k, and T with the gates
//   6, 4  loaders of q, and P, the dY slice and scale gamma, two chunks ahead
//         (the k conversion, the heaviest loader work, stays off the state
//         wave's SIMD)
// Two barriers open the walk (the loaders' first stores, then the helpers'
// first chunk); then one ends each of the n + 1 periods.  Period p processes
// chunk n - 1 - p.
// ===========================================================================
template <int DK>
struct alignas(16) RevSmem {
    static constexpr int NST = DK / 16;
    _Float16 K[2][C * DK];        // k of the state wave's chunk, rows swizzled
    _Float16 Tm[2][C * C];        // T, [t][i], rows swizzled
    float gate[2][3 * C];         // lam, -beta gamma, and gamma_last at [2 C]
    _Float16 Q[2][C * DK];        // q of the helpers' chunk
    _Float16 P[2][C * C];         // P, [t][i], rows swizzled
    _Float16 dY[2][C * 16];       // dY slice, [t][column]
    float hg[2][C];               // scale gamma
    float4v PdY[2][NB][64];       // scale P^T dY, accumulator tiles, lane-major
    float4v QB[2][NST][64];       // Q^T (scale gamma dY), the state's tiles, lane-major
    float SS[2][16][DK + 4];      // dS' of the chunk, [column][d_k row], for the copy wave
    float SR[2][16][C + 4];       // dR of the chunk, [column][token]
};

struct RevWalk {
    const uint16_t* q;        // this sequence's rows
    const uint16_t* k;
    const float* beta;        // this sequence and head: beta[t * H]
    const float* dy;          // this sequence's rows
    const float* g;           // this head's chunks in the backward workspace
    const float* Tm;          // T slots: fp16 T, then fp16 P
    long rowq, rowv;
    unsigned hq, hv;          // element offsets of the head (q, k) and the slice (dy)
    int H, T, nchunks;
    float scale;
};

// A operand of (X^T) for row block I of X's columns and token step ks, from
// a row-major swizzled [token][LD] fp16 tile X: lane (m + 16 g) gets
// X[32 ks + 16 (s / 4) + 4 g + s % 4][16 I + m] in slot s (the split-K token
// order of the accumulator tiles stacked along K).
template <int LD>
__device__ __forceinline__ half8 ld_tn(const _Float16* X, int I, int ks, int lane) {
    const int g = lane >> 4, x = lane & 15;
    const int o = swz<LD>(4 * g + (x >> 2), 16 * I + 4 * (x & 3));
    return cat(ld_tr4(X + ks * 32 * LD + o), ld_tr4(X + (ks * 32 + 16) * LD + o));
}

__device__ __forceinline__ rsrc_t rev_rsrc(const void* base, long elem_off, long bytes, bool live) {
    return make_rsrc(static_cast<const char*>(base) + (live ? elem_off : 0), live ? bytes : 0);
}

// bf16 rows (k or q) -> fp16 swizzled tile; pieces i = j * 64 + lane.
template <int DK, bool kQ>
struct RevRows {
    static constexpr int QC = DK / 8, N = C * QC / 64;
    int voff[N], loff[N];
    uint4 a[2][N];
    __device__ void init(int ls, const RevWalk& w) {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int i = j * 64 + ls, t = i / QC, cq = i % QC;
            voff[j] = static_cast<int>((static_cast<unsigned>(t) * static_cast<unsigned>(w.rowq) + w.hq + cq * 8u) * 2u);
            loff[j] = swz<DK>(t, cq * 8);
        }
    }
    template <int set>
    __device__ void load(const RevWalk& w, int chunk) {
        const bool live = chunk >= 0 && chunk < w.nchunks;
        const long t0 = static_cast<long>(chunk) * C;
        const rsrc_t r = rev_rsrc(kQ ? w.q : w.k, t0 * w.rowq * 2, (w.T - t0) * w.rowq * 2, live);
#pragma unroll
        for (int j = 0; j < N; ++j) a[set][j] = bload16(r, voff[j]);
    }
    template <int set, int buf>
    __device__ void store(RevSmem<DK>& sm) const {
        _Float16* dst = kQ ? sm.Q[buf] : sm.K[buf];
#pragma unroll
        for (int j = 0; j < N; ++j) st16(&dst[loff[j]], bf16x8_to_h8(a[set][j]));
    }
};

// fp16 64 x 64 workspace tile (T, or P in the second half of the chunk's T
// slot) -> swizzled LDS tile, 8 pieces per lane.
template <int DK, bool kP>
struct RevTile {
    int loff[8];
    int lane;
    uint4 a[2][8];
    __device__ void init(int ls) {
        lane = ls;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = j * 64 + ls;
            loff[j] = swz<C>(i >> 3, 8 * (i & 7));
        }
    }
    template <int set>
    __device__ void load(const RevWalk& w, int chunk) {
        const bool live = chunk >= 0 && chunk < w.nchunks;
        const rsrc_t r = rev_rsrc(w.Tm, static_cast<long>(chunk) * C * C * 4 + (kP ? C * C * 2 : 0), C * C * 2, live);
#pragma unroll
        for (int j = 0; j < 8; ++j) a[set][j] = bload16(r, (j * 64 + lane) * 16);
    }
    template <int set, int buf>
    __device__ void store(RevSmem<DK>& sm) const {
        _Float16* dst = kP ? sm.P[buf] : sm.Tm[buf];
#pragma unroll
        for (int j = 0; j < 8; ++j) st16(&dst[loff[j]], a[set][j]);
    }
};

// Per-token gate values of a chunk (lane = token): g_t, g_last and beta_t.
struct RevGates {
    float g[2], gl[2], b[2];
    template <int set>
    __device__ void load(const RevWalk& w, int chunk, int lane, bool need_beta) {
        const bool live = chunk >= 0 && chunk < w.nchunks;
        const long t0 = static_cast<long>(chunk) * C;
        const rsrc_t rg = rev_rsrc(w.g, t0 * 4, C * 4, live);
        g[set] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, lane * 4, 0, 0));
        gl[set] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (C - 1) * 4, 0, 0));
        if (need_beta) {
            const rsrc_t rb = rev_rsrc(w.beta, t0 * w.H * 4, (w.T - t0) * w.H * 4, live);
            b[set] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, lane * w.H * 4, 0, 0));
        }
    }
};

// The dY slice (fp32 rows) -> fp16 [t][16], 4 pieces per lane.
struct RevDy {
    int voff[4], loff[4];
    uint4 a[2][4];
    __device__ void init(int ls, const RevWalk& w) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = j * 64 + ls, t = i >> 2, c4 = i & 3;
            voff[j] = static_cast<int>((static_cast<unsigned>(t) * static_cast<unsigned>(w.rowv) + w.hv + 4u * c4) * 4u);
            loff[j] = t * 16 + 4 * c4;
        }
    }
    template <int set>
    __device__ void load(const RevWalk& w, int chunk) {
        const bool live = chunk >= 0 && chunk < w.nchunks;
        const long t0 = static_cast<long>(chunk) * C;
        const rsrc_t r = rev_rsrc(w.dy, t0 * w.rowv * 4, (w.T - t0) * w.rowv * 4, live);
#pragma unroll
        for (int j = 0; j < 4; ++j) a[set][j] = bload16(r, voff[j]);
    }
    template <int set, int buf, int DK>
    __device__ void store(RevSmem<DK>& sm) const {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<half4*>(&sm.dY[buf][loff[j]]) = to_h4(__builtin_bit_cast(float4v, a[set][j]));
    }
};

// Loader schedules.  State data (k, T, gates): the opening stores chunk
// n - 1 and has the next two in flight; period p stores the chunk of period
// p + 1 and loads the one of period p + 3.  Helper data (q, P, dY, scale
// gamma): the opening stores the chunks of periods 0 and 1; period p stores
// the chunk of period p + 2 and loads the one of period p + 4.  Loads past
// either end read zeros.
template <class L>
__device__ __forceinline__ void rev_state_schedule(L& ld, int n) {
    ld.template load<0>(n - 1);
    ld.template load<1>(n - 2);
    ld.template store<0, 0>();
    ld.template load<0>(n - 3);
    period_end();
    period_end();
    int p = 0;
    for (; p + 1 <= n; p += 2) {
        ld.template store<1, 1>();
        ld.template load<1>(n - 4 - p);
        period_end();
        ld.template store<0, 0>();
        ld.template load<0>(n - 5 - p);
        period_end();
    }
    if (p <= n) {
        ld.template store<1, 1>();
        ld.template load<1>(n - 4 - p);
        period_end();
    }
}
template <class L>
__device__ __forceinline__ void rev_help_schedule(L& ld, int n) {
    ld.template load<0>(n - 1);
    ld.template load<1>(n - 2);
    ld.template store<0, 0>();
    ld.template store<1, 1>();
    ld.template load<0>(n - 3);
    ld.template load<1>(n - 4);
    period_end();
    period_end();
    int p = 0;
    for (; p + 1 <= n; p += 2) {
        ld.template store<0, 0>();
        ld.template load<0>(n - 5 - p);
        period_end();
        ld.template store<1, 1>();
        ld.template load<1>(n - 6 - p);
        period_end();
    }
    if (p <= n) {
        ld.template store<0, 0>();
        ld.template load<0>(n - 5 - p);
        period_end();
    }
}

// Wave 7: k.  Wave 5: T and the state wave's gates.  Wave 6: q.  Wave 4: P,
// the dY slice and scale gamma.
template <int DK>
struct RevLoadK {
    RevRows<DK, false> rows;
    RevSmem<DK>* sm;
    const RevWalk* w;
    template <int set> __device__ void load(int chunk) { rows.template load<set>(*w, chunk); }
    template <int set, int buf> __device__ void store() { rows.template store<set, buf>(*sm); }
};
template <int DK>
struct RevLoadT {
    RevTile<DK, false> tile;
    RevGates gt;
    RevSmem<DK>* sm;
    const RevWalk* w;
    int lane;
    template <int set> __device__ void load(int chunk) {
        tile.template load<set>(*w, chunk);
        gt.template load<set>(*w, chunk, lane, true);
    }
    template <int set, int buf> __device__ void store() {
        tile.template store<set, buf>(*sm);
        const float g = gt.g[set], gl = gt.gl[set];
        sm->gate[buf][lane] = __expf(gl - g);
        sm->gate[buf][C + lane] = -gt.b[set] * __expf(g);
        if (lane == 0) sm->gate[buf][2 * C] = __expf(gl);
    }
};
template <int DK>
struct RevLoadQ {
    RevRows<DK, true> rows;
    RevSmem<DK>* sm;
    const RevWalk* w;
    template <int set> __device__ void load(int chunk) { rows.template load<set>(*w, chunk); }
    template <int set, int buf> __device__ void store() { rows.template store<set, buf>(*sm); }
};
template <int DK>
struct RevLoadP {
    RevTile<DK, true> tile;
    RevDy dyl;
    RevGates gt;
    RevSmem<DK>* sm;
    const RevWalk* w;
    int lane;
    template <int set> __device__ void load(int chunk) {
        tile.template load<set>(*w, chunk);
        dyl.template load<set>(*w, chunk);
        gt.template load<set>(*w, chunk, lane, false);
    }
    template <int set, int buf> __device__ void store() {
        tile.template store<set, buf>(*sm);
        dyl.template store<set, buf>(*sm);
        sm->hg[buf][lane] = w->scale * __expf(gt.g[set]);
    }
};

// One chunk of the dS chain (the chunk's data in buffer `buf`).
template <int DK, int buf>
__device__ __forceinline__ void rev_chunk(RevSmem<DK>& sm, StateRegs<DK>& st, int lane) {
    constexpr int KS = DK / 32, NST = DK / 16;
    const int lr = lane & 15, lq = lane >> 4;
    const _Float16* Kb = sm.K[buf];
    const float* gate = sm.gate[buf];
    // dS' out, for the copy wave (tile r, lane group lq: 4 consecutive rows)
#pragma unroll
    for (int r = 0; r < NST; ++r) *reinterpret_cast<float4v*>(&sm.SS[buf][lr][state_row<DK>(r, lq, 0)]) = st.S[r];
    // K dS' for the four token blocks
    float4v kd[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) kd[I] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int I = 0; I < NB; ++I)
            kd[I] = mma(ld8<DK>(Kb + I * 16 * DK, lr, 8 * ks_chunk<DK>(kk, lq)), st.Sb[kk], kd[I]);
    // the update's accumulator input: gamma_last dS' + Q^T (scale gamma dY)
    const float gl = gate[2 * C];
#pragma unroll
    for (int r = 0; r < NST; ++r) st.S[r] = gl * st.S[r] + sm.QB[buf][r][lane];
    // dE = scale P^T dY + lam o K dS'
    half4 eh[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        const float4v lam = *reinterpret_cast<const float4v*>(&gate[I * 16 + 4 * lq]);
        const float4v pd = sm.PdY[buf][I][lane];
        eh[I] = to_h4(pd[0] + lam[0] * kd[I][0], pd[1] + lam[1] * kd[I][1], pd[2] + lam[2] * kd[I][2],
                      pd[3] + lam[3] * kd[I][3]);
    }
    const half8 Eb0 = cat(eh[0], eh[1]), Eb1 = cat(eh[2], eh[3]);
    // dR = T^T dE; T^T is upper triangular, so row blocks 2 and 3 see only
    // tokens 32 .. 63
    float4v dr[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        dr[I] = mma(ld_tn<C>(sm.Tm[buf], I, 1, lane), Eb1, float4v{0.f, 0.f, 0.f, 0.f});
        if (I < 2) dr[I] = mma(ld_tn<C>(sm.Tm[buf], I, 0, lane), Eb0, dr[I]);
    }
#pragma unroll
    for (int I = 0; I < NB; ++I) *reinterpret_cast<float4v*>(&sm.SR[buf][lr][I * 16 + 4 * lq]) = dr[I];
    // -beta gamma o dR, the B operand of the update
    half4 bh[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        const float4v nb = *reinterpret_cast<const float4v*>(&gate[C + I * 16 + 4 * lq]);
        bh[I] = to_h4(nb * dr[I]);
    }
    const half8 Bb0 = cat(bh[0], bh[1]), Bb1 = cat(bh[2], bh[3]);
#pragma unroll
    for (int r = 0; r < NST; ++r) st.S[r] = mma(ld_kt<DK>(Kb, r, 0, lane), Bb0, st.S[r]);
#pragma unroll
    for (int r = 0; r < NST; ++r) st.S[r] = mma(ld_kt<DK>(Kb, r, 1, lane), Bb1, st.S[r]);
    state_refresh_operand(st);
}

// Helper h (0, 1) on the chunk in buffer hb: Q^T (scale gamma dY) for half
// of the state's tiles, and (helper 0) scale P^T dY.
template <int DK, int kHelper>
__device__ __forceinline__ void rev_helper(RevSmem<DK>& sm, int hb, int lane, float scale) {
    constexpr int NST = DK / 16, R0 = kHelper * NST / 2;
    const int lr = lane & 15, lq = lane >> 4;
    half4 dyh[NB], b1[NB];
#pragma unroll
    for (int J = 0; J < NB; ++J) {
        dyh[J] = ld_tr4(&sm.dY[hb][(J * 16 + 4 * lq + (lr >> 2)) * 16 + 4 * (lr & 3)]);
        const float4v hg = *reinterpret_cast<const float4v*>(&sm.hg[hb][J * 16 + 4 * lq]);
        b1[J] = to_h4(hg[0] * static_cast<float>(dyh[J][0]), hg[1] * static_cast<float>(dyh[J][1]),
                      hg[2] * static_cast<float>(dyh[J][2]), hg[3] * static_cast<float>(dyh[J][3]));
    }
    const half8 B0 = cat(b1[0], b1[1]), B1 = cat(b1[2], b1[3]);
#pragma unroll
    for (int r = R0; r < R0 + NST / 2; ++r) {
        float4v acc = mma(ld_kt<DK>(sm.Q[hb], r, 0, lane), B0, float4v{0.f, 0.f, 0.f, 0.f});
        acc = mma(ld_kt<DK>(sm.Q[hb], r, 1, lane), B1, acc);
        sm.QB[hb][r][lane] = acc;
    }
    if constexpr (kHelper == 0) {
        const half8 Y0 = cat(dyh[0], dyh[1]), Y1 = cat(dyh[2], dyh[3]);
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            float4v acc = mma(ld_tn<C>(sm.P[hb], I, 1, lane), Y1, float4v{0.f, 0.f, 0.f, 0.f});
            if (I < 2) acc = mma(ld_tn<C>(sm.P[hb], I, 0, lane), Y0, acc);
            sm.PdY[hb][I][lane] = scale * acc;
        }
    }
}

template <int DK>
__global__ __launch_bounds__(512) void rev_walk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                       const float* __restrict__ beta, const float* __restrict__ dy,
                                                       const float* __restrict__ dST, const float* __restrict__ ws_g,
                                                       const float* __restrict__ ws_T,
                                                       float* __restrict__ ws_dS, float* __restrict__ ws_dR,
                                                       float* __restrict__ dv_out, float* __restrict__ dS0, int B,
                                                       int T, int H, int nsl, float scale) {
    constexpr int DV = DK, NST = DK / 16;
    __shared__ RevSmem<DK> sm;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;
    const int xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
    const int bh = (jx / nsl) * kXcds + xcd;
    const int slice = jx % nsl;
    if (bh >= B * H) return;
    const int b = bh / H, h = bh % H;
    const int col0 = slice * 16;
    const long tok0 = static_cast<long>(b) * T;
    RevWalk w;
    w.rowq = static_cast<long>(H) * DK;
    w.rowv = static_cast<long>(H) * DV;
    w.q = q + tok0 * w.rowq;
    w.k = k + tok0 * w.rowq;
    w.beta = beta + tok0 * H + h;
    w.dy = dy + tok0 * w.rowv;
    w.T = T;
    w.H = H;
    w.nchunks = (T + C - 1) / C;
    const int n = w.nchunks;
    w.g = ws_g + static_cast<long>(bh) * n * C;
    w.Tm = ws_T + static_cast<long>(bh) * n * C * C;
    w.hq = static_cast<unsigned>(h * DK);
    w.hv = static_cast<unsigned>(h * DV + col0);
    w.scale = scale;

    if (wv == 0) {
        StateRegs<DK> st;
#pragma unroll
        for (int r = 0; r < NST; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                st.S[r][j] = dST ? dST[(static_cast<long>(bh) * DK + state_row<DK>(r, lq, j)) * DV + col0 + lr] : 0.f;
        state_refresh_operand(st);
        period_end();
        period_end();
        int p = 0;
        for (; p + 1 < n; p += 2) {
            rev_chunk<DK, 0>(sm, st, lane);
            period_end();
            rev_chunk<DK, 1>(sm, st, lane);
            period_end();
        }
        if (p < n) {
            rev_chunk<DK, 0>(sm, st, lane);
            period_end();
        }
        period_end();   // the copy wave's last period
        if (dS0) {
#pragma unroll
            for (int r = 0; r < NST; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    dS0[(static_cast<long>(bh) * DK + state_row<DK>(r, lq, j)) * DV + col0 + lr] = st.S[r][j];
        }
    } else if (wv == 1 || wv == 2) {
        period_end();
        if (n > 0) {
            if (wv == 1) rev_helper<DK, 0>(sm, 0, lane, scale);
            else rev_helper<DK, 1>(sm, 0, lane, scale);
        }
        period_end();
        for (int p = 0; p <= n; ++p) {
            if (p + 1 < n) {
                if (wv == 1) rev_helper<DK, 0>(sm, (p + 1) & 1, lane, scale);
                else rev_helper<DK, 1>(sm, (p + 1) & 1, lane, scale);
            }
            period_end();
        }
    } else if (wv == 3) {
        // dS' and dR go out rounded to fp16 (the gradient pass takes them as
        // fp16 operands)
        _Float16* dS16 = reinterpret_cast<_Float16*>(ws_dS);
        _Float16* dR16 = reinterpret_cast<_Float16*>(ws_dR);
        // period p loads beta of the chunk copied in period p + 1 into one
        // register and copies with the other (the loop runs in pairs, so no
        // register move waits for the load)
        auto copy_period = [&](int p, float& bload, const float& buse) {
            // issued before this period's stores: memory operations retire in
            // order, so a load issued after them would wait for them
            const int cn = n - 1 - p;
            const rsrc_t rb = rev_rsrc(w.beta, static_cast<long>(cn) * C * H * 4,
                                       (T - static_cast<long>(cn) * C) * H * 4, cn >= 0);
            bload = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, lane * H * 4, 0, 0));
            if (p >= 1) {
                // 16-byte row pieces: lane (4 row + c4) writes columns 4 c4 .. 4 c4 + 3
                const int c = n - p, cb = (p - 1) & 1, c4 = lane & 3, lrow = lane >> 2;
                const long bhn = static_cast<long>(bh) * n + c;
#pragma unroll
                for (int hh = 0; hh < DK / 16; ++hh) {
                    const int row = 16 * hh + lrow;
                    float4v x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = sm.SS[cb][4 * c4 + e][row];
                    *reinterpret_cast<half4*>(&dS16[(bhn * DK + row) * DV + col0 + 4 * c4]) = to_h4(x);
                }
#pragma unroll
                for (int hh = 0; hh < NB; ++hh) {
                    const int t = 16 * hh + lrow;
                    float4v x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = sm.SR[cb][4 * c4 + e][t];
                    *reinterpret_cast<half4*>(&dR16[(bhn * C + t) * DV + col0 + 4 * c4]) = to_h4(x);
                    const float bt = __shfl(buse, t);
                    if (static_cast<long>(c) * C + t < T)
                        *reinterpret_cast<float4v*>(&dv_out[((tok0 + static_cast<long>(c) * C + t) * H + h) * DV + col0 +
                                                            4 * c4]) = bt * x;
                }
            }
            period_end();
        };
        float b0 = 0.f, b1 = 0.f;
        period_end();
        period_end();
        int p = 0;
        for (; p + 1 <= n; p += 2) {
            copy_period(p, b0, b1);
            copy_period(p + 1, b1, b0);
        }
        if (p <= n) copy_period(p, b0, b1);
    } else if (wv == 7) {
        RevLoadK<DK> ld;
        ld.rows.init(lane, w);
        ld.sm = &sm;
        ld.w = &w;
        rev_state_schedule(ld, n);
    } else if (wv == 5) {
        RevLoadT<DK> ld;
        ld.tile.init(lane);
        ld.sm = &sm;
        ld.w = &w;
        ld.lane = lane;
        rev_state_schedule(ld, n);
    } else if (wv == 6) {
        RevLoadQ<DK> ld;
        ld.rows.init(lane, w);
        ld.sm = &sm;
        ld.w = &w;
        rev_help_schedule(ld, n);
    } else {   // wave 4
        RevLoadP<DK> ld;
        ld.tile.init(lane);
        ld.dyl.init(lane, w);
        ld.sm = &sm;
        ld.w = &w;
        ld.lane = lane;
        rev_help_schedule(ld, n);
    }
}

template <int DK>
static hipError_t launch_t(const PrefillArgs& a, float* save_S = nullptr, float* save_E = nullptr) {
    using Cfg = MainCfg<DK>;
    const int nchunks = (a.T + C - 1) / C;
    unsigned* status = static_cast<unsigned*>(a.workspace);
    _Float16* ws = status ? reinterpret_cast<_Float16*>(static_cast<char*>(a.workspace) + kStatusBytes) : nullptr;
    if (nchunks > 0) {
        // chunks per wave: one, unless the grid would pass kPrepGridWGs; at most 16
        const int BH = a.B * a.H;
        const long gx = (BH + kPrepWaves - 1) / kPrepWaves;
        const int cpw = static_cast<int>(
            std::min<long>(16, std::max<long>(1, (gx * nchunks + kPrepGridWGs - 1) / kPrepGridWGs)));
        const int gy = (nchunks + cpw - 1) / cpw;
        const long nblk = gx * ((gy + kXcds - 1) / kXcds) * kXcds;
        hipLaunchKernelGGL((prep_kernel<DK>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, a.stream,
                           static_cast<const uint16_t*>(a.k), a.alpha, a.beta, ws, status, a.T, a.H, BH, nchunks,
                           cpw, static_cast<int>(gx), gy);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nsl = a.dv / Cfg::SV;
    const int groups = (a.B * a.H + kXcds - 1) / kXcds;
    if constexpr (DK >= 64) {
        if (save_S) {
            hipLaunchKernelGGL((main_kernel<DK, true>), dim3(groups * kXcds * nsl), dim3(Cfg::NT), 0, a.stream,
                               static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                               static_cast<const uint16_t*>(a.v), ws, a.initial_state, a.final_state, nullptr,
                               a.B, a.T, a.H, a.dv, nsl, a.scale, status, save_S, save_E);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((main_kernel<DK>), dim3(groups * kXcds * nsl), dim3(Cfg::NT), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), ws, a.initial_state, a.final_state, a.y,
                       a.B, a.T, a.H, a.dv, nsl, a.scale, status, nullptr, nullptr);
    return hipGetLastError();
}

}  // namespace chunked

size_t prefill_bf16_workspace_bytes(int B, int T, int H) {
    const long nchunks = (T + chunked::C - 1) / chunked::C;
    return chunked::kStatusBytes + static_cast<size_t>(B) * H * nchunks * chunked::WS_CHUNK * sizeof(_Float16);
}

// The chunk-start states and E of every chunk ([b h chunk][d_k][d_v] and
// [b h chunk][token][d_v], rounded to fp16) from the same walk, for the
// backward pass; y is not formed.  d_k = d_v >= 64.
hipError_t launch_prefill_bf16_states(const PrefillArgs& a, float* S, float* E) {
    if (a.dk != a.dv) return hipErrorInvalidValue;
    switch (a.dk) {
        case 64: return chunked::launch_t<64>(a, S, E);
        case 128: return chunked::launch_t<128>(a, S, E);
        default: return hipErrorInvalidValue;
    }
}

// The backward's reverse walk (see rev_walk_kernel); d in {64, 128}.
hipError_t launch_bwd_reverse_walk(const RevWalkArgs& a) {
    if (a.T <= 0) return hipSuccess;
    const int nsl = a.d / 16;
    const int groups = (a.B * a.H + chunked::kXcds - 1) / chunked::kXcds;
    const dim3 grid(groups * chunked::kXcds * nsl);
    switch (a.d) {
        case 64:
            hipLaunchKernelGGL((chunked::rev_walk_kernel<64>), grid, dim3(512), 0, a.stream,
                               static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), a.beta, a.dy,
                               a.dST, a.g, a.Tm, a.dS, a.dR, a.dv, a.dS0, a.B, a.T, a.H, nsl, a.scale);
            break;
        case 128:
            hipLaunchKernelGGL((chunked::rev_walk_kernel<128>), grid, dim3(512), 0, a.stream,
                               static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), a.beta, a.dy,
                               a.dST, a.g, a.Tm, a.dS, a.dR, a.dv, a.dS0, a.B, a.T, a.H, nsl, a.scale);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
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
