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
// T' depends only on k, alpha and beta, so a chunk-parallel kernel
// (prep_kernel) computes it once per (head, chunk) into a workspace; the
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
//               transposed so it too feeds the MFMA from registers), then, once
//               the state wave has published E for the chunk, Y += P E -> y.
//   waves 3..7  loader waves: chunk c+1's q, k, v (bf16 -> fp16), k^T, T' and
//               the gates go to the other LDS buffer; one-word loads two to
//               three chunks ahead pull the lines into L2 so that these loads hit.
// Split-K operand layout: for a 16x16x32 MFMA, slot s of lane (m + 16 g) holds
// K-index 16*(s/4) + 4 g + s%4 of its row/column.  Two 16x16 accumulator tiles
// (lane (n + 16 g) holds rows 4 g .. 4 g + 3 of column n) stacked along K are
// exactly such a B operand, and A operands are read from LDS in the same order.
// LDS tiles are fp16 row-major with 16-byte chunks XOR-swizzled by row.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace chunked {

constexpr int C = 64;                    // tokens per chunk
constexpr int NB = C / 16;               // 16-token blocks per chunk
constexpr int NTB = NB * (NB + 1) / 2;   // lower 16x16 blocks of a chunk matrix
constexpr int TBLK = 256;                // halfs per 16x16 block
constexpr float kLogDecayFloor = -30.0f; // exp(-30) ~ 9e-14: alpha = 0 stays finite
constexpr int kXcds = 8;

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
    constexpr int kChunks = LD / 8;
    constexpr int kMask = (kChunks < 8 ? kChunks : 8) - 1;
    const int ch = col >> 3;
    return row * LD + (((ch ^ row) & kMask) | (ch & ~kMask)) * 8 + (col & 7);
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
// prep_kernel: T' = (I + A)^-1 diag(beta) for one (head, chunk).
// ===========================================================================
template <int DK>
struct PrepCfg {
    static constexpr int LDQ = DK + 8;   // padded rows (fp16)
    static constexpr int LDC = C + 8;
    static constexpr int LDA = C + 4;    // float rows, 16-byte aligned
    static constexpr int LDX = 16 + 8;
    static constexpr int NB = chunked::NB;
    static constexpr int NW = 4;
};

template <int DK>
struct PrepSmem {
    using Cfg = PrepCfg<DK>;
    _Float16 K[C * Cfg::LDQ];
    _Float16 A16[C * Cfg::LDC];
    _Float16 Tm[C * Cfg::LDC];
    _Float16 TT[C * Cfg::LDC];
    _Float16 X[Cfg::NW][16 * Cfg::LDX];
    float Af[C * Cfg::LDA];
    float g[C], beta[C];
};

// T = (I + A)^-1 for the unit lower-triangular chunk system, from A in
// sm.Af (float32) and sm.A16 (its fp16 copy).  The 16x16 diagonal blocks are
// inverted by forward substitution in float32 (one block per wave, one column
// per lane); then one block sub-diagonal per step,
//     T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ,
// whose terms all lie on earlier sub-diagonals.  Writes sm.Tm (row-major) and
// sm.TT (transposed).  Contains workgroup barriers: call from all 4 waves.
template <class Cfg, class Smem>
__device__ __forceinline__ void build_T(Smem& sm, int w, int l) {
    using M = Mma<_Float16>;
    constexpr int LDC = Cfg::LDC, LDA = Cfg::LDA, LDX = Cfg::LDX, NW = Cfg::NW;
    const int lr = l & 15, lq = l >> 4;
    if (w < NB && l < 16) {
        const int base = w * 16;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = (t == l) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < t; ++i) acc -= sm.Af[(base + t) * LDA + base + i] * x[i];
            x[t] = acc;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            sm.Tm[(base + t) * LDC + base + l] = static_cast<_Float16>(x[t]);
            sm.TT[(base + l) * LDC + base + t] = static_cast<_Float16>(x[t]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int lev = 1; lev < NB; ++lev) {
        for (int J = w; J + lev < NB; J += NW) {
            const int I = J + lev;
            const float4v x = M::range(sm.A16 + I * 16 * LDC, LDC, sm.TT + J * 16 * LDC, LDC, J * 16, I * 16,
                                       float4v{0.f, 0.f, 0.f, 0.f});
            _Float16* Xw = sm.X[w];
            *reinterpret_cast<half4*>(&Xw[lr * LDX + 4 * lq]) = to_h4(x);   // X transposed
            const float4v t = M::range(sm.Tm + I * 16 * LDC + I * 16, LDC, Xw, LDX, 0, 16,
                                       float4v{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.Tm[(I * 16 + 4 * lq + j) * LDC + J * 16 + lr] = static_cast<_Float16>(-t[j]);
            *reinterpret_cast<half4*>(&sm.TT[(J * 16 + lr) * LDC + I * 16 + 4 * lq]) =
                to_h4(-t[0], -t[1], -t[2], -t[3]);
        }
        __syncthreads();
    }
}

// Workspace layout: for each (b*H + h, chunk), the NTB lower 16x16 blocks of
// T' in the order (0,0),(1,0),(1,1),(2,0),...,(3,3), each row-major fp16.
template <int DK>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ k,
                                                   const float* __restrict__ alpha,
                                                   const float* __restrict__ beta,
                                                   _Float16* __restrict__ ws, int T, int H, int nchunks) {
    using Cfg = PrepCfg<DK>;
    using M = Mma<_Float16>;
    constexpr int LDQ = Cfg::LDQ, LDC = Cfg::LDC, LDA = Cfg::LDA;
    __shared__ PrepSmem<DK> sm;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lq = l >> 4;
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh % H;
    const int t0 = chunk * C;
    const long tok0 = static_cast<long>(b) * T;

    // k rows (bf16 -> fp16), zero past the end of the sequence
    for (int idx = tid; idx < C * DK / 8; idx += 256) {
        const int row = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (t0 + row < T) raw = *reinterpret_cast<const uint4*>(k + ((tok0 + t0 + row) * H + h) * DK + c8);
        const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
        half8 hv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            hv[2 * i] = static_cast<_Float16>(__uint_as_float(wds[i] << 16));
            hv[2 * i + 1] = static_cast<_Float16>(__uint_as_float(wds[i] & 0xffff0000u));
        }
        *reinterpret_cast<half8*>(&sm.K[row * LDQ + c8]) = hv;
    }
    if (w == 0) {
        float a = 1.f, be = 0.f;
        if (t0 + l < T) {
            const long off = (tok0 + t0 + l) * H + h;
            a = alpha[off];
            be = beta[off];
        }
        float lg = fmaxf(logf(a), kLogDecayFloor);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float t = __shfl_up(lg, off, 64);
            if (l >= off) lg += t;
        }
        sm.g[l] = lg;
        sm.beta[l] = be;
    }
    __syncthreads();

    // A = strictLower(diag(beta) (Gamma o K K^T)), tiles computed transposed
    // (K_J K_I^T) so that each lane holds 4 consecutive columns of one row.
    for (int tile = w; tile < NTB; tile += Cfg::NW) {
        int u = tile, I = 0;
        while (u > I) { u -= I + 1; ++I; }
        const int J = u;
        const float4v acc = M::range(sm.K + J * 16 * LDQ, LDQ, sm.K + I * 16 * LDQ, LDQ, 0, DK,
                                     float4v{0.f, 0.f, 0.f, 0.f});
        const int t = I * 16 + lr, i0 = J * 16 + 4 * lq;
        const float gt = sm.g[t], bt = sm.beta[t];
        float a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = (i0 + j < t) ? bt * expf(gt - sm.g[i0 + j]) * acc[j] : 0.f;
        *reinterpret_cast<float4*>(&sm.Af[t * LDA + i0]) = make_float4(a[0], a[1], a[2], a[3]);
        *reinterpret_cast<half4*>(&sm.A16[t * LDC + i0]) = to_h4(a[0], a[1], a[2], a[3]);
    }
    __syncthreads();
    build_T<Cfg>(sm, w, l);

    // T' = T diag(beta), lower blocks, 8 halfs per item
    _Float16* dst = ws + (static_cast<long>(bh) * nchunks + chunk) * NTB * TBLK;
    for (int idx = tid; idx < NTB * TBLK / 8; idx += 256) {
        const int blk = idx / 32, r = (idx % 32) / 2, hh = idx % 2;
        int u = blk, I = 0;
        while (u > I) { u -= I + 1; ++I; }
        const int J = u;
        const half8 tv = *reinterpret_cast<const half8*>(&sm.Tm[(I * 16 + r) * LDC + J * 16 + 8 * hh]);
        half8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[e] = static_cast<_Float16>(static_cast<float>(tv[e]) * sm.beta[J * 16 + 8 * hh + e]);
        *reinterpret_cast<half8*>(dst + blk * TBLK + r * 16 + 8 * hh) = o;
    }
}

// ===========================================================================
// main_kernel: the sequential chunk walk for one (head, 16-column slice).
// ===========================================================================
template <int DK>
struct MainCfg {
    static constexpr int SV = 16;                  // value columns per workgroup
    static constexpr int NT = 512;                 // 8 waves
    static constexpr int W_STATE = 0, W_OUT0 = 1, W_LOAD0 = 3, NLW = 5;
    static constexpr int LT = NLW * 64;            // loader threads
    static constexpr int QC = DK / 8;              // 16-byte chunks per q/k row
    static constexpr int N_V = 64 * (SV / 8);      // v items
    static constexpr int N_T = NTB * TBLK / 8;     // T' items
    static_assert(N_V <= LT && N_T <= LT, "one v item and one T' item per loader thread");
    static constexpr int KSTEP = DK >= 32 ? DK / 32 : 1; // 32-wide K steps over d_k
    static constexpr int NST = DK / 16;            // 16-row state tiles
};

template <int DK>
struct MainSmem {
    using Cfg = MainCfg<DK>;
    _Float16 Q[2][C * DK];
    _Float16 K[2][C * DK];
    _Float16 KT[2][DK * C];
    _Float16 Tp[2][C * C];
    _Float16 VT[2][Cfg::SV * C];
    _Float16 ST[2][Cfg::SV * DK];   // f16 state slice transposed, by chunk parity
    _Float16 ET[Cfg::SV * C];       // E of the current chunk, transposed
    float g[2][C], gam[2][C], dec[2][C];
    int flagE;
};

template <int DK>
struct Prefetch {
    static constexpr int NQ = (64 * MainCfg<DK>::QC + MainCfg<DK>::LT - 1) / MainCfg<DK>::LT;
    uint4 q[NQ], k[NQ];
    uint4 v, t;
    float alpha;
};

// Loader items: q and k as (16-byte chunk cq, token t) with t = item % 64, so
// the 64 lanes of a wave take 64 consecutive tokens of one chunk column (the
// k^T scatter then spreads over the banks); v as (chunk cv, token); T' as 320
// 16-byte pieces of its 10 lower blocks.
template <int DK>
__device__ __forceinline__ void loader_load(Prefetch<DK>& pf, int chunk, int lt, bool gate_wave, int lane,
                                            const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                            const float* alpha, const _Float16* ws, long tok0, int T, int H,
                                            int DV, int col0, int h, long wsbase) {
    using Cfg = MainCfg<DK>;
    const int t0 = chunk * C;
    const long rowbase = (tok0 + t0) * H + h;
#pragma unroll
    for (int i = 0; i < Prefetch<DK>::NQ; ++i) {
        const int idx = lt + i * Cfg::LT;
        const int cq = idx / 64, t = idx % 64;
        pf.q[i] = pf.k[i] = make_uint4(0, 0, 0, 0);
        if (idx < 64 * Cfg::QC && t0 + t < T) {
            const long off = (rowbase + static_cast<long>(t) * H) * DK + cq * 8;
            pf.q[i] = *reinterpret_cast<const uint4*>(q + off);
            pf.k[i] = *reinterpret_cast<const uint4*>(k + off);
        }
    }
    pf.v = make_uint4(0, 0, 0, 0);
    if (lt < Cfg::N_V) {
        const int cv = lt / 64, t = lt % 64;
        if (t0 + t < T)
            pf.v = *reinterpret_cast<const uint4*>(v + (rowbase + static_cast<long>(t) * H) * DV + col0 + cv * 8);
    }
    pf.t = make_uint4(0, 0, 0, 0);
    if (lt < Cfg::N_T)
        pf.t = *reinterpret_cast<const uint4*>(ws + wsbase + static_cast<long>(chunk) * NTB * TBLK + lt * 8);
    pf.alpha = 1.f;
    if (gate_wave && t0 + lane < T) pf.alpha = alpha[rowbase + static_cast<long>(lane) * H];
}

// One 4-byte load per 128-byte line of a chunk's q rows, k rows, v slice rows
// and T' blocks (about one or two per loader thread): brings them into L2
// ahead of the real loads.  Returns the loaded words XORed together.
template <int DK>
__device__ __forceinline__ uint32_t loader_touch(int chunk, int lt, const uint16_t* q, const uint16_t* k,
                                                 const uint16_t* v, const _Float16* ws, long tok0, int T, int H,
                                                 int DV, int col0, int h, long wsbase) {
    using Cfg = MainCfg<DK>;
    constexpr int LPR = DK * 2 >= 128 ? DK * 2 / 128 : 1;   // lines per q/k row
    constexpr int NQK = 2 * 64 * LPR, NV = 64, NTL = NTB * TBLK * 2 / 128;
    const int t0 = chunk * C;
    uint32_t x = 0;
#pragma unroll
    for (int rep = 0; rep < (NQK + NV + NTL + Cfg::LT - 1) / Cfg::LT; ++rep) {
        const int idx = lt + rep * Cfg::LT;
        const uint32_t* p = nullptr;
        if (idx < NQK) {
            const int which = idx / (64 * LPR), rem = idx % (64 * LPR), t = rem / LPR, part = rem % LPR;
            if (t0 + t < T)
                p = reinterpret_cast<const uint32_t*>((which ? k : q) + ((tok0 + t0 + t) * H + h) * DK + part * 64);
        } else if (idx < NQK + NV) {
            const int t = idx - NQK;
            if (t0 + t < T)
                p = reinterpret_cast<const uint32_t*>(v + ((tok0 + t0 + t) * H + h) * static_cast<long>(DV) + col0);
        } else if (idx < NQK + NV + NTL) {
            p = reinterpret_cast<const uint32_t*>(ws + wsbase + static_cast<long>(chunk) * NTB * TBLK +
                                                  (idx - NQK - NV) * 64);
        }
        if (p) x ^= *p;
    }
    return x;
}

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
__device__ __forceinline__ void loader_store(const Prefetch<DK>& pf, MainSmem<DK>& sm, int buf, int lt,
                                             bool gate_wave, int lane) {
    using Cfg = MainCfg<DK>;
#pragma unroll
    for (int i = 0; i < Prefetch<DK>::NQ; ++i) {
        const int idx = lt + i * Cfg::LT;
        if (idx < 64 * Cfg::QC) {
            const int cq = idx / 64, t = idx % 64;
            *reinterpret_cast<half8*>(&sm.Q[buf][swz<DK>(t, cq * 8)]) = bf16x8_to_h8(pf.q[i]);
            const half8 kh = bf16x8_to_h8(pf.k[i]);
            *reinterpret_cast<half8*>(&sm.K[buf][swz<DK>(t, cq * 8)]) = kh;
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.KT[buf][swz<C>(cq * 8 + e, t)] = kh[e];
        }
    }
    if (lt < Cfg::N_V) {
        const int cv = lt / 64, t = lt % 64;
        const half8 vh = bf16x8_to_h8(pf.v);
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.VT[buf][swz<C>(cv * 8 + e, t)] = vh[e];
    }
    if (lt < Cfg::N_T) {
        const int blk = lt / 32, r = (lt % 32) / 2, hh = lt % 2;
        // lower block index -> (I, J): (0,0),(1,0),(1,1),(2,0),(2,1),(2,2),(3,0),...
        const int I = blk >= 6 ? 3 : blk >= 3 ? 2 : blk >= 1 ? 1 : 0;
        const int J = blk - I * (I + 1) / 2;
        *reinterpret_cast<uint4*>(&sm.Tp[buf][swz<C>(I * 16 + r, J * 16 + 8 * hh)]) = pf.t;
    }
    if (gate_wave) {
        float lg = fmaxf(logf(pf.alpha), kLogDecayFloor);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float t = __shfl_up(lg, off, 64);
            if (lane >= off) lg += t;
        }
        const float glast = __shfl(lg, C - 1, 64);
        sm.g[buf][lane] = lg;
        sm.gam[buf][lane] = expf(lg);
        sm.dec[buf][lane] = expf(glast - lg);
    }
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

// One chunk of the state chain (state wave).
template <int DK>
__device__ __forceinline__ void state_chunk(MainSmem<DK>& sm, StateRegs<DK>& st, int chunk, int lane) {
    using Cfg = MainCfg<DK>;
    const int buf = chunk & 1;
    const int lr = lane & 15, lq = lane >> 4;
    const _Float16* Kb = sm.K[buf];
    // K S
    float4v ks[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        ks[I] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < Cfg::KSTEP; ++kk) {
            const half8 a = DK >= 32 ? ld_split<DK>(Kb, I * 16 + lr, kk * 32, lq)
                                     : ld_split_lo<DK>(Kb, I * 16 + lr, 0, lq);
            ks[I] = mma(a, st.Sb[kk], ks[I]);
        }
    }
    // R = V - gamma K S, as the split-K B operand of T' R
    half4 rh[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        const int t = I * 16 + 4 * lq;
        const float4 gm = *reinterpret_cast<const float4*>(&sm.gam[buf][t]);
        const half4 vv = ld4<C>(sm.VT[buf], lr, t);
        rh[I] = to_h4(static_cast<float>(vv[0]) - gm.x * ks[I][0], static_cast<float>(vv[1]) - gm.y * ks[I][1],
                      static_cast<float>(vv[2]) - gm.z * ks[I][2], static_cast<float>(vv[3]) - gm.w * ks[I][3]);
    }
    const half8 Rb0 = cat(rh[0], rh[1]), Rb1 = cat(rh[2], rh[3]);
    // E = T' R (T' is zero above the diagonal blocks)
    float4v e[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        e[I] = mma(ld_split<C>(sm.Tp[buf], I * 16 + lr, 0, lq), Rb0, float4v{0.f, 0.f, 0.f, 0.f});
        if (I >= 2) e[I] = mma(ld_split<C>(sm.Tp[buf], I * 16 + lr, 32, lq), Rb1, e[I]);
    }
    // publish E for the output waves; D E as the B operand of K^T (D E)
    half4 eh[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        const int t = I * 16 + 4 * lq;
        *reinterpret_cast<half4*>(&sm.ET[swz<C>(lr, t)]) = to_h4(e[I]);
        const float4 dc = *reinterpret_cast<const float4*>(&sm.dec[buf][t]);
        eh[I] = to_h4(dc.x * e[I][0], dc.y * e[I][1], dc.z * e[I][2], dc.w * e[I][3]);
    }
    __hip_atomic_store(&sm.flagE, chunk + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    const half8 Eb0 = cat(eh[0], eh[1]), Eb1 = cat(eh[2], eh[3]);
    // S = gamma_last S + K^T D E
    const float gl = sm.gam[buf][C - 1];
    _Float16* STn = sm.ST[buf ^ 1];
#pragma unroll
    for (int r = 0; r < Cfg::NST; ++r) {
        float4v u = mma(ld_split<C>(sm.KT[buf], r * 16 + lr, 0, lq), Eb0, float4v{0.f, 0.f, 0.f, 0.f});
        u = mma(ld_split<C>(sm.KT[buf], r * 16 + lr, 32, lq), Eb1, u);
#pragma unroll
        for (int j = 0; j < 4; ++j) st.S[r][j] = gl * st.S[r][j] + u[j];
        *reinterpret_cast<half4*>(&STn[swz<DK>(lr, r * 16 + 4 * lq)]) = to_h4(st.S[r]);
    }
    state_refresh_operand(st);
}

// One chunk of output (output wave `rp`: token blocks {0,3} or {1,2}).
template <int DK>
__device__ __forceinline__ void output_chunk(MainSmem<DK>& sm, int chunk, int rp, int lane, float* y,
                                             long tok0, int T, int H, int DV, int col0, int h, float scale,
                                             int* spin_error) {
    using Cfg = MainCfg<DK>;
    const int buf = chunk & 1;
    const int lr = lane & 15, lq = lane >> 4;
    const _Float16* Qb = sm.Q[buf];
    const _Float16* Kb = sm.K[buf];
    const _Float16* STb = sm.ST[buf];
    float4v yacc[2];
    half8 Pa[2][2];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int I = (ii == 0) ? rp : 3 - rp;
        // gamma Q S
        float4v qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < Cfg::KSTEP; ++kk) {
            if constexpr (DK >= 32)
                qs = mma(ld_split<DK>(Qb, I * 16 + lr, kk * 32, lq), ld_split<DK>(STb, lr, kk * 32, lq), qs);
            else
                qs = mma(ld_split_lo<DK>(Qb, I * 16 + lr, 0, lq), ld_split_lo<DK>(STb, lr, 0, lq), qs);
        }
        const float4 gm = *reinterpret_cast<const float4*>(&sm.gam[buf][I * 16 + 4 * lq]);
        yacc[ii] = float4v{gm.x * qs[0], gm.y * qs[1], gm.z * qs[2], gm.w * qs[3]};
        // P rows of block I, built transposed: lane holds row t, columns 4 lq .. 4 lq + 3 of block J
        const int t = I * 16 + lr;
        const float gt = sm.g[buf][t];
        half4 ph[NB];
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            ph[J] = half4{};
            if (J <= I) {
                float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kq = 0; kq < Cfg::KSTEP; ++kq) {
                    if constexpr (DK >= 32)
                        acc = mma(ld8<DK>(Kb, J * 16 + lr, kq * 32 + 8 * lq), ld8<DK>(Qb, I * 16 + lr, kq * 32 + 8 * lq),
                                  acc);
                    else
                        acc = mma(lq < 2 ? ld8<DK>(Kb, J * 16 + lr, 8 * lq) : half8{},
                                  lq < 2 ? ld8<DK>(Qb, I * 16 + lr, 8 * lq) : half8{}, acc);
                }
                const int i0 = J * 16 + 4 * lq;
                const float4 gi = *reinterpret_cast<const float4*>(&sm.g[buf][i0]);
                ph[J] = to_h4(i0 + 0 <= t ? expf(gt - gi.x) * acc[0] : 0.f,
                              i0 + 1 <= t ? expf(gt - gi.y) * acc[1] : 0.f,
                              i0 + 2 <= t ? expf(gt - gi.z) * acc[2] : 0.f,
                              i0 + 3 <= t ? expf(gt - gi.w) * acc[3] : 0.f);
            }
        }
        Pa[ii][0] = cat(ph[0], ph[1]);
        Pa[ii][1] = cat(ph[2], ph[3]);
    }
    // wait until the state wave has published E for this chunk
    for (int it = 0; __hip_atomic_load(&sm.flagE, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <= chunk; ++it) {
        if (it > (1 << 22)) { *spin_error = 1; break; }
        __builtin_amdgcn_s_sleep(1);
    }
    const half8 Eb0 = ld_split<C>(sm.ET, lr, 0, lq), Eb1 = ld_split<C>(sm.ET, lr, 32, lq);
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int I = (ii == 0) ? rp : 3 - rp;
        float4v yv = mma(Pa[ii][0], Eb0, yacc[ii]);
        if (I >= 2) yv = mma(Pa[ii][1], Eb1, yv);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = chunk * C + I * 16 + 4 * lq + j;
            if (t < T) y[((tok0 + t) * H + h) * static_cast<long>(DV) + col0 + lr] = scale * yv[j];
        }
    }
}

template <int DK>
__global__ __launch_bounds__(512) void main_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, const float* __restrict__ alpha,
                                                   const float* __restrict__ beta, const _Float16* __restrict__ ws,
                                                   const float* __restrict__ S0, float* __restrict__ S_out,
                                                   float* __restrict__ y, int B, int T, int H, int DV, int nsl,
                                                   float scale) {
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
    const long wsbase = static_cast<long>(bh) * nchunks * NTB * TBLK;

    const bool is_state = (w == Cfg::W_STATE);
    const bool is_out = (w >= Cfg::W_OUT0 && w < Cfg::W_OUT0 + 2);
    const bool is_load = (w >= Cfg::W_LOAD0);
    const int lt = (w - Cfg::W_LOAD0) * 64 + lane;
    const bool gate_wave = (w == Cfg::W_LOAD0 + Cfg::NLW - 1);

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
        for (int c = 0; c < nchunks; ++c) {
            state_chunk<DK>(sm, st, c, lane);
            __syncthreads();
        }
        if (S_out) {
#pragma unroll
            for (int r = 0; r < Cfg::NST; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    S_out[(static_cast<long>(bh) * DK + r * 16 + 4 * lq + j) * DV + col0 + lr] = st.S[r][j];
        }
    } else if (is_out) {
        int spin_error = 0;
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            output_chunk<DK>(sm, c, w - Cfg::W_OUT0, lane, y, tok0, T, H, DV, col0, h, scale, &spin_error);
            __syncthreads();
        }
    } else {
        // loader: during chunk c, chunk c+1 is loaded (L2 hits) and stored to
        // the other buffer; chunk c+3 is touched so that it is in L2 by then.
        Prefetch<DK> pf;
        uint32_t sink = 0;
        auto ld = [&](int c) {
            loader_load<DK>(pf, c, lt, gate_wave, lane, q, k, v, alpha, ws, tok0, T, H, DV, col0, h, wsbase);
        };
        auto touch = [&](int c) {
            return c < nchunks ? loader_touch<DK>(c, lt, q, k, v, ws, tok0, T, H, DV, col0, h, wsbase) : 0u;
        };
        uint32_t tA = touch(1), tB = touch(2);
        if (nchunks > 0) {
            ld(0);
            loader_store<DK>(pf, sm, 0, lt, gate_wave, lane);
        }
        __syncthreads();
        auto step = [&](int c, uint32_t& slot) {
            if (c + 1 < nchunks) ld(c + 1);
            sink ^= slot;             // touched two chunks ago: long since arrived
            slot = touch(c + 3);
            if (c + 1 < nchunks) loader_store<DK>(pf, sm, (c + 1) & 1, lt, gate_wave, lane);
            __syncthreads();
        };
        for (int c = 0; c < nchunks; c += 2) {
            step(c, tA);
            if (c + 1 < nchunks) step(c + 1, tB);
        }
        sink ^= tA ^ tB;
        if (sink == 0x9e3779b9u && T < 0) y[0] = 0.f;   // keeps the touch loads; never true (T >= 0)
    }
}

template <int DK>
static hipError_t launch_t(const PrefillArgs& a) {
    using Cfg = MainCfg<DK>;
    const int nchunks = (a.T + C - 1) / C;
    _Float16* ws = static_cast<_Float16*>(a.workspace);
    if (nchunks > 0) {
        hipLaunchKernelGGL((prep_kernel<DK>), dim3(nchunks, a.B * a.H), dim3(256), 0, a.stream,
                           static_cast<const uint16_t*>(a.k), a.alpha, a.beta, ws, a.T, a.H, nchunks);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nsl = a.dv / Cfg::SV;
    const int groups = (a.B * a.H + kXcds - 1) / kXcds;
    hipLaunchKernelGGL((main_kernel<DK>), dim3(groups * kXcds * nsl), dim3(Cfg::NT), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.alpha, a.beta, ws, a.initial_state, a.final_state, a.y,
                       a.B, a.T, a.H, a.dv, nsl, a.scale);
    return hipGetLastError();
}

}  // namespace chunked

size_t prefill_bf16_workspace_bytes(int B, int T, int H) {
    const long nchunks = (T + chunked::C - 1) / chunked::C;
    return static_cast<size_t>(B) * H * nchunks * chunked::NTB * chunked::TBLK * sizeof(_Float16);
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
