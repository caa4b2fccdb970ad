// Chunked prefill of the gated delta rule on gfx950 (slinene ai-papers-daily
// page on Qwen3.8-Next, Module A: the delta-form recurrence, evaluated here in
// its chunkwise WY / UT-transform form).
//
// Chunkwise form.  For a chunk of C tokens starting from state S, with
// g_t = sum_{i<=t} log alpha_i (inside the chunk), gamma_t = exp(g_t),
// Gamma_ti = exp(g_t - g_i) for i <= t, and d_t = exp(g_last - g_t):
//   A_ti = beta_t Gamma_ti k_t.k_i (i < t),   T = (I + A)^-1 (unit lower)
//   R    = diag(beta) (V - diag(gamma) K S)
//   E    = T R                                 (rows: beta_t * miss of token t)
//   Y    = diag(gamma) Q S + P E,  P_ti = Gamma_ti q_t.k_i (i <= t)
//   S'   = gamma_last S + K^T diag(d) E
// Every product except the 16x16 diagonal blocks of T runs on MFMA.
//
// Parallel decomposition.  The recurrence is separable over value columns,
// so one workgroup owns a slice of SV columns of one (batch, head) state and
// walks its chunks in order, keeping the float32 state slice in registers for
// the whole sequence (plus a copy in LDS as an MFMA operand).  The
// slices of one head recompute the state-independent Gram products; they are
// placed on one XCD so that the q/k chunk loads they share hit that XCD's L2.
//
// This kernel serves float32 inputs (bf16 inputs take the kernels of
// prefill_chunked.hip).  Every product runs on float32 MFMA with float32
// operands and accumulation, with 64-token chunks for d_k <= 32 and 32-token
// chunks for d_k = 64 and 128, where the float32 tiles of a 64-token chunk do
// not fit the LDS.
//
// Workgroup: 4 waves.  Per chunk (barriers between stages):
//   0. chunk c's q, k, v, alpha, beta (prefetched into registers during chunk
//      c-1) go to LDS; wave 0 turns alpha into the in-chunk log-decay prefix;
//   1. Gram tiles K K^T -> A, Q K^T -> P (lower blocks only), K S -> R and
//      Q S -> the output accumulator;
//   2. T: diagonal 16x16 blocks by forward substitution (float32), then one
//      sub-diagonal of blocks per step, T_IJ = -T_II (sum_K A_IK T_KJ);
//   3. E = T R;
//   4. Y += P E (stored), S' = gamma_last S + K^T diag(d) E.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// log(alpha) is floored so that alpha = 0 gives a finite log-decay; exp of the
// floor (9e-14) is far below float32 resolution of any surviving term.
constexpr float kLogDecayFloor = -30.0f;
constexpr int kXcds = 8;

template <int DK_, int SV_, int C_>
struct PrefillCfg {
    static constexpr int DK = DK_, SV = SV_, C = C_;
    using Op = float;
    static constexpr int NW = 4, NT = 256;
    static constexpr int PAD = 16 / sizeof(Op);
    static constexpr int LDQ = DK + PAD;  // rows over d_k (Q, K, S^T)
    static constexpr int LDC = C + PAD;   // rows over chunk tokens
    static constexpr int LDA = C + 1;     // float32 A
    static constexpr int LDX = 16 + PAD;  // per-wave 16x16 scratch
    static constexpr int NB = C / 16;     // 16-token blocks per chunk
    static constexpr int NSV = SV / 16;   // 16-column tiles per slice
    static constexpr int NG = NB * (NB + 1) / 2;
    static constexpr int NS_TILES = (DK / 16) * NSV;
    static constexpr int NST = (NS_TILES + NW - 1) / NW;   // state tiles per wave
    static constexpr int NYB = (NB + NW - 1) / NW;         // output row blocks per wave
    static constexpr int EPL = 4;                          // input elements per 16-byte load
    static constexpr int QK_LOADS = (C * DK / EPL + NT - 1) / NT;
    static constexpr int V_LOADS = (C * SV / EPL + NT - 1) / NT;
};

template <class Cfg>
struct PrefillSmem {
    using Op = typename Cfg::Op;
    Op Q[Cfg::C * Cfg::LDQ];
    Op K[Cfg::C * Cfg::LDQ];
    Op KT[Cfg::DK * Cfg::LDC];
    Op P[Cfg::C * Cfg::LDC];
    Op Tm[Cfg::C * Cfg::LDC];   // T, row-major
    Op TT[Cfg::C * Cfg::LDC];   // T transposed
    Op A16[Cfg::C * Cfg::LDC];  // A as an MFMA operand
    Op ST[Cfg::SV * Cfg::LDQ];  // state slice transposed
    Op RT[Cfg::SV * Cfg::LDC];
    Op ET[Cfg::SV * Cfg::LDC];
    Op EdT[Cfg::SV * Cfg::LDC];
    Op X[Cfg::NW][16 * Cfg::LDX];
    float Af[Cfg::C * Cfg::LDA];
    float V[Cfg::C * Cfg::SV];
    float g[Cfg::C], gam[Cfg::C], beta[Cfg::C], dec[Cfg::C];
};

__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// One 16-byte global load as EPL = 4 floats.
__device__ __forceinline__ void unpack16(const uint4& r, float* out) {
    out[0] = __uint_as_float(r.x); out[1] = __uint_as_float(r.y);
    out[2] = __uint_as_float(r.z); out[3] = __uint_as_float(r.w);
}

template <class Cfg>
struct ChunkRegs {
    uint4 q[Cfg::QK_LOADS], k[Cfg::QK_LOADS], v[Cfg::V_LOADS];
    float alpha, beta;
};

// T = (I + A)^-1 for the unit lower-triangular chunk system, from the float32
// A in sm.Af (and its MFMA copy sm.A16).  The 16x16 diagonal blocks are
// inverted by forward substitution in float32 (one block per wave, one column
// per lane); then one block sub-diagonal per step,
//     T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ,
// whose terms all lie on earlier sub-diagonals.  Writes T to sm.Tm (row-major)
// and sm.TT (transposed).  Contains workgroup barriers: call from all waves.
template <class Cfg>
__device__ __forceinline__ void build_T(PrefillSmem<Cfg>& sm, int w, int l) {
    using Op = typename Cfg::Op;
    using M = Mma<Op>;
    constexpr int NB = Cfg::NB, NW = Cfg::NW, LDC = Cfg::LDC, LDA = Cfg::LDA, LDX = Cfg::LDX;
    const int lr = l & 15, lq = l >> 4;
    // ---- stage 2a: diagonal blocks of T by forward substitution ---------
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
            sm.Tm[(base + t) * LDC + base + l] = static_cast<Op>(x[t]);
            sm.TT[(base + l) * LDC + base + t] = static_cast<Op>(x[t]);
        }
    }
    __syncthreads();

    // ---- stage 2b: one sub-diagonal of T blocks per step ----------------
#pragma unroll
    for (int lev = 1; lev < NB; ++lev) {
        for (int J = w; J + lev < NB; J += NW) {
            const int I = J + lev;
            // X = sum_{K=J}^{I-1} A_IK T_KJ
            const float4v x = M::range(sm.A16 + I * 16 * LDC, LDC, sm.TT + J * 16 * LDC, LDC, J * 16,
                                       I * 16, float4v{0.f, 0.f, 0.f, 0.f});
            Op* Xw = sm.X[w];
            store4(&Xw[lr * LDX + 4 * lq], x[0], x[1], x[2], x[3]);   // X transposed
            const float4v t = M::range(sm.Tm + I * 16 * LDC + I * 16, LDC, Xw, LDX, 0, 16,
                                       float4v{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.Tm[(I * 16 + 4 * lq + j) * LDC + J * 16 + lr] = static_cast<Op>(-t[j]);
            store4(&sm.TT[(J * 16 + lr) * LDC + I * 16 + 4 * lq], -t[0], -t[1], -t[2], -t[3]);
        }
        __syncthreads();
    }

}

template <class Cfg>
__global__ __launch_bounds__(256) void prefill_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ S0, float* __restrict__ ST_out, float* __restrict__ y,
    int B, int T, int H, int DV, int nsl, float scale) {
    using Op = typename Cfg::Op;
    using M = Mma<Op>;
    constexpr int C = Cfg::C, DK = Cfg::DK, SV = Cfg::SV, NW = Cfg::NW, NB = Cfg::NB;
    constexpr int LDQ = Cfg::LDQ, LDC = Cfg::LDC, LDA = Cfg::LDA, LDX = Cfg::LDX, EPL = Cfg::EPL;
    __shared__ PrefillSmem<Cfg> sm;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lq = l >> 4;   // accumulator: rows 4*lq + j, column lr

    // workgroup -> (head, slice): consecutive block ids go to consecutive XCDs,
    // so the nsl slices of one head get ids that are equal modulo kXcds
    const int xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
    const int bh = (jx / nsl) * kXcds + xcd;
    const int slice = jx % nsl;
    if (bh >= B * H) return;
    const int b = bh / H, h = bh % H;
    const int col0 = slice * SV;
    const long rowstride_qk = static_cast<long>(H) * DK;
    const long rowstride_v = static_cast<long>(H) * DV;
    const long tok0 = static_cast<long>(b) * T;

    // ---- state slice: float32 master in registers (accumulator layout) ----
    float4v Sacc[Cfg::NST];
#pragma unroll
    for (int i = 0; i < Cfg::NST; ++i) {
        const int ti = w + i * NW;
        Sacc[i] = float4v{0.f, 0.f, 0.f, 0.f};
        if (ti < Cfg::NS_TILES) {
            const int rt = ti / Cfg::NSV, ct = ti % Cfg::NSV;
            const int n = ct * 16 + lr;
            if (S0) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    Sacc[i][j] = S0[(static_cast<long>(bh) * DK + rt * 16 + 4 * lq + j) * DV + col0 + n];
            }
            store4(&sm.ST[n * LDQ + rt * 16 + 4 * lq], Sacc[i][0], Sacc[i][1], Sacc[i][2], Sacc[i][3]);
        }
    }

    ChunkRegs<Cfg> rg;
    auto load_chunk = [&](int c) {
        const int t0 = c * C;
#pragma unroll
        for (int i = 0; i < Cfg::QK_LOADS; ++i) {
            const int idx = tid + i * Cfg::NT;
            const int row = idx / (DK / EPL), cv = idx % (DK / EPL);
            rg.q[i] = rg.k[i] = make_uint4(0, 0, 0, 0);
            if (idx < C * DK / EPL && t0 + row < T) {
                const long off = ((tok0 + t0 + row) * H + h) * DK + cv * EPL;
                rg.q[i] = *reinterpret_cast<const uint4*>(static_cast<const float*>(q) + off);
                rg.k[i] = *reinterpret_cast<const uint4*>(static_cast<const float*>(k) + off);
            }
        }
#pragma unroll
        for (int i = 0; i < Cfg::V_LOADS; ++i) {
            const int idx = tid + i * Cfg::NT;
            const int row = idx / (SV / EPL), cv = idx % (SV / EPL);
            rg.v[i] = make_uint4(0, 0, 0, 0);
            if (idx < C * SV / EPL && t0 + row < T) {
                const long off = ((tok0 + t0 + row) * H + h) * static_cast<long>(DV) + col0 + cv * EPL;
                rg.v[i] = *reinterpret_cast<const uint4*>(static_cast<const float*>(v) + off);
            }
        }
        rg.alpha = 1.f;
        rg.beta = 0.f;
        if (w == 0 && l < C && t0 + l < T) {
            const long off = (tok0 + t0 + l) * H + h;
            rg.alpha = alpha[off];
            rg.beta = beta[off];
        }
    };

    auto store_chunk = [&]() {
#pragma unroll
        for (int i = 0; i < Cfg::QK_LOADS; ++i) {
            const int idx = tid + i * Cfg::NT;
            if (idx < C * DK / EPL) {
                const int row = idx / (DK / EPL), c0 = (idx % (DK / EPL)) * EPL;
                float fq[EPL], fk[EPL];
                unpack16(rg.q[i], fq);
                unpack16(rg.k[i], fk);
#pragma unroll
                for (int e = 0; e < EPL; e += 4) {
                    store4(&sm.Q[row * LDQ + c0 + e], fq[e], fq[e + 1], fq[e + 2], fq[e + 3]);
                    store4(&sm.K[row * LDQ + c0 + e], fk[e], fk[e + 1], fk[e + 2], fk[e + 3]);
                }
#pragma unroll
                for (int e = 0; e < EPL; ++e) sm.KT[(c0 + e) * LDC + row] = static_cast<Op>(fk[e]);
            }
        }
#pragma unroll
        for (int i = 0; i < Cfg::V_LOADS; ++i) {
            const int idx = tid + i * Cfg::NT;
            if (idx < C * SV / EPL) {
                const int row = idx / (SV / EPL), c0 = (idx % (SV / EPL)) * EPL;
                float fv[EPL];
                unpack16(rg.v[i], fv);
#pragma unroll
                for (int e = 0; e < EPL; ++e) sm.V[row * SV + c0 + e] = fv[e];
            }
        }
        if (w == 0) {
            // in-chunk inclusive prefix sum of the floored log-decay
            float lg = (l < C) ? fmaxf(logf(rg.alpha), kLogDecayFloor) : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float t = __shfl_up(lg, off, 64);
                if (l >= off) lg += t;
            }
            const float glast = __shfl(lg, C - 1, 64);
            if (l < C) {
                sm.g[l] = lg;
                sm.gam[l] = expf(lg);
                sm.beta[l] = rg.beta;
                sm.dec[l] = expf(glast - lg);
            }
        }
    };

    const int nchunks = (T + C - 1) / C;
    if (nchunks > 0) load_chunk(0);

    for (int c = 0; c < nchunks; ++c) {
        store_chunk();
        __syncthreads();
        if (c + 1 < nchunks) load_chunk(c + 1);

        // ---- stage 1: Gram tiles (lower blocks), K S -> R, Q S -> Y --------
        float4v Yacc[Cfg::NYB][Cfg::NSV];
        for (int tile = w; tile < 2 * Cfg::NG; tile += NW) {
            const bool isP = tile >= Cfg::NG;
            int u = isP ? tile - Cfg::NG : tile;
            int I = 0;
            while (u > I) { u -= I + 1; ++I; }
            const int J = u;
            const Op* Arow = (isP ? sm.Q : sm.K) + I * 16 * LDQ;
            float4v acc = M::range(Arow, LDQ, sm.K + J * 16 * LDQ, LDQ, 0, DK, float4v{0.f, 0.f, 0.f, 0.f});
            const int i = J * 16 + lr;
            const float gi = sm.g[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = I * 16 + 4 * lq + j;
                if (isP) {
                    const float val = (t >= i) ? expf(sm.g[t] - gi) * acc[j] : 0.f;
                    sm.P[t * LDC + i] = static_cast<Op>(val);
                } else {
                    const float val = (t > i) ? sm.beta[t] * expf(sm.g[t] - gi) * acc[j] : 0.f;
                    sm.Af[t * LDA + i] = val;
                    sm.A16[t * LDC + i] = static_cast<Op>(val);
                }
            }
        }
#pragma unroll
        for (int yb = 0; yb < Cfg::NYB; ++yb) {
            const int I = w + yb * NW;
            if (I < NB) {
#pragma unroll
                for (int ct = 0; ct < Cfg::NSV; ++ct) {
                    const float4v z4 = {0.f, 0.f, 0.f, 0.f};
                    const float4v ks = M::range(sm.K + I * 16 * LDQ, LDQ, sm.ST + ct * 16 * LDQ, LDQ, 0, DK, z4);
                    const float4v qs = M::range(sm.Q + I * 16 * LDQ, LDQ, sm.ST + ct * 16 * LDQ, LDQ, 0, DK, z4);
                    const int n = ct * 16 + lr;
                    float r[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = I * 16 + 4 * lq + j;
                        r[j] = sm.beta[t] * (sm.V[t * SV + n] - sm.gam[t] * ks[j]);
                        Yacc[yb][ct][j] = sm.gam[t] * qs[j];
                    }
                    store4(&sm.RT[n * LDC + I * 16 + 4 * lq], r[0], r[1], r[2], r[3]);
                }
            }
        }
        __syncthreads();

        build_T<Cfg>(sm, w, l);

        // ---- stage 3: E = T R ------------------------------------------------
        for (int I = w; I < NB; I += NW) {
#pragma unroll
            for (int ct = 0; ct < Cfg::NSV; ++ct) {
                const float4v e = M::range(sm.Tm + I * 16 * LDC, LDC, sm.RT + ct * 16 * LDC, LDC, 0,
                                           (I + 1) * 16, float4v{0.f, 0.f, 0.f, 0.f});
                const int n = ct * 16 + lr, t0 = I * 16 + 4 * lq;
                store4(&sm.ET[n * LDC + t0], e[0], e[1], e[2], e[3]);
                store4(&sm.EdT[n * LDC + t0], sm.dec[t0] * e[0], sm.dec[t0 + 1] * e[1],
                       sm.dec[t0 + 2] * e[2], sm.dec[t0 + 3] * e[3]);
            }
        }
        __syncthreads();

        // ---- stage 4: Y = gamma Q S + P E (stored); S' = gamma_last S + K^T D E
#pragma unroll
        for (int yb = 0; yb < Cfg::NYB; ++yb) {
            const int I = w + yb * NW;
            if (I < NB) {
#pragma unroll
                for (int ct = 0; ct < Cfg::NSV; ++ct) {
                    const float4v yv = M::range(sm.P + I * 16 * LDC, LDC, sm.ET + ct * 16 * LDC, LDC, 0,
                                                (I + 1) * 16, Yacc[yb][ct]);
                    const int n = ct * 16 + lr;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = c * C + I * 16 + 4 * lq + j;
                        if (t < T) y[((tok0 + t) * H + h) * static_cast<long>(DV) + col0 + n] = scale * yv[j];
                    }
                }
            }
        }
        const float gl = sm.gam[C - 1];
#pragma unroll
        for (int i = 0; i < Cfg::NST; ++i) {
            const int ti = w + i * NW;
            if (ti < Cfg::NS_TILES) {
                const int rt = ti / Cfg::NSV, ct = ti % Cfg::NSV;
                const float4v upd = M::range(sm.KT + rt * 16 * LDC, LDC, sm.EdT + ct * 16 * LDC, LDC, 0, C,
                                             float4v{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int j = 0; j < 4; ++j) Sacc[i][j] = gl * Sacc[i][j] + upd[j];
                store4(&sm.ST[(ct * 16 + lr) * LDQ + rt * 16 + 4 * lq], Sacc[i][0], Sacc[i][1], Sacc[i][2],
                       Sacc[i][3]);
            }
        }
        __syncthreads();
    }

    if (ST_out) {
#pragma unroll
        for (int i = 0; i < Cfg::NST; ++i) {
            const int ti = w + i * NW;
            if (ti < Cfg::NS_TILES) {
                const int rt = ti / Cfg::NSV, ct = ti % Cfg::NSV;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ST_out[(static_cast<long>(bh) * DK + rt * 16 + 4 * lq + j) * DV + col0 + ct * 16 + lr] =
                        Sacc[i][j];
            }
        }
    }
}

template <int DK, int SV>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
    // C = 64 wherever the float32 tiles fit the 160 KB of LDS (d_k <= 32);
    // at d_k = 64 and 128 they do not, and the walk takes 32-token chunks
    using Cfg = PrefillCfg<DK, SV, DK <= 32 ? 64 : 32>;
    const int nsl = a.dv / SV;
    const int groups = (a.B * a.H + kXcds - 1) / kXcds;
    const long blocks = static_cast<long>(groups) * kXcds * nsl;
    hipLaunchKernelGGL((prefill_kernel<Cfg>), dim3(static_cast<unsigned>(blocks)), dim3(Cfg::NT), 0, a.stream,
                       a.q, a.k, a.v, a.alpha, a.beta, a.initial_state, a.final_state, a.y, a.B, a.T, a.H,
                       a.dv, nsl, a.scale);
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_prefill_dk(const PrefillArgs& a) {
    // One workgroup per (head, SV-column slice).  Narrow slices spread a few
    // heads over the 256 CUs; once there are enough heads, wider slices cut
    // the Gram work that every slice of a head repeats.
    constexpr int kCUs = 256;
    const long bh = static_cast<long>(a.B) * a.H;
    if (a.dv >= 32 && bh * (a.dv / 16) > kCUs) return launch_prefill_t<DK, 32>(a);
    return launch_prefill_t<DK, 16>(a);
}

hipError_t launch_prefill(const PrefillArgs& a) {
    if (a.bf16) return launch_prefill_bf16(a);
    switch (a.dk) {
        case 16: return launch_prefill_dk<16>(a);
        case 32: return launch_prefill_dk<32>(a);
        case 64: return launch_prefill_dk<64>(a);
        case 128: return launch_prefill_dk<128>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
