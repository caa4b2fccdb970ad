// Multi-token (speculative) decode of the gated delta rule.
//
// The rainbus digest of "On the Design of Qwen3.8-Next Architecture" (its
// prerequisites section, the paragraph on multi-token prediction and
// speculative decoding) describes drafting several tokens at once and
// verifying them with the main model in parallel.  For the
// recurrent mixer a draft block of K tokens is K ordinary steps of the delta
// form (slinene ai-papers-daily page, Module A) taken from a live state; when
// the first j drafts are accepted, the live state must become the state after
// exactly those j steps.
//
// verify: one pass over the live state S_0 (read only).  With
//     G_t    = alpha_1 ... alpha_t          D(i, t) = alpha_{i+1} ... alpha_t
//     u_i    = beta_i e_i                   (the write of token i)
// the recurrence unrolls inside the block to
//     e_t = v_t - G_t S_0^T k_t - sum_{i<t}  D(i, t) (k_i . k_t) u_i
//     y_t = scale (G_t S_0^T q_t + sum_{i<=t} D(i, t) (k_i . q_t) u_i)
// so every output needs only the 2K column sums S_0^T k_t and S_0^T q_t (one
// read of the state, like a single decode step) plus K x K scalar dot
// products of the block's keys and queries.  The per-token misses e_t go out
// for the commit; optionally every prefix state S_t goes out too (K state
// writes, for callers that keep snapshots instead of committing).
//
// commit: S <- G_j S + sum_{i<j} D(i, j) k_i u_i^T for the j accepted drafts,
// one read and one write of the state, the same bytes as a decode step; a
// sequence with nothing accepted is not touched at all.
//
// Thread layout as in the single-token decode kernel: a thread owns one
// float4 column group of kRpt state rows spaced kRowGroups apart, so one load
// instruction of the workgroup covers kRowGroups consecutive rows.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <int DK, int DV>
struct MtpShape {
    static constexpr int kColGroups = DV / 4;
    static constexpr int kVec = DK * kColGroups;
    static constexpr int kRpt = kVec / 256 > 0 ? kVec / 256 : 1;
    static constexpr int kThreads = kVec / kRpt;
    static constexpr int kRowGroups = kThreads / kColGroups;
    static constexpr int kWaves = kThreads / 64;
};

__device__ __forceinline__ float4v fma4(float a, float4v x, float4v acc) {
    return float4v{acc.x + a * x.x, acc.y + a * x.y, acc.z + a * x.z, acc.w + a * x.w};
}

// Sum over the 16 lanes of a DPP row (quad permutations, then the half-row
// and row mirrors); every lane of the row ends with the total.
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false));  // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false));  // row_mirror
    return x;
}

// KM: compile-time upper bound of the block length K (tokens K..KM-1 are
// padding: zero q, k, v, alpha = 1, beta = 0, outputs not written).
// kPrefix: also write every prefix state (keeps the state slice in registers
// to the end; without it the slice dies after the column sums).
// kCommit: first commit the accepted prefix of the previous block (pk, pa,
// pb, pe, pacc; Kp tokens) onto the state slice in registers and write it
// back, then verify the new block from the committed state: one read and at
// most one write of the state for a whole draft round.
struct PendingBlock {
    const void* k;          // [N, Kp, H, d_k]
    const float* alpha;     // [N, Kp, H]
    const float* beta;
    const float* e;         // [N, Kp, H, d_v]
    const int* accepted;    // [N]
    int Kp;
};

template <int DK, int DV, int KM, bool kBf16, bool kPrefix, bool kCommit = false>
__global__ __launch_bounds__((MtpShape<DK, DV>::kThreads)) void mtp_verify_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, float* __restrict__ state,
    float* __restrict__ y, float* e_out, float* __restrict__ prefix, int K, int H,
    float scale, PendingBlock pend) {
    using Sh = MtpShape<DK, DV>;
    constexpr int KQ = 2 * KM;                 // k_0..k_{KM-1}, q_0..q_{KM-1}
    constexpr int kIn = (KQ * DK + Sh::kThreads - 1) / Sh::kThreads;
    constexpr int kVin = (KM * Sh::kColGroups + Sh::kThreads - 1) / Sh::kThreads;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int cg = tid % Sh::kColGroups;
    const int rg = tid / Sh::kColGroups;
    const int nh = blockIdx.x;
    const int n = nh / H, h = nh - n * H;

    // the block's q, k, v and gates first: the set-up below then waits only
    // for these, while the state stream issued after them is still in flight.
    // Token t of the block, head h, is row ((n K + t) H + h).  Every load is
    // unconditional (indices clamped into the block, padding selected to zero
    // afterwards) so that no branch makes the compiler wait for each load.
    float xin[kIn];
#pragma unroll
    for (int m = 0; m < kIn; ++m) {
        const int i = tid + m * Sh::kThreads;
        const int ic = i < KQ * DK ? i : KQ * DK - 1;
        const int t2 = ic / DK, r = ic - t2 * DK;
        const int t = t2 < KM ? t2 : t2 - KM;
        const int tc = t < K ? t : K - 1;
        const float x = load_in<kBf16>(t2 < KM ? k : q, (static_cast<long>(n * K + tc) * H + h) * DK + r);
        xin[m] = t < K ? x : 0.f;
    }
    float4v vin[kVin];
#pragma unroll
    for (int m = 0; m < kVin; ++m) {
        const int i = tid + m * Sh::kThreads;
        const int ic = i < KM * Sh::kColGroups ? i : KM * Sh::kColGroups - 1;
        const int t = ic / Sh::kColGroups, c = ic - t * Sh::kColGroups;
        const int tc = t < K ? t : K - 1;
        const long b = (static_cast<long>(n * K + tc) * H + h) * DV + 4 * c;
        const float4v x = float4v{load_in<kBf16>(v, b), load_in<kBf16>(v, b + 1), load_in<kBf16>(v, b + 2),
                                  load_in<kBf16>(v, b + 3)};
        vin[m] = t < K ? x : float4v{0.f, 0.f, 0.f, 0.f};
    }
    const int tg = tid < K ? tid : K - 1;
    const long g = static_cast<long>(n * K + tg) * H + h;
    const float a_ld = alpha[g], b_ld = beta[g];
    const float ain = tid < K ? a_ld : 1.f;
    const float bin = tid < K ? b_ld : 0.f;

    // the previous block's accepted writes (kCommit): u_t = beta_t e_t times
    // the decay still to come within the accepted prefix, and its keys
    constexpr int kPin = (KM * DK + Sh::kThreads - 1) / Sh::kThreads;
    int jacc = 0;
    float Gp = 1.f;
    float4v pu[KM];
    float xpk[kPin];
    if constexpr (kCommit) {
        jacc = pend.accepted[n];
        jacc = jacc < 0 ? 0 : (jacc > pend.Kp ? pend.Kp : jacc);
#pragma unroll
        for (int t = KM - 1; t >= 0; --t) {
            pu[t] = float4v{0.f, 0.f, 0.f, 0.f};
            if (t < jacc) {
                const long gp = static_cast<long>(n * pend.Kp + t) * H + h;
                const float4v et = *reinterpret_cast<const float4v*>(pend.e + gp * DV + 4 * cg);
                pu[t] = (Gp * pend.beta[gp]) * et;
                Gp *= pend.alpha[gp];
            }
        }
#pragma unroll
        for (int m = 0; m < kPin; ++m) {
            const int i = tid + m * Sh::kThreads;
            const int ic = i < KM * DK ? i : KM * DK - 1;
            const int t = ic / DK, r = ic - t * DK;
            const int tc = t < jacc ? t : 0;
            const float x = load_in<kBf16>(pend.k, (static_cast<long>(n * pend.Kp + tc) * H + h) * DK + r);
            xpk[m] = t < jacc ? x : 0.f;
        }
    }

    // the state slice of this thread: a read-once stream
    float4v* S = reinterpret_cast<float4v*>(state + static_cast<long>(nh) * DK * DV);
    float4v s[Sh::kRpt];
#pragma unroll
    for (int j = 0; j < Sh::kRpt; ++j)
        s[j] = __builtin_nontemporal_load(&S[(rg + j * Sh::kRowGroups) * Sh::kColGroups + cg]);

    __shared__ __align__(16) float skp[kCommit ? DK : 1][KM];       // previous block's keys (kCommit)
    __shared__ __align__(16) float skq[DK][KQ];                    // row r: k_t[r] then q_t[r]
    __shared__ float4v sv[KM][Sh::kColGroups];
    __shared__ float4v red[Sh::kWaves][KQ][Sh::kColGroups];
    __shared__ float skk[KM][KM], sqk[KM][KM];                     // k_i.k_t (i < t), k_i.q_t (i <= t)
    __shared__ float sa[KM], sb[KM];

#pragma unroll
    for (int m = 0; m < kIn; ++m) {
        const int i = tid + m * Sh::kThreads;
        const int t2 = i / DK, r = i - t2 * DK;
        if (i < KQ * DK) skq[r][t2] = xin[m];
    }
#pragma unroll
    for (int m = 0; m < kVin; ++m) {
        const int i = tid + m * Sh::kThreads;
        const int t = i / Sh::kColGroups, c = i - t * Sh::kColGroups;
        if (i < KM * Sh::kColGroups) sv[t][c] = vin[m];
    }
    if (tid < KM) {
        sa[tid] = ain;
        sb[tid] = bin;
    }
    if constexpr (kCommit) {
#pragma unroll
        for (int m = 0; m < kPin; ++m) {
            const int i = tid + m * Sh::kThreads;
            const int t = i / DK, r = i - t * DK;
            if (i < KM * DK) skp[r][t] = xpk[m];
        }
    }
    __syncthreads();
    if constexpr (kCommit) {
        // commit: S <- G_j S + sum_{t<j} k_t u_t^T, written back when anything was accepted
        if (jacc > 0) {
#pragma unroll
            for (int j = 0; j < Sh::kRpt; ++j) {
                const int r = rg + j * Sh::kRowGroups;
                float4v o = Gp * s[j];
#pragma unroll
                for (int t = 0; t < KM; ++t) o = fma4(skp[r][t], pu[t], o);
                s[j] = o;
                __builtin_nontemporal_store(o, &S[r * Sh::kColGroups + cg]);
            }
        }
    }

    // K x K dot products of the block, 16 lanes each: pair (a, b) gives
    // k_a.k_b when a < b and k_b.q_a when a >= b
    {
        constexpr int kGroups = Sh::kThreads / 16;
        const int grp = tid >> 4, sub = tid & 15;
#pragma unroll
        for (int d0 = 0; d0 < KM * KM; d0 += kGroups) {
            const int d = d0 + grp;
            const int a = d / KM, b = d - a * KM;
            const int c0 = a < b ? a : b, c1 = a < b ? b : KM + a;
            float x = 0.f;
            if (d < KM * KM) {
#pragma unroll
                for (int r = sub; r < DK; r += 16) x += skq[r][c0] * skq[r][c1];
            }
            x = row16_sum(x);
            if (sub == 0 && d < KM * KM) {
                if (a < b) skk[a][b] = x;
                else sqk[b][a] = x;
            }
        }
    }

    // column sums S_0^T k_t and S_0^T q_t over this thread's rows
    float4v acc[KQ];
#pragma unroll
    for (int c = 0; c < KQ; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < Sh::kRpt; ++j) {
        const float4v* row = reinterpret_cast<const float4v*>(&skq[rg + j * Sh::kRowGroups][0]);
#pragma unroll
        for (int c4 = 0; c4 < KQ / 4; ++c4) {
            const float4v w = row[c4];
            acc[4 * c4 + 0] = fma4(w.x, s[j], acc[4 * c4 + 0]);
            acc[4 * c4 + 1] = fma4(w.y, s[j], acc[4 * c4 + 1]);
            acc[4 * c4 + 2] = fma4(w.z, s[j], acc[4 * c4 + 2]);
            acc[4 * c4 + 3] = fma4(w.w, s[j], acc[4 * c4 + 3]);
        }
    }
    // lanes of one wave that share a column group differ by multiples of kColGroups
#pragma unroll
    for (int off = Sh::kColGroups; off < 64; off <<= 1) {
#pragma unroll
        for (int c = 0; c < KQ; ++c) {
            acc[c].x += __shfl_xor(acc[c].x, off);
            acc[c].y += __shfl_xor(acc[c].y, off);
            acc[c].z += __shfl_xor(acc[c].z, off);
            acc[c].w += __shfl_xor(acc[c].w, off);
        }
    }
    if (lane < Sh::kColGroups) {
#pragma unroll
        for (int c = 0; c < KQ; ++c) red[wave][c][lane] = acc[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < KQ; ++c) {
        float4v t = red[0][c][cg];
#pragma unroll
        for (int w = 1; w < Sh::kWaves; ++w) t += red[w][c][cg];
        acc[c] = t;
    }

    // the block's recurrence, unrolled (t and i are compile-time; K is uniform)
    float4v u[KM];
    float dec[KM];
    float G = 1.f;
    const bool writer = rg == 0;
#pragma unroll
    for (int t = 0; t < KM; ++t) {
        u[t] = float4v{0.f, 0.f, 0.f, 0.f};
        dec[t] = 1.f;
        if (t < K) {
            const float a = sa[t];
            G *= a;
#pragma unroll
            for (int i = 0; i < t; ++i) dec[i] *= a;
            float4v m = sv[t][cg] - G * acc[t];
#pragma unroll
            for (int i = 0; i < t; ++i) m = fma4(-dec[i] * skk[i][t], u[i], m);
            u[t] = sb[t] * m;
            float4v yt = G * acc[KM + t];
#pragma unroll
            for (int i = 0; i <= t; ++i) yt = fma4(dec[i] * sqk[i][t], u[i], yt);
            if (writer) {
                const long o = (static_cast<long>(n * K + t) * H + h) * DV + 4 * cg;
                *reinterpret_cast<float4v*>(y + o) = scale * yt;
                if (e_out) *reinterpret_cast<float4v*>(e_out + o) = m;
            }
        }
    }

    // optional prefix states S_t = alpha_t S_{t-1} + k_t u_t^T
    if constexpr (kPrefix) {
#pragma unroll
        for (int t = 0; t < KM; ++t) {
            if (t < K) {
                const float a = sa[t];
                float4v* P = reinterpret_cast<float4v*>(
                    prefix + (static_cast<long>(n * K + t) * H + h) * DK * DV);
#pragma unroll
                for (int j = 0; j < Sh::kRpt; ++j) {
                    const int r = rg + j * Sh::kRowGroups;
                    s[j] = fma4(skq[r][t], u[t], a * s[j]);
                    __builtin_nontemporal_store(s[j], &P[r * Sh::kColGroups + cg]);
                }
            }
        }
    }
}

template <int DK, int DV, int KM, bool kBf16>
__global__ __launch_bounds__((MtpShape<DK, DV>::kThreads)) void mtp_commit_kernel(
    const void* __restrict__ k, const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ e, const int* __restrict__ accepted, float* __restrict__ state, int K,
    int H) {
    using Sh = MtpShape<DK, DV>;
    const int tid = threadIdx.x;
    const int cg = tid % Sh::kColGroups;
    const int rg = tid / Sh::kColGroups;
    const int nh = blockIdx.x;
    const int n = nh / H, h = nh - n * H;
    int j = accepted[n];
    j = j < 0 ? 0 : (j > K ? K : j);
    if (j == 0) return;                    // nothing accepted: the state stays as it is

    float4v* S = reinterpret_cast<float4v*>(state + static_cast<long>(nh) * DK * DV);
    float4v s[Sh::kRpt];
#pragma unroll
    for (int r = 0; r < Sh::kRpt; ++r) s[r] = S[(rg + r * Sh::kRowGroups) * Sh::kColGroups + cg];

    __shared__ __align__(16) float sk[DK][KM];
    for (int i = tid; i < KM * DK; i += Sh::kThreads) {
        const int t = i / DK, r = i - t * DK;
        sk[r][t] = t < j ? load_in<kBf16>(k, (static_cast<long>(n * K + t) * H + h) * DK + r) : 0.f;
    }
    // u_t = beta_t e_t scaled by the decay still to come, D(t, j)
    float4v u[KM];
    float G = 1.f;
#pragma unroll
    for (int t = KM - 1; t >= 0; --t) {
        u[t] = float4v{0.f, 0.f, 0.f, 0.f};
        if (t < j) {
            const long g = static_cast<long>(n * K + t) * H + h;
            const float4v et = *reinterpret_cast<const float4v*>(e + g * DV + 4 * cg);
            u[t] = (G * beta[g]) * et;
            G *= alpha[g];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < Sh::kRpt; ++r) {
        const int row = rg + r * Sh::kRowGroups;
        float4v o = G * s[r];
#pragma unroll
        for (int t = 0; t < KM; ++t) o = fma4(sk[row][t], u[t], o);
        __builtin_nontemporal_store(o, &S[row * Sh::kColGroups + cg]);
    }
}

template <int DK, int DV, int KM, bool kBf16>
static hipError_t launch_mtp_t(const MtpArgs& a) {
    using Sh = MtpShape<DK, DV>;
    const dim3 grid(static_cast<unsigned>(a.N * a.H)), block(Sh::kThreads);
    if (a.commit)
        hipLaunchKernelGGL((mtp_commit_kernel<DK, DV, KM, kBf16>), grid, block, 0, a.stream, a.k, a.alpha,
                           a.beta, a.e, a.accepted, a.state, a.K, a.H);
    else if (a.pend_accepted)
        hipLaunchKernelGGL((mtp_verify_kernel<DK, DV, KM, kBf16, false, true>), grid, block, 0, a.stream, a.q, a.k,
                           a.v, a.alpha, a.beta, a.state, a.y, a.e, nullptr, a.K, a.H, a.scale,
                           PendingBlock{a.pend_k, a.pend_alpha, a.pend_beta, a.pend_e, a.pend_accepted, a.Kp});
    else if (a.prefix)
        hipLaunchKernelGGL((mtp_verify_kernel<DK, DV, KM, kBf16, true>), grid, block, 0, a.stream, a.q, a.k,
                           a.v, a.alpha, a.beta, a.state, a.y, a.e, a.prefix, a.K, a.H, a.scale, PendingBlock{});
    else
        hipLaunchKernelGGL((mtp_verify_kernel<DK, DV, KM, kBf16, false>), grid, block, 0, a.stream, a.q, a.k,
                           a.v, a.alpha, a.beta, a.state, a.y, a.e, a.prefix, a.K, a.H, a.scale, PendingBlock{});
    return hipGetLastError();
}

template <int DK, int DV, bool kBf16>
static hipError_t launch_mtp_k(const MtpArgs& a) {
    const int km = a.pend_accepted && a.Kp > a.K ? a.Kp : a.K;
    return km <= 4 ? launch_mtp_t<DK, DV, 4, kBf16>(a) : launch_mtp_t<DK, DV, 8, kBf16>(a);
}

template <bool kBf16>
static hipError_t launch_mtp_dt(const MtpArgs& a) {
#define GDN_MTP_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch_mtp_k<DK_, DV_, kBf16>(a);
#define GDN_MTP_ROW(DK_) GDN_MTP_CASE(DK_, 16) GDN_MTP_CASE(DK_, 32) GDN_MTP_CASE(DK_, 64) GDN_MTP_CASE(DK_, 128)
    GDN_MTP_ROW(16) GDN_MTP_ROW(32) GDN_MTP_ROW(64) GDN_MTP_ROW(128)
#undef GDN_MTP_ROW
#undef GDN_MTP_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_mtp(const MtpArgs& a) {
    return a.bf16 ? launch_mtp_dt<true>(a) : launch_mtp_dt<false>(a);
}

}  // namespace gdn
