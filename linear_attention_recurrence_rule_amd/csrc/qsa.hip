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
//   qsa_prep_kernel   one wave per row (a query head or a pooled key), two
//                     dimensions per lane; the rotation angle is formed and
//                     reduced modulo 2 pi in double precision, so that long
//                     positions keep their phase.
//   qsa_score_kernel  64 queries x 64 blocks per workgroup, one head at a
//                     time through LDS: bf16 MFMA 16x16x32 (exact products,
//                     fp32 sums) or fp32 MFMA 16x16x4 for fp32 operands; ReLU
//                     per head, summed, written for complete blocks only.
//   qsa_select_kernel one wave per query: a value-range histogram finds the
//                     bin of the K_B-th score, its few candidates are ranked
//                     exactly (exact radix select on the order-preserving
//                     bits as the fallback), then an ordered compaction.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// prep: grid (rows / 4), 256 threads, one wave per row.  Rows [0, B n H) are
// query heads, rows [B n H, B n H + B nb) pooled keys.
// ---------------------------------------------------------------------------
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
    const long row = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const long nq = static_cast<long>(B) * n * H;
    const int nb = n / r;
    const long nk = static_cast<long>(B) * nb;
    if (row >= nq + nk) return;                      // whole waves drop out together
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
    const float ss = wave_sum(x[0] * x[0] + x[1] * x[1]);
    const float inv = 1.f / sqrtf(ss / static_cast<float>(D) + eps);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int d = lane + 64 * e;
        x[e] *= inv;
        if (w && d < D) x[e] *= w[d];
    }
    // partial rotary embedding: dimension d < rope_dims pairs with d +- half
    const int half = rope_dims / 2;
    float y[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int d = lane + 64 * e;
        // the partner value lives in lane (d +- half) mod 64, slot (d +- half) / 64
        const int pd = d < half ? d + half : d - half;
        const int pl = (pd >= 0 ? pd : 0) & 63, pe = (pd >= 0 ? pd : 0) >> 6;
        const float p0 = __shfl(x[0], pl), p1 = __shfl(x[1], pl);
        const float partner = pe ? p1 : p0;
        y[e] = x[e];
        if (d < rope_dims) {
            const int j = d < half ? d : d - half;
            const double ang = static_cast<double>(pos) * exp2(-2.0 * j / rope_dims * log2_base);
            const double red = ang - 6.283185307179586 * floor(ang * 0.15915494309189535);
            const float c = cosf(static_cast<float>(red)), s = sinf(static_cast<float>(red));
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

// ---------------------------------------------------------------------------
// scores, four query heads: the rows of the query tile are taken in their
// memory order (query, head), so the four rows a lane holds in each 16x16
// MFMA output tile are the four heads of one query and the ReLU-sum over
// heads stays inside the lane.  A workgroup keeps 32 queries (128 rows) in
// LDS and streams the visible 64-block key tiles through two LDS buffers,
// loading the next tile into registers while the current one is used.
// grid (ceil(n / 32), B), 256 threads; the longest query tiles go first.
// ---------------------------------------------------------------------------
template <int D, bool kBf16>
__global__ __launch_bounds__(256) void qsa_score4_kernel(const void* __restrict__ q, const void* __restrict__ kbar,
                                                         float* __restrict__ scores, float* __restrict__ rowmax, int n,
                                                         int r, int nb, long ldS) {
    constexpr int TQ = 32, TR = 4 * TQ, TB = 64;
    constexpr int ES = kBf16 ? 2 : 4;
    constexpr int LD = D + (kBf16 ? 8 : 4);
    constexpr int kVec = 16 / ES;                    // elements per 16-byte load
    constexpr int kKPer = TB * D / kVec / 256;       // 16-byte key loads per thread and tile
    const int ntq = (n + TQ - 1) / TQ;
    const int qt = ntq - 1 - static_cast<int>(blockIdx.x), b = blockIdx.y;
    const int i0 = qt * TQ;
    const int ilast = min(i0 + TQ, n) - 1;
    const int mvis = (ilast + 1) / r;                // blocks visible to the tile's last query
    if (mvis == 0) return;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;

    __shared__ __align__(16) unsigned char sQ[TR * LD * ES];
    __shared__ __align__(16) unsigned char sK[2][TB * LD * ES];
    __shared__ __align__(16) float sOut[4][8][TB + 4];          // each wave's 8 rows of the tile's scores

    const unsigned char* qb = static_cast<const unsigned char*>(q);
    const unsigned char* kb = static_cast<const unsigned char*>(kbar);
    for (int idx = tid; idx < TR * D / kVec; idx += 256) {
        const int rr = idx / (D / kVec), cc = idx - rr * (D / kVec);
        const int i = i0 + rr / 4;
        float4v v = {0.f, 0.f, 0.f, 0.f};
        if (i < n) v = *reinterpret_cast<const float4v*>(qb + ((static_cast<long>(b) * n + i0) * 4 * D + rr * D + cc * kVec) * ES);
        *reinterpret_cast<float4v*>(sQ + (rr * LD + cc * kVec) * ES) = v;
    }
    float4v pre[kKPer];
    auto fetch = [&](int bt) {
#pragma unroll
        for (int u = 0; u < kKPer; ++u) {
            const int idx = tid + 256 * u, rr = idx / (D / kVec), cc = idx - rr * (D / kVec);
            const int blk = min(bt * TB + rr, nb - 1);
            pre[u] = *reinterpret_cast<const float4v*>(kb + ((static_cast<long>(b) * nb + blk) * D + cc * kVec) * ES);
        }
    };
    auto publish = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kKPer; ++u) {
            const int idx = tid + 256 * u, rr = idx / (D / kVec), cc = idx - rr * (D / kVec);
            *reinterpret_cast<float4v*>(sK[buf] + (rr * LD + cc * kVec) * ES) = pre[u];
        }
    };
    const int nbt = (mvis + TB - 1) / TB;
    float rmax[2] = {0.f, 0.f};
    fetch(0);
    publish(0);
    __syncthreads();
    for (int bt = 0; bt < nbt; ++bt) {
        const int buf = bt & 1;
        fetch(bt + 1 < nbt ? bt + 1 : bt);
        const int b0 = bt * TB;
        float4v acc[2][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = float4v{0.f, 0.f, 0.f, 0.f};
        if constexpr (kBf16) {
            const __bf16* A = reinterpret_cast<const __bf16*>(sQ) + (32 * wave + (l & 15)) * LD + 8 * (l >> 4);
            const __bf16* Bt = reinterpret_cast<const __bf16*>(sK[buf]) + (l & 15) * LD + 8 * (l >> 4);
#pragma unroll
            for (int k = 0; k < D; k += 32) {
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(A + k);
                const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(A + 16 * LD + k);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const bf16x8 bv = *reinterpret_cast<const bf16x8*>(Bt + 16 * nt * LD + k);
                    acc[0][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bv, acc[0][nt], 0, 0, 0);
                    acc[1][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bv, acc[1][nt], 0, 0, 0);
                }
            }
        } else {
            const float* A = reinterpret_cast<const float*>(sQ) + (32 * wave + (l & 15)) * LD + (l >> 4) * (D / 4);
            const float* Bt = reinterpret_cast<const float*>(sK[buf]) + (l & 15) * LD + (l >> 4) * (D / 4);
#pragma unroll 8
            for (int k = 0; k < D / 4; ++k) {
                const float a0 = A[k], a1 = A[16 * LD + k];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const float bv = Bt[16 * nt * LD + k];
                    acc[0][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, bv, acc[0][nt], 0, 0, 0);
                    acc[1][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bv, acc[1][nt], 0, 0, 0);
                }
            }
        }
        // the tile's scores go out as whole 256-byte row pieces through a
        // wave-private LDS staging area, with streaming stores; entries past a
        // row's visible blocks are written too (within the row's padded
        // storage) and never read
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int i = i0 + 8 * wave + 4 * mt + (l >> 4);
            const int vis = (i + 1) / r;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int blk = b0 + 16 * nt + (l & 15);
                const float sc = fmaxf(acc[mt][nt][0], 0.f) + fmaxf(acc[mt][nt][1], 0.f) +
                                 fmaxf(acc[mt][nt][2], 0.f) + fmaxf(acc[mt][nt][3], 0.f);
                if (blk < vis) rmax[mt] = fmaxf(rmax[mt], sc);
                sOut[wave][4 * mt + (l >> 4)][16 * nt + (l & 15)] = sc;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int f = l + 64 * p, row = f >> 4, c4 = f & 15;
            const int i = i0 + 8 * wave + row;
            if (i < n)
                __builtin_nontemporal_store(*reinterpret_cast<const float4v*>(&sOut[wave][row][4 * c4]),
                                            reinterpret_cast<float4v*>(&scores[(static_cast<long>(b) * n + i) * ldS + b0 + 4 * c4]));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        publish(buf ^ 1);
        __syncthreads();
    }
    // per-row maximum of the visible scores (16 lanes share a row)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        float x = rmax[mt];
        x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false)));
        x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false)));
        x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false)));
        x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false)));
        const int i = i0 + 8 * wave + 4 * mt + (l >> 4);
        if ((l & 15) == 0 && i < n) rowmax[static_cast<long>(b) * n + i] = x;
    }
}

// ---------------------------------------------------------------------------
// select: grid (ceil(n / 4), B), 256 threads, one wave per query.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned order_key(float f) {   // order-preserving bits of a float
    const unsigned u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-level helpers: one wave owns one query row, so no workgroup barriers
// are needed.  LDS writes and reads of one wave execute in order; the fences
// below only keep the compiler from moving them across each other.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ unsigned wave_suffix_incl(unsigned x) {     // sum over lanes >= this lane
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const unsigned y = __shfl_down(x, off);
        if (lane + off < 64) x += y;
    }
    return x;
}
__device__ __forceinline__ unsigned wave_prefix_excl(unsigned v) {     // sum over lanes < this lane
    const int lane = threadIdx.x & 63;
    unsigned x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const unsigned y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x - v;
}
__device__ __forceinline__ unsigned wave_sum_u(unsigned x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// Bin beta of an nbins histogram with count(> beta) < need <= count(>= beta);
// *above = count(> beta).  Lane l covers bins [l per, l per + per).
__device__ __forceinline__ unsigned wave_threshold(const unsigned* hist, int per, unsigned need, unsigned* above) {
    const int lane = threadIdx.x & 63;
    unsigned c = 0;
    for (int j = 0; j < per; ++j) c += hist[lane * per + j];
    const unsigned incl = wave_suffix_incl(c), excl = incl - c;
    unsigned bin = 0, acc = excl;
    const bool mine = excl < need && need <= incl;
    if (mine) {
        for (int j = per - 1; j >= 0; --j) {
            const unsigned hv = hist[lane * per + j];
            if (acc + hv >= need) {
                bin = lane * per + j;
                break;
            }
            acc += hv;
        }
    }
    const int src = __ffsll(static_cast<long long>(__ballot(mine))) - 1;
    *above = __shfl(acc, src);
    return __shfl(bin, src);
}

// The row of query i: m valid scores, storage padded to whole float4s.
// `visit(j, value)` is called for every j < m; four float4 loads per lane are
// in flight at a time.
template <class F>
__device__ __forceinline__ void for_each_score(const float* row, int m, const F& visit) {
    const int lane = threadIdx.x & 63;
    const int m4 = (m + 3) / 4;
    for (int v0 = 0; v0 < m4; v0 += 256) {
        float4v x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = reinterpret_cast<const float4v*>(row)[min(v0 + lane + 64 * u, m4 - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = v0 + lane + 64 * u;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (v < m4 && 4 * v + e < m) visit(4 * v + e, x[u][e]);
        }
    }
}

// Wave-uniform walk over the row in float4 groups, in ascending order: lane
// l gets group v0 + l, 64 groups (256 entries) per step, four steps' loads in
// flight; `f(v, x, base)` runs for every step on the whole wave (groups past
// the row end get v >= m4 and entries the caller must skip by j < m), with a
// running counter the caller advances.
template <class F>
__device__ __forceinline__ void for_groups(const float* row, int m, const F& f) {
    const int lane = threadIdx.x & 63;
    const int m4 = (m + 3) / 4;
    unsigned base = 0;
    for (int v0 = 0; v0 < m4; v0 += 256) {
        float4v x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = reinterpret_cast<const float4v*>(row)[min(v0 + lane + 64 * u, m4 - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (v0 + 64 * u < m4) f(v0 + lane + 64 * u, x[u], base);
    }
}

constexpr int kBins = 2048;

// Exact radix select (11 + 11 + 10 bits of the order key), used when the
// value histogram leaves more than 64 candidates in the threshold bin (ties,
// degenerate rows): returns the cut, the KB-th largest (key, index).
__device__ void radix_cut_wave(const float* row, int m, int KB, unsigned* hist, unsigned& ckey, int& cidx) {
    const int lane = threadIdx.x & 63;
    unsigned need = KB, above;
    for (int j = lane; j < kBins; j += 64) hist[j] = 0;
    wave_sync();
    for_each_score(row, m, [&](int, float v) { atomicAdd(&hist[order_key(v) >> 21], 1u); });
    wave_sync();
    const unsigned b1 = wave_threshold(hist, kBins / 64, need, &above);
    need -= above;
    wave_sync();
    for (int j = lane; j < kBins; j += 64) hist[j] = 0;
    wave_sync();
    for_each_score(row, m, [&](int, float v) {
        const unsigned u = order_key(v);
        if ((u >> 21) == b1) atomicAdd(&hist[(u >> 10) & 0x7FFu], 1u);
    });
    wave_sync();
    const unsigned b2 = wave_threshold(hist, kBins / 64, need, &above);
    need -= above;
    const unsigned pre = (b1 << 11) | b2;
    wave_sync();
    for (int j = lane; j < 1024; j += 64) hist[j] = 0;
    wave_sync();
    for_each_score(row, m, [&](int, float v) {
        const unsigned u = order_key(v);
        if ((u >> 10) == pre) atomicAdd(&hist[u & 0x3FFu], 1u);
    });
    wave_sync();
    const unsigned b3 = wave_threshold(hist, 1024 / 64, need, &above);
    need -= above;                                   // keys equal to ustar still to take (>= 1)
    const unsigned ustar = (pre << 10) | b3;
    // the need-th largest index among the keys equal to ustar, scanning down
    // in groups of 64 consecutive entries (ties go to the later block)
    unsigned seen = 0;
    int found = -1;
    for (int g0 = ((m - 1) / 64) * 64; g0 >= 0 && found < 0; g0 -= 64) {
        const int j = g0 + lane;
        const bool eq = j < m && order_key(row[j]) == ustar;
        const unsigned long long mask = __ballot(eq);
        const unsigned cnt = static_cast<unsigned>(__popcll(mask));
        if (seen + cnt >= need) {
            // lanes above j among the equal ones, counted from the top
            const unsigned rank = seen + static_cast<unsigned>(__popcll(mask >> lane)) ;   // includes this lane
            const bool hit = eq && rank == need;
            found = __shfl(j, __ffsll(static_cast<long long>(__ballot(hit))) - 1);
        }
        seen += cnt;
    }
    ckey = ustar;
    cidx = found;
}

// One wave per query row; four rows per workgroup.  A value-range histogram
// (2048 equal bins over [0, row max]; the scores are sums of ReLUs, never
// negative) finds the bin holding the K_B-th largest score; zeros, which all
// share bin 0, are counted per lane rather than with atomics.  The threshold
// bin's candidates (a handful for continuous scores) are ranked against each
// other by (score, index) to find the cut; more than 64 of them fall back to
// the exact radix select.  The selected blocks then go out in ascending order.
__global__ __launch_bounds__(256) void qsa_select_kernel(const float* __restrict__ scores,
                                                         const float* __restrict__ rowmax, int* __restrict__ idx,
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
    const float* row = scores + (static_cast<long>(b) * n + i) * ldS;
    __shared__ unsigned shist[4][kBins];
    __shared__ unsigned sck[4][64];
    __shared__ int sci[4][64];
    unsigned* hist = shist[w];

    float mx = 0.f;
    if (rowmax) {
        mx = rowmax[static_cast<long>(b) * n + i];   // from the scoring pass
    } else {
        for_each_score(row, m, [&](int, float v) { mx = fmaxf(mx, v); });
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    }
    for (int j = lane; j < kBins; j += 64) hist[j] = 0;
    wave_sync();

    unsigned ckey = 0;
    int cidx = 0;
    bool fast = mx > 0.f;
    if (fast) {
        const float scale = static_cast<float>(kBins) / mx;
        auto bin_of = [&](float v) {
            return v == 0.f ? 0u : static_cast<unsigned>(min(kBins - 1, static_cast<int>(v * scale)));
        };
        unsigned zeros = 0;
        for_each_score(row, m, [&](int, float v) {
            if (v == 0.f) ++zeros;
            else atomicAdd(&hist[bin_of(v)], 1u);
        });
        zeros = wave_sum_u(zeros);
        if (lane == 0 && zeros) atomicAdd(&hist[0], zeros);
        wave_sync();
        unsigned above;
        const unsigned beta = wave_threshold(hist, kBins / 64, KB, &above);
        const unsigned cb = hist[beta];
        fast = cb <= 64;
        if (fast) {
            // collect the threshold bin's entries (any order: they are ranked next)
            for_groups(row, m, [&](int v, const float4v& x, unsigned& base) {
                unsigned inm = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * v + e < m && bin_of(x[e]) == beta) inm |= 1u << e;
                const unsigned cnt = __popc(inm);
                unsigned slot = base + wave_prefix_excl(cnt);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (inm & (1u << e)) {
                        sck[w][slot] = order_key(x[e]);
                        sci[w][slot] = 4 * v + e;
                        ++slot;
                    }
                base += wave_sum_u(cnt);
            });
            wave_sync();
            const unsigned need = KB - above;        // taken from this bin, 1 .. cb
            unsigned k0 = 0;
            int i0 = 0;
            bool hit = false;
            if (lane < static_cast<int>(cb)) {
                k0 = sck[w][lane];
                i0 = sci[w][lane];
                unsigned rank = 0;
                for (unsigned c = 0; c < cb; ++c) {
                    const unsigned k1 = sck[w][c];
                    rank += k1 > k0 || (k1 == k0 && sci[w][c] > i0);
                }
                hit = rank == need - 1;
            }
            const int src = __ffsll(static_cast<long long>(__ballot(hit))) - 1;
            ckey = __shfl(k0, src);
            cidx = __shfl(i0, src);
        }
    }
    if (!fast) {
        wave_sync();
        radix_cut_wave(row, m, KB, hist, ckey, cidx);
    }

    // ordered compaction: entries with (key, j) >= (ckey, cidx), ascending
    for_groups(row, m, [&](int v, const float4v& x, unsigned& base) {
        unsigned selm = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * v + e;
            const unsigned u = order_key(x[e]);
            if (j < m && (u > ckey || (u == ckey && j >= cidx))) selm |= 1u << e;
        }
        const unsigned cnt = __popc(selm);
        unsigned pos = base + wave_prefix_excl(cnt);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (selm & (1u << e)) out[pos++] = 4 * v + e;
        base += wave_sum_u(cnt);
    });
}

}  // namespace qsa

// Workspace: the fp32 scores, rows padded to 64 blocks, then the per-row maxima.
size_t qsa_select_workspace_bytes(int B, int n, int r) {
    const long nb = n / r;
    const long ld = (nb + 63) / 64 * 64;
    return static_cast<size_t>(B) * n * ld * 4 + ((static_cast<size_t>(B) * n * 4 + 255) & ~static_cast<size_t>(255));
}

template <bool kBf16>
static hipError_t launch_qsa_prep_t(const QsaPrepArgs& a) {
    const long rows = static_cast<long>(a.B) * a.n * a.H + static_cast<long>(a.B) * (a.n / a.r);
    hipLaunchKernelGGL((qsa::qsa_prep_kernel<kBf16>), dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0,
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
    float* rowmax = scores + static_cast<long>(a.B) * a.n * ld;
    const bool four = a.H == 4;
    if (nb > 0 && four)
        hipLaunchKernelGGL((qsa::qsa_score4_kernel<D, kBf16>), dim3((a.n + 31) / 32, a.B), dim3(256), 0, a.stream, a.q,
                           a.kbar, scores, rowmax, a.n, a.r, nb, ld);
    else if (nb > 0)
        hipLaunchKernelGGL((qsa::qsa_score_kernel<D, kBf16>), dim3((a.n + 63) / 64, (nb + 63) / 64, a.B), dim3(256), 0,
                           a.stream, a.q, a.kbar, scores, a.n, a.H, a.r, nb, ld);
    hipLaunchKernelGGL(qsa::qsa_select_kernel, dim3((a.n + 3) / 4, a.B), dim3(256), 0, a.stream, scores,
                       four ? rowmax : nullptr, a.idx, a.n, a.r, a.KB, ld);
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
    return a.bf16 ? launch_qsa_select_dt<true>(a) : launch_qsa_select_dt<false>(a);
}

}  // namespace gdn
