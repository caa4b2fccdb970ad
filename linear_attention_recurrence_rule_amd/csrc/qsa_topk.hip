// QSA top-K_B block selection for four query heads, without materialising
// the scores (slinene ai-papers-daily page on "On the Design of Qwen3.8-Next
// Architecture", Module B: block-causal scores
//     I_ib = sum_h ReLU(<q_i^h, kbar_b>)   over the complete blocks b r + r - 1 <= i,
// and the K_B = ceil(K / r) best blocks per query, ties going to the later
// block, reported in ascending order and -1 padded).
//
// A 64K-token sequence has 5.4e8 (query, block) scores, 2.1 GB in fp32, and a
// 1M-token one 1.4e11, so the scores are recomputed instead of stored:
//   qsa_kmax_kernel   max_b |kbar_b| per sequence.  With sum_h |q_i^h| it
//                     bounds every score of query i from above.
//   qsa_pass4_kernel  (histogram pass) scores with the same MFMA tiles as the
//                     materialised path, into a 256-bin histogram per query:
//                     bin 0 holds exact zeros, bins 2 .. 255 are 1/16-octave
//                     ranges of the float below the query's bound (15.9
//                     octaves), bin 1 is everything further down.  Long rows
//                     (16 key tiles or more) read one key tile in eight.  The
//                     result per query is a band [tlo, thi) of bit patterns
//                     meant to hold the K_B-th largest score: the exact
//                     threshold bin when every tile was read, else the bins
//                     of the sample ranks p K_B -+ (3.5 sqrt(p K_B) + 2).
//   qsa_pass4_kernel  (emit pass) every visible tile again: blocks at or above
//                     tlo are listed (bit pattern, block) in per-lane
//                     sub-lists of the query.
//   qsa_merge_kernel  one wave per query: the K_B - (outright count) best
//                     candidates are found by radix selection on the bit
//                     patterns (ties to the later block), and the union with the
//                     outright blocks goes out ascending through an LDS
//                     bitmap.  A band that missed (too few or too many taken
//                     outright) or an overflowing list queues the query.
//   qsa_exact_kernel  the queued queries, one workgroup each: the row's scores
//                     are recomputed (same MFMA step) into a scratch row and
//                     selected exactly there.
// The sub-lists take B n 16 (K_B / 16 + kCapB / 16 + 32) 8 bytes: 1.1 GB at
// 64K tokens, K_B = 512.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include "qsa_wave.hpp"

#include <type_traits>

namespace gdn {
namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kTB = 64;              // key blocks per tile
constexpr int kHB = 256;             // histogram bins per query

// sum over the four heads of ReLU(score); ReLU as a signed-integer max with 0
// on the bit pattern (negative floats, -0 included, are negative integers).
// Each term is +0 or a positive float, so the sum has its sign bit clear and
// its bit pattern orders like its value.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }
__device__ __forceinline__ float relu_sum(const float4v& a) {
    return relu(a[0]) + relu(a[1]) + relu(a[2]) + relu(a[3]);
}

// ---------------------------------------------------------------------------
// grid (1), 256 threads: zero the per-sequence key maxima and the queue count.
// grid (ceil(nb / 256), B), 256 threads: kmax[b] = max_j |kbar_j| (as bits:
// non-negative floats order like their bit patterns).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void qsa_zero_kernel(float* __restrict__ kmax, int B, int* __restrict__ qcount) {
    for (int j = threadIdx.x; j < B; j += 256) kmax[j] = 0.f;
    if (threadIdx.x == 0) *qcount = 0;
}

template <int D, bool kBf16>
__global__ __launch_bounds__(256) void qsa_kmax_kernel(const void* __restrict__ kbar, float* __restrict__ kmax,
                                                       int nb) {
    constexpr int ES = kBf16 ? 2 : 4, kVec = 16 / ES;
    const int b = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
    float ss = 0.f;
    if (j < nb) {
        const unsigned char* p = static_cast<const unsigned char*>(kbar) + (static_cast<long>(b) * nb + j) * D * ES;
#pragma unroll
        for (int e0 = 0; e0 < D; e0 += kVec) {
            const float4v raw = *reinterpret_cast<const float4v*>(p + e0 * ES);
            if constexpr (kBf16) {
                const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += static_cast<float>(x[e]) * static_cast<float>(x[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) ss += raw[e] * raw[e];
            }
        }
    }
    float x = sqrtf(ss);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned*>(kmax + b), __float_as_uint(x));
}

// ---------------------------------------------------------------------------
// Query fragments of one wave's 32 (query, head) tile rows, loaded from
// global memory once and kept in registers.  Rows are taken in memory order
// (query, head), so the four rows a lane holds in a 16x16 MFMA output tile
// are the four heads of one query and the ReLU-sum over heads stays in the
// lane (lane l holds query 8 w + 4 mt + l / 16, block column l % 16).
// ---------------------------------------------------------------------------
template <int D, bool kBf16, int MT>
struct QFrag;
template <int D, int MT>
struct QFrag<D, true, MT> {
    bf16x8 a[MT][D / 32];  // lane (r + 16 g): row r of 16-row group mt, elements 32 kk + 8 g .. + 8
};
template <int D, int MT>
struct QFrag<D, false, MT> {
    float a[MT][D / 4];    // lane (r + 16 g): row r, elements g D / 4 + k (split-K fp32 layout)
};

// A wave holds MT groups of 16 tile rows, 4 MT queries.
template <int D, bool kBf16, int MT>
__device__ __forceinline__ void load_qfrag(QFrag<D, kBf16, MT>& f, const void* q, int b, int n, int i0, int wave,
                                           int l, float (&sq)[MT]) {
    const int r = l & 15, g = l >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int R = 16 * MT * wave + 16 * mt + r;     // tile row: query R / 4, head R % 4
        const bool ok = i0 + R / 4 < n;
        const long base = ((static_cast<long>(b) * n + i0) * 4 + R) * D;
        float s = 0.f;
        if constexpr (kBf16) {
            const __bf16* p = static_cast<const __bf16*>(q) + base + 8 * g;
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                f.a[mt][kk] = ok ? *reinterpret_cast<const bf16x8*>(p + 32 * kk) : bf16x8{};
#pragma unroll
                for (int e = 0; e < 8; ++e) s += static_cast<float>(f.a[mt][kk][e]) * static_cast<float>(f.a[mt][kk][e]);
            }
        } else {
            const float* p = static_cast<const float*>(q) + base + g * (D / 4);
#pragma unroll
            for (int k4 = 0; k4 < D / 16; ++k4) {
                const float4v v = ok ? *reinterpret_cast<const float4v*>(p + 4 * k4) : float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f.a[mt][4 * k4 + e] = v[e];
                    s += v[e] * v[e];
                }
            }
        }
        sq[mt] = s;
    }
}

// Scores of one 64-block key tile for this wave's 4 MT queries:
// acc[mt][nt][h] = <q_i^h, kbar_blk>, i = i0 + 4 MT w + 4 mt + l / 16,
// blk = b0 + 16 nt + l % 16.  sK: 64 key rows of LD elements.
template <int D, bool kBf16, int LD, int MT>
__device__ __forceinline__ void tile_scores(const QFrag<D, kBf16, MT>& f, const unsigned char* sK, int l,
                                            float4v (&acc)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = float4v{0.f, 0.f, 0.f, 0.f};
    if constexpr (kBf16 && MT > 2) {
        // four or more groups reuse each B fragment enough to hide its read
        const __bf16* Bt = reinterpret_cast<const __bf16*>(sK) + (l & 15) * LD + 8 * (l >> 4);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const bf16x8 bv = *reinterpret_cast<const bf16x8*>(Bt + 16 * nt * LD + 32 * kk);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[mt][kk], bv, acc[mt][nt], 0, 0, 0);
            }
    } else if constexpr (kBf16) {
        // every B fragment of the tile is read before the first MFMA, so the
        // LDS latency is paid once per tile
        const __bf16* Bt = reinterpret_cast<const __bf16*>(sK) + (l & 15) * LD + 8 * (l >> 4);
        bf16x8 bv[D / 32][4];
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) bv[kk][nt] = *reinterpret_cast<const bf16x8*>(Bt + 16 * nt * LD + 32 * kk);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[mt][kk], bv[kk][nt], acc[mt][nt], 0, 0, 0);
    } else {
        const float* Bt = reinterpret_cast<const float*>(sK) + (l & 15) * LD + (l >> 4) * (D / 4);
#pragma unroll 8
        for (int k = 0; k < D / 4; ++k) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const float bv = Bt[16 * nt * LD + k];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[mt][k], bv, acc[mt][nt], 0, 0, 0);
            }
        }
    }
}

__device__ __forceinline__ float quad_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));
    return x;
}
__device__ __forceinline__ unsigned row16_sum_u(unsigned x) {    // sum over a row of 16 lanes
    x += static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0xB1, 0xf, 0xf, false));
    x += static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x4E, 0xf, 0xf, false));
    x += static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x141, 0xf, 0xf, false));
    x += static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x140, 0xf, 0xf, false));
    return x;
}

// Bins on the bit pattern u of a non-negative score (sign bit cleared, so
// that -0 reads as 0): bin 0 is u = 0; fine index u >> 19; bin b >= 2 starts
// at fine index lo + b - 2; bin 1 holds the positives below bin 2.  Lower
// edge (as a bit pattern) of bin b; bin 1 starts at the smallest positive.
__device__ __forceinline__ int ubin(unsigned u, int lo) {
    if (u == 0u) return 0;
    const int fi = static_cast<int>(u >> 19);
    return fi < lo ? 1 : min(kHB - 1, 2 + fi - lo);
}
__device__ __forceinline__ unsigned bin_edge(int b, int lo) {
    if (b <= 0) return 0u;
    if (b == 1) return 1u;
    const int fi = lo + b - 2;
    return fi > 0 ? static_cast<unsigned>(fi) << 19 : 1u;
}
// upper edge of bin b (the lower edge of bin b + 1; the top bin has none)
__device__ __forceinline__ unsigned bin_top(int b, int lo) {
    return b >= kHB - 1 ? 0xFFFFFFFFu : bin_edge(b + 1, lo);
}

// Key tiles of a query tile: all of them, or for long rows one tile in eight
// (tile 8 j + (5 j mod 8) of group j; the last group may be partial).
constexpr int kSampleFrom = 16;      // tiles below which the histogram pass reads every tile
constexpr int kCapB = 1024;          // candidates a query can rank in the merge
constexpr int kSlots = kCapB / 64;
constexpr int kMapWords = 256;       // merge: output bitmap chunk (16384 blocks)
__device__ __forceinline__ int sampled_tile(int j) { return 8 * j + ((5 * j) & 7); }

// ---------------------------------------------------------------------------
// Both scoring passes, 256 threads: the histogram pass with 4 waves x 8
// queries, grid (ceil(n / 32), B); the emit pass with 4 waves x 16 queries,
// grid (ceil(n / 64), B), so that each B fragment read from LDS feeds four
// MFMAs.  The longest query tiles go first.  The key tiles stream through
// two LDS buffers with register prefetch.
//   kEmit = false: histogram pass.  For each query with m > K_B it keeps the
//     band [tlo, thi) of score bit patterns that should hold its K_B-th
//     largest score: exact bin edges when every tile was read, otherwise the
//     bins of the sample ranks p K_B -+ (3.5 sqrt(p K_B) + 2), p the sampled
//     fraction of the query's blocks.
//   kEmit = true: emit pass over every visible tile.  Every block with
//     u >= tlo is listed as (bit pattern, block); the merge tells the
//     outright ones (u >= thi) from the candidates.  Each lane keeps its own
//     sub-list per query (the blocks of its residue mod 16), so no slot is
//     shared; the uncapped lengths are kept, which catches an overflow.
// ---------------------------------------------------------------------------
template <int D, bool kBf16, bool kEmit>
__global__ __launch_bounds__(256, kBf16 ? 2 : 1)   // bf16: two workgroups per CU
void qsa_pass4_kernel(const void* __restrict__ q, const void* __restrict__ kbar, const float* __restrict__ kmax,
                      uint2* __restrict__ info, int* __restrict__ cnt, uint2* __restrict__ list, int n, int r,
                      int nb, int KB, int cap) {
    constexpr int ES = kBf16 ? 2 : 4;
    constexpr int LD = D + (kBf16 ? 8 : 4);
    constexpr int kVec = 16 / ES;                    // elements per 16-byte load
    constexpr int kKPer = kTB * D / kVec / 256;      // 16-byte key loads per thread and tile
    constexpr int MT = kEmit ? 4 : 2;                // 16-row groups (4 queries each) per wave
    constexpr int TQ = 16 * MT;                      // queries per workgroup
    const int ntq = (n + TQ - 1) / TQ;
    const int qt = ntq - 1 - static_cast<int>(blockIdx.x), b = blockIdx.y;
    const int i0 = qt * TQ;
    const int ilast = min(i0 + TQ, n) - 1;
    const int mvis = (ilast + 1) / r;                // blocks visible to the tile's last query
    if (mvis <= KB) return;                          // every query of the tile keeps all its blocks
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, g = l >> 4;

    __shared__ __align__(16) unsigned char sK[2][kTB * LD * ES];
    __shared__ unsigned sH[kEmit ? 1 : TQ][kHB];

    QFrag<D, kBf16, MT> f;
    float sq[MT];
    load_qfrag<D, kBf16, MT>(f, q, b, n, i0, wave, l, sq);

    // this lane's MT queries
    int qi[MT], vis[MT];
    bool act[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        qi[mt] = i0 + 4 * MT * wave + 4 * mt + g;
        vis[mt] = qi[mt] < n ? (qi[mt] + 1) / r : 0;
        act[mt] = vis[mt] > KB;
    }
    const int nbt = (mvis + kTB - 1) / kTB;
    const bool sampled = !kEmit && nbt >= kSampleFrom;
    const int nsteps = sampled ? (nbt + 7) / 8 : nbt;
    auto tile_of = [&](int j) { return sampled ? sampled_tile(j) : j; };

    int lo[MT];
    unsigned tlo[MT];                                // emit pass: 0xFFFFFFFF (above every sum) keeps nothing
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        lo[mt] = 0;
        tlo[mt] = 0xFFFFFFFFu;
    }
    if constexpr (!kEmit) {
        // bound: sum_h |q^h| max_j |kbar_j|; lanes r = 4 u + h of group mt hold (query u, head h)
        const float km = kmax[b];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float s = sq[mt];
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            const float qn = quad_sum(sqrtf(s));     // sum over the four heads of query (l % 16) / 4
            const float ub = __shfl(qn, 4 * g) * km; // this lane's query in the output layout
            lo[mt] = static_cast<int>(((__float_as_uint(ub) >> 23) & 255u) + 1u) * 16 - (kHB - 2);
        }
        for (int j = l; j < 4 * MT * kHB; j += 64) sH[4 * MT * wave + j / kHB][j % kHB] = 0u;
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if (act[mt]) tlo[mt] = info[static_cast<long>(b) * n + qi[mt]].x;
    }
    // emit pass: this lane's sub-list of each of its queries (the blocks of residue l % 16)
    uint2* lrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        lrow[mt] = list + ((static_cast<long>(b) * n + (qi[mt] < n ? qi[mt] : 0)) * 16 + (l & 15)) * cap;
    // the wave's first query sees the fewest blocks: a tile below its count is
    // visible to all the wave's queries
    const int q_lo = i0 + 4 * MT * wave;
    const int vis_lo = q_lo < n ? (q_lo + 1) / r : 0;
    unsigned zc[MT];                                 // histogram pass: zeros seen by this lane
    int nl[MT];                                      // emit pass: this lane's sub-list lengths
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) zc[mt] = nl[mt] = 0;

    const unsigned char* kb = static_cast<const unsigned char*>(kbar);
    // key tiles: two register sets, loaded two steps ahead of their use
    float4v pre[2][kKPer];
    auto fetch = [&](float4v (&p)[kKPer], int bt) {
        bt = min(bt, nbt - 1);
#pragma unroll
        for (int u = 0; u < kKPer; ++u) {
            const int idx = tid + 256 * u, rr = idx / (D / kVec), c = idx - rr * (D / kVec);
            const int blk = min(bt * kTB + rr, nb - 1);
            p[u] = *reinterpret_cast<const float4v*>(kb + ((static_cast<long>(b) * nb + blk) * D + c * kVec) * ES);
        }
    };
    auto publish = [&](const float4v (&p)[kKPer], int buf) {
#pragma unroll
        for (int u = 0; u < kKPer; ++u) {
            const int idx = tid + 256 * u, rr = idx / (D / kVec), c = idx - rr * (D / kVec);
            *reinterpret_cast<float4v*>(sK[buf] + (rr * LD + c * kVec) * ES) = p[u];
        }
    };
    // emit pass: the blocks of one tile with u >= tlo go to the lane sub-lists;
    // a full tile (one every query of the wave sees whole) needs no per-block bound
    auto emit = [&](const float4v (&acc)[MT][4], int b0, auto full) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int blk = b0 + 16 * nt + (l & 15);
                const unsigned u = __float_as_uint(relu_sum(acc[mt][nt]));
                const bool keep = u >= tlo[mt] && (decltype(full)::value || blk < vis[mt]);
                if (keep && nl[mt] < cap)
                    lrow[mt][static_cast<unsigned>(nl[mt])] = make_uint2(u, static_cast<unsigned>(blk));
                nl[mt] += static_cast<int>(keep);
            }
        }
    };
    // step j: scores of key tile tile_of(j) from LDS buffer j & 1
    auto step = [&](int j, int buf) {
        const int bt = tile_of(j);                   // may pass nbt in the last sampled group
        const int b0 = bt * kTB;
        float4v acc[MT][4];
        tile_scores<D, kBf16, LD, MT>(f, sK[buf], l, acc);
        if constexpr (!kEmit) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const int blk = b0 + 16 * nt + (l & 15);
                    const unsigned u = __float_as_uint(relu_sum(acc[mt][nt]));
                    if (act[mt] && blk < vis[mt]) {
                        if (u == 0u) ++zc[mt];
                        else atomicAdd(&sH[4 * MT * wave + 4 * mt + g][ubin(u, lo[mt])], 1u);
                    }
                }
            }
        } else {
            if (b0 + kTB <= vis_lo) emit(acc, b0, std::true_type{});
            else emit(acc, b0, std::false_type{});
        }
    };
    fetch(pre[0], tile_of(0));
    publish(pre[0], 0);
    if (nsteps > 1) fetch(pre[1], tile_of(1));
    __syncthreads();
    // pairs of steps, so that the register sets and LDS buffers are fixed per step
    for (int j = 0; j < nsteps; j += 2) {
        if (j + 2 < nsteps) fetch(pre[0], tile_of(j + 2));
        step(j, 0);
        if (j + 1 < nsteps) publish(pre[1], 1);      // tile j + 1, loaded a step ago
        __syncthreads();
        if (j + 1 >= nsteps) break;
        if (j + 3 < nsteps) fetch(pre[1], tile_of(j + 3));
        step(j + 1, 1);
        if (j + 2 < nsteps) publish(pre[0], 0);      // tile j + 2
        __syncthreads();
    }
    if constexpr (!kEmit) {
        // zeros: one plain store per query (bin 0 gets no atomics)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const unsigned z = row16_sum_u(zc[mt]);
            if ((l & 15) == 0) sH[4 * MT * wave + 4 * mt + g][0] = z;
        }
        wave_sync();
#pragma unroll
        for (int rr = 0; rr < 4 * MT; ++rr) {
            const int i = i0 + 4 * MT * wave + rr;
            const int m = i < n ? (i + 1) / r : 0;
            if (m > KB) {                            // wave-uniform
                const unsigned* h = sH[4 * MT * wave + rr];
                const int lor = __shfl(lo[rr >> 2], 16 * (rr & 3));
                unsigned c4 = 0;
#pragma unroll
                for (int t = 0; t < kHB / 64; ++t) c4 += h[l * (kHB / 64) + t];
                const unsigned total = wave_sum_u(c4);            // sampled visible blocks
                unsigned khi = static_cast<unsigned>(KB), klo = static_cast<unsigned>(KB);
                if (sampled) {
                    const float k = static_cast<float>(KB) * static_cast<float>(total) / static_cast<float>(m);
                    // 3.5 standard deviations of the sampled rank: at 64K tokens
                    // no row then misses the band (at 3, a few did, and the
                    // exact pass that takes them cost ~120 us); at 4 and more
                    // some rows pass the 1024-candidate cap of the merge
                    const float dlt = 3.5f * sqrtf(k) + 2.f;
                    khi = k - dlt >= 1.f ? static_cast<unsigned>(k - dlt) : 0u;
                    klo = static_cast<unsigned>(ceilf(k + dlt));
                }
                unsigned above;
                unsigned th = 0xFFFFFFFFu, tl = 0u;
                if (khi >= 1u) th = bin_top(static_cast<int>(wave_threshold(h, kHB / 64, khi, &above)), lor);
                if (klo <= total) tl = bin_edge(static_cast<int>(wave_threshold(h, kHB / 64, klo, &above)), lor);
                if (l == 0) info[static_cast<long>(b) * n + i] = make_uint2(tl, th);
            }
        }
    } else {
        // per query: the 16 sub-list lengths (uncapped)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if (act[mt]) cnt[(static_cast<long>(b) * n + qi[mt]) * 16 + (l & 15)] = nl[mt];
    }
}

// ---------------------------------------------------------------------------
// merge: grid (ceil(n / 4), B), 256 threads, one wave per query.  The
// query's 16 sub-lists hold every block with u >= tlo; those with u >= thi
// are taken outright, the rest are candidates.  The candidates are gathered
// (LDS) and held in registers (slot t of lane l: candidate 64 t + l); the
// need-th largest bit pattern, need = K_B - (outright count), is found by
// radix selection, 10 bits a round, and among the ties at the cut the later
// blocks are taken (bisection on the index).
// The taken blocks are marked in an LDS bitmap, 16384 blocks at a time, and
// written out in ascending order.  A band that missed (need outside
// [1, candidates]) or an overflowing sub-list queues the query.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 4) void qsa_merge_kernel(const uint2* __restrict__ info, const int* __restrict__ cnt,
                                                        const uint2* __restrict__ list, int* __restrict__ idx,
                                                        int* __restrict__ queue, int* __restrict__ qcount, int n,
                                                        int r, int KB, int cap) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i = blockIdx.x * 4 + w, b = blockIdx.y;
    if (i >= n) return;                              // whole waves drop out
    const int m = (i + 1) / r;
    const long row = static_cast<long>(b) * n + i;
    int* out = idx + row * KB;
    if (m <= KB) {                                   // every candidate is selected
        for (int j = lane; j < KB; j += 64) out[j] = j < m ? j : -1;
        return;
    }
    __shared__ __align__(16) unsigned sKey[4][kCapB];
    __shared__ int sBlk[4][kCapB];
    __shared__ unsigned long long sMap[4][kMapWords];
    const unsigned thi = info[row].y;
    // lane l reads sub-list l % 16, entry pairs l / 16 + 4 t (16 bytes each):
    // 2 kBatch entries per lane in flight
    constexpr int kBatch = 8;
    const int sl = lane & 15;
    const int len = cnt[row * 16 + sl];
    const bool over = __ballot(len > cap) != 0ull;
    int maxlen = len;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) maxlen = max(maxlen, __shfl_xor(maxlen, off));
    const uint2* lst = list + (row * 16 + sl) * cap;
    const bool one_chunk = m <= 64 * kMapWords;
    // visit(u, blk) for every listed entry, kBatch loads per lane at a time
    auto load_pairs = [&](int k0, uint2 (&e)[2 * kBatch]) {
#pragma unroll
        for (int t = 0; t < kBatch; ++t) {
            const int k = k0 + 2 * ((lane >> 4) + 4 * t);
            uint4 v = make_uint4(0u, 0xFFFFFFFFu, 0u, 0xFFFFFFFFu);
            if (k < len) v = *reinterpret_cast<const uint4*>(lst + k);
            e[2 * t] = make_uint2(v.x, v.y);
            e[2 * t + 1] = k + 1 < len ? make_uint2(v.z, v.w) : make_uint2(0u, 0xFFFFFFFFu);
        }
    };
    auto for_entries = [&](auto visit) {
        for (int k0 = 0; k0 < maxlen; k0 += 8 * kBatch) {
            uint2 e[2 * kBatch];
            load_pairs(k0, e);
#pragma unroll
            for (int t = 0; t < 2 * kBatch; ++t) visit(e[t].x, static_cast<int>(e[t].y));
        }
    };
    auto mark = [&](int d, int c0) { atomicOr(&sMap[w][(d - c0) >> 6], 1ull << ((d - c0) & 63)); };
    // pass A: count the outright entries (marking them when the row fits one
    // bitmap chunk) and gather the candidates in list order
    if (one_chunk)
        for (int j = lane; j < (m + 63) / 64; j += 64) sMap[w][j] = 0ull;
    wave_sync();
    unsigned nc = 0, nd = 0;
    if (!over) {
        for (int k0 = 0; k0 < maxlen; k0 += 8 * kBatch) {
            uint2 e[2 * kBatch];
            load_pairs(k0, e);
            unsigned mine = 0, outr = 0;
#pragma unroll
            for (int t = 0; t < 2 * kBatch; ++t) {
                const int d = static_cast<int>(e[t].y);
                if (d >= 0 && e[t].x < thi) ++mine;
                if (d >= 0 && e[t].x >= thi) {
                    ++outr;
                    if (one_chunk) mark(d, 0);
                }
            }
            unsigned pos = nc + wave_prefix_excl(mine);
#pragma unroll
            for (int t = 0; t < 2 * kBatch; ++t) {
                const int d = static_cast<int>(e[t].y);
                if (d >= 0 && e[t].x < thi) {
                    if (pos < static_cast<unsigned>(kCapB)) {
                        sKey[w][pos] = e[t].x;
                        sBlk[w][pos] = d;
                    }
                    ++pos;
                }
            }
            nc += wave_sum_u(mine);
            nd += wave_sum_u(outr);
        }
    }
    const int need = KB - static_cast<int>(nd);
    if (over || need < 1 || need > static_cast<int>(nc) || nc > static_cast<unsigned>(kCapB)) {
        if (lane == 0) queue[atomicAdd(qcount, 1)] = static_cast<int>(row);   // overflow, or the band missed
        return;
    }
    wave_sync();
    const int ns = (static_cast<int>(nc) + 63) / 64;
    unsigned key[kSlots];
    int bi[kSlots];
    unsigned kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int t = 0; t < kSlots; ++t) {
        const int j = 64 * t + lane;
        const bool real = t < ns && j < static_cast<int>(nc);
        key[t] = real ? sKey[w][j] : 0u;
        bi[t] = real ? sBlk[w][j] : -1;
        if (real) {
            kmn = min(kmn, key[t]);
            kmx = max(kmx, key[t]);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        kmn = min(kmn, static_cast<unsigned>(__shfl_xor(static_cast<int>(kmn), off)));
        kmx = max(kmx, static_cast<unsigned>(__shfl_xor(static_cast<int>(kmx), off)));
    }
    auto count_if = [&](auto pred) {
        unsigned c = 0;
#pragma unroll
        for (int t = 0; t < kSlots; ++t)
            if (t < ns) c += static_cast<unsigned>(__popcll(__ballot(bi[t] >= 0 && pred(key[t], bi[t]))));
        return c;
    };
    // the need-th largest key T, count(key > T) < need <= count(key >= T), by
    // radix selection on key - base: a 1024-bin histogram of the keys still in
    // [base, base + rng] (in this wave's sKey row, free now that the
    // candidates are in registers), then the bin that holds the rank-th
    // largest becomes the range; a range of at most 1024 values is decided
    // exactly.  Three rounds cover the usual band of about 2^21 patterns.
    static_assert(kCapB == 1024, "the histogram takes one sKey row");
    unsigned* hist = sKey[w];
    unsigned base = kmn, rng = kmx - kmn;
    unsigned rank = static_cast<unsigned>(need);     // from the top, inside the range
    for (;;) {
        const int bits = rng ? 32 - __clz(static_cast<int>(rng)) : 0;
        const int shift = bits > 10 ? bits - 10 : 0;
        wave_sync();
#pragma unroll
        for (int j = 0; j < 4; ++j) reinterpret_cast<uint4*>(hist)[lane * 4 + j] = make_uint4(0u, 0u, 0u, 0u);
        wave_sync();
#pragma unroll
        for (int t = 0; t < kSlots; ++t) {
            const unsigned d = key[t] - base;        // keys below base wrap past rng
            if (t < ns && bi[t] >= 0 && d <= rng) atomicAdd(&hist[d >> shift], 1u);
        }
        wave_sync();
        unsigned above;
        const unsigned bin = wave_threshold(hist, kCapB / 64, rank, &above);
        rank -= above;
        base += bin << shift;
        if (shift == 0) break;
        rng = min(rng - (bin << shift), (1u << shift) - 1u);
    }
    const unsigned T = base;
    const unsigned take_eq = static_cast<unsigned>(need) - count_if([&](unsigned k, int) { return k > T; });
    // among the keys equal to T, the take_eq latest blocks: largest X with count(idx >= X) >= take_eq
    // (X = 0 when every one of them is taken, the usual case)
    const unsigned eq = count_if([&](unsigned k, int) { return k == T; });
    int xlo = 0, xhi = eq == take_eq ? 1 : m;
    while (xhi - xlo > 1) {
        const int mid = (xlo + xhi) >> 1;
        if (count_if([&](unsigned k, int j) { return k == T && j >= mid; }) >= take_eq) xlo = mid;
        else xhi = mid;
    }
    const int X = xlo;
    // ascending union, one bitmap chunk at a time (one chunk: marked in pass A);
    // with K_B <= kCapB the output is staged in sBlk (the candidates are in
    // registers by now) and copied out in order
    const bool staged = KB <= kCapB;
    int* sOut = sBlk[w];
    wave_sync();
    unsigned written = 0;
    for (int c0 = 0; c0 < m; c0 += 64 * kMapWords) {
        const int c1 = min(m, c0 + 64 * kMapWords);
        const int nw = (c1 - c0 + 63) / 64;
        if (!one_chunk) {
            for (int j = lane; j < nw; j += 64) sMap[w][j] = 0ull;
            wave_sync();
            for_entries([&](unsigned u, int d) {
                if (d >= 0 && u >= thi && d >= c0 && d < c1) mark(d, c0);
            });
        }
#pragma unroll
        for (int t = 0; t < kSlots; ++t) {
            const int d = bi[t];
            if (t < ns && d >= c0 && d < c1 && (key[t] > T || (key[t] == T && d >= X))) mark(d, c0);
        }
        wave_sync();
        for (int w0 = 0; w0 < nw; w0 += 64) {
            const int wi = w0 + lane;
            unsigned long long word = wi < nw ? sMap[w][wi] : 0ull;
            const unsigned cw = static_cast<unsigned>(__popcll(word));
            unsigned pos = written + wave_prefix_excl(cw);
            while (word) {
                const int bit = __ffsll(static_cast<long long>(word)) - 1;
                if (pos < static_cast<unsigned>(KB)) {
                    if (staged) sOut[pos] = c0 + 64 * wi + bit;
                    else out[pos] = c0 + 64 * wi + bit;
                }
                ++pos;
                word &= word - 1ull;
            }
            written += wave_sum_u(cw);
        }
        wave_sync();
    }
    if (staged)
        for (int j = lane; j < KB; j += 64) out[j] = sOut[j];
}

// ---------------------------------------------------------------------------
// exact pass: grid (kExactWGs), 16 waves; workgroup x takes the queued
// queries x, x + kExactWGs, ...  The waves score the row 16 blocks at a time
// with the MFMA step of the scoring passes (the query's heads as A rows 0..3;
// eight groups' key loads in flight) into LDS (rows up to kExactLds blocks)
// or the workgroup's scratch row (ld floats), then the workgroup selects on
// it exactly (select_row_wg).
// ---------------------------------------------------------------------------
constexpr int kExactWGs = 256;

// Workgroup-cooperative form of select_row (the same rules and result) for
// the exact pass: the NW waves share the value histogram and the gathering of
// the threshold bin, wave 0 ranks that bin (or runs the radix select), and the
// ordered compaction runs per contiguous wave segment of the row, a count pass
// and then the writes at the segment's offset.  sw holds NW + 8 words.
template <int NW>
__device__ void select_row_wg(const float* row, int m, int KB, float mx, int* out, unsigned* hist, unsigned* sck,
                              int* sci, unsigned* sw) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int m4 = (m + 3) / 4;
    const int seg = ((m4 + NW - 1) / NW + 63) / 64 * 64;   // float4 groups per wave, whole steps
    const int g_lo = min(m4, w * seg), g_hi = min(m4, g_lo + seg);
    auto for_seg = [&](auto f) {                           // f(v, x, ok) on whole-wave steps
        for (int v0 = g_lo; v0 < g_hi; v0 += 64) {
            const int v = v0 + lane;
            const float4v x = reinterpret_cast<const float4v*>(row)[min(v, m4 - 1)];
            f(v, x, v < g_hi);
        }
    };
    for (int j = threadIdx.x; j < kBins; j += 64 * NW) hist[j] = 0;
    if (threadIdx.x < 8) sw[NW + threadIdx.x] = 0;
    __syncthreads();
    bool fast = mx > 0.f;
    if (fast) {
        const float scale = static_cast<float>(kBins) / mx;
        auto bin_of = [&](float v) {
            return v == 0.f ? 0u : static_cast<unsigned>(min(kBins - 1, static_cast<int>(v * scale)));
        };
        unsigned zeros = 0;
        for_seg([&](int v, const float4v& x, bool ok) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (!ok || 4 * v + e >= m) continue;
                if (x[e] == 0.f) ++zeros;
                else atomicAdd(&hist[bin_of(x[e])], 1u);
            }
        });
        zeros = wave_sum_u(zeros);
        if (lane == 0 && zeros) atomicAdd(&hist[0], zeros);
        __syncthreads();
        if (w == 0) {
            unsigned above;
            const unsigned beta = wave_threshold(hist, kBins / 64, KB, &above);
            if (lane == 0) {
                sw[NW] = beta;
                sw[NW + 1] = above;
                sw[NW + 2] = hist[beta];
            }
        }
        __syncthreads();
        const unsigned beta = sw[NW], above = sw[NW + 1], cb = sw[NW + 2];
        fast = cb <= 64;
        if (fast) {
            // gather the threshold bin's entries (any order: they are ranked next)
            for_seg([&](int v, const float4v& x, bool ok) {
                unsigned inm = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (ok && 4 * v + e < m && bin_of(x[e]) == beta) inm |= 1u << e;
                const unsigned cnt = __popc(inm);
                const unsigned tot = wave_sum_u(cnt);
                if (tot == 0) return;
                unsigned base = 0;
                if (lane == 0) base = atomicAdd(&sw[NW + 3], tot);
                unsigned slot = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(base))) +
                                wave_prefix_excl(cnt);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (inm & (1u << e)) {
                        sck[slot] = order_key(x[e]);
                        sci[slot] = 4 * v + e;
                        ++slot;
                    }
            });
            __syncthreads();
            if (w == 0) {
                const unsigned need = KB - above;    // taken from this bin, 1 .. cb
                unsigned k0 = 0;
                int i0 = 0;
                bool hit = false;
                if (lane < static_cast<int>(cb)) {
                    k0 = sck[lane];
                    i0 = sci[lane];
                    unsigned rank = 0;
                    for (unsigned c = 0; c < cb; ++c) {
                        const unsigned k1 = sck[c];
                        rank += k1 > k0 || (k1 == k0 && sci[c] > i0);
                    }
                    hit = rank == need - 1;
                }
                const int src = __ffsll(static_cast<long long>(__ballot(hit))) - 1;
                const unsigned ck = __shfl(k0, src);
                const int ci = __shfl(i0, src);
                if (lane == 0) {
                    sw[NW + 4] = ck;
                    sw[NW + 5] = static_cast<unsigned>(ci);
                }
            }
        }
    }
    if (!fast && w == 0) {
        unsigned ck;
        int ci;
        radix_cut_wave(row, m, KB, hist, ck, ci);
        if (lane == 0) {
            sw[NW + 4] = ck;
            sw[NW + 5] = static_cast<unsigned>(ci);
        }
    }
    __syncthreads();
    const unsigned ckey = sw[NW + 4];
    const int cidx = static_cast<int>(sw[NW + 5]);
    // ordered compaction of the entries with (key, j) >= (ckey, cidx)
    auto sel = [&](int v, const float4v& x, bool ok) {
        unsigned sm = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * v + e;
            const unsigned u = order_key(x[e]);
            if (ok && j < m && (u > ckey || (u == ckey && j >= cidx))) sm |= 1u << e;
        }
        return sm;
    };
    unsigned mine = 0;
    for_seg([&](int v, const float4v& x, bool ok) { mine += __popc(sel(v, x, ok)); });
    mine = wave_sum_u(mine);
    if (lane == 0) sw[w] = mine;
    __syncthreads();
    unsigned base = 0;
    for (int i = 0; i < w; ++i) base += sw[i];
    for_seg([&](int v, const float4v& x, bool ok) {
        const unsigned sm = sel(v, x, ok);
        const unsigned cnt = __popc(sm);
        unsigned pos = base + wave_prefix_excl(cnt);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (sm & (1u << e)) out[pos++] = 4 * v + e;
        base += wave_sum_u(cnt);
    });
}
constexpr int kExactWaves = 16;      // waves per workgroup of the exact pass
constexpr int kExactLds = 24576;     // rows up to this many blocks are scored into LDS

template <int D, bool kBf16>
__global__ __launch_bounds__(1024) void qsa_exact_kernel(const void* __restrict__ q, const void* __restrict__ kbar,
                                                        const int* __restrict__ queue,
                                                        const int* __restrict__ qcount, float* __restrict__ scratch,
                                                        long ld, int* __restrict__ idx, int n, int r, int nb, int KB) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
    const int total = *qcount;
    __shared__ unsigned shist[kBins];
    __shared__ unsigned sck[64];
    __shared__ int sci[64];
    __shared__ float smax[kExactWaves];
    __shared__ unsigned sw[kExactWaves + 8];
    __shared__ __align__(16) float srow[kExactLds];
    for (int t = blockIdx.x; t < total; t += kExactWGs) {
        const long row = queue[t];
        const int b = static_cast<int>(row / n), i = static_cast<int>(row % n);
        const int m = (i + 1) / r;
        float* sr = m <= kExactLds ? srow : scratch + static_cast<long>(blockIdx.x) * ld;
        QFrag<D, kBf16, 1> f;
        float sqd[1];
        load_qfrag<D, kBf16, 1>(f, q, b, n, i, 0, lane, sqd);   // A rows 0..3: (i, head 0..3)
        float mx = 0.f;
        constexpr int kG = kBf16 ? 4 : 2;            // 16-block groups per batch
        for (int g0 = 16 * kG * w; g0 < m; g0 += 16 * kG * kExactWaves) {
            float4v acc[kG];
#pragma unroll
            for (int u = 0; u < kG; ++u) acc[u] = float4v{0.f, 0.f, 0.f, 0.f};
            if constexpr (kBf16) {
                bf16x8 bv[kG][D / 32];
#pragma unroll
                for (int u = 0; u < kG; ++u) {
                    const int blk = min(g0 + 16 * u + (lane & 15), m - 1);
                    const __bf16* Bt = static_cast<const __bf16*>(kbar) + (static_cast<long>(b) * nb + blk) * D + 8 * g;
#pragma unroll
                    for (int kk = 0; kk < D / 32; ++kk) bv[u][kk] = *reinterpret_cast<const bf16x8*>(Bt + 32 * kk);
                }
                // all loads in flight before the first use (the scheduler would otherwise
                // reuse one register set and wait on every load)
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < kG; ++u)
#pragma unroll
                    for (int kk = 0; kk < D / 32; ++kk)
                        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[0][kk], bv[u][kk], acc[u], 0, 0, 0);
            } else {
#pragma unroll
                for (int u = 0; u < kG; ++u) {
                    const int blk = min(g0 + 16 * u + (lane & 15), m - 1);
                    const float* Bt = static_cast<const float*>(kbar) + (static_cast<long>(b) * nb + blk) * D + g * (D / 4);
#pragma unroll 8
                    for (int k = 0; k < D / 4; ++k)
                        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[0][k], Bt[k], acc[u], 0, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < kG; ++u) {
                const int blk = g0 + 16 * u + (lane & 15);
                if (g == 0 && blk < m) {
                    const float sc = relu_sum(acc[u]);
                    sr[blk] = sc;
                    mx = fmaxf(mx, sc);
                }
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if (lane == 0) smax[w] = mx;
        // the row is read back by wave 0; the barrier's workgroup-scope ordering
        // covers the scratch row too (all waves of a workgroup share one CU)
        __syncthreads();
        float rmx = 0.f;
#pragma unroll
        for (int j = 0; j < kExactWaves; ++j) rmx = fmaxf(rmx, smax[j]);
        select_row_wg<kExactWaves>(sr, m, KB, rmx, idx + row * KB, shist, sck, sci, sw);
        __syncthreads();
    }
}

// Sub-list capacity (per query and lane): K_B / 16 + kCapB / 16 or fewer
// entries on average, with room to spare.
static int sub_cap(int KB) { return ((KB + 15) / 16 + kCapB / 16 + 32 + 1) & ~1; }

// Workspace carving (each piece 256-byte aligned).
struct TopkLayout {
    size_t kmax, qcount, info, cnt, queue, list, scratch, total;
};
static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
static TopkLayout topk_layout(int B, int n, int r, int KB) {
    const size_t rows = static_cast<size_t>(B) * n;
    const size_t nb = static_cast<size_t>(n / r);
    const size_t nbw = (nb + 63) / 64;
    const size_t ld = nbw > 0 ? nbw * 64 : 64;
    TopkLayout t;
    size_t o = 0;
    t.kmax = o;    o += align256(4 * static_cast<size_t>(B));
    t.qcount = o;  o += 256;
    t.info = o;    o += align256(rows * sizeof(uint2));
    t.cnt = o;     o += align256(rows * 16 * 4);
    t.queue = o;   o += align256(rows * 4);
    t.list = o;    o += align256(rows * 16 * static_cast<size_t>(sub_cap(KB)) * sizeof(uint2));
    t.scratch = o; o += align256(static_cast<size_t>(kExactWGs) * ld * 4);
    t.total = o;
    return t;
}

}  // namespace qsa

size_t qsa_select4_workspace_bytes(int B, int n, int r, int KB) { return qsa::topk_layout(B, n, r, KB).total; }

template <int D, bool kBf16>
static hipError_t launch_select4_t(const QsaSelectArgs& a) {
    using namespace qsa;
    const int nb = a.n / a.r;
    const int nbw = (nb + 63) / 64;
    const TopkLayout t = topk_layout(a.B, a.n, a.r, a.KB);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    float* kmax = reinterpret_cast<float*>(ws + t.kmax);
    int* qcount = reinterpret_cast<int*>(ws + t.qcount);
    uint2* info = reinterpret_cast<uint2*>(ws + t.info);
    int* cnt = reinterpret_cast<int*>(ws + t.cnt);
    const int cap = sub_cap(a.KB);
    int* queue = reinterpret_cast<int*>(ws + t.queue);
    uint2* list = reinterpret_cast<uint2*>(ws + t.list);
    float* scratch = reinterpret_cast<float*>(ws + t.scratch);
    const long ld = nbw > 0 ? static_cast<long>(nbw) * 64 : 64;
    const dim3 gh((a.n + 31) / 32, a.B), ge((a.n + 63) / 64, a.B), gq((a.n + 3) / 4, a.B);
    hipLaunchKernelGGL(qsa_zero_kernel, dim3(1), dim3(256), 0, a.stream, kmax, a.B, qcount);
    if (nb > a.KB) {                                 // otherwise every query keeps all its blocks
        hipLaunchKernelGGL((qsa_kmax_kernel<D, kBf16>), dim3((nb + 255) / 256, a.B), dim3(256), 0, a.stream, a.kbar,
                           kmax, nb);
        hipLaunchKernelGGL((qsa_pass4_kernel<D, kBf16, false>), gh, dim3(256), 0, a.stream, a.q, a.kbar, kmax, info,
                           cnt, list, a.n, a.r, nb, a.KB, cap);
        hipLaunchKernelGGL((qsa_pass4_kernel<D, kBf16, true>), ge, dim3(256), 0, a.stream, a.q, a.kbar, kmax, info,
                           cnt, list, a.n, a.r, nb, a.KB, cap);
    }
    hipLaunchKernelGGL(qsa_merge_kernel, gq, dim3(256), 0, a.stream, info, cnt, list, a.idx, queue, qcount, a.n,
                       a.r, a.KB, cap);
    if (nb > a.KB)
        hipLaunchKernelGGL((qsa_exact_kernel<D, kBf16>), dim3(kExactWGs), dim3(64 * kExactWaves), 0, a.stream, a.q,
                           a.kbar,
                           queue, qcount, scratch, ld, a.idx, a.n, a.r, nb, a.KB);
    return hipGetLastError();
}

template <bool kBf16>
static hipError_t launch_select4_dt(const QsaSelectArgs& a) {
    switch (a.D) {
        case 32: return launch_select4_t<32, kBf16>(a);
        case 64: return launch_select4_t<64, kBf16>(a);
        case 128: return launch_select4_t<128, kBf16>(a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_qsa_select4(const QsaSelectArgs& a) {
    return a.bf16 ? launch_select4_dt<true>(a) : launch_select4_dt<false>(a);
}

}  // namespace gdn
