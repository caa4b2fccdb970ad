// Wave-level building blocks of the QSA block selection (gfx950): one wave
// owns one query row of scores, so no workgroup barriers are needed.  The
// selection picks the K_B largest scores of a row, ties going to the later
// block (slinene ai-papers-daily page on Qwen3.8-Next, Module B: top-K_B block
// selection), and writes the chosen block indices in ascending order.
#pragma once

#include "gdn_device.hpp"

namespace gdn {
namespace qsa {

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
// Wave-wide sums and scans with DPP lane moves (no LDS round trips): shifts
// by 1, 2, 4 and 8 lanes within each row of 16 (zeros shifted in), then the
// last lane of rows 0 and 2 added into rows 1 and 3, then lane 31 into rows 2
// and 3.
template <int kCtrl, int kRowMask, bool kZeroFill>
__device__ __forceinline__ unsigned dpp_u(unsigned v) {
    return static_cast<unsigned>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, kRowMask, 0xf, kZeroFill));
}
__device__ __forceinline__ unsigned wave_scan_incl_u(unsigned x) {      // sum over lanes <= this lane
    x += dpp_u<0x111, 0xf, true>(x);    // row_shr:1
    x += dpp_u<0x112, 0xf, true>(x);    // row_shr:2
    x += dpp_u<0x114, 0xf, true>(x);    // row_shr:4
    x += dpp_u<0x118, 0xf, true>(x);    // row_shr:8
    x += dpp_u<0x142, 0xa, false>(x);   // row_bcast:15
    x += dpp_u<0x143, 0xc, false>(x);   // row_bcast:31
    return x;
}
__device__ __forceinline__ unsigned wave_sum_u(unsigned x) {
    return static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(wave_scan_incl_u(x)), 63));
}
__device__ __forceinline__ unsigned wave_prefix_excl(unsigned v) {     // sum over lanes < this lane
    return wave_scan_incl_u(v) - v;
}
__device__ __forceinline__ unsigned wave_suffix_incl(unsigned x) {     // sum over lanes >= this lane
    const unsigned incl = wave_scan_incl_u(x);
    return static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63)) - incl + x;
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

// Exact selection on one materialised row of m >= K_B + 1 non-negative scores
// (sums of ReLUs): a value-range histogram (2048 equal bins over [0, row
// max]; zeros, which all share bin 0, are counted per lane rather than with
// atomics) finds the bin holding the K_B-th largest score; its candidates (a
// handful for continuous scores) are ranked against each other by (score,
// index) to find the cut; more than 64 of them fall back to the exact radix
// select.  The selected blocks then go out in ascending order to out[0, K_B).
// mx is the row maximum, or negative when unknown.  hist holds kBins words,
// sck and sci 64 entries each, all private to the calling wave.
__device__ __forceinline__ void select_row(const float* row, int m, int KB, float mx, int* out, unsigned* hist,
                                           unsigned* sck, int* sci) {
    const int lane = threadIdx.x & 63;
    if (mx < 0.f) {                                  // not known: one pass for it
        mx = 0.f;
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
                        sck[slot] = order_key(x[e]);
                        sci[slot] = 4 * v + e;
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
}  // namespace gdn
