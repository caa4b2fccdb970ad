// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, wave64 reductions and MFMA tile steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bfloat16 <-> float32 (round to nearest even on the way down).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// (gfx950 converts with v_cvt_pk_bf16_f32, two values per instruction)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(lo), static_cast<__bf16>(hi)});
}

// Load element i of an input that is either float32 or bfloat16.
template <bool kBf16>
__device__ __forceinline__ float load_in(const void* p, long i) {
    if constexpr (kBf16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// ---------------------------------------------------------------------------
// MFMA tile steps.  A 16x16 output tile C is accumulated as C += A * B where
// A (16 x K) is read row-major from LDS with leading dimension lda, and B
// (K x 16) is read from its transpose Bt (16 x K, row-major, ldb), so both
// operands are read as short contiguous runs along K.  Accumulator layout
// (all 16x16 MFMAs on CDNA): lane l holds C[4*(l/16) + j][l % 16], j = 0..3.
// Within one instruction, lane l supplies A row l%16 and B column l%16 for the
// K-slice selected by l/16; both operands use the same slice numbering, so the
// contraction is exact whatever order the hardware sums the slices in.
// ---------------------------------------------------------------------------
template <class T> struct Mma;

template <> struct Mma<_Float16> {
    static constexpr int kStep = 32;
    __device__ __forceinline__ static float4v step32(const _Float16* A, int lda, const _Float16* Bt,
                                                     int ldb, int k0, float4v acc) {
        const int l = threadIdx.x & 63;
        const half8 a = *reinterpret_cast<const half8*>(A + (l & 15) * lda + k0 + 8 * (l >> 4));
        const half8 b = *reinterpret_cast<const half8*>(Bt + (l & 15) * ldb + k0 + 8 * (l >> 4));
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
    // acc += A[:, k0:k0+16] * B[k0:k0+16, :] issued as a 16x16x32 step whose
    // upper K half is zero (the lanes holding it load nothing).
    __device__ __forceinline__ static float4v step32_lo(const _Float16* A, int lda, const _Float16* Bt,
                                                        int ldb, int k0, float4v acc) {
        const int l = threadIdx.x & 63;
        half8 a = {}, b = {};
        if ((l >> 4) < 2) {
            a = *reinterpret_cast<const half8*>(A + (l & 15) * lda + k0 + 8 * (l >> 4));
            b = *reinterpret_cast<const half8*>(Bt + (l & 15) * ldb + k0 + 8 * (l >> 4));
        }
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
    // acc += A[:, k0:k1] * B[k0:k1, :], k0 and k1 multiples of 16.  Every step
    // of one accumulation chain uses the same MFMA shape: a 16x16x16 step fed
    // the accumulator of a 16x16x32 step just before it has produced wrong
    // sums on gfx950, so a 16-wide remainder becomes a half-zero 32-wide step.
    __device__ __forceinline__ static float4v range(const _Float16* A, int lda, const _Float16* Bt,
                                                    int ldb, int k0, int k1, float4v acc) {
        int k = k0;
        for (; k + 32 <= k1; k += 32) acc = step32(A, lda, Bt, ldb, k, acc);
        if (k < k1) acc = step32_lo(A, lda, Bt, ldb, k, acc);
        return acc;
    }
};

template <> struct Mma<float> {
    static constexpr int kStep = 4;
    __device__ __forceinline__ static float4v step4(const float* A, int lda, const float* Bt, int ldb,
                                                    int k0, float4v acc) {
        const int l = threadIdx.x & 63;
        const float a = A[(l & 15) * lda + k0 + (l >> 4)];
        const float b = Bt[(l & 15) * ldb + k0 + (l >> 4)];
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    // acc += A[:, k0:k1] * B[k0:k1, :], k0 and k1 multiples of 4.
    __device__ __forceinline__ static float4v range(const float* A, int lda, const float* Bt, int ldb,
                                                    int k0, int k1, float4v acc) {
        for (int k = k0; k < k1; k += 4) acc = step4(A, lda, Bt, ldb, k, acc);
        return acc;
    }
};

}  // namespace gdn
