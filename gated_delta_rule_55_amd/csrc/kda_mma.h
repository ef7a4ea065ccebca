// kda_mma.h -- 16x16 matrix-core tile products for gfx950 with a chosen
// operand precision.
//
// Fragment convention (one wave, one 16x16 output tile, a K step of 32):
//   lane l supplies row (l % 16) of A and column (l % 16) of B, and the 8
//   values a[e], b[e] (e = 0..7) at k = 8 (l / 16) + e of the step.
//   The accumulator holds C[4 (l / 16) + r][l % 16], r = 0..3.
// The 16x16x32 f16/bf16 instructions take the 8 values packed; the fp32
// instruction 16x16x4 takes one value per lane and is issued 8 times, step e
// pairing a[e] with b[e] -- a permutation of k that both operands share, so
// the sum over the 32 values of k is the same.
#pragma once

#include "kda_common.h"

namespace kda {

enum class Prec {
    F32,     // fp32 operands (matrix-core fp32)
    F16,     // both operands rounded to fp16
    F16X3,   // both split into fp16 hi + lo: hi*hi + hi*lo + lo*hi
    BF16X3,  // both split into bf16 hi + lo (fp32 exponent range)
    BF16X2A  // A split into bf16 hi + lo, B exact in bf16: hi*B + lo*B
};

__device__ __forceinline__ f16x8 pack_f16(const float (&x)[8]) {
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = static_cast<_Float16>(x[e]);
    return r;
}

__device__ __forceinline__ bf16x8 pack_bf16(const float (&x)[8]) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(x[e]);
    return r;
}

// hi = round(x), lo = round(x - hi)
__device__ __forceinline__ void split_f16(const float (&x)[8], f16x8 &hi, f16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const _Float16 h = static_cast<_Float16>(x[e]);
        hi[e] = h;
        lo[e] = static_cast<_Float16>(x[e] - static_cast<float>(h));
    }
}

__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = static_cast<__bf16>(x[e]);
        hi[e] = h;
        lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
    }
}

__device__ __forceinline__ f32x4 mfma_f16(const f16x8 &a, const f16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += A_step * B_step for one K step of 32 (see the fragment convention).
template <Prec P>
__device__ __forceinline__ void mma(f32x4 &acc, const float (&a)[8], const float (&b)[8]) {
    if constexpr (P == Prec::F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
    } else if constexpr (P == Prec::F16) {
        acc = mfma_f16(pack_f16(a), pack_f16(b), acc);
    } else if constexpr (P == Prec::F16X3) {
        f16x8 ah, al, bh, bl;
        split_f16(a, ah, al);
        split_f16(b, bh, bl);
        acc = mfma_f16(al, bh, acc);
        acc = mfma_f16(ah, bl, acc);
        acc = mfma_f16(ah, bh, acc);
    } else if constexpr (P == Prec::BF16X3) {
        bf16x8 ah, al, bh, bl;
        split_bf16(a, ah, al);
        split_bf16(b, bh, bl);
        acc = mfma_bf16(al, bh, acc);
        acc = mfma_bf16(ah, bl, acc);
        acc = mfma_bf16(ah, bh, acc);
    } else {  // BF16X2A
        bf16x8 ah, al;
        split_bf16(a, ah, al);
        const bf16x8 bb = pack_bf16(b);
        acc = mfma_bf16(al, bb, acc);
        acc = mfma_bf16(ah, bb, acc);
    }
}

}  // namespace kda
