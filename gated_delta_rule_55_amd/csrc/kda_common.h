// kda_common.h -- small device helpers shared by the KDA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Raw bfloat16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Input element loader: bf16 (raw bits) or fp32.
template <bool kBf16>
__device__ __forceinline__ float load_in(const void *p, int64_t i) {
    if constexpr (kBf16) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    } else {
        return static_cast<const float *>(p)[i];
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// -softplus(x) = -(max(x, 0) + log(1 + e^-|x|)), natural log; +inf -> -inf, -inf -> 0
__device__ __forceinline__ float neg_softplus(float x) {
    return -(fmaxf(x, 0.f) + kLn2 * __log2f(1.f + fast_exp2(-fabsf(x) * kLog2e)));
}

// 1 / (1 + e^-x); -inf -> 0, +inf -> 1
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + fast_exp2(-x * kLog2e)); }

}  // namespace kda
