// kda_layer.hip -- the KDA layer's output epilogue over the prefill output.
//
// The KDA-layer item of the model-architecture list on the page "Kimi Linear
// 高效注意力架构" ends the layer with a sigmoid output gate and RMSNorm.  Per
// (token, head) row of Dv = 128 values:
//
//     out = o / sqrt(mean_j o_j^2 + eps) * w * sigmoid(g)
//
// with w [Dv] fp32 shared by all heads and g [.., Dv] bf16 (the output-gate
// projection).  The prefill's state pass produces each row in eight 16-column
// slabs from eight workgroups, so the norm of a row is only known once all of
// them are done; this streaming pass applies it in place afterwards (one read
// of o and g, one write of o).  Half a wave owns a row: lane l % 32 holds
// columns 4 (l % 32) .. 4 (l % 32) + 3, loaded as one 16-byte vector.
#include "kda_prefill.h"

namespace kda {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kEpiThreads = 256;
constexpr int kEpiDv = 128;

__global__ void __launch_bounds__(kEpiThreads)
layer_epilogue_kernel(float *__restrict__ o, const uint16_t *__restrict__ g, const float *__restrict__ w,
                      int64_t rows, float eps) {
    const int lane = threadIdx.x % kWave, c4 = lane % 32;
    const f32x4 wv = reinterpret_cast<const f32x4 *>(w)[c4];
    const int64_t half = (static_cast<int64_t>(blockIdx.x) * kEpiThreads + threadIdx.x) / 32;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kEpiThreads / 32;
    // every lane runs the same number of iterations (rows are taken in pairs by
    // whole waves), so the shuffles below always see their partners
    const int64_t wave_rows = (rows + 1) / 2 * 2;
    for (int64_t row0 = half - half % 2; row0 < wave_rows; row0 += stride) {
        const int64_t row = row0 + half % 2;
        const bool ok = row < rows;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        u32x2 gb = {0u, 0u};
        if (ok) {
            x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(o + row * kEpiDv) + c4);
            gb = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(g + row * kEpiDv) + c4);
        }
        float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) ss += __shfl_xor(ss, off);
        const float sc = 1.f / sqrtf(ss * (1.f / kEpiDv) + eps);
        const float gv[4] = {__uint_as_float(gb.x << 16), __uint_as_float(gb.x & 0xffff0000u),
                             __uint_as_float(gb.y << 16), __uint_as_float(gb.y & 0xffff0000u)};
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = x[e] * sc * wv[e] * sigmoid_f(gv[e]);
        if (ok) __builtin_nontemporal_store(y, reinterpret_cast<f32x4 *>(o + row * kEpiDv) + c4);
    }
}

}  // namespace

hipError_t launch_layer_epilogue(float *o, const uint16_t *g, const float *w, int64_t rows, float eps,
                                 hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    // 8 rows per workgroup per pass; a grid of a few waves per SIMD streams the rest
    const int64_t want = (rows + 7) / 8;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
    const unsigned grid = static_cast<unsigned>(want < cap ? want : cap);
    hipLaunchKernelGGL(layer_epilogue_kernel, dim3(grid), dim3(kEpiThreads), 0, stream, o, g, w, rows, eps);
    return hipGetLastError();
}

}  // namespace kda
