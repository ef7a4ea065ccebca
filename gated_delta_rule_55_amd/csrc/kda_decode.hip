// kda_decode.hip -- one recurrent step of KDA for N x H independent states.
//
// Per (sequence n, head h) the state S [Dk x Dv] fp32 is streamed from HBM
// once, decayed, reduced twice over d_k, updated with the rank-1 delta write
// and streamed back once (state-update equation of the section "Kimi Delta
// Attention (KDA)" on the page "Kimi Linear 高效注意力架构", with the fixed
// per-head state of its linear-complexity bullet):
//
//   S'  = Diag(exp(log_alpha)) S                  decay rows (key channels)
//   p   = S'^T k,  r = S'^T q                     two column reductions
//   u   = beta (v - p)
//   S   = S' + k u^T                              == (I - b k k^T) S' + b k v^T
//   o   = S^T q = r + (k . q) u
//
// The Gated DeltaNet step (one scalar gate per head, the recurrence the same
// page compares KDA against) is the same kernel with that gate read once per
// (n, h) and applied to every row.
//
// One workgroup of min(512, Dk*Dv/4) threads per (n, h).  Thread t owns 4 adjacent columns
// (one float4) of RPT rows spaced RG apart, so each wave reads and writes whole
// contiguous rows (coalesced 16-byte accesses).  Reductions: butterfly
// shuffles inside a wave over the lanes that share a column group, then LDS
// across waves.  All arithmetic is fp32.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

constexpr int kDecodeThreads = 512;

// SG: one scalar gate per (n, h) (log_alpha [N, H]) instead of one per key
// channel (log_alpha [N, H, Dk]).
template <int DK, int DV, bool kBf16, bool SG>
__global__ void __launch_bounds__(kDecodeThreads)
decode_step_kernel(const void *__restrict__ q, const void *__restrict__ k,
                   const void *__restrict__ v, const float *__restrict__ log_alpha,
                   const float *__restrict__ beta, float *__restrict__ state,
                   float *__restrict__ o) {
    constexpr int CG = DV / 4;                                  // float4 column groups
    constexpr int NT = (DK * DV / 4 < kDecodeThreads) ? DK * DV / 4 : kDecodeThreads;  // threads
    constexpr int RG = NT / CG;                                 // row groups
    constexpr int RPT = DK / RG;                                // rows per thread
    constexpr int NW = (NT + kWave - 1) / kWave;                // waves holding rows
    static_assert(CG <= kWave && kWave % CG == 0, "column groups must tile a wave");
    static_assert(RG * RPT == DK, "rows must tile the state");

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ f32x4 s_red[NW][CG][2];
    __shared__ float s_kq[NW][CG];

    const int t = threadIdx.x;
    const int64_t unit = blockIdx.x;  // n * H + h
    const int cg = t % CG;
    const int rg = t / CG;
    f32x4 *S = reinterpret_cast<f32x4 *>(state + unit * DK * DV);

    // the state stream is issued first; the token's vectors load under it
    f32x4 sv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) sv[i] = __builtin_nontemporal_load(&S[(rg + i * RG) * CG + cg]);
    const float b = beta[unit];
    f32x4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = load_in<kBf16>(v, unit * DV + 4 * cg + e);
    for (int c = t; c < DK; c += blockDim.x) {
        s_k[c] = load_in<kBf16>(k, unit * DK + c);
        s_q[c] = load_in<kBf16>(q, unit * DK + c);
        const float g = SG ? log_alpha[unit] : log_alpha[unit * DK + c];
        s_a[c] = fast_exp2(g * kLog2e);  // exp(-inf) -> 0
    }
    __syncthreads();

    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + i * RG;
        const float a = s_a[row], kr = s_k[row], qr = s_q[row];
        sv[i] *= a;
        p += sv[i] * kr;
        r += sv[i] * qr;
        kq += kr * qr;
    }
    // reduce over the lanes of this wave that share column group cg
#pragma unroll
    for (int off = CG; off < kWave; off <<= 1) {
        if (off >= NT) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] += __shfl_xor(p[e], off);
            r[e] += __shfl_xor(r[e], off);
        }
        kq += __shfl_xor(kq, off);
    }
    const int w = t / kWave, lane = t % kWave;
    if (lane < CG) {
        s_red[w][lane][0] = p;
        s_red[w][lane][1] = r;
        s_kq[w][lane] = kq;
    }
    __syncthreads();
    p = s_red[0][cg][0];
    r = s_red[0][cg][1];
    kq = s_kq[0][cg];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) {
        p += s_red[ww][cg][0];
        r += s_red[ww][cg][1];
        kq += s_kq[ww][cg];
    }
    const f32x4 u = b * (vv - p);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + i * RG;
        __builtin_nontemporal_store(sv[i] + s_k[row] * u, &S[row * CG + cg]);
    }
    if (rg == 0) reinterpret_cast<f32x4 *>(o + unit * DV)[cg] = r + kq * u;
}

template <int DK, int DV, bool kBf16>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    constexpr int NT = (DK * DV / 4 < kDecodeThreads) ? DK * DV / 4 : kDecodeThreads;
    const dim3 grid(static_cast<unsigned>(a.N * a.H));
    if (a.scalar_gate)
        hipLaunchKernelGGL((decode_step_kernel<DK, DV, kBf16, true>), grid, dim3(NT), 0, stream, a.q,
                           a.k, a.v, a.log_alpha, a.beta, a.state, a.o);
    else
        hipLaunchKernelGGL((decode_step_kernel<DK, DV, kBf16, false>), grid, dim3(NT), 0, stream, a.q,
                           a.k, a.v, a.log_alpha, a.beta, a.state, a.o);
    return hipGetLastError();
}

template <bool kBf16>
static hipError_t dispatch_dv(const DecodeArgs &a, hipStream_t s) {
#define KDA_DV_CASES(DKV)                                          \
    switch (a.Dv) {                                                \
        case 16: return launch_decode_t<DKV, 16, kBf16>(a, s);     \
        case 32: return launch_decode_t<DKV, 32, kBf16>(a, s);     \
        case 64: return launch_decode_t<DKV, 64, kBf16>(a, s);     \
        case 128: return launch_decode_t<DKV, 128, kBf16>(a, s);   \
        default: return hipErrorInvalidValue;                      \
    }
    switch (a.Dk) {
        case 16: KDA_DV_CASES(16)
        case 32: KDA_DV_CASES(32)
        case 64: KDA_DV_CASES(64)
        case 128: KDA_DV_CASES(128)
        default: return hipErrorInvalidValue;
    }
#undef KDA_DV_CASES
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    if (a.N * static_cast<int64_t>(a.H) == 0) return hipSuccess;
    return a.bf16 ? dispatch_dv<true>(a, stream) : dispatch_dv<false>(a, stream);
}

}  // namespace kda
