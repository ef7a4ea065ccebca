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
// (n, h) and applied to every row.  The general diagonal-plus-low-rank step
// (the form the same section contrasts KDA with) is
//
//   e = b^T S,  S' = Diag(exp(log_alpha)) S,  S = S' + a e^T + k v^T
//   o = S^T q = S'^T q + (a . q) e + (k . q) v
//
// with the first reduction taken over the undecayed state.
//
// One workgroup of min(1024, Dk*Dv/4) threads per (n, h).  Thread t owns 4 adjacent columns
// (one float4) of RPT rows spaced RG apart, so each wave reads and writes whole
// contiguous rows (coalesced 16-byte accesses).  Reductions: butterfly
// shuffles inside a wave over the lanes that share a column group, then LDS
// across waves.  All arithmetic is fp32.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

constexpr int kDecodeThreads = 1024;  // 16 waves: 4 float4 of the state per thread at d = 128

// Gate modes: 0 KDA (log_alpha [N, H, Dk]); 1 Gated DeltaNet (one log_alpha per
// (n, h), [N, H]); 2 KDA layer: q and k arrive unnormalised and are divided by
// sqrt(|x|^2 + l2_eps), alpha = exp(-softplus(x_alpha)), beta = sigmoid(x_beta)
// from bf16 projections, and the output is o / sqrt(mean o^2 + norm_eps) * w *
// sigmoid(g) (the KDA-layer item of the page's model-architecture list).
template <int DK, int DV, bool kBf16, int GM>
__global__ void __launch_bounds__(kDecodeThreads) decode_step_kernel(DecodeArgs a) {
    constexpr int CG = DV / 4;                                  // float4 column groups
    constexpr int NT = (DK * DV / 4 < kDecodeThreads) ? DK * DV / 4 : kDecodeThreads;  // threads
    constexpr int RG = NT / CG;                                 // row groups
    constexpr int RPT = DK / RG;                                // rows per thread
    constexpr int NW = (NT + kWave - 1) / kWave;                // waves holding rows
    constexpr int NWK = (DK + kWave - 1) / kWave;               // waves holding a key channel
    static_assert(CG <= kWave && kWave % CG == 0, "column groups must tile a wave");
    static_assert(RG * RPT == DK, "rows must tile the state");
    static_assert(NT >= DK, "one thread per key channel");

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ f32x4 s_red[NW][CG][2];
    __shared__ float s_kq[NW][CG], s_aq[GM == 3 ? NW : 1][CG];
    __shared__ float s_nrm[NWK][2];

    const int t = threadIdx.x;
    const int64_t unit = blockIdx.x;  // n * H + h
    const int cg = t % CG;
    const int rg = t / CG;
    const int w = t / kWave, lane = t % kWave;
    f32x4 *S = reinterpret_cast<f32x4 *>(a.state + unit * DK * DV);

    // the state stream is issued first; the token's vectors load under it
    f32x4 sv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) sv[i] = __builtin_nontemporal_load(&S[(rg + i * RG) * CG + cg]);
    // zero, in a form the compiler does not treat as uniform: the (n, h) scalars below
    // become vector loads issued here with the token's others (as scalar loads they
    // would be placed after the whole state stream has arrived)
    const int z0 = static_cast<int>(__builtin_amdgcn_mbcnt_lo(0u, 0u));
    const float b = GM == 2 ? sigmoid_f(bf16_bits_to_f32(a.x_beta[unit])) : GM == 3 ? 1.f : a.beta[unit + z0];
    f32x4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = load_in<kBf16>(a.v, unit * DV + 4 * cg + e);
    // Per-row token values: gate mode 2 needs the norms of k and q over all rows
    // first, so it goes through LDS and a barrier; the other modes read the rows
    // a thread owns directly (cache-resident), after the state stream is issued,
    // and need no barrier before the reductions.
    float kk = 0.f, qq = 0.f;
    float rkv[GM == 2 ? 1 : RPT], rqv[GM == 2 ? 1 : RPT], rav[GM == 2 ? 1 : RPT];
    float rla[GM == 3 ? RPT : 1], rlb[GM == 3 ? RPT : 1];
    if constexpr (GM != 2) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg + i * RG;
            rkv[i] = load_in<kBf16>(a.k, unit * DK + row);
            rqv[i] = load_in<kBf16>(a.q, unit * DK + row);
            const float g = GM == 1 ? a.log_alpha[unit + z0] : a.log_alpha[unit * DK + row];
            rav[i] = fast_exp2(g * kLog2e);  // exp(-inf) -> 0
            if constexpr (GM == 3) {
                rla[i] = load_in<kBf16>(a.lr_a, unit * DK + row);
                rlb[i] = load_in<kBf16>(a.lr_b, unit * DK + row);
            }
        }
    }
    if (GM == 2 && t < DK) {
        const float kc = load_in<kBf16>(a.k, unit * DK + t), qc = load_in<kBf16>(a.q, unit * DK + t);
        s_k[t] = kc;
        s_q[t] = qc;
        kk = kc * kc;
        qq = qc * qc;
        s_a[t] = fast_exp2(neg_softplus(bf16_bits_to_f32(a.x_alpha[unit * DK + t])) * kLog2e);
    }
    if constexpr (GM == 2) {
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            kk += __shfl_xor(kk, off);
            qq += __shfl_xor(qq, off);
        }
        if (lane == 0 && w < NWK) {
            s_nrm[w][0] = kk;
            s_nrm[w][1] = qq;
        }
        __syncthreads();
    }
    float rk = 1.f, rq = 1.f;  // 1 / |k|, 1 / |q| (gate mode 2)
    if constexpr (GM == 2) {
        float nk = 0.f, nq = 0.f;
#pragma unroll
        for (int ww = 0; ww < NWK; ++ww) {
            nk += s_nrm[ww][0];
            nq += s_nrm[ww][1];
        }
        rk = 1.f / sqrtf(nk + a.l2_eps);
        rq = 1.f / sqrtf(nq + a.l2_eps);
    }

    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f, aq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + i * RG;
        float al, kr, qr;
        if constexpr (GM == 2) {
            al = s_a[row];
            kr = s_k[row] * rk;
            qr = s_q[row] * rq;
        } else {
            al = rav[i];
            kr = rkv[i];
            qr = rqv[i];
        }
        if constexpr (GM == 3) {
            p += sv[i] * rlb[i];  // e = b^T S before the decay
            aq += rla[i] * qr;
        }
        sv[i] *= al;
        if constexpr (GM != 3) p += sv[i] * kr;
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
        if constexpr (GM == 3) aq += __shfl_xor(aq, off);
    }
    if (lane < CG) {
        s_red[w][lane][0] = p;
        s_red[w][lane][1] = r;
        s_kq[w][lane] = kq;
        if constexpr (GM == 3) s_aq[w][lane] = aq;
    }
    __syncthreads();
    p = s_red[0][cg][0];
    r = s_red[0][cg][1];
    kq = s_kq[0][cg];
    if constexpr (GM == 3) aq = s_aq[0][cg];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) {
        p += s_red[ww][cg][0];
        r += s_red[ww][cg][1];
        kq += s_kq[ww][cg];
        if constexpr (GM == 3) aq += s_aq[ww][cg];
    }
    // KDA: S += k u^T with u = beta (v - p);  DPLR: S += a e^T + k v^T with e = p
    const f32x4 u = GM == 3 ? vv : b * (vv - p);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + i * RG;
        const float kr = GM == 2 ? s_k[row] * rk : rkv[GM == 2 ? 0 : i];
        f32x4 nv = sv[i] + kr * u;
        if constexpr (GM == 3) nv += rla[i] * p;
        __builtin_nontemporal_store(nv, &S[row * CG + cg]);
    }
    if (rg == 0) {
        f32x4 ot = r + kq * u;
        if constexpr (GM == 3) ot += aq * p;
        if constexpr (GM == 2) {
            // RMSNorm over the DV columns held by lanes 0 .. CG-1 of wave 0
            float ss = ot[0] * ot[0] + ot[1] * ot[1] + ot[2] * ot[2] + ot[3] * ot[3];
#pragma unroll
            for (int off = 1; off < CG; off <<= 1) ss += __shfl_xor(ss, off);
            const float sc = 1.f / sqrtf(ss / DV + a.norm_eps);
            const f32x4 wv = reinterpret_cast<const f32x4 *>(a.norm_weight)[cg];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ot[e] = ot[e] * sc * wv[e] * sigmoid_f(bf16_bits_to_f32(a.out_gate[unit * DV + 4 * cg + e]));
        }
        reinterpret_cast<f32x4 *>(a.o + unit * DV)[cg] = ot;
    }
}

template <int DK, int DV, bool kBf16>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    constexpr int NT = (DK * DV / 4 < kDecodeThreads) ? DK * DV / 4 : kDecodeThreads;
    const dim3 grid(static_cast<unsigned>(a.N * a.H));
    switch (a.gate_mode) {
        case 0: hipLaunchKernelGGL((decode_step_kernel<DK, DV, kBf16, 0>), grid, dim3(NT), 0, stream, a); break;
        case 1: hipLaunchKernelGGL((decode_step_kernel<DK, DV, kBf16, 1>), grid, dim3(NT), 0, stream, a); break;
        case 3: hipLaunchKernelGGL((decode_step_kernel<DK, DV, kBf16, 3>), grid, dim3(NT), 0, stream, a); break;
        case 2:
            if constexpr (kBf16) {
                hipLaunchKernelGGL((decode_step_kernel<DK, DV, kBf16, 2>), grid, dim3(NT), 0, stream, a);
                break;
            } else {
                return hipErrorInvalidValue;  // the layer's projections are bf16
            }
        default: return hipErrorInvalidValue;
    }
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
