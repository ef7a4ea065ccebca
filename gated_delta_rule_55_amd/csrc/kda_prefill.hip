// kda_prefill.hip -- chunked KDA prefill on gfx950.
//
// The recurrence of the section "Kimi Delta Attention (KDA)" on the page
// "Kimi Linear 高效注意力架构" is run chunk by chunk (chunk C tokens), as its
// bullet on the hardware-efficient chunked algorithm describes (DPLR with
// a = b = k, so the WY/UT form needs one triangular inverse per chunk).  Per
// chunk, with local tokens i, j, incoming state S0 and per-channel cumulative
// log-decay G_i = sum_{m<=i} g_m, Gamma = exp(G):
//
//   A_ij = beta_i sum_c k_ic k_jc e^{G_ic - G_jc}    (j < i)
//   P_ij =        sum_c q_ic k_jc e^{G_ic - G_jc}    (j <= i)
//   T    = (I + A)^-1,   T' = T Diag(beta)
//   W    = T' (K * Gamma),     U' = T' V
//   Q'   = Q * Gamma - P W,    O_intra = P U'
//   U    = U' - W S0,  O = Q' S0 + O_intra,  S1 = Diag(Gamma_last) S0 + Kt^T U
//   with Kt_j = k_j e^{G_last - G_j}.
//
// Q' folds P into the readout operator so the sequential pass needs no P and
// O does not wait for U.  Everything that depends on the chunk alone (the
// "intra" work) runs fully parallel in intra_kernel and is written to the
// workspace as one package per (chunk, head) in the matrix-core fragment
// layouts of the state pass; state_kernel then walks the chunks of each
// (sequence, head) in order, one 16-column slab of the state per workgroup
// (columns of S are independent given the package), keeping the fp32 state
// slab in registers.
//
// Exponent safety: the factored products e^{G_i - G_m} e^{G_m - G_j} use a
// per-tile reference m.  Off-diagonal 16x16 tiles take m = the last token of
// the column tile, so both factors are <= 1.  Diagonal tiles take the tile's
// token 7; a channel whose half-span there exceeds kSafeSpan2 (log2 units) is
// removed from the factored product and added exactly per element.  A token
// whose log_alpha is -inf on every channel is a reset: its g counts as 0 in
// the exponents and masks zero the coupling across it; other -inf values are
// clamped to -88.
//
// Operand precision (fp32 accumulation everywhere): with bf16 inputs the
// intra products use bf16 hi/lo splits (three products), [W; Q'] S uses fp16,
// Kt^T U uses fp16 hi/lo splits; with fp32 inputs every product is fp32.
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"
#include "kda_mma.h"

namespace kda {

constexpr float kGFloor = -88.0f;               // clamp for partial -inf decays
constexpr float kSafeSpan2 = 110.0f;            // max |exponent| (log2) of a factor
constexpr float kNegInf = -__builtin_huge_valf();

struct IntraParams {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    const int32_t *cu_seqlens, *chunk_offsets;  // varlen only
    int64_t T;
    int32_t H, N;
    char *ws;
    size_t pkg_bytes;
    PackageLayout L;
};

struct StateParams {
    const float *init_state;
    const int32_t *cu_seqlens, *chunk_offsets;
    float *o, *final_state;
    int64_t T;
    int32_t H, N;
    const char *ws;
    size_t pkg_bytes;
    PackageLayout L;
};

template <int C, int DK, int DV, bool BF>
struct Cfg {
    static constexpr int NT16 = C / 16;            // 16-token row tiles of a chunk
    static constexpr int CP = C < 32 ? 32 : C;     // token dimension padded to a K step
    static constexpr int DKP = DK < 32 ? 32 : DK;
    static constexpr int DVP = DV < 32 ? 32 : DV;
    static constexpr int GK = DKP / 32;            // 32-wide channel groups
    static constexpr int GV = DVP / 32;
    static constexpr int GS = DK + 4;              // LDS row strides (elements)
    static constexpr int KS = DK + 8;
    static constexpr int VS = DV + 8;
    static constexpr int AS = CP + 4;
    static constexpr int XS = CP + 4;
    using In = std::conditional_t<BF, uint16_t, float>;
    using Op = std::conditional_t<BF, _Float16, float>;  // stored operand type
    static constexpr Prec kIntra = BF ? Prec::BF16X3 : Prec::F32;
    static constexpr Prec kIntraV = BF ? Prec::BF16X2A : Prec::F32;
};

// Stores 8 operand values (converted to the package's operand type) as one
// 16-byte (fp16) or two 16-byte (fp32) vector stores.
template <typename Op>
__device__ __forceinline__ void store8(Op *dst, const float (&v)[8]) {
    if constexpr (sizeof(Op) == 2) {
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(v[e]);
        *reinterpret_cast<f16x8 *>(dst) = h;
    } else {
        *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
}

template <bool BF>
__device__ __forceinline__ float in_to_f32(typename std::conditional_t<BF, uint16_t, float> x) {
    if constexpr (BF) return bf16_bits_to_f32(x);
    else return x;
}

// Locates the chunk handled by slot x: its first flattened token and length.
// Returns false when x is past the last chunk (varlen grids are an upper bound).
__device__ __forceinline__ bool locate_chunk(int64_t x, int C, int64_t T, int32_t N,
                                             const int32_t *cu, const int32_t *off,
                                             int64_t &tok0, int &nvalid) {
    if (cu == nullptr) {
        const int64_t cps = (T + C - 1) / C;
        const int64_t n = x / cps, c = x % cps;
        tok0 = n * T + c * C;
        const int64_t rem = T - c * C;
        nvalid = static_cast<int>(rem < C ? rem : C);
        return true;
    }
    if (x >= off[N]) return false;
    int lo = 0, hi = N;  // off[lo] <= x < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= x) lo = mid;
        else hi = mid;
    }
    const int64_t c = x - off[lo];
    tok0 = cu[lo] + c * C;
    const int64_t rem = cu[lo + 1] - tok0;
    nvalid = static_cast<int>(rem < C ? rem : C);
    return true;
}

// -----------------------------------------------------------------------------
// varlen plan: chunk_offsets[n] = sum_{m<n} ceil(len_m / C)
// -----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) plan_kernel(const int32_t *__restrict__ cu, int32_t N, int C,
                                                   int32_t *__restrict__ off) {
    __shared__ int32_t part[256];
    const int t = threadIdx.x;
    const int per = (N + 255) / 256;
    const int b = t * per, e = min(N, b + per);
    int32_t s = 0;
    for (int n = b; n < e; ++n) s += (cu[n + 1] - cu[n] + C - 1) / C;
    part[t] = s;
    __syncthreads();
    if (t == 0) {
        int32_t run = 0;
        for (int i = 0; i < 256; ++i) {
            const int32_t v = part[i];
            part[i] = run;
            run += v;
        }
    }
    __syncthreads();
    int32_t run = part[t];
    for (int n = b; n < e; ++n) {
        off[n] = run;
        run += (cu[n + 1] - cu[n] + C - 1) / C;
    }
    if (t == 255) off[N] = run;
}

// -----------------------------------------------------------------------------
// intra-chunk package
// -----------------------------------------------------------------------------
template <int C, int DK, int DV, bool BF>
__global__ void __launch_bounds__(256) intra_kernel(IntraParams p) {
    using F = Cfg<C, DK, DV, BF>;
    using In = typename F::In;
    using Op = typename F::Op;
    constexpr int NT16 = F::NT16, CP = F::CP, DKP = F::DKP;

    __shared__ __align__(16) float sG[C][F::GS];
    __shared__ __align__(16) In sK[C][F::KS];
    __shared__ __align__(16) In sQ[C][F::KS];
    __shared__ __align__(16) In sV[C][F::VS];
    __shared__ __align__(16) float sA[C][F::AS];
    __shared__ __align__(16) float sP[C][F::AS];
    __shared__ __align__(16) float sX[4][32][F::XS];
    __shared__ float sBeta[C];
    __shared__ int sLru[C];
    __shared__ int sLastReset;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    const int h = blockIdx.y;
    const int64_t x = blockIdx.x;
    int64_t tok0;
    int nvalid;
    if (!locate_chunk(x, C, p.T, p.N, p.cu_seqlens, p.chunk_offsets, tok0, nvalid)) return;
    const int H = p.H;
    char *pkg = p.ws + (static_cast<size_t>(x) * H + h) * p.pkg_bytes;

    // ---- 1. stage the chunk in LDS; pad rows >= nvalid with identity tokens
    {
        constexpr int GV4 = DK / 4;
        for (int idx = tid; idx < C * GV4; idx += 256) {
            const int i = idx / GV4, c4 = idx % GV4;
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
            if (i < nvalid)
                g = *reinterpret_cast<const f32x4 *>(p.log_alpha + ((tok0 + i) * H + h) * DK + 4 * c4);
            *reinterpret_cast<f32x4 *>(&sG[i][4 * c4]) = g;
        }
        constexpr int EPV = 16 / sizeof(In);  // elements per 16-byte vector
        constexpr int KV = DK / EPV, VV = DV / EPV;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        for (int idx = tid; idx < C * KV; idx += 256) {
            const int i = idx / KV, c = (idx % KV) * EPV;
            f32x4 kv = z, qv = z;
            if (i < nvalid) {
                const int64_t off = ((tok0 + i) * H + h) * DK + c;
                kv = *reinterpret_cast<const f32x4 *>(static_cast<const In *>(p.k) + off);
                qv = *reinterpret_cast<const f32x4 *>(static_cast<const In *>(p.q) + off);
            }
            *reinterpret_cast<f32x4 *>(&sK[i][c]) = kv;
            *reinterpret_cast<f32x4 *>(&sQ[i][c]) = qv;
        }
        for (int idx = tid; idx < C * VV; idx += 256) {
            const int i = idx / VV, c = (idx % VV) * EPV;
            f32x4 vv = z;
            if (i < nvalid)
                vv = *reinterpret_cast<const f32x4 *>(static_cast<const In *>(p.v) +
                                                      ((tok0 + i) * H + h) * DV + c);
            *reinterpret_cast<f32x4 *>(&sV[i][c]) = vv;
        }
        for (int idx = tid; idx < C * F::AS; idx += 256) {
            (&sA[0][0])[idx] = 0.f;
            (&sP[0][0])[idx] = 0.f;
        }
        for (int i = tid; i < C; i += 256) sBeta[i] = i < nvalid ? p.beta[(tok0 + i) * H + h] : 0.f;
    }
    __syncthreads();

    // ---- 2. resets (log_alpha = -inf on every channel) and their masks
    if (w == 0) {
        bool reset = false;
        if (lane < nvalid) {
            reset = true;
            for (int c = 0; c < DK; ++c) reset = reset && (sG[lane][c] == kNegInf);
        }
        const uint64_t mask = __ballot(reset);
        if (lane < C) {
            const uint64_t upto = lane == 63 ? mask : (mask & ((uint64_t(1) << (lane + 1)) - 1));
            sLru[lane] = upto ? 63 - __clzll(upto) : -1;
        }
        if (lane == 0) sLastReset = mask ? 63 - __clzll(mask) : -1;
    }
    __syncthreads();
    for (int idx = tid; idx < C * DK; idx += 256) {
        const int i = idx / DK, c = idx % DK;
        const float g = sG[i][c];
        sG[i][c] = (sLru[i] == i) ? 0.f : fmaxf(g, kGFloor) * kLog2e;
    }
    __syncthreads();
    // cumulative log2-decay per channel
    if (tid < DK) {
        float run = 0.f;
        for (int i = 0; i < C; ++i) {
            run += sG[i][tid];
            sG[i][tid] = run;
        }
    }
    __syncthreads();

    auto Kf = [&](int i, int c) { return in_to_f32<BF>(sK[i][c]); };
    auto Qf = [&](int i, int c) { return in_to_f32<BF>(sQ[i][c]); };
    auto Vf = [&](int i, int c) { return in_to_f32<BF>(sV[i][c]); };

    // ---- 3. A and P, 16x16 tiles on the lower triangle
    {
        constexpr int NTILES = NT16 * (NT16 + 1) / 2;
        for (int t = w; t < NTILES; t += 4) {
            int I = 0, J = t;
            while (J > I) { J -= I + 1; ++I; }
            const bool diag = I == J;
            const int m = diag ? 16 * I + 7 : 16 * J + 15;
            const int ia = 16 * I + l16, jb = 16 * J + l16;
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            bool unsafe_any = false;
#pragma unroll
            for (int ks = 0; ks < DKP / 32; ++ks) {
                float xk[8], xq[8], y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int c = 32 * ks + 8 * kg + e;
                    xk[e] = xq[e] = y[e] = 0.f;
                    if (c < DK) {
                        const float gm = sG[m][c];
                        float fa = fast_exp2(sG[ia][c] - gm);
                        float fb = fast_exp2(gm - sG[jb][c]);
                        if (diag) {
                            const float span = fmaxf(sG[16 * I][c] - gm, gm - sG[16 * I + 15][c]);
                            if (!(span <= kSafeSpan2)) {
                                fa = 0.f;
                                fb = 0.f;
                                unsafe_any = true;
                            }
                        }
                        xk[e] = Kf(ia, c) * fa;
                        xq[e] = Qf(ia, c) * fa;
                        y[e] = Kf(jb, c) * fb;
                    }
                }
                mma<F::kIntra>(accA, xk, y);
                mma<F::kIntra>(accP, xq, y);
            }
            if (diag && __ballot(unsafe_any)) {
                // exact per-element terms for channels taken out above
                for (int c = 0; c < DK; ++c) {
                    const float gm = sG[m][c];
                    const float span = fmaxf(sG[16 * I][c] - gm, gm - sG[16 * I + 15][c]);
                    if (span <= kSafeSpan2) continue;
                    const int j = 16 * J + l16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * I + 4 * kg + r;
                        const float ex = fast_exp2(fminf(sG[i][c] - sG[j][c], 0.f));
                        accA[r] += Kf(i, c) * Kf(j, c) * ex;
                        accP[r] += Qf(i, c) * Kf(j, c) * ex;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * kg + r, j = 16 * J + l16;
                const bool keep = sLru[i] <= j;  // no reset in (j, i]
                sA[i][j] = (j < i && keep) ? sBeta[i] * accA[r] : 0.f;
                sP[i][j] = (j <= i && keep) ? accP[r] : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- 4. T = (I + A)^-1 in place (unit lower triangular), then T' = T Diag(beta)
    if (w < NT16 && lane < 16) {
        const int base = 16 * w, col = lane;
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float val = (i == col) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) val -= sA[base + i][base + j] * t[j];
            t[i] = val;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (i >= col) sA[base + i][base + col] = t[i];
    }
    __syncthreads();
    for (int I = 1; I < NT16; ++I) {
        float *X = &sX[0][0][0];  // I blocks of 16x16 scratch
        const int i = tid >> 4, j = tid & 15;
        for (int J = 0; J < I; ++J) {
            float acc = 0.f;
            for (int K = J; K < I; ++K)
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    acc += sA[16 * I + i][16 * K + kk] * sA[16 * K + kk][16 * J + j];
            X[J * 256 + i * 16 + j] = acc;
        }
        __syncthreads();
        for (int J = 0; J < I; ++J) {
            float acc = 0.f;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) acc += sA[16 * I + i][16 * I + kk] * X[J * 256 + kk * 16 + j];
            sA[16 * I + i][16 * J + j] = -acc;
        }
        __syncthreads();
    }
    for (int idx = tid; idx < C * C; idx += 256) {
        const int i = idx / C, j = idx % C;
        sA[i][j] *= sBeta[j];
    }
    __syncthreads();

    // ---- 5/6. per-wave jobs: channel groups (W, Q') and value groups (U', O_intra)
    float(*X)[F::XS] = sX[w];
    auto a_frag = [&](const float(*M)[F::AS], int I, int s, float (&a)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = M[16 * I + l16][32 * s + 8 * kg + e];
    };
    for (int job = w; job < F::GK + F::GV; job += 4) {
        if (job < F::GK) {
            const int g = job;
            // W = T' (K * Gamma) for the 32 channels of group g, kept transposed in X
            for (int hc = 0; hc < 2; ++hc) {
                const int ct = 2 * g + hc;
                if (16 * ct >= DK) break;
                const int c = 16 * ct + l16;
#pragma unroll
                for (int I = 0; I < NT16; ++I) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < CP / 32; ++s) {
                        float a[8], b[8];
                        a_frag(sA, I, s, a);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int j = 32 * s + 8 * kg + e;
                            b[e] = (j < C && sLru[j] < 0) ? Kf(j, c) * fast_exp2(sG[j][c]) : 0.f;
                        }
                        mma<F::kIntra>(acc, a, b);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) X[16 * hc + l16][16 * I + 4 * kg + r] = acc[r];
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            // Q' = Q * Gamma - P W   (registers)
            f32x4 qp[2][NT16];
#pragma unroll
            for (int hc = 0; hc < 2; ++hc) {
                const int ct = 2 * g + hc;
                const int c = 16 * ct + l16;
#pragma unroll
                for (int I = 0; I < NT16; ++I) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    if (16 * ct < DK) {
#pragma unroll
                        for (int s = 0; s < CP / 32; ++s) {
                            float a[8], b[8];
                            a_frag(sP, I, s, a);
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const int j = 32 * s + 8 * kg + e;
                                b[e] = j < C ? X[16 * hc + l16][j] : 0.f;
                            }
                            mma<F::kIntra>(acc, a, b);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int i = 16 * I + 4 * kg + r;
                            const float qg = sLru[i] < 0 ? Qf(i, c) * fast_exp2(sG[i][c]) : 0.f;
                            acc[r] = qg - acc[r];
                        }
                    }
                    qp[hc][I] = acc;
                }
            }
            // WQ fragments, W part: row 16 I + l16, channels 32 g + 8 kg + e
            Op *wq = reinterpret_cast<Op *>(pkg + p.L.wq);
#pragma unroll
            for (int I = 0; I < NT16; ++I) {
                float v8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int cl = 8 * kg + e;
                    v8[e] = (32 * g + cl < DK) ? X[cl][16 * I + l16] : 0.f;
                }
                store8(wq + ((static_cast<size_t>(I) * (DKP / 32) + g) * 64 + lane) * 8, v8);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
            for (int hc = 0; hc < 2; ++hc)
#pragma unroll
                for (int I = 0; I < NT16; ++I)
#pragma unroll
                    for (int r = 0; r < 4; ++r) X[16 * hc + l16][16 * I + 4 * kg + r] = qp[hc][I][r];
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
            for (int I = 0; I < NT16; ++I) {
                float v8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int cl = 8 * kg + e;
                    v8[e] = (32 * g + cl < DK) ? X[cl][16 * I + l16] : 0.f;
                }
                store8(wq + ((static_cast<size_t>(NT16 + I) * (DKP / 32) + g) * 64 + lane) * 8, v8);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        } else {
            const int g = job - F::GK;
            f32x4 *up = reinterpret_cast<f32x4 *>(pkg + p.L.up);
            f32x4 *oi = reinterpret_cast<f32x4 *>(pkg + p.L.oi);
            // U' = T' V for the 32 value columns of group g
            for (int hc = 0; hc < 2; ++hc) {
                const int ct = 2 * g + hc;
                if (16 * ct >= DV) break;
                const int c = 16 * ct + l16;
#pragma unroll
                for (int I = 0; I < NT16; ++I) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < CP / 32; ++s) {
                        float a[8], b[8];
                        a_frag(sA, I, s, a);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int j = 32 * s + 8 * kg + e;
                            b[e] = j < C ? Vf(j, c) : 0.f;
                        }
                        mma<F::kIntraV>(acc, a, b);
                    }
                    up[(static_cast<size_t>(ct) * NT16 + I) * 64 + lane] = acc;
#pragma unroll
                    for (int r = 0; r < 4; ++r) X[16 * hc + l16][16 * I + 4 * kg + r] = acc[r];
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            // O_intra = P U'
            for (int hc = 0; hc < 2; ++hc) {
                const int ct = 2 * g + hc;
                if (16 * ct >= DV) break;
#pragma unroll
                for (int I = 0; I < NT16; ++I) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < CP / 32; ++s) {
                        float a[8], b[8];
                        a_frag(sP, I, s, a);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int j = 32 * s + 8 * kg + e;
                            b[e] = j < C ? X[16 * hc + l16][j] : 0.f;
                        }
                        mma<F::kIntra>(acc, a, b);
                    }
                    oi[(static_cast<size_t>(ct) * NT16 + I) * 64 + lane] = acc;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
    }

    // ---- 7. decayed keys Kt (A operand of Kt^T U) and Gamma_last
    {
        const int last_reset = sLastReset;
        constexpr int NKT = (DK / 16) * (CP / 32);
        Op *kt = reinterpret_cast<Op *>(pkg + p.L.kt);
        constexpr int PARTS = BF ? 2 : 1;
        for (int blk = w; blk < NKT; blk += 4) {
            const int ct = blk / (CP / 32), ks = blk % (CP / 32);
            const int c = 16 * ct + l16;
            const float glast = sG[C - 1][c];
            float val[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 32 * ks + 8 * kg + e;
                val[e] = (j < C && j >= last_reset) ? Kf(j, c) * fast_exp2(glast - sG[j][c]) : 0.f;
            }
            Op *dst = kt + ((static_cast<size_t>(ct) * (CP / 32) + ks) * PARTS * 64 + lane) * 8;
            if constexpr (BF) {
                f16x8 hi, lo;
                split_f16(val, hi, lo);
                *reinterpret_cast<f16x8 *>(dst) = hi;
                *reinterpret_cast<f16x8 *>(dst + 64 * 8) = lo;
            } else {
                store8(dst, val);
            }
        }
        float *gl = reinterpret_cast<float *>(pkg + p.L.gl);
        for (int c = tid; c < DK; c += 256) gl[c] = last_reset >= 0 ? 0.f : fast_exp2(sG[C - 1][c]);
    }
}

// -----------------------------------------------------------------------------
// sequential state pass: one workgroup per (sequence, head, 16-column slab)
// -----------------------------------------------------------------------------
template <int C, int DK, int DV, bool BF>
__global__ void __launch_bounds__(256) state_kernel(StateParams p) {
    using F = Cfg<C, DK, DV, BF>;
    using Op = typename F::Op;
    constexpr int NT16 = F::NT16, CP = F::CP, DKP = F::DKP;
    constexpr int NTK = DK / 16;                 // 16-row tiles of the state
    constexpr int SPW = (NTK + 3) / 4;           // state tiles per wave
    constexpr int NRT = 2 * NT16;                // row tiles of [W; Q']
    constexpr int RPW = (NRT + 3) / 4;           // [W; Q'] row tiles per wave
    constexpr int PARTS = BF ? 2 : 1;
    constexpr int SSS = DKP + 8;                 // LDS strides (elements)
    constexpr int SUS = CP + 8;

    __shared__ __align__(16) Op sS[16][SSS];          // state slab as a B operand [col][channel]
    __shared__ __align__(16) Op sU[PARTS][16][SUS];   // U (hi, lo) as a B operand [col][token]

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    const int n = blockIdx.x, h = blockIdx.y, ct = blockIdx.z;
    const int H = p.H;

    int64_t tok_base, L, slot_base;
    if (p.cu_seqlens) {
        tok_base = p.cu_seqlens[n];
        L = p.cu_seqlens[n + 1] - tok_base;
        slot_base = p.chunk_offsets[n];
    } else {
        tok_base = static_cast<int64_t>(n) * p.T;
        L = p.T;
        slot_base = static_cast<int64_t>(n) * ((p.T + C - 1) / C);
    }
    const int64_t nchunks = (L + C - 1) / C;

    for (int idx = tid; idx < 16 * SSS; idx += 256) (&sS[0][0])[idx] = static_cast<Op>(0.f);
    for (int idx = tid; idx < PARTS * 16 * SUS; idx += 256) (&sU[0][0][0])[idx] = static_cast<Op>(0.f);

    const int col = 16 * ct + l16;
    const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * DV;
    f32x4 S[SPW];
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl) {
        const int tk = w + 4 * sl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * tk + 4 * kg + r;
            S[sl][r] = (tk < NTK && p.init_state) ? p.init_state[sbase + static_cast<size_t>(row) * DV + col]
                                                   : 0.f;
        }
    }
    __syncthreads();
    auto put_state = [&]() {
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk < NTK) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[l16][16 * tk + 4 * kg + r] = static_cast<Op>(S[sl][r]);
            }
        }
    };
    put_state();

    for (int64_t c = 0; c < nchunks; ++c) {
        const char *pkg = p.ws + (static_cast<size_t>(slot_base + c) * H + h) * p.pkg_bytes;
        const int64_t rem = L - c * C;
        const int nvalid = static_cast<int>(rem < C ? rem : C);
        __syncthreads();  // sS holds this chunk's incoming state

        // (a) [W; Q'] S0 for this wave's row tiles; U = U' - W S0, O = O_intra + Q' S0
#pragma unroll
        for (int rw = 0; rw < RPW; ++rw) {
            const int rt = w + 4 * rw;
            if (rt >= NRT) break;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const Op *wq = reinterpret_cast<const Op *>(pkg + p.L.wq);
#pragma unroll
            for (int ks = 0; ks < DKP / 32; ++ks) {
                const Op *af = wq + ((static_cast<size_t>(rt) * (DKP / 32) + ks) * 64 + lane) * 8;
                if constexpr (BF) {
                    const f16x8 a = *reinterpret_cast<const f16x8 *>(af);
                    const f16x8 b = *reinterpret_cast<const f16x8 *>(&sS[l16][32 * ks + 8 * kg]);
                    acc = mfma_f16(a, b, acc);
                } else {
                    float a[8], b[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        a[e] = af[e];
                        b[e] = sS[l16][32 * ks + 8 * kg + e];
                    }
                    mma<Prec::F32>(acc, a, b);
                }
            }
            if (rt < NT16) {
                const f32x4 upv = reinterpret_cast<const f32x4 *>(pkg + p.L.up)[(static_cast<size_t>(ct) * NT16 + rt) * 64 + lane];
                const f32x4 u = upv - acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * rt + 4 * kg + r;
                    const Op hi = static_cast<Op>(u[r]);
                    sU[0][l16][j] = hi;
                    if constexpr (BF) sU[1][l16][j] = static_cast<Op>(u[r] - static_cast<float>(hi));
                }
            } else {
                const int I = rt - NT16;
                const f32x4 oiv = reinterpret_cast<const f32x4 *>(pkg + p.L.oi)[(static_cast<size_t>(ct) * NT16 + I) * 64 + lane];
                const f32x4 ov = oiv + acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * kg + r;
                    if (i < nvalid) p.o[((tok_base + c * C + i) * H + h) * DV + col] = ov[r];
                }
            }
        }
        __syncthreads();  // sU complete; all reads of sS done

        // (c) S1 = Diag(Gamma_last) S0 + Kt^T U for this wave's state tiles
        const float *gl = reinterpret_cast<const float *>(pkg + p.L.gl);
        const Op *kt = reinterpret_cast<const Op *>(pkg + p.L.kt);
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk >= NTK) break;
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = gl[16 * tk + 4 * kg + r] * S[sl][r];
#pragma unroll
            for (int ks = 0; ks < CP / 32; ++ks) {
                const Op *af = kt + ((static_cast<size_t>(tk) * (CP / 32) + ks) * PARTS * 64 + lane) * 8;
                if constexpr (BF) {
                    const f16x8 ah = *reinterpret_cast<const f16x8 *>(af);
                    const f16x8 al = *reinterpret_cast<const f16x8 *>(af + 64 * 8);
                    const f16x8 bh = *reinterpret_cast<const f16x8 *>(&sU[0][l16][32 * ks + 8 * kg]);
                    const f16x8 bl = *reinterpret_cast<const f16x8 *>(&sU[1][l16][32 * ks + 8 * kg]);
                    acc = mfma_f16(al, bh, acc);
                    acc = mfma_f16(ah, bl, acc);
                    acc = mfma_f16(ah, bh, acc);
                } else {
                    float a[8], b[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        a[e] = af[e];
                        b[e] = sU[0][l16][32 * ks + 8 * kg + e];
                    }
                    mma<Prec::F32>(acc, a, b);
                }
            }
            S[sl] = acc;
        }
        put_state();
    }

    if (p.final_state) {
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk >= NTK) break;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * tk + 4 * kg + r;
                p.final_state[sbase + static_cast<size_t>(row) * DV + col] = S[sl][r];
            }
        }
    }
}

// -----------------------------------------------------------------------------
// launch
// -----------------------------------------------------------------------------
template <int C, int DK, int DV, bool BF>
static hipError_t launch_t(const PrefillArgs &a, hipStream_t stream) {
    const PackageLayout L = package_layout(C, DK, DV, BF);
    if (a.cu_seqlens) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens, a.N, C,
                           a.chunk_offsets);
    }
    if (a.n_slots > 0) {
        IntraParams ip{a.q, a.k, a.v, a.log_alpha, a.beta, a.cu_seqlens, a.chunk_offsets,
                       a.T, a.H, a.N, a.workspace, a.pkg_bytes, L};
        hipLaunchKernelGGL((intra_kernel<C, DK, DV, BF>), dim3(static_cast<unsigned>(a.n_slots), a.H),
                           dim3(256), 0, stream, ip);
    }
    StateParams sp{a.init_state, a.cu_seqlens, a.chunk_offsets, a.o, a.final_state,
                   a.T, a.H, a.N, a.workspace, a.pkg_bytes, L};
    hipLaunchKernelGGL((state_kernel<C, DK, DV, BF>), dim3(a.N, a.H, DV / 16), dim3(256), 0, stream, sp);
    return hipGetLastError();
}

template <int C, bool BF>
static hipError_t dispatch_d(const PrefillArgs &a, hipStream_t s) {
    if (a.Dk != a.Dv) return hipErrorInvalidValue;
    switch (a.Dk) {
        case 16: return launch_t<C, 16, 16, BF>(a, s);
        case 32: return launch_t<C, 32, 32, BF>(a, s);
        case 64: return launch_t<C, 64, 64, BF>(a, s);
        case 128:
            // the fp32 path holds q, k, v in fp32 in LDS; 64-token chunks at
            // d = 128 do not fit (prefill_effective_chunk maps them to 32)
            if constexpr (BF || C <= 32) return launch_t<C, 128, 128, BF>(a, s);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

int prefill_effective_chunk(int C, int Dk, int Dv, bool bf16) {
    if (!bf16 && (Dk > 64 || Dv > 64) && C > 32) return 32;
    return C;
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    const bool bf = a.bf16;
    switch (a.C) {
        case 16: return bf ? dispatch_d<16, true>(a, stream) : dispatch_d<16, false>(a, stream);
        case 32: return bf ? dispatch_d<32, true>(a, stream) : dispatch_d<32, false>(a, stream);
        case 64: return bf ? dispatch_d<64, true>(a, stream) : dispatch_d<64, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
