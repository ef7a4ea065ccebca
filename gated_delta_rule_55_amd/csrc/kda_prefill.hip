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
// Kt^T U uses fp16 Kt and fp16 hi/lo U (two products); with fp32 inputs every
// product is fp32.
#include <algorithm>

#include "kda_prefill.h"

namespace kda {

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

hipError_t launch_plan(const int32_t *cu_seqlens, int32_t N, int C, int32_t *chunk_offsets, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu_seqlens, N, C, chunk_offsets);
    return hipGetLastError();
}

// -----------------------------------------------------------------------------
// intra-chunk package
// -----------------------------------------------------------------------------
// Layout conventions shared with state_kernel:
//   * the WQ fragment for row tile rt and 32-channel step ks gives lane l the
//     token 16 rt + l%16 and the channels 32 ks + 4 (l/16) + e (e < 4) and
//     32 ks + 16 + 4 (l/16) + (e - 4) (e >= 4); the state pass stores its state
//     slab with the same channel order, so the pairing of k values matches.
//   * T' = T Diag(beta) and R = P T' are stored as one 128 x 64 operand
//     M = [T'; -R], so [W; Q'] = [0; Q*Gamma] + M (K*Gamma) and
//     [U'; -O_intra] = M V; M is lower triangular in the token index.
// One chunk's inputs as held in registers by one thread (the kernel loads the
// next work item's inputs while it computes the current one).
template <int C, int DK, int DV, bool BF>
struct IntraInputs {
    using In = typename Cfg<C, DK, DV, BF>::In;
    static constexpr int SEG = kIntraThreads / DK, TPS = (C + SEG - 1) / SEG;
    static constexpr int EPV = 16 / sizeof(In);
    static constexpr int KV = DK / EPV, VV = DV / EPV;
    static constexpr int NKV = (C * KV + kIntraThreads - 1) / kIntraThreads;
    static constexpr int NVV = (C * VV + kIntraThreads - 1) / kIntraThreads;
    float g[TPS];
    f32x4 k[NKV], q[NKV], v[NVV];
    float beta;
    int64_t tok0;
    int nvalid;
    bool valid;

    __device__ __forceinline__ void load(const IntraParams &p, int64_t item, int tid) {
        const int H = p.H;
        const int64_t slot = item / H;
        const int h = static_cast<int>(item % H);
        valid = locate_chunk(slot, C, p.T, p.N, p.cu_seqlens, p.chunk_offsets, tok0, nvalid);
        if (!valid) nvalid = 0;
        const int cc = tid % DK, seg = tid / DK;
#pragma unroll
        for (int u = 0; u < TPS; ++u) {
            const int i = seg * TPS + u;
            g[u] = (i < nvalid) ? p.log_alpha[((tok0 + i) * H + h) * p.g_row + cc * p.g_ch] : 0.f;
        }
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < NKV; ++r) {
            const int idx = tid + kIntraThreads * r;
            const int i = idx / KV, c = (idx % KV) * EPV;
            k[r] = q[r] = z;
            if (idx < C * KV && i < nvalid) {
                const int64_t off = ((tok0 + i) * H + h) * DK + c;
                k[r] = *reinterpret_cast<const f32x4 *>(static_cast<const In *>(p.k) + off);
                q[r] = *reinterpret_cast<const f32x4 *>(static_cast<const In *>(p.q) + off);
            }
        }
#pragma unroll
        for (int r = 0; r < NVV; ++r) {
            const int idx = tid + kIntraThreads * r;
            const int i = idx / VV, c = (idx % VV) * EPV;
            v[r] = z;
            if (idx < C * VV && i < nvalid)
                v[r] = *reinterpret_cast<const f32x4 *>(static_cast<const In *>(p.v) +
                                                        ((tok0 + i) * H + h) * DV + c);
        }
        beta = (tid < nvalid) ? p.beta[(tok0 + tid) * H + h] : 0.f;
    }
};


template <int C, int DK, int DV, bool BF>
__global__ void __launch_bounds__(kIntraThreads) intra_kernel(IntraParams p, int64_t n_items) {
    using F = Cfg<C, DK, DV, BF>;
    using In = typename F::In;
    using Op = typename F::Op;
    using Inputs = IntraInputs<C, DK, DV, BF>;
    constexpr int NT16 = F::NT16, CP = F::CP, DKP = F::DKP;
    constexpr int AS = CP + 8;                       // fp32 row stride of A/T and P/R
    constexpr int MS = BF ? CP + 8 : CP + 4;         // row stride of M (elements)
    constexpr int SEG = Inputs::SEG;                 // token segments of the cumsum
    constexpr int TPS = Inputs::TPS;                 // tokens per segment
    constexpr int KSK = DKP / 32, KSC = CP / 32;
    constexpr int PARTS = BF ? 2 : 1;
    constexpr int NW = kIntraThreads / kWave;
    using MT = std::conditional_t<BF, __bf16, float>;

    __shared__ __align__(16) float sG[C][F::GS];
    __shared__ __align__(16) In sK[C][F::KS];
    __shared__ __align__(16) In sQ[C][F::KS];
    __shared__ __align__(16) In sV[C][F::VS];
    __shared__ __align__(16) float sAP[2][C][AS];  // A -> T and P -> R (fp32); then M
    __shared__ float sBeta[C];
    __shared__ int sLru[C];
    __shared__ int sAllInf[C];
    __shared__ float sSeg[SEG][DK];
    __shared__ uint32_t sNotInf[SEG];
    __shared__ int sUnsafe[NT16];
    __shared__ int sLastReset;
    static_assert(sizeof(MT) * PARTS * 2 * C * MS <= sizeof(float) * 2 * C * AS, "M overlay");
    MT *Mp = reinterpret_cast<MT *>(&sAP[0][0][0]);  // [PARTS][2C][MS]
    float(*sA)[AS] = sAP[0];
    float(*sP)[AS] = sAP[1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    const int cc = tid % DK, seg = tid / DK;

    int64_t item = p.item0 + blockIdx.x;
    const int64_t stride = gridDim.x;
    for (; item < n_items; item += stride) {
      const int64_t item_next = item + stride;
      Inputs cur;
      cur.load(p, item, tid);
      if (cur.valid) {
        const int nvalid = cur.nvalid;
        float gr[TPS];
#pragma unroll
        for (int u = 0; u < TPS; ++u) gr[u] = cur.g[u];
        char *pkg = p.ws + static_cast<size_t>(item - p.item0) * p.pkg_bytes;
        __syncthreads();  // the previous chunk's LDS reads are done

    // ---- 1. stage k, q, v in LDS from registers (rows >= nvalid hold zeros)
    {
#pragma unroll
        for (int r = 0; r < Inputs::NKV; ++r) {
            const int idx = tid + kIntraThreads * r;
            if (idx < C * Inputs::KV) {
                const int i = idx / Inputs::KV, c = (idx % Inputs::KV) * Inputs::EPV;
                *reinterpret_cast<f32x4 *>(&sK[i][c]) = cur.k[r];
                *reinterpret_cast<f32x4 *>(&sQ[i][c]) = cur.q[r];
            }
        }
#pragma unroll
        for (int r = 0; r < Inputs::NVV; ++r) {
            const int idx = tid + kIntraThreads * r;
            if (idx < C * Inputs::VV) {
                const int i = idx / Inputs::VV, c = (idx % Inputs::VV) * Inputs::EPV;
                *reinterpret_cast<f32x4 *>(&sV[i][c]) = cur.v[r];
            }
        }
        if (tid < C) {
            sBeta[tid] = cur.beta;
            sAllInf[tid] = tid < nvalid ? 1 : 0;
        }
        if (tid < SEG) sNotInf[tid] = 0u;
    }
    __syncthreads();

    // ---- 2. resets: a token whose log_alpha is -inf on every channel
    {
        static_assert(TPS <= 32, "one bit per token of a segment");
        uint32_t notinf = 0;
#pragma unroll
        for (int u = 0; u < TPS; ++u) notinf |= static_cast<uint32_t>(!(gr[u] == kNegInf)) << u;
        // OR over the lanes of this wave holding the same segment (DK or 64 lanes)
#pragma unroll
        for (int off = 1; off < (DK < kWave ? DK : kWave); off <<= 1) notinf |= __shfl_xor(notinf, off);
        if ((tid & ((DK < kWave ? DK : kWave) - 1)) == 0) atomicOr(&sNotInf[seg], notinf);
    }
    __syncthreads();
    if (tid < C) {
        const int sg = tid / TPS, u = tid % TPS;
        if ((sNotInf[sg] >> u) & 1u) sAllInf[tid] = 0;
    }
    __syncthreads();
    if (w == 0) {
        const bool reset = lane < C && sAllInf[lane] != 0;
        const uint64_t mask = __ballot(reset);
        if (lane < C) {
            const uint64_t upto = lane == 63 ? mask : (mask & ((uint64_t(1) << (lane + 1)) - 1));
            sLru[lane] = upto ? 63 - __clzll(upto) : -1;
        }
        if (lane == 0) sLastReset = mask ? 63 - __clzll(mask) : -1;
    }
    __syncthreads();

    // ---- 3. cumulative log2-decay per channel (segmented scan in registers)
    {
        float run = 0.f;
#pragma unroll
        for (int u = 0; u < TPS; ++u) {
            const int i = seg * TPS + u;
            const float g = (i < C && sLru[i] == i) ? 0.f : fmaxf(gr[u], kGFloor) * kLog2e;
            run += g;
            gr[u] = run;
        }
        sSeg[seg][cc] = run;
    }
    __syncthreads();
    {
        float base = 0.f;
        for (int s2 = 0; s2 < seg; ++s2) base += sSeg[s2][cc];
#pragma unroll
        for (int u = 0; u < TPS; ++u) {
            const int i = seg * TPS + u;
            if (i < C) sG[i][cc] = gr[u] + base;
        }
    }
    for (int idx = tid; idx < 2 * C * AS / 4; idx += kIntraThreads)
        reinterpret_cast<f32x4 *>(&sAP[0][0][0])[idx] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (tid < NT16) sUnsafe[tid] = 0;
    __syncthreads();
    // diagonal tiles whose half-span exceeds the safe factor range on some channel
    for (int idx = tid; idx < NT16 * DK; idx += kIntraThreads) {
        const int I = idx / DK, c = idx % DK;
        const float gm = sG[16 * I + 7][c];
        if (!(fmaxf(sG[16 * I][c] - gm, gm - sG[16 * I + 15][c]) <= kSafeSpan2)) sUnsafe[I] = 1;
    }
    __syncthreads();

    auto Kf = [&](int i, int c) { return in_to_f32<BF>(sK[i][c]); };
    auto Qf = [&](int i, int c) { return in_to_f32<BF>(sQ[i][c]); };
    auto Vf = [&](int i, int c) { return in_to_f32<BF>(sV[i][c]); };
    auto ld8f = [&](const float *src, float (&o)[8]) {
        const f32x4 a = reinterpret_cast<const f32x4 *>(src)[0];
        const f32x4 b = reinterpret_cast<const f32x4 *>(src)[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[e] = a[e];
            o[4 + e] = b[e];
        }
    };
    auto ld8in = [&](const In *src, float (&o)[8]) {
        if constexpr (BF) {
            const u16x8 r = *reinterpret_cast<const u16x8 *>(src);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = bf16_bits_to_f32(r[e]);
        } else {
            ld8f(src, o);
        }
    };

    // ---- 4. A and P, 16x16 tiles on the lower triangle (factored exponents)
    // First touch one word of every 128-byte line of the next item's inputs so
    // that its loads hit L2 when it starts (the words are consumed at the end).
    const float touch = touch_next_item<C, DK, DV, BF>(p, item_next, n_items, tid);
    {
        constexpr int NTILES = NT16 * (NT16 + 1) / 2;
        // factored tile product; kSlow also drops channels whose diagonal-tile
        // half-span is outside the safe factor range (added exactly below)
        auto tile_ap = [&](int I, int J, int m, f32x4 &accA, f32x4 &accP, auto slow_tag) {
            constexpr bool kSlow = decltype(slow_tag)::value;
            const int ia = 16 * I + l16, jb = 16 * J + l16;
#pragma unroll 1
            for (int ks = 0; ks < DKP / 32; ++ks) {
                const int c0 = 32 * ks + 8 * kg;
                float xk[8], xq[8], y[8];
                if (DK >= 32 || c0 < DK) {
                    float gi[8], gm[8], gj[8], ki[8], qi[8], kj[8];
                    ld8f(&sG[ia][c0], gi);
                    ld8f(&sG[m][c0], gm);
                    ld8f(&sG[jb][c0], gj);
                    ld8in(&sK[ia][c0], ki);
                    ld8in(&sQ[ia][c0], qi);
                    ld8in(&sK[jb][c0], kj);
                    float gf[8], gl[8];
                    if constexpr (kSlow) {
                        ld8f(&sG[16 * I][c0], gf);
                        ld8f(&sG[16 * I + 15][c0], gl);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float fa = fast_exp2(gi[e] - gm[e]);
                        float fb = fast_exp2(gm[e] - gj[e]);
                        if constexpr (kSlow) {
                            const bool uns = !(fmaxf(gf[e] - gm[e], gm[e] - gl[e]) <= kSafeSpan2);
                            fa = uns ? 0.f : fa;
                            fb = uns ? 0.f : fb;
                        }
                        xk[e] = ki[e] * fa;
                        xq[e] = qi[e] * fa;
                        y[e] = kj[e] * fb;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) xk[e] = xq[e] = y[e] = 0.f;
                }
                mma<Prec::F32>(accA, xk, y);
                mma<Prec::F32>(accP, xq, y);
            }
        };
        for (int t = w; t < NTILES; t += NW) {
            int I = 0, J = t;
            while (J > I) { J -= I + 1; ++I; }
            const bool diag = I == J;
            const int m = diag ? 16 * I + 7 : 16 * J + 15;
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            if (diag && sUnsafe[I]) {
                tile_ap(I, J, m, accA, accP, std::true_type{});
                // exact per-element terms for the channels taken out
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
            } else {
                tile_ap(I, J, m, accA, accP, std::false_type{});
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

    // ---- 5. T = (I + A)^-1 (unit lower triangular), in place over A
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
    // off-diagonal blocks: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ  (fp32 matrix cores)
    for (int I = 1; I < NT16; ++I) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        const int J = w;
        if (J < I) {
            f32x4 xv = {0.f, 0.f, 0.f, 0.f};
            for (int K = J; K < I; ++K) {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int kk = 4 * s4 + kg;
                    xv = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[16 * I + l16][16 * K + kk],
                                                               sA[16 * K + kk][16 * J + l16], xv, 0, 0, 0);
                }
            }
            // y = T_II x, with x's rows 4 kg + r held by this lane as xv[r]
#pragma unroll
            for (int r = 0; r < 4; ++r)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[16 * I + l16][16 * I + 4 * kg + r], xv[r], y,
                                                          0, 0, 0);
        }
        __syncthreads();
        if (J < I) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sA[16 * I + 4 * kg + r][16 * J + l16] = -y[r];
        }
        __syncthreads();
    }

    // ---- 6. R = P T' and M = [T'; -R] (T' = T Diag(beta)) as matrix-core operands
    {
        constexpr int NB = NT16 * (NT16 + 1) / 2;
        constexpr int BPW = (NB + NW - 1) / NW;
        f32x4 tv[BPW], rv[BPW];
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int t = w + NW * b;
            tv[b] = rv[b] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t < NB) {
                int I = 0, J = t;
                while (J > I) { J -= I + 1; ++I; }
                const float bj = sBeta[16 * J + l16];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int K = J; K <= I; ++K) {
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        const int kk = 4 * s4 + kg;
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sP[16 * I + l16][16 * K + kk],
                                                                    sA[16 * K + kk][16 * J + l16], acc, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    rv[b][r] = -acc[r] * bj;
                    tv[b][r] = sA[16 * I + 4 * kg + r][16 * J + l16] * bj;
                }
            }
        }
        __syncthreads();  // every fp32 read of A/T and P is done: M overlays them
        for (int idx = tid; idx < PARTS * 2 * C * MS * static_cast<int>(sizeof(MT)) / 16; idx += kIntraThreads)
            reinterpret_cast<f32x4 *>(Mp)[idx] = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int t = w + NW * b;
            if (t < NB) {
                int I = 0, J = t;
                while (J > I) { J -= I + 1; ++I; }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * I + 4 * kg + r, col = 16 * J + l16;
                    const float vals[2] = {tv[b][r], rv[b][r]};
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const size_t o = static_cast<size_t>(hh * C + row) * MS + col;
                        if constexpr (BF) {
                            const __bf16 hi = static_cast<__bf16>(vals[hh]);
                            Mp[o] = hi;
                            Mp[static_cast<size_t>(2 * C) * MS + o] =
                                static_cast<__bf16>(vals[hh] - static_cast<float>(hi));
                        } else {
                            Mp[o] = vals[hh];
                        }
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- 7. package: [W; Q'] fragments, Kt fragments, U', O_intra, Gamma_last
    const int last_reset = sLastReset;
    // B fragment of M^T for row tile rt and token step s: row 16 rt + l16 of M
    auto m_frag_bf = [&](int rt, int s, bf16x8 &hi, bf16x8 &lo) {
        const size_t o = static_cast<size_t>(16 * rt + l16) * MS + 32 * s + 8 * kg;
        hi = *reinterpret_cast<const bf16x8 *>(Mp + o);
        lo = *reinterpret_cast<const bf16x8 *>(Mp + static_cast<size_t>(2 * C) * MS + o);
    };
    auto m_frag_f = [&](int rt, int s, float (&a)[8]) {
        ld8f(reinterpret_cast<const float *>(Mp) + static_cast<size_t>(16 * rt + l16) * MS + 32 * s + 8 * kg, a);
    };
    Op *wq = reinterpret_cast<Op *>(pkg + p.L.wq);
    Op *kt = reinterpret_cast<Op *>(pkg + p.L.kt);
    constexpr int NJOBS = KSK + DV / 16;
    for (int job = w; job < NJOBS; job += NW) {
        if (job < KSK) {
            // channels 32 ks .. 32 ks + 31: W^T = Kg^T T'^T and Q'^T = Qg^T + Kg^T (-R)^T
            const int ks = job;
            bf16x8 ka_hi[2][KSC], ka_lo[2][KSC];
            float ka_f[2][KSC][8];
#pragma unroll
            for (int hc = 0; hc < 2; ++hc) {
                const int c = 32 * ks + 16 * hc + l16;
#pragma unroll
                for (int s = 0; s < KSC; ++s) {
                    float kgv[8], ktv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = 32 * s + 8 * kg + e;
                        kgv[e] = ktv[e] = 0.f;
                        if (c < DK && j < C) {
                            const float kk = Kf(j, c), gj = sG[j][c];
                            kgv[e] = sLru[j] < 0 ? kk * fast_exp2(gj) : 0.f;
                            ktv[e] = j >= last_reset ? kk * fast_exp2(sG[C - 1][c] - gj) : 0.f;
                        }
                    }
                    if (c < DK) {
                        const int ct = 2 * ks + hc;
                        store8(kt + ((static_cast<size_t>(ct) * KSC + s) * 64 + lane) * 8, ktv);
                    }
                    if constexpr (BF) split_bf16(kgv, ka_hi[hc][s], ka_lo[hc][s]);
                    else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) ka_f[hc][s][e] = kgv[e];
                    }
                }
            }
#pragma unroll 2
            for (int rt = 0; rt < 2 * NT16; ++rt) {
                const int I = rt < NT16 ? rt : rt - NT16;
                const int nks = (16 * I + 15) / 32 + 1;  // token steps with nonzeros
                f32x4 acc[2];
#pragma unroll
                for (int hc = 0; hc < 2; ++hc) {
                    acc[hc] = f32x4{0.f, 0.f, 0.f, 0.f};
                    const int c0 = 32 * ks + 16 * hc + 4 * kg;
                    if (rt >= NT16 && c0 < DK) {  // Q * Gamma for token 16 I + l16
                        const int i = 16 * I + l16;
                        if (sLru[i] < 0) {
                            const f32x4 gv = *reinterpret_cast<const f32x4 *>(&sG[i][c0]);
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[hc][r] = Qf(i, c0 + r) * fast_exp2(gv[r]);
                        }
                    }
                }
#pragma unroll
                for (int s = 0; s < KSC; ++s) {
                    if (s >= nks) break;
                    if constexpr (BF) {
                        bf16x8 mh, ml;
                        m_frag_bf(rt, s, mh, ml);
#pragma unroll
                        for (int hc = 0; hc < 2; ++hc) {
                            acc[hc] = mfma_bf16(ka_lo[hc][s], mh, acc[hc]);
                            acc[hc] = mfma_bf16(ka_hi[hc][s], ml, acc[hc]);
                            acc[hc] = mfma_bf16(ka_hi[hc][s], mh, acc[hc]);
                        }
                    } else {
                        float mf[8];
                        m_frag_f(rt, s, mf);
#pragma unroll
                        for (int hc = 0; hc < 2; ++hc) mma<Prec::F32>(acc[hc], ka_f[hc][s], mf);
                    }
                }
                float v8[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v8[r] = acc[0][r];
                    v8[4 + r] = acc[1][r];
                }
                store8(wq + ((static_cast<size_t>(rt) * KSK + ks) * 64 + lane) * 8, v8);
            }
        } else {
            // value columns 16 ct .. 16 ct + 15: [U'; -O_intra] = M V
            const int ct = job - KSK;
            const int c = 16 * ct + l16;
            float vb[KSC][8];
#pragma unroll
            for (int s = 0; s < KSC; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 32 * s + 8 * kg + e;
                    vb[s][e] = j < C ? Vf(j, c) : 0.f;
                }
            f32x4 *up = reinterpret_cast<f32x4 *>(pkg + p.L.up);
            f32x4 *oi = reinterpret_cast<f32x4 *>(pkg + p.L.oi);
#pragma unroll 2
            for (int rt = 0; rt < 2 * NT16; ++rt) {
                const int I = rt < NT16 ? rt : rt - NT16;
                const int nks = (16 * I + 15) / 32 + 1;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KSC; ++s) {
                    if (s >= nks) break;
                    if constexpr (BF) {
                        bf16x8 mh, ml;
                        m_frag_bf(rt, s, mh, ml);
                        const bf16x8 vv = pack_bf16(vb[s]);
                        acc = mfma_bf16(ml, vv, acc);
                        acc = mfma_bf16(mh, vv, acc);
                    } else {
                        float mf[8];
                        m_frag_f(rt, s, mf);
                        mma<Prec::F32>(acc, mf, vb[s]);
                    }
                }
                if (rt < NT16) up[(static_cast<size_t>(ct) * NT16 + I) * 64 + lane] = acc;
                else oi[(static_cast<size_t>(ct) * NT16 + I) * 64 + lane] = -acc;
            }
        }
    }
    float *glp = reinterpret_cast<float *>(pkg + p.L.gl);
    for (int c = tid; c < DK; c += kIntraThreads) glp[c] = last_reset >= 0 ? 0.f : fast_exp2(sG[C - 1][c]);
    if (n_items < 0) glp[0] = touch;  // never true: keeps the touch loads alive
      }  // cur.valid
    }
}

// -----------------------------------------------------------------------------
// sequential state pass: one workgroup per (sequence, head, 16-column slab)
// -----------------------------------------------------------------------------
// 8 matrix-core operand values of one lane: fp16 (bf16 path) or fp32.
template <bool BF>
struct Vec8;
template <>
struct Vec8<true> {
    f16x8 v;
};
template <>
struct Vec8<false> {
    f32x4 a, b;
};

template <bool BF>
__device__ __forceinline__ Vec8<BF> ld_vec8(const void *p) {
    Vec8<BF> r;
    if constexpr (BF) {
        r.v = *reinterpret_cast<const f16x8 *>(p);
    } else {
        r.a = reinterpret_cast<const f32x4 *>(p)[0];
        r.b = reinterpret_cast<const f32x4 *>(p)[1];
    }
    return r;
}

__device__ __forceinline__ void unpack8(const Vec8<false> &x, float (&o)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o[e] = x.a[e];
        o[4 + e] = x.b[e];
    }
}

// The part of one chunk's package a wave of the state pass consumes, held in
// registers so the next chunk's loads are in flight while this one computes.
// LR2: the DPLR form (kda_dplr.hip), whose state update adds a second
// low-rank term: the Kt section holds 2 CP tokens, [A-tilde; K-tilde], and the
// chunk's values V (the package's VX section) follow U in the contraction.
template <int C, int DK, int DV, bool BF, bool LR2 = false>
struct StateFrags {
    using F = Cfg<C, DK, DV, BF>;
    static constexpr int NTK = DK / 16, SPW = (NTK + 3) / 4;
    static constexpr int NRT = 2 * F::NT16, RPW = (NRT + 3) / 4;
    static constexpr int KSK = F::DKP / 32, KSC = F::CP / 32, PARTS = BF ? 2 : 1;  // U hi/lo
    static constexpr int KSC2 = LR2 ? 2 * KSC : KSC;
    Vec8<BF> wq[RPW][KSK];
    f32x4 uo[RPW];
    Vec8<BF> kt[SPW][KSC2];
    f32x4 gl[SPW];
    f32x4 vx[LR2 ? RPW : 1];  // LR2: V rows 16 rt + 4 (lane / 16) + r, column 16 ct + lane % 16

    __device__ __forceinline__ void load(const char *pkg, const PackageLayout &L, int w, int lane,
                                         int ct) {
        using Op = typename F::Op;
        constexpr int NT16 = F::NT16;
        const Op *wqp = reinterpret_cast<const Op *>(pkg + L.wq);
#pragma unroll
        for (int rw = 0; rw < RPW; ++rw) {
            const int rt = w + 4 * rw;
            if (NRT % 4 == 0 || rt < NRT) {  // compile-time true when tiles divide evenly
#pragma unroll
                for (int ks = 0; ks < KSK; ++ks)
                    wq[rw][ks] = ld_vec8<BF>(wqp + ((static_cast<size_t>(rt) * KSK + ks) * 64 + lane) * 8);
                const size_t off = rt < NT16 ? L.up : L.oi;
                const int I = rt < NT16 ? rt : rt - NT16;
                uo[rw] = reinterpret_cast<const f32x4 *>(pkg + off)[(static_cast<size_t>(ct) * NT16 + I) * 64 + lane];
                if constexpr (LR2) {
                    // V rows of tile I (bf16 on the 16-bit path); loaded for every
                    // row tile and kept for the U tiles only, so the load is not
                    // under a branch
                    const size_t vi = (static_cast<size_t>(ct) * NT16 + I) * 64 + lane;
                    f32x4 v;
                    if constexpr (BF) {
                        const uint2 r = reinterpret_cast<const uint2 *>(pkg + L.vx)[vi];
                        v = f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                                  __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
                    } else {
                        v = reinterpret_cast<const f32x4 *>(pkg + L.vx)[vi];
                    }
                    vx[rw] = rt < NT16 ? v : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
        const Op *ktp = reinterpret_cast<const Op *>(pkg + L.kt);
        const float *glp = reinterpret_cast<const float *>(pkg + L.gl);
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (NTK % 4 == 0 || tk < NTK) {
#pragma unroll
                for (int ks = 0; ks < KSC2; ++ks)
                    kt[sl][ks] = ld_vec8<BF>(ktp + ((static_cast<size_t>(tk) * KSC2 + ks) * 64 + lane) * 8);
                gl[sl] = *reinterpret_cast<const f32x4 *>(glp + 16 * tk + 4 * (lane >> 4));
            }
        }
    }
};

// SAVE: the saving variant (the backward's forward pass) writes the state
// entering each chunk to p.chunk_states and stores no output.  LR2: the DPLR
// form (see StateFrags).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf,
                                                                 true));
}
// orders a wave's own LDS accesses around a change of a buffer's role
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// sum over each group of four lanes, in every lane of the group
__device__ __forceinline__ float quad_sum(float x) {
    x += dpp_mov<0xb1>(x);    // quad_perm [1, 0, 3, 2]
    return x + dpp_mov<0x4e>(x);  // quad_perm [2, 3, 0, 1]
}

// The KDA layer's fused epilogue (LAYER): a row's sum of o^2 is spread over the
// eight slab workgroups of its head, so each writes its per-row partial sums
// into the workspace's row-norm exchange (one 64-bit word per row, the call's
// tag in the high half, written with a relaxed device-scope atomic store) and
// scales its own rows of the chunk kLayerLag chunk steps later, once the other
// slabs' words of that chunk carry the tag (read with relaxed device-scope
// atomic loads, which bypass L1).  The state passes' grid (state_grid) puts the
// eight slabs of a (sequence, head) unit on one XCD and next to each other in
// that XCD's dispatch order, so all eight are resident together whenever the
// XCD holds eight workgroups: no slab waits on one that cannot start.  Every
// wait is bounded; a wave whose wait runs out writes NaN rows from then on.
constexpr int kLayerLag = 4;             // chunk steps between writing and reading partials
constexpr int kLayerSpinLimit = 1 << 16; // polls of one chunk's partials before giving up

template <int C, int DK, int DV, bool BF, bool SAVE, bool LR2, bool LAYER = false>
__device__ __forceinline__ void state_body(const StateParams &p) {
    using F = Cfg<C, DK, DV, BF>;
    using Op = typename F::Op;
    using Frags = StateFrags<C, DK, DV, BF, LR2>;
    constexpr int NT16 = F::NT16, CP = F::CP, DKP = F::DKP;
    constexpr int NTK = Frags::NTK, SPW = Frags::SPW, NRT = Frags::NRT, RPW = Frags::RPW;
    constexpr int KSK = Frags::KSK, KSC = Frags::KSC2, PARTS = Frags::PARTS;
    constexpr int SSS = DKP + 8;                 // LDS strides (elements)
    constexpr int SUS = (LR2 ? 2 * CP : CP) + 8;

    __shared__ __align__(16) Op sS[16][SSS];          // state slab as a B operand [col][channel]
    __shared__ __align__(16) Op sU[PARTS][16][SUS];   // U (hi, lo) as a B operand [col][token]
    // LAYER: each wave's 16 x 16 tile of o, turned from the accumulator layout
    // (lane l: rows 4 (l / 16) .. + 3 of column l % 16) into rows of four
    // columns (lane l: row 4 (l / 16) + (l % 16) / 4, columns 4 (l % 4) .. + 3):
    // a row's partial sum is then a sum over four lanes, and the lane reads its
    // output gate and writes its output as one vector each
    __shared__ __align__(16) float sO[LAYER ? 4 : 1][16][16];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    const int H = p.H;
    static_assert(!LAYER || DV == 128, "the layer's eight 16-column slabs");
    int n, h, ct;
    if (!state_unit<DV / 16>(p.N, H, n, h, ct)) return;  // so are its siblings

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
    // this launch's chunks of the sequence: [cb, ce)
    const int64_t cb = p.s0 > slot_base ? p.s0 - slot_base : 0;
    const int64_t ce = p.s1 - slot_base < nchunks ? p.s1 - slot_base : nchunks;
    if (nchunks == 0 ? !p.do_empty : cb >= ce) return;
    auto pkg_of = [&](int64_t c) {
        return p.ws + (static_cast<size_t>(slot_base + c - p.s0) * H + h) * p.pkg_bytes;
    };

    for (int idx = tid; idx < 16 * SSS; idx += 256) (&sS[0][0])[idx] = static_cast<Op>(0.f);
    for (int idx = tid; idx < PARTS * 16 * SUS; idx += 256) (&sU[0][0][0])[idx] = static_cast<Op>(0.f);

    const int col = 16 * ct + l16;
    const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * DV;

    // LAYER: o of a chunk waits kLayerLag steps for the other slabs' partial
    // sums; this wave's 16 rows of it (o and the output gate's bf16 bits, in
    // the row layout of sO below) wait in a queue: entry i holds chunk
    // c - kLayerLag + i at step c, so no chunk index is kept
    constexpr int QN = LAYER ? kLayerLag : 1;
    f32x4 qov[QN];
    uint2 qg[QN];
#pragma unroll
    for (int i = 0; i < QN; ++i) {
        qov[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        qg[i] = uint2{0u, 0u};
    }
    bool gave_up = false;
    const int orow4 = 4 * kg + (l16 >> 2), ocol4 = 4 * (l16 & 3);  // this lane's row and columns of an o tile
    f32x4 w4 = {0.f, 0.f, 0.f, 0.f};  // LAYER: RMSNorm weights of those columns (none needed at T = 0)
    if constexpr (LAYER)
        if (p.norm_weight) w4 = *reinterpret_cast<const f32x4 *>(p.norm_weight + 16 * ct + ocol4);
    // the state entering chunk cb: the initial state, or the one carried in
    const float *s_in = cb == 0 ? (p.init_state ? p.init_state + sbase : nullptr)
                                : p.carry_in + static_cast<size_t>(h) * DK * DV;
    f32x4 S[SPW];
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl) {
        const int tk = w + 4 * sl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * tk + 4 * kg + r;
            S[sl][r] = (tk < NTK && s_in) ? s_in[static_cast<size_t>(row) * DV + col] : 0.f;
        }
    }
    __syncthreads();
    // The state slab is stored [col][channel] with the channel order of the WQ
    // fragments: within each 32-channel step, position 8 g + 4 half + r holds
    // channel 16 half + 4 g + r.
    auto put_state = [&]() {
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk < NTK) {
                const int pos = 32 * (tk >> 1) + 8 * kg + 4 * (tk & 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[l16][pos + r] = static_cast<Op>(S[sl][r]);
            }
        }
    };
    put_state();

    // LAYER: this lane's two partial-sum words of chunk c - kLayerLag, loaded
    // at the start of step c, before chunk c + 2's package, so that waiting for
    // them at the end of the step never waits for package loads still in flight
    uint64_t pwa = 0, pwb = 0;
    // (lane l: slabs 2 (l % 4) and 2 (l % 4) + 1 of its o row, 16 w + orow4)
    auto poll_words = [&](int64_t pc) {
        return p.norm_xchg + (static_cast<size_t>(slot_base + pc - p.s0) * H + h) * (norm_xchg_bytes(C, DV) / 8) +
               2 * (l16 & 3) * CP + 16 * w + orow4;
    };
    auto poll_issue = [&](int64_t c) {
        if constexpr (LAYER) {
            if (c - kLayerLag >= cb) {
                const uint64_t *np = poll_words(c - kLayerLag);
                pwa = __hip_atomic_load(np, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                pwb = __hip_atomic_load(np + CP, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    };

    // LAYER: scales and stores this wave's 16 rows of chunk pc once the eight
    // slabs' partial sums of that chunk are readable
    // (loaded: the words were loaded for this chunk at the start of the step;
    // otherwise they are loaded here)
    auto finish = [&](const f32x4 ov, const uint2 g, const int64_t pc, bool loaded) {
        const int I = w;  // the wave's Q' row tile is w + NT16
        const int64_t rem = L - pc * C;
        const int nv = static_cast<int>(rem < C ? rem : C);
        const uint64_t *np = poll_words(pc);
        uint64_t a = pwa, b = pwb;
        if (!gave_up) {
            for (int it = 0;; ++it) {
                if (!loaded || it > 0) {
                    if (it > 0) __builtin_amdgcn_s_sleep(2);
                    a = __hip_atomic_load(np, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    b = __hip_atomic_load(np + CP, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                const bool ok = static_cast<uint32_t>(a >> 32) == p.layer_tag &&
                                static_cast<uint32_t>(b >> 32) == p.layer_tag;
                if (__ballot(!ok) == 0) break;
                if (it >= kLayerSpinLimit) {
                    gave_up = true;
                    break;
                }
            }
        }
        const float ss = quad_sum(__uint_as_float(static_cast<uint32_t>(a)) + __uint_as_float(static_cast<uint32_t>(b)));
        const float rs = gave_up ? __builtin_nanf("") : 1.f / sqrtf(ss * (1.f / DV) + p.norm_eps);
        const float gv[4] = {__uint_as_float(g.x << 16), __uint_as_float(g.x & 0xffff0000u),
                             __uint_as_float(g.y << 16), __uint_as_float(g.y & 0xffff0000u)};
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = ov[e] * rs * w4[e] * sigmoid_f(gv[e]);
        const int row = 16 * I + orow4;
        if (row < nv) *reinterpret_cast<f32x4 *>(p.o + ((tok_base + pc * C + row) * H + h) * DV + 16 * ct + ocol4) = y;
    };

    // one chunk of the recurrence on this slab, operands from registers;
    // kPartial: the sequence's last chunk has fewer than C tokens (its o stores
    // are masked; full chunks store unconditionally so the hot loop has no
    // data-dependent branches around memory operations)
    auto step = [&](const Frags &f, int64_t c, auto partial_tag) {
        constexpr bool kPartial = decltype(partial_tag)::value;
        const int64_t rem = L - c * C;
        const int nvalid = static_cast<int>(rem < C ? rem : C);
        f32x4 cov = {0.f, 0.f, 0.f, 0.f};
        uint2 cg = {0u, 0u};
        if constexpr (SAVE) {
          if (p.chunk_states) {
            float *cs = p.chunk_states + (static_cast<size_t>(slot_base + c - p.s0) * H + h) * DK * DV;
#pragma unroll
            for (int sl = 0; sl < SPW; ++sl) {
                const int tk = w + 4 * sl;
                if (tk < NTK) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) cs[static_cast<size_t>(16 * tk + 4 * kg + r) * DV + col] = S[sl][r];
                }
            }
          }
        }
        __syncthreads();  // sS holds this chunk's incoming state

        // (a) [W; Q'] S0 for this wave's row tiles; U = U' - W S0, O = O_intra + Q' S0
#pragma unroll
        for (int rw = 0; rw < RPW; ++rw) {
            const int rt = w + 4 * rw;
            if (NRT % 4 != 0 && rt >= NRT) break;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSK; ++ks) {
                if constexpr (BF) {
                    const f16x8 b = *reinterpret_cast<const f16x8 *>(&sS[l16][32 * ks + 8 * kg]);
                    acc = mfma_f16(f.wq[rw][ks].v, b, acc);
                } else {
                    float a[8], b[8];
                    unpack8(f.wq[rw][ks], a);
#pragma unroll
                    for (int e = 0; e < 8; ++e) b[e] = sS[l16][32 * ks + 8 * kg + e];
                    mma<Prec::F32>(acc, a, b);
                }
            }
            if (rt < NT16) {
                const f32x4 u = f.uo[rw] - acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * rt + 4 * kg + r;
                    const Op hi = static_cast<Op>(u[r]);
                    sU[0][l16][j] = hi;
                    if constexpr (BF) sU[1][l16][j] = static_cast<Op>(u[r] - static_cast<float>(hi));
                    if constexpr (LR2) {
                        const float x = f.vx[rw][r];
                        const Op xh = static_cast<Op>(x);
                        sU[0][l16][CP + j] = xh;
                        if constexpr (BF) sU[1][l16][CP + j] = static_cast<Op>(x - static_cast<float>(xh));
                    }
                }
            } else if constexpr (LAYER) {
                // o in the row layout (sO); this slab's sum of o^2 per row,
                // published for the other slabs; o and the output gate wait in
                // the queue
                const int I = rt - NT16;
                const f32x4 ov = f.uo[rw] + acc;
                float(*t)[16] = sO[w];
#pragma unroll
                for (int r = 0; r < 4; ++r) t[4 * kg + r][l16] = ov[r];
                wave_lds_sync();
                const f32x4 o4 = *reinterpret_cast<const f32x4 *>(&t[orow4][ocol4]);
                const int row = 16 * I + orow4;  // o row of this lane in the chunk
                const float ps = quad_sum(o4[0] * o4[0] + o4[1] * o4[1] + o4[2] * o4[2] + o4[3] * o4[3]);
                if ((l16 & 3) == 0) {
                    uint64_t *np =
                        p.norm_xchg + (static_cast<size_t>(slot_base + c - p.s0) * H + h) * (norm_xchg_bytes(C, DV) / 8);
                    const uint64_t word = (static_cast<uint64_t>(p.layer_tag) << 32) | __float_as_uint(ps);
                    __hip_atomic_store(np + ct * CP + row, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                if (!kPartial || row < nvalid)
                    cg = *reinterpret_cast<const uint2 *>(p.out_gate + ((tok_base + c * C + row) * H + h) * DV +
                                                          16 * ct + ocol4);
                cov = o4;
            } else if constexpr (!SAVE) {
                const int I = rt - NT16;
                const f32x4 ov = f.uo[rw] + acc;
                float *orow = p.o + ((tok_base + c * C + 16 * I + 4 * kg) * H + h) * DV + col;
                if constexpr (!kPartial) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) orow[static_cast<size_t>(r) * H * DV] = ov[r];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (16 * I + 4 * kg + r < nvalid) orow[static_cast<size_t>(r) * H * DV] = ov[r];
                }
            }
        }
        __syncthreads();  // sU complete; all reads of sS done

        // (c) S1 = Diag(Gamma_last) S0 + Kt^T U for this wave's state tiles
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (NTK % 4 != 0 && tk >= NTK) break;
            f32x4 acc = f.gl[sl] * S[sl];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                if constexpr (BF) {
                    const f16x8 bh = *reinterpret_cast<const f16x8 *>(&sU[0][l16][32 * ks + 8 * kg]);
                    const f16x8 bl = *reinterpret_cast<const f16x8 *>(&sU[1][l16][32 * ks + 8 * kg]);
                    acc = mfma_f16(f.kt[sl][ks].v, bl, acc);
                    acc = mfma_f16(f.kt[sl][ks].v, bh, acc);
                } else {
                    float a[8], b[8];
                    unpack8(f.kt[sl][ks], a);
#pragma unroll
                    for (int e = 0; e < 8; ++e) b[e] = sU[0][l16][32 * ks + 8 * kg + e];
                    mma<Prec::F32>(acc, a, b);
                }
            }
            S[sl] = acc;
        }
        put_state();
        if constexpr (LAYER) {
            // chunk c - kLayerLag leaves the queue, chunk c joins it
            if (c - kLayerLag >= cb) finish(qov[0], qg[0], c - kLayerLag, true);
#pragma unroll
            for (int i = 0; i + 1 < QN; ++i) {
                qov[i] = qov[i + 1];
                qg[i] = qg[i + 1];
            }
            qov[QN - 1] = cov;
            qg[QN - 1] = cg;
        }
    };

    // software pipeline, three packages deep: chunk c + 2 loads while chunk c
    // computes (a ring of three register buffers, so no buffer is copied while
    // its loads are in flight)
    using Full = std::false_type;
    using Part = std::true_type;
    const int64_t nfull = L / C < ce ? L / C : ce;  // chunks with C valid tokens
    Frags f0, f1, f2;
    auto load = [&](Frags &f, int64_t cc) { f.load(pkg_of(cc), p.L, w, lane, ct); };
    if (ce > cb) load(f0, cb);
    if (ce > cb + 1) load(f1, cb + 1);
    int64_t c = cb;
    for (; c + 4 < nfull; c += 3) {  // chunks c .. c + 2 are full; c + 3 and c + 4 exist
        poll_issue(c);
        load(f2, c + 2);
        step(f0, c, Full{});
        poll_issue(c + 1);
        load(f0, c + 3);
        step(f1, c + 1, Full{});
        poll_issue(c + 2);
        load(f1, c + 4);
        step(f2, c + 2, Full{});
    }
    // tail: f0 holds chunk c and f1 chunk c + 1 (when it exists)
    for (; c < ce; ++c) {
        poll_issue(c);
        if (c + 2 < ce) load(f2, c + 2);
        if (c < nfull) step(f0, c, Full{});
        else step(f0, c, Part{});
        f0 = f1;
        f1 = f2;
    }

    if constexpr (LAYER) {  // the last chunks' rows, oldest first
        // chunks ce - kLayerLag .. ce - 1 (those that exist) are still queued
#pragma unroll
        for (int i = 0; i < QN; ++i)
            if (ce - QN + i >= cb) finish(qov[i], qg[i], ce - QN + i, false);
    }

    // the state leaving chunk ce - 1: the final state, or the one carried out
    float *s_out = ce == nchunks ? (p.final_state ? p.final_state + sbase : nullptr)
                                 : (p.carry_out ? p.carry_out + static_cast<size_t>(h) * DK * DV : nullptr);
    if (s_out) {
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk >= NTK) break;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * tk + 4 * kg + r;
                s_out[static_cast<size_t>(row) * DV + col] = S[sl][r];
            }
        }
    }
}

template <int C, int DK, int DV, bool BF, bool SAVE = false>
__global__ void __launch_bounds__(256) state_kernel(StateParams p) {
    state_body<C, DK, DV, BF, SAVE, false>(p);
}

// The KDA layer's state pass with its RMSNorm and output-gate epilogue fused
// (one-dimensional grid, see state_body).
__global__ void __launch_bounds__(256) layer_state_kernel(StateParams p) {
    state_body<64, 128, 128, true, false, false, true>(p);
}

template <int C, int DK, int DV, bool BF>
__global__ void __launch_bounds__(256) dplr_state_kernel(StateParams p) {
    state_body<C, DK, DV, BF, false, true>(p);
}

// -----------------------------------------------------------------------------
// launch
// -----------------------------------------------------------------------------

// The intra-chunk pass: the packages of chunk slots [s0, s1) (every head) into
// pkgs, slot s0's first (the prefill: every slot, into a.workspace).  The
// varlen plan is made only where plan is set.
template <int C, int DK, int DV, bool BF>
static hipError_t launch_intra_t(const PrefillArgs &a, hipStream_t stream, int64_t s0, int64_t s1, char *pkgs,
                                 bool plan) {
    const PackageLayout L = package_layout(C, DK, DV, BF);
    if (a.cu_seqlens && plan) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens, a.N, C,
                           a.chunk_offsets);
    }
    if (s1 > s0) {
        IntraParams ip{a.q, a.k, a.v, a.log_alpha, a.beta, a.cu_seqlens, a.chunk_offsets,
                       a.T, a.H, a.N, pkgs, a.pkg_bytes, L,
                       a.gate_mode == 1 ? 1 : DK, a.gate_mode == 1 ? 0 : 1,
                       a.gate_mode, a.x_alpha, a.x_beta, a.l2_eps, s0 * a.H};
        // persistent: a few workgroups per compute unit walk the (chunk, head)
        // items, each loading the next item's inputs while computing one
        const int64_t n_items = s1 * a.H;
        if constexpr (C == 64 && DK == 128 && DV == 128 && BF) {
            const hipError_t e = launch_intra_wide(ip, n_items, stream);
            if (e != hipSuccess) return e;
        } else {
        if (a.gate_mode == 2) return hipErrorInvalidValue;  // the layer runs on the wide kernel only
        static thread_local int per_cu = 0;  // resident workgroups per CU for this instantiation
        if (per_cu == 0) {
            int nb = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, intra_kernel<C, DK, DV, BF>, kIntraThreads, 0) !=
                    hipSuccess || nb <= 0)
                nb = 1;
            per_cu = nb;
        }
        const int64_t grid = std::min<int64_t>((s1 - s0) * a.H, static_cast<int64_t>(device_cu_count()) * per_cu);
        hipLaunchKernelGGL((intra_kernel<C, DK, DV, BF>), dim3(static_cast<unsigned>(grid)), dim3(kIntraThreads), 0,
                           stream, ip, n_items);
        }
    }
    return hipSuccess;
}

template <int C, int DK, int DV, bool BF>
static hipError_t launch_t(const PrefillArgs &a, hipStream_t stream) {
    const hipError_t ei = launch_intra_t<C, DK, DV, BF>(a, stream, 0, a.n_slots, a.workspace, true);
    if (ei != hipSuccess) return ei;
    StateParams sp{a.init_state, a.cu_seqlens, a.chunk_offsets, a.o, a.final_state, nullptr,
                   a.T, a.H, a.N, a.workspace, a.pkg_bytes, package_layout(C, DK, DV, BF)};
    if constexpr (C == 64 && DK == 128 && DV == 128 && BF) {
        if (a.gate_mode == 2) {
            sp.out_gate = a.out_gate;
            sp.norm_weight = a.norm_weight;
            sp.norm_eps = a.norm_eps;
            sp.layer_tag = a.layer_tag;
            sp.norm_xchg = reinterpret_cast<uint64_t *>(a.norm_xchg);
            if (a.T > 0 && (sp.norm_xchg == nullptr || sp.out_gate == nullptr || sp.norm_weight == nullptr))
                return hipErrorInvalidValue;
            dim3 grid;
            if (!state_grid(a.N, a.H, DV, grid)) return hipErrorInvalidValue;
            hipLaunchKernelGGL(layer_state_kernel, grid, dim3(256), 0, stream, sp);
            return hipGetLastError();
        }
    }
    if (a.gate_mode == 2) return hipErrorInvalidValue;  // the layer runs at C = 64, d = 128, bf16 only
    dim3 grid;
    if (!state_grid(a.N, a.H, DV, grid)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((state_kernel<C, DK, DV, BF>), grid, dim3(256), 0, stream, sp);
    return hipGetLastError();
}

template <int C, int DK, int DV, bool BF>
hipError_t launch_forward_segment(const PrefillArgs &a, const FwdSegment &g, hipStream_t stream) {
    if (g.intra) {
        const hipError_t ei = launch_intra_t<C, DK, DV, BF>(a, stream, g.s0, g.s1, g.pkgs, g.plan);
        if (ei != hipSuccess) return ei;
    }
    StateParams sp{a.init_state, a.cu_seqlens, a.chunk_offsets, nullptr, nullptr, g.chunk_states,
                   a.T, a.H, a.N, g.pkgs, a.pkg_bytes, package_layout(C, DK, DV, BF),
                   g.s0, g.s1, g.carry_in, g.carry_out, g.do_empty};
    dim3 grid;
    if (!state_grid(a.N, a.H, DV, grid)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((state_kernel<C, DK, DV, BF, true>), grid, dim3(256), 0, stream, sp);
    return hipGetLastError();
}
template <int C, int D, bool BF>
hipError_t launch_dplr_state(const StateParams &sp, hipStream_t stream) {
    dim3 grid;
    if (!state_grid(sp.N, sp.H, D, grid)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dplr_state_kernel<C, D, D, BF>), grid, dim3(256), 0, stream, sp);
    return hipGetLastError();
}
#define KDA_DPLR_STATE(C, D) \
    template hipError_t launch_dplr_state<C, D, true>(const StateParams &, hipStream_t); \
    template hipError_t launch_dplr_state<C, D, false>(const StateParams &, hipStream_t);
KDA_DPLR_STATE(16, 16) KDA_DPLR_STATE(16, 32) KDA_DPLR_STATE(16, 64) KDA_DPLR_STATE(16, 128)
KDA_DPLR_STATE(32, 16) KDA_DPLR_STATE(32, 32) KDA_DPLR_STATE(32, 64) KDA_DPLR_STATE(32, 128)
KDA_DPLR_STATE(64, 16) KDA_DPLR_STATE(64, 32) KDA_DPLR_STATE(64, 64)
template hipError_t launch_dplr_state<64, 128, true>(const StateParams &, hipStream_t);
#undef KDA_DPLR_STATE

// the shapes the backward supports: d_k = d_v, the chunk the forward uses
#define KDA_FWD_STATES(C, D, BF) \
    template hipError_t launch_forward_segment<C, D, D, BF>(const PrefillArgs &, const FwdSegment &, hipStream_t);
KDA_FWD_STATES(16, 16, true) KDA_FWD_STATES(16, 32, true) KDA_FWD_STATES(16, 64, true) KDA_FWD_STATES(16, 128, true)
KDA_FWD_STATES(32, 16, true) KDA_FWD_STATES(32, 32, true) KDA_FWD_STATES(32, 64, true) KDA_FWD_STATES(32, 128, true)
KDA_FWD_STATES(64, 16, true) KDA_FWD_STATES(64, 32, true) KDA_FWD_STATES(64, 64, true) KDA_FWD_STATES(64, 128, true)
KDA_FWD_STATES(16, 16, false) KDA_FWD_STATES(16, 32, false) KDA_FWD_STATES(16, 64, false) KDA_FWD_STATES(16, 128, false)
KDA_FWD_STATES(32, 16, false) KDA_FWD_STATES(32, 32, false) KDA_FWD_STATES(32, 64, false) KDA_FWD_STATES(32, 128, false)
KDA_FWD_STATES(64, 16, false) KDA_FWD_STATES(64, 32, false) KDA_FWD_STATES(64, 64, false)
#undef KDA_FWD_STATES

template <int C, int DK, bool BF>
static hipError_t dispatch_dv(const PrefillArgs &a, hipStream_t s) {
    // the fp32 path holds q, k, v and the decay in fp32 in LDS: 64-token chunks
    // with d_k or d_v = 128 do not fit (prefill_effective_chunk maps them to 32)
    switch (a.Dv) {
        case 16: return launch_t<C, DK, 16, BF>(a, s);
        case 32: return launch_t<C, DK, 32, BF>(a, s);
        case 64: return launch_t<C, DK, 64, BF>(a, s);
        case 128:
            if constexpr (BF || C <= 32) return launch_t<C, DK, 128, BF>(a, s);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <int C, bool BF>
static hipError_t dispatch_d(const PrefillArgs &a, hipStream_t s) {
    switch (a.Dk) {
        case 16: return dispatch_dv<C, 16, BF>(a, s);
        case 32: return dispatch_dv<C, 32, BF>(a, s);
        case 64: return dispatch_dv<C, 64, BF>(a, s);
        case 128:
            if constexpr (BF || C <= 32) return dispatch_dv<C, 128, BF>(a, s);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
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
