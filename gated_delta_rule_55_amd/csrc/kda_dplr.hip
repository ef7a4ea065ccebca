// kda_dplr.hip -- chunked prefill of the general diagonal-plus-low-rank (DPLR)
// recurrence on gfx950.
//
//   S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
//
// is the general form the section "Kimi Delta Attention (KDA)" of the page
// "Kimi Linear 高效注意力架构" sets KDA against (its bullet on the
// hardware-efficient chunked algorithm: tying both low-rank vectors to the key
// removes work and about halves kernel time; KDA is a = -beta k,
// b = alpha * k, v -> beta v).  Per chunk, with incoming state S0, per-channel
// G_i = sum_{m<=i} log alpha_m and Gb_i = G_{i-1} (Gb_0 = 0), the low-rank
// readouts u_i = b_i^T S_{i-1} satisfy
//
//   u_i  = (b_i e^{Gb_i})^T S0 + sum_{j<i} Aab_ij u_j + sum_{j<i} Abk_ij v_j
//   Aab_ij = sum_c b_ic a_jc e^{Gb_ic - G_jc},   Abk_ij the same with k_j,
//
// so with T = (I - Aab)^-1 and X = B e^{Gb}:  U = W S0 + U',  W = T X,
// U' = T Abk V, and
//
//   O  = Q' S0 + O_intra,   Q' = Q e^{G} + Pqa W,   O_intra = (Pqa T Abk + Pqk) V
//   S1 = Diag(e^{G_last}) S0 + At^T U + Kt^T V,   At_j = a_j e^{G_last - G_j}
//   Pqa_ij = sum_c q_ic a_jc e^{G_ic - G_jc} (j <= i),   Pqk with k_j, Kt with k_j.
//
// Against KDA's chunk that is four decayed Gram matrices instead of two, three
// products of C x C matrices instead of one, and a state update of rank 2C
// instead of C.  dplr_intra_kernel writes one package per (chunk, head) in the
// layouts of the KDA state pass, which then walks the chunks in its DPLR form
// (W stored negated; [At; Kt] against [U; V] as one contraction over 2C tokens,
// V from the package's VX section).
//
// Gram matrices: 16x16 block pairs with a reference token m,
// e^{x_i - G_j} = e^{x_i - G_m} e^{G_m - G_j}: below the diagonal m is the last
// token of the column block (both factors <= 1), on it the block's token 7
// (factors <= e^30; channels spanning more are added with the exact exponential
// per pair).  On the 16-bit path (d >= 32) the Gram blocks, and (C >= 32) the
// package's products against X and V, are bf16 hi/lo matrix-core products (V is
// exact in bf16, so only its partner is split); the fp32 path keeps fp32
// matrix cores below the diagonal and the exact exponential per pair on it.
// T and the C x C products run on the fp32 matrix cores on both paths, and all
// accumulation is fp32.  A token whose log_alpha is -inf on
// every channel zeroes the diagonal part of its transition but not the
// low-rank part: it adds 0 to G, and the couplings it cuts are masked (Aab, Abk
// and X through a reset strictly before token i; P, At, Kt through one in
// (j, i]).  Other -inf values are clamped to -88.
#include <algorithm>

#include "kda_prefill.h"

namespace kda {
namespace {

constexpr int kDplrThreads = 512;  // 8 waves
// half-span of the cumulative decay around a diagonal block's reference token
// up to which that block goes through the matrix cores: e^30, in the kernel's
// base-2 units of G
constexpr float kDplrDiagSpan = 30.0f * kLog2e;
constexpr int kDplrWaves = kDplrThreads / 64;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

struct DplrIntraParams {
    const void *q, *k, *v, *a, *b;
    const float *log_alpha;
    const int32_t *cu_seqlens, *chunk_offsets;
    int64_t T;
    int32_t H, N;
    char *ws;
    size_t pkg_bytes;
    PackageLayout L;
};

template <bool BF>
__device__ __forceinline__ float ld_in(const void *p, int64_t i) {
    if constexpr (BF) return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    else return static_cast<const float *>(p)[i];
}

// Elements i .. i + 3 of an input (i a multiple of 4): one 8-byte (bf16) or
// 16-byte (fp32) load.
template <bool BF>
__device__ __forceinline__ f32x4 ld_in4(const void *p, int64_t i) {
    if constexpr (BF) {
        const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
        return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
    } else {
        return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p) + i);
    }
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += A B for one 16x16 tile over K = 16 (one 16-wide block of the
// contraction): a(r, k) = A[r][k], b(k, n) = B[k][n]; lane l supplies row /
// column l % 16 at k = 4 s + l / 16 and holds C[4 (l / 16) + r][l % 16].
template <typename FA, typename FB>
__device__ __forceinline__ void mm16(f32x4 &acc, FA &&a, FB &&b, int lane) {
    const int r = lane & 15, kk = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma4(a(r, 4 * s + kk), b(4 * s + kk, r), acc);
}

template <int C, int D, bool BF>
__global__ void __launch_bounds__(kDplrThreads) dplr_intra_kernel(DplrIntraParams p) {
    using F = Cfg<C, D, D, BF>;
    using Op = typename F::Op;
    constexpr int NTI = C / 16, NTD = D / 16, CP = F::CP, DKP = F::DKP;
    constexpr int KSC2 = 2 * (CP / 32), KSK = DKP / 32;
    constexpr int GS = D + 4, MS = C + 4;  // rows 16-byte aligned
    constexpr int NSB = NTI * 10;  // 4x4 sub-blocks on or below the diagonal of the diagonal blocks
    constexpr int NQ = D / 16 < 8 ? D / 16 < 1 ? 1 : D / 16 : 8;  // channel parts per sub-block
    constexpr int CQ = D / NQ;
    static_assert(NTI <= 4, "one wave per row / column tile of a chunk");
    static_assert(NSB * NQ <= kDplrThreads && 64 % NQ == 0 && CQ % 4 == 0, "diagonal work layout");

    // the package's products on the 16-bit path: bf16 matrix cores with the
    // four C x C matrices as hi/lo planes, 32 tokens per step
    constexpr bool kPk16 = BF && C % 32 == 0;
    constexpr int MP = C + 8;  // bf16 row stride of the hi/lo planes (16-byte rows)
    constexpr size_t kMF = sizeof(float) * 4 * C * MS, kMB = kPk16 ? sizeof(__bf16) * 8 * C * MP : 0;
    __shared__ __align__(16) float sG[C][GS];  // G, cumulative log-decay in base 2 (log2 e times the natural one)
    constexpr bool kGram16 = BF && D >= 32;  // the bf16 matrix-core Gram path
    // alpha_i = e^{G_i - G_{i-1}} (16-bit Gram path): q's factor is b's times alpha_i
    __shared__ __align__(16) float sAl[kGram16 ? C : 1][GS];
    // -Aab -> T, Abk -> T Abk, Pqa -> Pqa T, Pqk -> Pqa T Abk + Pqk (fp32); on the
    // 16-bit path overlaid at the end by the same four as bf16 hi/lo planes
    __shared__ __align__(16) unsigned char sMraw[kMF > kMB ? kMF : kMB];
    auto sM = reinterpret_cast<float (*)[C][MS]>(sMraw);
    __bf16 *Mp = reinterpret_cast<__bf16 *>(sMraw);  // plane 2 m + (0 hi, 1 lo) of matrix m: C x MP
    constexpr int NSEG = kDplrThreads / D < C / 4 ? kDplrThreads / D : C / 4, RPS = C / NSEG;
    __shared__ float sSeg[NSEG][D];  // per-segment decay sums of the scan
    __shared__ int sRst[C], sCnt[C];
    __shared__ int sLast;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    const int H = p.H;
    int64_t slot, hh;
    divmod_nonneg(static_cast<int64_t>(blockIdx.x), H, slot, hh);
    const int h = static_cast<int>(hh);
    int64_t tok0;
    int nvalid;
    if (!locate_chunk(slot, C, p.T, p.N, p.cu_seqlens, p.chunk_offsets, tok0, nvalid)) return;
    char *pkg = p.ws + static_cast<size_t>(blockIdx.x) * p.pkg_bytes;
    // Inputs of token i (0 for i >= nvalid).  The load itself is unconditional,
    // from a row inside the chunk, and the value selected after it: a load
    // under a branch gets a wait of its own before the branch rejoins, which
    // would serialise every load of the loops below.
    auto row = [&](int i) { return ((tok0 + (i < nvalid ? i : nvalid - 1)) * H + h) * D; };
    auto in = [&](const void *x, int i, int c) {
        const float v = ld_in<BF>(x, row(i) + c);
        return i < nvalid ? v : 0.f;
    };
    auto in4 = [&](const void *x, int i, int c) {  // channels c .. c + 3 of token i
        const f32x4 v = ld_in4<BF>(x, row(i) + c);
        return i < nvalid ? v : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // the same split in two: the raw load (one 8-byte bf16 or 16-byte fp32
    // vector, held while a loop step computes) and its widening
    using Raw4 = std::conditional_t<BF, uint2, f32x4>;
    auto raw4 = [&](const void *x, int i, int c) {
        if constexpr (BF) return *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + row(i) + c);
        else return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(x) + row(i) + c);
    };
    auto widen4 = [&](const Raw4 &r, int i) {
        f32x4 v;
        if constexpr (BF)
            v = f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
                      __uint_as_float(r.y & 0xffff0000u)};
        else v = r;
        return i < nvalid ? v : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    auto g4 = [&](int i, int c) {  // G[i][c .. c + 3], G[-1] = 0
        return i >= 0 ? *reinterpret_cast<const f32x4 *>(&sG[i][c]) : f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // The first Gram job of this wave (a block pair below the diagonal, else
    // its diagonal block) has its first channel step of b, q, a, k loaded now,
    // ahead of the decay scan (16-bit Gram path).
    constexpr int NPAIR = NTI * (NTI - 1) / 2;
    static_assert(NPAIR <= kDplrWaves && NTI <= kDplrWaves, "at most one job of each kind per wave");
    const bool has_pair = kDplrWaves - 1 - w < NPAIR;
    uint4 pre[4];
    if constexpr (BF && D >= 32) {
        int fI = w < NTI ? w : 0, fJ = fI;
        if (has_pair) {
            fI = 1;
            fJ = kDplrWaves - 1 - w;
            while (fJ >= fI) {
                fJ -= fI;
                ++fI;
            }
        }
        const int c = 8 * kg;
        pre[0] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.b) + row(16 * fI + l16) + c);
        pre[1] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.q) + row(16 * fI + l16) + c);
        pre[2] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.a) + row(16 * fJ + l16) + c);
        pre[3] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.k) + row(16 * fJ + l16) + c);
    }

    // ---- cumulative decay and resets (the chunk's log_alpha in 16-byte
    //      vectors, every load issued before the first is used)
    {
        constexpr int NV = C * D / 4, NL = (NV + kDplrThreads - 1) / kDplrThreads;
        f32x4 la[NL];
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int x = 4 * (tid + kDplrThreads * u), i = (x < C * D ? x : 0) / D, c = (x < C * D ? x : 0) % D;
            la[u] = *reinterpret_cast<const f32x4 *>(p.log_alpha + row(i) + c);
        }
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int x = 4 * (tid + kDplrThreads * u), i = x / D, c = x % D;
            if (x < C * D) *reinterpret_cast<f32x4 *>(&sG[i][c]) = i < nvalid ? la[u] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    for (int i = tid; i < C; i += kDplrThreads) sRst[i] = i < nvalid ? 1 : 0;
    for (int x = tid; x < 4 * C * MS; x += kDplrThreads) (&sM[0][0][0])[x] = 0.f;
    __syncthreads();
    for (int x = tid; x < C * D; x += kDplrThreads) {
        const int i = x / D, c = x % D;
        if (i < nvalid && sG[i][c] != kNegInf) sRst[i] = 0;
    }
    __syncthreads();
    // the scan in NSEG segments of RPS tokens per channel, then the segments' offsets
    const int sc = tid % D, sseg = tid / D;
    if (sseg < NSEG) {
        float acc = 0.f;
        for (int r = 0; r < RPS; ++r) {
            const int i = sseg * RPS + r;
            const float dg = sRst[i] ? 0.f : fmaxf(sG[i][sc], kGFloor) * kLog2e;
            if constexpr (kGram16) sAl[i][sc] = fast_exp2(dg);
            acc += dg;
            sG[i][sc] = acc;
        }
        sSeg[sseg][sc] = acc;
    }
    if (w == kDplrWaves - 1) {  // reset counts by one wave-wide ballot (C <= 64 tokens)
        const unsigned long long rm = __ballot(lane < C && sRst[lane] != 0);
        if (lane < C) sCnt[lane] = __popcll(rm & ((2ull << lane) - 1ull));
        if (lane == 0) sLast = rm ? 63 - __clzll(rm) : -1;
    }
    __syncthreads();
    if (sseg > 0 && sseg < NSEG) {
        float off = 0.f;
        for (int q = 0; q < sseg; ++q) off += sSeg[q][sc];
        for (int r = 0; r < RPS; ++r) sG[sseg * RPS + r][sc] += off;
    }
    __syncthreads();
    auto cnt_before = [&](int i) { return sCnt[i] - sRst[i]; };  // resets at tokens < i

    // One Gram block pair (I, J) on the 16-bit path with bf16 hi/lo matrix-core
    // products (three per K step of 32 channels, about 16 significant bits per
    // operand as the KDA Gram tiles): rows i = 16 I + l16 of the left operands
    // b e^{Gb_i - G_m} and q e^{G_i - G_m}, columns j = 16 J + l16 of the right
    // ones a e^{G_m - G_j} and k e^{G_m - G_j}.  Below the diagonal m is the last
    // token of J; on it (kDiag) m is the block's token 7, and channels whose span
    // around m exceeds kDplrDiagSpan are left out (zero operands) and reported
    // in `unsafe` (bit c % 32 of word c / 32).  Each lane loads 8 consecutive
    // channels of its token as one 16-byte vector, the next step's while one
    // computes.
    auto gram16 = [&](int I, int J, auto diag_tag, auto pre_tag, f32x4 &aab, f32x4 &abk, f32x4 &pqa,
                      f32x4 &pqk, uint32_t (&unsafe)[4]) {
        constexpr bool kDiag = decltype(diag_tag)::value, kPre = decltype(pre_tag)::value;
        const int m = kDiag ? 16 * J + 7 : 16 * J + 15, i = 16 * I + l16, j = 16 * J + l16;
        auto raw8 = [&](const void *x, int ii, int c) {
            return *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + row(ii) + c);
        };
        // (tokens past nvalid read the last valid row; their Gram entries are
        // zeroed where the blocks are stored)
        auto widen8 = [&](const uint4 &r, float (&v)[8]) {
            const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                v[2 * q2] = __uint_as_float(wd[q2] << 16);
                v[2 * q2 + 1] = __uint_as_float(wd[q2] & 0xffff0000u);
            }
        };
        uint4 rb[2], rq[2], ra[2], rk[2];
        auto issue = [&](int st, int sl) {
            const int c = 32 * st + 8 * kg;
            rb[sl] = raw8(p.b, i, c);
            rq[sl] = raw8(p.q, i, c);
            ra[sl] = raw8(p.a, j, c);
            rk[sl] = raw8(p.k, j, c);
        };
        if constexpr (kPre) {  // step 0 loaded at the start of the kernel
            rb[0] = pre[0];
            rq[0] = pre[1];
            ra[0] = pre[2];
            rk[0] = pre[3];
        } else {
            issue(0, 0);
        }
#pragma unroll
        for (int st = 0; st < D / 32; ++st) {
            if (st + 1 < D / 32) issue(st + 1, (st + 1) & 1);
            const int c = 32 * st + 8 * kg;  // this lane's channels c .. c + 7
            float bv[8], qv[8], av[8], kv[8];
            widen8(rb[st & 1], bv);
            widen8(rq[st & 1], qv);
            widen8(ra[st & 1], av);
            widen8(rk[st & 1], kv);
            float lb[8], lq[8], xa[8], xk[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int c4 = c + 4 * hh;
                const f32x4 gm = g4(m, c4), gbi = g4(i - 1, c4), gj = g4(j, c4);
                const f32x4 al = *reinterpret_cast<const f32x4 *>(&sAl[i][c4]);
                f32x4 gfirst = gm, glast = gm;
                if constexpr (kDiag) {
                    gfirst = g4(16 * J - 1, c4);
                    glast = g4(16 * J + 15, c4);
                }
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int e = 4 * hh + e4;
                    bool safe = true;
                    if constexpr (kDiag) {
                        safe = gfirst[e4] - gm[e4] <= kDplrDiagSpan && gm[e4] - glast[e4] <= kDplrDiagSpan;
                        const uint64_t ub = __ballot(!safe);  // lanes 16 g: channel 32 st + 8 g + e
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            if ((ub >> (16 * g)) & 1u) {
                                const int ch = 32 * st + 8 * g + e;
                                unsafe[ch >> 5] |= 1u << (ch & 31);
                            }
                    }
                    const float e3 = safe ? fast_exp2(gm[e4] - gj[e4]) : 0.f;
                    const float fb = safe ? fast_exp2(gbi[e4] - gm[e4]) : 0.f;
                    lb[e] = bv[e] * fb;
                    lq[e] = qv[e] * (fb * al[e4]);
                    xa[e] = av[e] * e3;
                    xk[e] = kv[e] * e3;
                }
            }
            bf16x8 lbh, lbl, lqh, lql, xah, xal, xkh, xkl;
            split_bf16(lb, lbh, lbl);
            split_bf16(lq, lqh, lql);
            split_bf16(xa, xah, xal);
            split_bf16(xk, xkh, xkl);
            aab = mfma_bf16(lbl, xah, aab);
            aab = mfma_bf16(lbh, xal, aab);
            aab = mfma_bf16(lbh, xah, aab);
            abk = mfma_bf16(lbl, xkh, abk);
            abk = mfma_bf16(lbh, xkl, abk);
            abk = mfma_bf16(lbh, xkh, abk);
            pqa = mfma_bf16(lql, xah, pqa);
            pqa = mfma_bf16(lqh, xal, pqa);
            pqa = mfma_bf16(lqh, xah, pqa);
            pqk = mfma_bf16(lql, xkh, pqk);
            pqk = mfma_bf16(lqh, xkl, pqk);
            pqk = mfma_bf16(lqh, xkh, pqk);
        }
    };

    // ---- Gram blocks below the diagonal, one 16x16 block pair per wave
    {
        // (the last waves first: the diagonal work below fills the first ones)
        for (int pr = kDplrWaves - 1 - w; pr < NPAIR; pr += kDplrWaves) {
            int I = 1, J = pr;
            while (J >= I) {
                J -= I;
                ++I;
            }
            const int m = 16 * J + 15, i = 16 * I + l16, j = 16 * J + l16;
            f32x4 aab = {0.f, 0.f, 0.f, 0.f}, abk = aab, pqa = aab, pqk = aab;
            if constexpr (kGram16) {
                uint32_t none[4] = {0u, 0u, 0u, 0u};
                gram16(I, J, std::false_type{}, std::true_type{}, aab, abk, pqa, pqk, none);
            } else {
            // the next step's b, q, a, k are loaded while one computes
            Raw4 rb[2], rq[2], ra4[2], rk4[2];
            auto issue = [&](int t, int sl) {
                const int c = 16 * t + 4 * kg;
                rb[sl] = raw4(p.b, i, c);
                rq[sl] = raw4(p.q, i, c);
                ra4[sl] = raw4(p.a, j, c);
                rk4[sl] = raw4(p.k, j, c);
            };
            issue(0, 0);
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
                if (t + 1 < D / 16) issue(t + 1, (t + 1) & 1);
                const int c = 16 * t + 4 * kg;  // this lane's channels c .. c + 3
                const f32x4 gm = g4(m, c), gbi = g4(i - 1, c), gi = g4(i, c), gj = g4(j, c);
                const f32x4 bv = widen4(rb[t & 1], i), qv = widen4(rq[t & 1], i), av = widen4(ra4[t & 1], j),
                            kv = widen4(rk4[t & 1], j);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float e3 = fast_exp2(gm[e] - gj[e]);
                    const float lb = bv[e] * fast_exp2(gbi[e] - gm[e]), lq = qv[e] * fast_exp2(gi[e] - gm[e]);
                    const float ra = av[e] * e3, rk = kv[e] * e3;
                    aab = mfma4(lb, ra, aab);
                    abk = mfma4(lb, rk, abk);
                    pqa = mfma4(lq, ra, pqa);
                    pqk = mfma4(lq, rk, pqk);
                }
            }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ii = 16 * I + 4 * kg + r;
                const bool live = ii < nvalid && j < nvalid;
                const bool okA = live && cnt_before(ii) == sCnt[j], okP = live && sCnt[ii] == sCnt[j];
                sM[0][ii][j] = okA ? -aab[r] : 0.f;
                sM[1][ii][j] = okA ? abk[r] : 0.f;
                sM[2][ii][j] = okP ? pqa[r] : 0.f;
                sM[3][ii][j] = okP ? pqk[r] : 0.f;
            }
        }
    }
    // ---- diagonal blocks on the 16-bit path: on the matrix cores as the blocks
    //      below, one wave per block, with the block's token 7 as the reference
    //      m (e^{x_i - G_j} = e^{x_i - G_m} e^{G_m - G_j}, both factors at most
    //      e^{kDplrDiagSpan}); a channel whose cumulative decay spans more than
    //      that on either side of m is left out of the products (zero operands)
    //      and added exactly afterwards.  The entries above the diagonal come
    //      out finite and are masked.
    if constexpr (BF) {
        for (int J = w; J < NTI; J += kDplrWaves) {
            const int m = 16 * J + 7, i = 16 * J + l16, j = i;
            f32x4 aab = {0.f, 0.f, 0.f, 0.f}, abk = aab, pqa = aab, pqk = aab;
            uint32_t unsafe[4] = {0u, 0u, 0u, 0u};  // bit c % 32 of word c / 32: channel c
            if constexpr (kGram16) {
                if (has_pair) gram16(J, J, std::true_type{}, std::false_type{}, aab, abk, pqa, pqk, unsafe);
                else gram16(J, J, std::true_type{}, std::true_type{}, aab, abk, pqa, pqk, unsafe);
            } else {
            Raw4 rb[2], rq[2], ra4[2], rk4[2];
            auto issue = [&](int t, int sl) {
                const int c = 16 * t + 4 * kg;
                rb[sl] = raw4(p.b, i, c);
                rq[sl] = raw4(p.q, i, c);
                ra4[sl] = raw4(p.a, j, c);
                rk4[sl] = raw4(p.k, j, c);
            };
            issue(0, 0);
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
                if (t + 1 < D / 16) issue(t + 1, (t + 1) & 1);
                const int c = 16 * t + 4 * kg;  // this lane's channels c .. c + 3
                const f32x4 gm = g4(m, c), gfirst = g4(16 * J - 1, c), glast = g4(16 * J + 15, c);
                const f32x4 gbi = g4(i - 1, c), gi = g4(i, c), gj = g4(j, c);
                const f32x4 bv = widen4(rb[t & 1], i), qv = widen4(rq[t & 1], i), av = widen4(ra4[t & 1], j),
                            kv = widen4(rk4[t & 1], j);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool safe = gfirst[e] - gm[e] <= kDplrDiagSpan && gm[e] - glast[e] <= kDplrDiagSpan;
                    const float e3 = safe ? fast_exp2(gm[e] - gj[e]) : 0.f;
                    const float lb = safe ? bv[e] * fast_exp2(gbi[e] - gm[e]) : 0.f;
                    const float lq = safe ? qv[e] * fast_exp2(gi[e] - gm[e]) : 0.f;
                    const float ra = av[e] * e3, rk = kv[e] * e3;
                    aab = mfma4(lb, ra, aab);
                    abk = mfma4(lb, rk, abk);
                    pqa = mfma4(lq, ra, pqa);
                    pqk = mfma4(lq, rk, pqk);
                    const uint64_t ub = __ballot(!safe);  // lanes 16 g: channel 16 t + 4 g + e
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        if ((ub >> (16 * g)) & 1u) {
                            const int ch = 16 * t + 4 * g + e;
                            unsafe[ch >> 5] |= 1u << (ch & 31);
                        }
                }
            }
            }
            // rare: the left-out channels, exact decay per term
#pragma unroll
            for (int word = 0; word < 4; ++word) {
                uint32_t bits = unsafe[word];
                while (bits) {
                    const int ch = 32 * word + __builtin_ctz(bits);
                    bits &= bits - 1u;
                    const float aj = in(p.a, j, ch), kj = in(p.k, j, ch);
                    const float gjc = sG[j][ch];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int ii = 16 * J + 4 * kg + r;
                        const float bi = in(p.b, ii, ch), qi = in(p.q, ii, ch);
                        const float gbc = ii > 0 ? sG[ii - 1][ch] : 0.f;
                        const float eA = fast_exp2(fminf(gbc - gjc, 0.f)), eP = fast_exp2(fminf(sG[ii][ch] - gjc, 0.f));
                        aab[r] += bi * aj * eA;
                        abk[r] += bi * kj * eA;
                        pqa[r] += qi * aj * eP;
                        pqk[r] += qi * kj * eP;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ii = 16 * J + 4 * kg + r;
                const bool live = ii < nvalid && j < nvalid;
                const bool okA = live && j < ii && cnt_before(ii) == sCnt[j];
                const bool okP = live && j <= ii && sCnt[ii] == sCnt[j];
                sM[0][ii][j] = okA ? -aab[r] : 0.f;
                sM[1][ii][j] = okA ? abk[r] : 0.f;
                sM[2][ii][j] = okP ? pqa[r] : 0.f;
                sM[3][ii][j] = okP ? pqk[r] : 0.f;
            }
        }
    }
    // ---- diagonal blocks on the fp32 path, exact decay per term: one 4x4
    //      sub-block per group of NQ adjacent lanes, each lane a part of the
    //      channels; the parts are summed by lane exchange in a fixed order
    if constexpr (!BF) {
        const int sb = tid / NQ, qt = tid % NQ;
        int li = 0, lj = sb % 10;
        while (lj > li) {
            lj -= li + 1;
            ++li;
        }
        const int bi = 4 * (sb / 10) + li, bj = 4 * (sb / 10) + lj;
        float acc[4][4][4] = {};  // [Aab, Abk, Pqa, Pqk][x][y]
        if (sb < NSB) {
#pragma unroll 1
            for (int c = qt * CQ; c < (qt + 1) * CQ; c += 4) {
                f32x4 gi[4], gbi[4], gj[4], qv[4], bv[4], av[4], kv[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int i = 4 * bi + x, j = 4 * bj + x;
                    gi[x] = g4(i, c);
                    gbi[x] = g4(i - 1, c);
                    gj[x] = g4(j, c);
                    qv[x] = in4(p.q, i, c);
                    bv[x] = in4(p.b, i, c);
                    av[x] = in4(p.a, j, c);
                    kv[x] = in4(p.k, j, c);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int x = 0; x < 4; ++x)
#pragma unroll
                        for (int y = 0; y < 4; ++y) {
                            const float eA = fast_exp2(fminf(gbi[x][e] - gj[y][e], 0.f));
                            const float eP = fast_exp2(fminf(gi[x][e] - gj[y][e], 0.f));
                            acc[0][x][y] += bv[x][e] * av[y][e] * eA;
                            acc[1][x][y] += bv[x][e] * kv[y][e] * eA;
                            acc[2][x][y] += qv[x][e] * av[y][e] * eP;
                            acc[3][x][y] += qv[x][e] * kv[y][e] * eP;
                        }
            }
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y)
#pragma unroll
                    for (int d = 1; d < NQ; d <<= 1) acc[mt][x][y] += __shfl_xor(acc[mt][x][y], d);
        if (sb < NSB && qt == 0) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) {
                    const int i = 4 * bi + x, j = 4 * bj + y;
                    const bool okA = j < i && cnt_before(i) == sCnt[j];
                    const bool okP = j <= i && sCnt[i] == sCnt[j];
                    sM[0][i][j] = okA ? -acc[0][x][y] : 0.f;
                    sM[1][i][j] = okA ? acc[1][x][y] : 0.f;
                    sM[2][i][j] = okP ? acc[2][x][y] : 0.f;
                    sM[3][i][j] = okP ? acc[3][x][y] : 0.f;
                }
        }
    }
    __syncthreads();

    // ---- T = (I + sM[0])^-1 = (I - Aab)^-1 in place: diagonal 16x16 blocks by
    //      forward substitution (one lane per column), then block rows in order,
    //      T_IJ = -T_II sum_{J <= K < I} (-Aab)_IK T_KJ
    if (w < NTI && lane < 16) {
        const int base = 16 * w, col = lane;
        float tv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float val = i == col ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) val -= sM[0][base + i][base + j] * tv[j];
            tv[i] = val;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sM[0][base + i][base + col] = i >= col ? tv[i] : 0.f;
    }
    __syncthreads();
    for (int I = 1; I < NTI; ++I) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        const int J = w;
        if (J < I) {
            f32x4 xv = {0.f, 0.f, 0.f, 0.f};
            for (int K = J; K < I; ++K)
                mm16(xv, [&](int r, int k) { return sM[0][16 * I + r][16 * K + k]; },
                     [&](int k, int n) { return sM[0][16 * K + k][16 * J + n]; }, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) y = mfma4(sM[0][16 * I + l16][16 * I + 4 * kg + r], xv[r], y);
        }
        __syncthreads();
        if (J < I) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sM[0][16 * I + 4 * kg + r][16 * J + l16] = -y[r];
        }
        __syncthreads();
    }

    // ---- R = Pqa T, then T Abk and R Abk + Pqk, tile by tile over all the
    //      waves: the 16x16 tiles (I, Jc), Jc <= I, heaviest (I - Jc largest)
    //      first, wave w taking tiles w, w + 8, ...  Each product is formed in
    //      registers and written in place only after every wave has read its
    //      operands (barrier between).
    {
        constexpr int NTL = NTI * (NTI + 1) / 2, TPW = (NTL + kDplrWaves - 1) / kDplrWaves;
        auto tile_of = [](int t, int &I, int &Jc) {
            int d = NTI - 1, n = 1;
            while (t >= n) {
                t -= n;
                --d;
                ++n;
            }
            Jc = t;
            I = t + d;
        };
        f32x4 a1[TPW], a2[TPW], tv[TPW], rv[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = w + kDplrWaves * u;
            a1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t < NTL) {
                int I, Jc;
                tile_of(t, I, Jc);
                for (int K = Jc; K <= I; ++K)
                    mm16(a1[u], [&](int r, int k) { return sM[2][16 * I + r][16 * K + k]; },
                         [&](int k, int n) { return sM[0][16 * K + k][16 * Jc + n]; }, lane);
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = w + kDplrWaves * u;
            if (t < NTL) {
                int I, Jc;
                tile_of(t, I, Jc);
#pragma unroll
                for (int r = 0; r < 4; ++r) sM[2][16 * I + 4 * kg + r][16 * Jc + l16] = a1[u][r];
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = w + kDplrWaves * u;
            a1[u] = a2[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t < NTL) {
                int I, Jc;
                tile_of(t, I, Jc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    a2[u][r] = sM[3][16 * I + 4 * kg + r][16 * Jc + l16];
                    tv[u][r] = sM[0][16 * I + 4 * kg + r][16 * Jc + l16];
                    rv[u][r] = sM[2][16 * I + 4 * kg + r][16 * Jc + l16];
                }
                for (int K = Jc; K <= I; ++K) {
                    auto bk = [&](int k, int n) { return sM[1][16 * K + k][16 * Jc + n]; };
                    mm16(a1[u], [&](int r, int k) { return sM[0][16 * I + r][16 * K + k]; }, bk, lane);
                    mm16(a2[u], [&](int r, int k) { return sM[2][16 * I + r][16 * K + k]; }, bk, lane);
                }
            }
        }
        __syncthreads();  // every fp32 read of the four matrices is done
        if constexpr (kPk16) {
            // the planes: this wave's tiles of T, T Abk, R, R Abk + Pqk from
            // registers, and zeros in the tiles (I, I + 1), I even, that the
            // 32-token steps of row tile I also read
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int t = w + kDplrWaves * u;
                if (t < NTL) {
                    int I, Jc;
                    tile_of(t, I, Jc);
                    const f32x4 *mats[4] = {&tv[u], &a1[u], &rv[u], &a2[u]};
#pragma unroll
                    for (int m = 0; m < 4; ++m)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float x = (*mats[m])[r];
                            const __bf16 hi = static_cast<__bf16>(x);
                            const int o = ((2 * m) * C + 16 * I + 4 * kg + r) * MP + 16 * Jc + l16;
                            Mp[o] = hi;
                            Mp[o + C * MP] = static_cast<__bf16>(x - static_cast<float>(hi));
                        }
                }
            }
            constexpr int NZ = 8 * (NTI / 2) * 16 * 2;  // 16-byte pieces: planes x tiles x rows x 2
            for (int z = tid; z < NZ; z += kDplrThreads) {
                const int half = z & 1, rr = (z >> 1) & 15, zt = (z >> 5) % (NTI / 2), pl = (z >> 5) / (NTI / 2);
                const int I = 2 * zt;
                *reinterpret_cast<uint4 *>(Mp + (pl * C + 16 * I + rr) * MP + 16 * (I + 1) + 8 * half) =
                    uint4{0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int t = w + kDplrWaves * u;
                if (t < NTL) {
                    int I, Jc;
                    tile_of(t, I, Jc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        sM[1][16 * I + 4 * kg + r][16 * Jc + l16] = a1[u][r];
                        sM[3][16 * I + 4 * kg + r][16 * Jc + l16] = a2[u][r];
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- the package.  Channel-tile jobs: -W = -T X and Q' = Q e^G + R X in
    //      the WQ layout, [At; Kt] in the KT layout.  Value-tile jobs: U' =
    //      (T Abk) V and O_intra = (R Abk + Pqk) V in the UP / OI layouts.
    Op *wq = reinterpret_cast<Op *>(pkg + p.L.wq);
    Op *kt = reinterpret_cast<Op *>(pkg + p.L.kt);
    f32x4 *up = reinterpret_cast<f32x4 *>(pkg + p.L.up);
    f32x4 *oi = reinterpret_cast<f32x4 *>(pkg + p.L.oi);
    f32x4 *vx = reinterpret_cast<f32x4 *>(pkg + p.L.vx);
    constexpr int NCT = DKP / 16;
    const int last_rst = sLast, cnt_last = sCnt[C - 1];
    auto store4 = [&](Op *dst, const f32x4 &v) {
        if constexpr (BF) {
            *reinterpret_cast<f16x4 *>(dst) = f16x4{static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]),
                                                     static_cast<_Float16>(v[2]), static_cast<_Float16>(v[3])};
        } else {
            *reinterpret_cast<f32x4 *>(dst) = v;
        }
    };
    // row 16 rt + l16 of matrix m's planes at tokens 32 s + 8 kg .. + 7
    auto m_frag = [&](int m, int rt, int s, bf16x8 &hi, bf16x8 &lo) {
        const int o = (2 * m * C + 16 * rt + l16) * MP + 32 * s + 8 * kg;
        hi = *reinterpret_cast<const bf16x8 *>(Mp + o);
        lo = *reinterpret_cast<const bf16x8 *>(Mp + o + C * MP);
    };
    auto raw1 = [&](const void *x, int i, int c) {  // bf16 bits of x[token i][c], clamped row
        return static_cast<const uint16_t *>(x)[row(i) + c];
    };
    constexpr int KS = C / 32 > 0 ? C / 32 : 1;  // 32-token steps of the 16-bit products
    for (int job = w; job < NCT + NTD; job += kDplrWaves) {
        if (job < NCT) {
            const int ct = job, ks = ct >> 1, hc = ct & 1;
            if (ct >= NTD) {  // channels past Dk (Dk = 16): zero operands
                for (int rt = 0; rt < 2 * NTI; ++rt)
                    store4(wq + ((static_cast<size_t>(rt) * KSK + ks) * 64 + lane) * 8 + 4 * hc,
                           f32x4{0.f, 0.f, 0.f, 0.f});
                continue;
            }
            const int cx = 16 * ct + l16;  // this lane's channel as the left operand
            if constexpr (kPk16) {
                // X^T operand: X[32 s + 8 kg + e][cx], split in bf16 hi/lo; the
                // products M X over the 32-token steps holding row tile I's nonzeros
                uint16_t braw[KS][8];
                f32x4 qraw[NTI];
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
                    for (int e = 0; e < 8; ++e) braw[s2][e] = raw1(p.b, 32 * s2 + 8 * kg + e, cx);
#pragma unroll
                for (int t = 0; t < NTI; ++t) qraw[t] = in4(p.q, 16 * t + l16, 16 * ct + 4 * kg);
                __builtin_amdgcn_sched_barrier(0);
                bf16x8 xh[KS], xl[KS];
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2) {
                    float xv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = 32 * s2 + 8 * kg + e;
                        const float gb = j > 0 ? sG[j - 1][cx] : 0.f;
                        const float bv = __uint_as_float(static_cast<uint32_t>(braw[s2][e]) << 16);
                        xv[e] = j < nvalid && cnt_before(j) == 0 ? bv * fast_exp2(gb) : 0.f;
                    }
                    split_bf16(xv, xh[s2], xl[s2]);
                }
                f32x4 qg[NTI];
#pragma unroll
                for (int I = 0; I < NTI; ++I) {
                    const int i = 16 * I + l16, c0 = 16 * ct + 4 * kg;
                    const f32x4 gv = g4(i, c0);
                    const bool live = sCnt[i] == 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) qg[I][r] = live ? qraw[I][r] * fast_exp2(gv[r]) : 0.f;
                }
#pragma unroll
                for (int rt = 0; rt < 2 * NTI; ++rt) {
                    const int I = rt < NTI ? rt : rt - NTI, m = rt < NTI ? 0 : 2;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2)
                        if (32 * s2 <= 16 * I + 15) {
                            bf16x8 mh, ml;
                            m_frag(m, I, s2, mh, ml);
                            acc = mfma_bf16(xl[s2], mh, acc);
                            acc = mfma_bf16(xh[s2], ml, acc);
                            acc = mfma_bf16(xh[s2], mh, acc);
                        }
                    // acc[r] = (M X)[token 16 I + l16][channel 16 ct + 4 kg + r]
                    store4(wq + ((static_cast<size_t>(rt) * KSK + ks) * 64 + lane) * 8 + 4 * hc,
                           rt < NTI ? -acc : acc + qg[I]);
                }
            } else {
            // this job's b and q values, all loads issued before any is used (the
            // scheduling barrier keeps the compiler from sinking each load to its
            // use, which would wait out every load's latency in turn)
            f32x4 braw[NTI], qraw[NTI];
#pragma unroll
            for (int t = 0; t < NTI; ++t) {
#pragma unroll
                for (int e = 0; e < 4; ++e) braw[t][e] = in(p.b, 16 * t + 4 * kg + e, cx);
                qraw[t] = in4(p.q, 16 * t + l16, 16 * ct + 4 * kg);
            }
            __builtin_amdgcn_sched_barrier(0);
            // X^T fragment: xf[t][e] = X[16 t + 4 kg + e][cx]
            f32x4 xf[NTI];
#pragma unroll
            for (int t = 0; t < NTI; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * t + 4 * kg + e;
                    const float gb = j > 0 ? sG[j - 1][cx] : 0.f;
                    xf[t][e] = cnt_before(j) == 0 ? braw[t][e] * fast_exp2(gb) : 0.f;
                }
            // the Q e^G terms of the Q' rows
            f32x4 qg[NTI];
#pragma unroll
            for (int I = 0; I < NTI; ++I) {
                const int i = 16 * I + l16, c0 = 16 * ct + 4 * kg;
                const f32x4 gv = g4(i, c0);
                const bool live = sCnt[i] == 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) qg[I][r] = live ? qraw[I][r] * fast_exp2(gv[r]) : 0.f;
            }
            for (int rt = 0; rt < 2 * NTI; ++rt) {
                const int I = rt < NTI ? rt : rt - NTI, mt = rt < NTI ? 0 : 2;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < NTI; ++t)
                    if (t <= I) {
                        const f32x4 mv = *reinterpret_cast<const f32x4 *>(&sM[mt][16 * I + l16][16 * t + 4 * kg]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc = mfma4(xf[t][e], mv[e], acc);
                    }
                // acc[r] = (M X)[token 16 I + l16][channel 16 ct + 4 kg + r]
                f32x4 val;
                if (rt < NTI) {
                    val = -acc;
                } else {
                    f32x4 q4 = qg[0];
#pragma unroll
                    for (int J = 1; J < NTI; ++J)
                        if (J == I) q4 = qg[J];
                    val = acc + q4;
                }
                store4(wq + ((static_cast<size_t>(rt) * KSK + ks) * 64 + lane) * 8 + 4 * hc, val);
            }
            }
            // [At; Kt]: channel cx, tokens 32 s + 8 kg + e of each half; the a and
            // k values loaded in one batch first
            float akraw[KSC2][8];
#pragma unroll
            for (int s = 0; s < KSC2; ++s) {
                const bool second = s >= KSC2 / 2;
                const int s0 = second ? s - KSC2 / 2 : s;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 32 * s0 + 8 * kg + e;
                    akraw[s][e] = in(second ? p.k : p.a, j < C ? j : C - 1, cx);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < KSC2; ++s) {
                const bool second = s >= KSC2 / 2;
                const int s0 = second ? s - KSC2 / 2 : s;
                float v8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 32 * s0 + 8 * kg + e, jj = j < C ? j : C - 1;
                    v8[e] = (j < C && sCnt[jj] == cnt_last) ? akraw[s][e] * fast_exp2(sG[C - 1][cx] - sG[jj][cx]) : 0.f;
                }
                store8(kt + ((static_cast<size_t>(ct) * KSC2 + s) * 64 + lane) * 8, v8);
            }
        } else {
            const int vt = job - NCT, col = 16 * vt + l16;
            // V fragment: vf[t][e] = V[16 t + 4 kg + e][col], loaded in one batch
            // (on the 16-bit path also V[32 s + 8 kg + e][col] as the B operand
            // of the bf16 products: V is exact in bf16, only M is split)
            f32x4 vf[NTI];
            uint16_t vraw[kPk16 ? KS : 1][8];
#pragma unroll
            for (int t = 0; t < NTI; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) vf[t][e] = in(p.v, 16 * t + 4 * kg + e, col);
            if constexpr (kPk16) {
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
                    for (int e = 0; e < 8; ++e) vraw[s2][e] = raw1(p.v, 32 * s2 + 8 * kg + e, col);
            }
            __builtin_amdgcn_sched_barrier(0);
            bf16x8 vb[kPk16 ? KS : 1];
            if constexpr (kPk16) {
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2) {
                    uint32_t wd[4];
#pragma unroll
                    for (int q2 = 0; q2 < 4; ++q2) {
                        const int j = 32 * s2 + 8 * kg + 2 * q2;
                        const uint32_t lo = j < nvalid ? vraw[s2][2 * q2] : 0u;
                        const uint32_t hi = j + 1 < nvalid ? vraw[s2][2 * q2 + 1] : 0u;
                        wd[q2] = lo | (hi << 16);
                    }
                    vb[s2] = __builtin_bit_cast(bf16x8, (uint4{wd[0], wd[1], wd[2], wd[3]}));
                }
            }
            for (int rt = 0; rt < 2 * NTI; ++rt) {
                const int I = rt < NTI ? rt : rt - NTI, mt = rt < NTI ? 1 : 3;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (kPk16) {
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2)
                        if (32 * s2 <= 16 * I + 15) {
                            bf16x8 mh, ml;
                            m_frag(mt, I, s2, mh, ml);
                            acc = mfma_bf16(ml, vb[s2], acc);
                            acc = mfma_bf16(mh, vb[s2], acc);
                        }
                } else {
#pragma unroll
                for (int t = 0; t < NTI; ++t)
                    if (t <= I) {
                        const f32x4 mv = *reinterpret_cast<const f32x4 *>(&sM[mt][16 * I + l16][16 * t + 4 * kg]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc = mfma4(mv[e], vf[t][e], acc);
                    }
                }
                f32x4 *dst = rt < NTI ? up : oi;
                dst[(static_cast<size_t>(vt) * NTI + I) * 64 + lane] = acc;
                // V itself for the state pass: vf[I] holds rows 16 I + 4 kg + e of
                // column col, the UP layout of row tile I
                if (rt < NTI) {
                    const size_t vi = (static_cast<size_t>(vt) * NTI + I) * 64 + lane;
                    if constexpr (BF) {  // exact: V is bf16 (the low halves are zero)
                        const f32x4 x = vf[I];
                        reinterpret_cast<uint2 *>(vx)[vi] =
                            uint2{(__float_as_uint(x[0]) >> 16) | (__float_as_uint(x[1]) & 0xffff0000u),
                                  (__float_as_uint(x[2]) >> 16) | (__float_as_uint(x[3]) & 0xffff0000u)};
                    } else {
                        vx[vi] = vf[I];
                    }
                }
            }
        }
    }
    float *glp = reinterpret_cast<float *>(pkg + p.L.gl);
    for (int c = tid; c < D; c += kDplrThreads) glp[c] = last_rst >= 0 ? 0.f : fast_exp2(sG[C - 1][c]);
}

template <int C, int D, bool BF>
hipError_t launch_dplr_t(const PrefillArgs &a, hipStream_t stream) {
    const PackageLayout L = dplr_package_layout(C, D, D, BF);
    if (a.cu_seqlens) {
        const hipError_t e = launch_plan(a.cu_seqlens, a.N, C, a.chunk_offsets, stream);
        if (e != hipSuccess) return e;
    }
    if (a.n_slots > 0) {
        DplrIntraParams ip{a.q, a.k, a.v, a.lr_a, a.lr_b, a.log_alpha, a.cu_seqlens, a.chunk_offsets,
                           a.T, a.H, a.N, a.workspace, a.pkg_bytes, L};
        const int64_t n_items = a.n_slots * a.H;
        if (n_items > 0x7fffffff) return hipErrorInvalidValue;
        hipLaunchKernelGGL((dplr_intra_kernel<C, D, BF>), dim3(static_cast<unsigned>(n_items)),
                           dim3(kDplrThreads), 0, stream, ip);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    StateParams sp{a.init_state, a.cu_seqlens, a.chunk_offsets, a.o, a.final_state, nullptr,
                   a.T, a.H, a.N, a.workspace, a.pkg_bytes, L};
    return launch_dplr_state<C, D, BF>(sp, stream);
}

template <int C, bool BF>
hipError_t dispatch_dplr_d(const PrefillArgs &a, hipStream_t s) {
    switch (a.Dk) {
        case 16: return launch_dplr_t<C, 16, BF>(a, s);
        case 32: return launch_dplr_t<C, 32, BF>(a, s);
        case 64: return launch_dplr_t<C, 64, BF>(a, s);
        case 128:
            if constexpr (BF || C <= 32) return launch_dplr_t<C, 128, BF>(a, s);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_dplr(const PrefillArgs &a, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    if (a.Dk != a.Dv) return hipErrorInvalidValue;
    const bool bf = a.bf16;
    switch (a.C) {
        case 16: return bf ? dispatch_dplr_d<16, true>(a, stream) : dispatch_dplr_d<16, false>(a, stream);
        case 32: return bf ? dispatch_dplr_d<32, true>(a, stream) : dispatch_dplr_d<32, false>(a, stream);
        case 64: return bf ? dispatch_dplr_d<64, true>(a, stream) : dispatch_dplr_d<64, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
