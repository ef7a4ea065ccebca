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
// Gram matrices: 16x16 blocks below the diagonal on the fp32 matrix cores with
// the reference m = the last token of the column block, e^{x_i - G_j} =
// e^{x_i - G_m} e^{G_m - G_j} (both factors <= 1); the diagonal blocks with the
// exact exponential of every pair.  A token whose log_alpha is -inf on every
// channel zeroes the diagonal part of its transition but not the low-rank
// part: it adds 0 to G, and the couplings it cuts are masked (Aab, Abk and X
// through a reset strictly before token i; P, At, Kt through one in (j, i]).
// Other -inf values are clamped to -88.  All arithmetic of this kernel is fp32.
#include <algorithm>

#include "kda_prefill.h"

namespace kda {
namespace {

constexpr int kDplrThreads = 512;  // 8 waves
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

    __shared__ __align__(16) float sG[C][GS];  // G, cumulative log-decay
    __shared__ __align__(16) float sM[4][C][MS];  // -Aab -> T, Abk -> T Abk, Pqa -> Pqa T, Pqk -> Pqa T Abk + Pqk
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
    auto in = [&](const void *x, int i, int c) {
        return i < nvalid ? ld_in<BF>(x, ((tok0 + i) * H + h) * D + c) : 0.f;
    };
    auto in4 = [&](const void *x, int i, int c) {  // channels c .. c + 3 of token i
        return i < nvalid ? ld_in4<BF>(x, ((tok0 + i) * H + h) * D + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    auto g4 = [&](int i, int c) {  // G[i][c .. c + 3], G[-1] = 0
        return i >= 0 ? *reinterpret_cast<const f32x4 *>(&sG[i][c]) : f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // ---- cumulative decay and resets
    for (int x = tid; x < C * D; x += kDplrThreads) {
        const int i = x / D, c = x % D;
        sG[i][c] = i < nvalid ? p.log_alpha[((tok0 + i) * H + h) * D + c] : 0.f;
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
            acc += sRst[i] ? 0.f : fmaxf(sG[i][sc], kGFloor);
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

    // ---- Gram blocks below the diagonal, one 16x16 block pair per wave
    {
        constexpr int NPAIR = NTI * (NTI - 1) / 2;
        // (the last waves first: the diagonal work below fills the first ones)
        for (int pr = kDplrWaves - 1 - w; pr < NPAIR; pr += kDplrWaves) {
            int I = 1, J = pr;
            while (J >= I) {
                J -= I;
                ++I;
            }
            const int m = 16 * J + 15, i = 16 * I + l16, j = 16 * J + l16;
            f32x4 aab = {0.f, 0.f, 0.f, 0.f}, abk = aab, pqa = aab, pqk = aab;
#pragma unroll 2
            for (int t = 0; t < D / 16; ++t) {
                const int c = 16 * t + 4 * kg;  // this lane's channels c .. c + 3
                const f32x4 gm = g4(m, c), gbi = g4(i - 1, c), gi = g4(i, c), gj = g4(j, c);
                const f32x4 bv = in4(p.b, i, c), qv = in4(p.q, i, c), av = in4(p.a, j, c), kv = in4(p.k, j, c);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float e3 = __expf(gm[e] - gj[e]);
                    const float lb = bv[e] * __expf(gbi[e] - gm[e]), lq = qv[e] * __expf(gi[e] - gm[e]);
                    const float ra = av[e] * e3, rk = kv[e] * e3;
                    aab = mfma4(lb, ra, aab);
                    abk = mfma4(lb, rk, abk);
                    pqa = mfma4(lq, ra, pqa);
                    pqk = mfma4(lq, rk, pqk);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ii = 16 * I + 4 * kg + r;
                const bool okA = cnt_before(ii) == sCnt[j], okP = sCnt[ii] == sCnt[j];
                sM[0][ii][j] = okA ? -aab[r] : 0.f;
                sM[1][ii][j] = okA ? abk[r] : 0.f;
                sM[2][ii][j] = okP ? pqa[r] : 0.f;
                sM[3][ii][j] = okP ? pqk[r] : 0.f;
            }
        }
    }
    // ---- diagonal blocks, exact decay per term: one 4x4 sub-block per group of
    //      NQ adjacent lanes, each lane a part of the channels; the parts are
    //      summed by lane exchange in a fixed order
    {
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
                            const float eA = __expf(fminf(gbi[x][e] - gj[y][e], 0.f));
                            const float eP = __expf(fminf(gi[x][e] - gj[y][e], 0.f));
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
        __syncthreads();
    }

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

    // ---- R = Pqa T in place (a wave per row block: it alone reads and writes those rows)
    if (w < NTI) {
        const int I = w;
        f32x4 acc[NTI];
#pragma unroll
        for (int Jc = 0; Jc < NTI; ++Jc) {
            acc[Jc] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (Jc <= I)
                for (int K = Jc; K <= I; ++K)
                    mm16(acc[Jc], [&](int r, int k) { return sM[2][16 * I + r][16 * K + k]; },
                         [&](int k, int n) { return sM[0][16 * K + k][16 * Jc + n]; }, lane);
        }
#pragma unroll
        for (int Jc = 0; Jc < NTI; ++Jc)
            if (Jc <= I) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sM[2][16 * I + 4 * kg + r][16 * Jc + l16] = acc[Jc][r];
            }
    }
    __syncthreads();
    // ---- T Abk and R Abk + Pqk in place (a wave per column block of Abk)
    if (w < NTI) {
        const int Jc = w;
        f32x4 m1[NTI], m2[NTI];
#pragma unroll
        for (int I = 0; I < NTI; ++I) {
            m1[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) m2[I][r] = sM[3][16 * I + 4 * kg + r][16 * Jc + l16];
            if (I >= Jc)
                for (int K = Jc; K <= I; ++K) {
                    auto bk = [&](int k, int n) { return sM[1][16 * K + k][16 * Jc + n]; };
                    mm16(m1[I], [&](int r, int k) { return sM[0][16 * I + r][16 * K + k]; }, bk, lane);
                    mm16(m2[I], [&](int r, int k) { return sM[2][16 * I + r][16 * K + k]; }, bk, lane);
                }
        }
#pragma unroll
        for (int I = 0; I < NTI; ++I)
            if (I >= Jc) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sM[1][16 * I + 4 * kg + r][16 * Jc + l16] = m1[I][r];
                    sM[3][16 * I + 4 * kg + r][16 * Jc + l16] = m2[I][r];
                }
            }
    }
    __syncthreads();

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
            // X^T fragment: xf[t][e] = X[16 t + 4 kg + e][cx]
            f32x4 xf[NTI];
#pragma unroll
            for (int t = 0; t < NTI; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * t + 4 * kg + e;
                    const float gb = j > 0 ? sG[j - 1][cx] : 0.f;
                    xf[t][e] = cnt_before(j) == 0 ? in(p.b, j, cx) * __expf(gb) : 0.f;
                }
            // the Q e^G terms of the Q' rows, loaded before the products
            f32x4 qg[NTI];
#pragma unroll
            for (int I = 0; I < NTI; ++I) {
                const int i = 16 * I + l16, c0 = 16 * ct + 4 * kg;
                const f32x4 qv = in4(p.q, i, c0), gv = g4(i, c0);
                const bool live = sCnt[i] == 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) qg[I][r] = live ? qv[r] * __expf(gv[r]) : 0.f;
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
            // [At; Kt]: channel cx, tokens 32 s + 8 kg + e of each half
#pragma unroll
            for (int s = 0; s < KSC2; ++s) {
                const bool second = s >= KSC2 / 2;
                const int s0 = second ? s - KSC2 / 2 : s;
                float v8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 32 * s0 + 8 * kg + e;
                    float x = 0.f;
                    if (j < C && sCnt[j] == cnt_last)
                        x = in(second ? p.k : p.a, j, cx) * __expf(sG[C - 1][cx] - sG[j][cx]);
                    v8[e] = x;
                }
                store8(kt + ((static_cast<size_t>(ct) * KSC2 + s) * 64 + lane) * 8, v8);
            }
        } else {
            const int vt = job - NCT, col = 16 * vt + l16;
            // V fragment: vf[t][e] = V[16 t + 4 kg + e][col]
            f32x4 vf[NTI];
#pragma unroll
            for (int t = 0; t < NTI; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) vf[t][e] = in(p.v, 16 * t + 4 * kg + e, col);
            for (int rt = 0; rt < 2 * NTI; ++rt) {
                const int I = rt < NTI ? rt : rt - NTI, mt = rt < NTI ? 1 : 3;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < NTI; ++t)
                    if (t <= I) {
                        const f32x4 mv = *reinterpret_cast<const f32x4 *>(&sM[mt][16 * I + l16][16 * t + 4 * kg]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc = mfma4(mv[e], vf[t][e], acc);
                    }
                f32x4 *dst = rt < NTI ? up : oi;
                dst[(static_cast<size_t>(vt) * NTI + I) * 64 + lane] = acc;
                // V itself for the state pass: vf[I] holds rows 16 I + 4 kg + e of
                // column col, the UP layout of row tile I
                if (rt < NTI) vx[(static_cast<size_t>(vt) * NTI + I) * 64 + lane] = vf[I];
            }
        }
    }
    float *glp = reinterpret_cast<float *>(pkg + p.L.gl);
    for (int c = tid; c < D; c += kDplrThreads) glp[c] = last_rst >= 0 ? 0.f : __expf(sG[C - 1][c]);
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
