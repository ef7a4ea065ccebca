// kda_backward.hip -- chunked backward of the KDA prefill on gfx950.
//
// Gradients of the recurrence of the section "Kimi Delta Attention (KDA)" on
// the page "Kimi Linear 高效注意力架构" (the training workload the page names),
// taken through the same chunked form the forward uses.  Per chunk, with incoming state S0,
// outgoing state S1 and the forward's quantities (G, Gamma, A = Diag(beta) Abar,
// T = (I + A)^-1, P, W, U' as in kda_prefill.hip):
//
//   R = V - (K*Gamma) S0,  X = Diag(beta) R,  U = T X
//   O = (Q*Gamma) S0 + P U,  S1 = Diag(Gamma_C) S0 + Kt^T U
//
// Given dO and dS1, reverse mode gives
//
//   dS0  = Diag(Gamma_C) dS1 + Q'^T dO - W^T (Kt dS1)          (state pass)
//   dU   = P^T dO + Kt dS1,   dX = T^T dU,   dR = Diag(beta) dX = dV
//   dT   = dU X^T,   dA = -T^T dT T^T (strictly lower),   dAbar = Diag(beta) dA
//   dP   = dO U^T (lower),   d(Q*Gamma) = dO S0^T,   d(K*Gamma) = -dR S0^T,
//   dKt  = U dS1^T,   dGamma_C = rowsum(S0 * dS1)
//   dbeta_i = sum_v R_iv dX_iv + sum_j dA_ij Abar_ij
//
// and the decayed Gram products (e_ijc = exp(G_ic - G_jc), i >= j)
//
//   dq_i += sum_j dP_ij e_ij k_j,   dk_j += sum_i dP_ij e_ij q_i,
//   dk_i += sum_j dAbar_ij e_ij k_j,   dk_j += sum_i dAbar_ij e_ij k_i,
//
// each pair term f contributing +f to dG_i and -f to dG_j; dlog_alpha is the
// reverse cumulative sum of dG over the chunk (0 at -inf gates and resets).
//
// Passes: the forward's intra-chunk packages and a state pass that saves the
// state entering every chunk (kda_prefill.hip), then bwd_state_kernel walks
// each (sequence, head, 16-column slab) backwards writing dS1 of every chunk
// and dS0 of the sequence, then intra_bwd_kernel computes every gradient of
// one (chunk, head) at a time.  Products after the package run on the fp32
// matrix cores with fp32 accumulation (on the 16-bit path the reverse state
// pass uses fp16 hi/lo operands); the decay factors of a 16-token block pair
// go through a reference token (both factors <= 1 below the diagonal; on the
// diagonal, 16-bit path only, the block's token 7 with an exact per-pair
// fallback for channels whose decay spans more than e^40).
#include <algorithm>
#include <type_traits>

#include "kda_prefill.h"

namespace kda {
namespace {

constexpr int kBwdThreads = 256;

// acc += A B for one 16x16 output tile on the fp32 matrix cores, K a multiple
// of 4: a(r, k) is element (r, k) of the tile's 16 rows of A, b(k, n) element
// (k, n) of its 16 columns of B.  Lane l supplies row / column l % 16 at
// k = 4 s + l / 16 of step s; the accumulator holds C[4 (l / 16) + r][l % 16].
// The operands of up to 16 steps are loaded as one batch before their
// products, so a batch costs one memory round trip.
template <int K, typename FA, typename FB>
__device__ __forceinline__ void mm_f32(f32x4 &acc, FA &&a, FB &&b, int lane) {
    const int r = lane & 15, kk = lane >> 4;
    constexpr int BATCH = K / 4 < 16 ? K / 4 : 16;
    static_assert(K % (4 * BATCH) == 0, "K is a multiple of the batch");
    for (int k0 = 0; k0 < K; k0 += 4 * BATCH) {
        float av[BATCH], bv[BATCH];
#pragma unroll
        for (int s = 0; s < BATCH; ++s) {
            av[s] = a(r, k0 + 4 * s + kk);
            bv[s] = b(k0 + 4 * s + kk, r);
        }
#pragma unroll
        for (int s = 0; s < BATCH; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc, 0, 0, 0);
    }
}

// The same product with the operands read 4 k at a time: a4(r, k0) returns
// A[r][k0 .. k0 + 3] and b4(k0, n) B[k0 .. k0 + 3][n] (a 16-byte load where the
// operand is contiguous in k).  Step (t, j) gives lane l the k = 16 t + 4 (l / 16) + j,
// the same for both operands, so the steps still cover every k once.  K is a
// multiple of 16.
template <int K, typename FA, typename FB>
__device__ __forceinline__ void mm_f32_v(f32x4 &acc, FA &&a4, FB &&b4, int lane) {
    const int r = lane & 15, kk = lane >> 4;
    constexpr int NT = K / 16, BATCH = NT < 4 ? NT : 4;
    static_assert(K % 16 == 0 && NT % BATCH == 0, "K is a multiple of 16 and of the batch");
    for (int t0 = 0; t0 < NT; t0 += BATCH) {
        f32x4 av[BATCH], bv[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            av[b] = a4(r, 16 * (t0 + b) + 4 * kk);
            bv[b] = b4(16 * (t0 + b) + 4 * kk, r);
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[b][j], bv[b][j], acc, 0, 0, 0);
    }
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// One lane's share of an operand over a whole contraction of K, in the order
// of mm_f32_v: v[t][j] is its value at k = 16 t + 4 (lane / 16) + j, and
// f4(k0, n) as mm_f32_v's b4.  Loaded once, it serves every output tile that
// shares the operand.
template <int K>
struct Frag {
    f32x4 v[K / 16];
};

template <int K, typename F4>
__device__ __forceinline__ Frag<K> frag_of(F4 &&f4, int lane) {
    Frag<K> f;
    const int r = lane & 15, kk = lane >> 4;
#pragma unroll
    for (int t = 0; t < K / 16; ++t) f.v[t] = f4(16 * t + 4 * kk, r);
    return f;
}

// mm_f32_v with B given as a preloaded fragment
template <int K, typename FA>
__device__ __forceinline__ void mm_f32_vb(f32x4 &acc, FA &&a4, const Frag<K> &bf, int lane) {
    const int r = lane & 15, kk = lane >> 4;
    constexpr int NT = K / 16, BATCH = NT;  // the whole left-hand fragment in one batch
#pragma unroll
    for (int t0 = 0; t0 < NT; t0 += BATCH) {
        f32x4 av[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) av[b] = a4(r, 16 * (t0 + b) + 4 * kk);
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[b][j], bf.v[t0 + b][j], acc, 0, 0, 0);
    }
}

// The tiles t = t0, t0 + step, .. < tend of products acc_t = A_t B with B a
// preloaded fragment, software-pipelined: tile t + step's left-hand fragment
// (a4t(t, r, k0) as mm_f32_v's a4) and its epilogue inputs (pre(t), 4 values)
// are loaded before tile t's products, so their latency overlaps them.
// epi(t, acc, pre_t) consumes a tile.
template <int K, typename FA, typename FP, typename FE>
__device__ __forceinline__ void tiles_vb(int t0, int tend, int step, FA &&a4t, const Frag<K> &bf, FP &&pre,
                                         FE &&epi, int lane) {
    const int r = lane & 15, kk = lane >> 4;
    constexpr int NT = K / 16;
    f32x4 cur[NT], nxt[NT], pc = {0.f, 0.f, 0.f, 0.f}, pn = pc;
    if (t0 < tend) {
#pragma unroll
        for (int b = 0; b < NT; ++b) cur[b] = a4t(t0, r, 16 * b + 4 * kk);
        pc = pre(t0);
    }
    for (int t = t0; t < tend; t += step) {
        if (t + step < tend) {
#pragma unroll
            for (int b = 0; b < NT; ++b) nxt[b] = a4t(t + step, r, 16 * b + 4 * kk);
            pn = pre(t + step);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[b][j], bf.v[b][j], acc, 0, 0, 0);
        epi(t, acc, pc);
#pragma unroll
        for (int b = 0; b < NT; ++b) cur[b] = nxt[b];
        pc = pn;
    }
}

// sum over the 16 lanes of each row group (lanes 16 g .. 16 g + 15)
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// -----------------------------------------------------------------------------
// state pass, backwards: one workgroup per (sequence, head, 16-column slab)
// -----------------------------------------------------------------------------
// 8 package operand values of one lane (fp16 on the 16-bit path, fp32 otherwise)
template <bool BF>
struct Raw8;
template <>
struct Raw8<true> {
    f16x8 v;
    __device__ __forceinline__ void load(const void *p) { v = *reinterpret_cast<const f16x8 *>(p); }
    __device__ __forceinline__ float at(int e) const { return static_cast<float>(v[e]); }
};
template <>
struct Raw8<false> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const void *p) {
        a = reinterpret_cast<const f32x4 *>(p)[0];
        b = reinterpret_cast<const f32x4 *>(p)[1];
    }
    __device__ __forceinline__ float at(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// One chunk's operands of the backward state pass as this thread loads them:
// its blocks of the package's W / Q' and Kt fragments, its share of Gamma_C
// and of the dO slab.  The next (earlier) chunk's are loaded while one computes.
template <int C, int D, bool BF>
struct BwdFrags {
    using F = Cfg<C, D, D, BF>;
    using Op = typename F::Op;
    static constexpr int NT16 = C / 16, NTK = D / 16, KSK = F::DKP / 32, KSC = F::CP / 32, NRT = 2 * NT16;
    static constexpr int WQB = (NRT * KSK + 3) / 4, KTB = (NTK * KSC + 3) / 4;
    static constexpr int DOE = (C * 16 + kBwdThreads - 1) / kBwdThreads, GLE = (D + kBwdThreads - 1) / kBwdThreads;
    Raw8<BF> wq[WQB], kt[KTB];
    float dO[DOE], gl[GLE];

    __device__ __forceinline__ void load(const BwdStateParams &p, const char *pkg, int64_t row0, int nvalid, int ct,
                                         int h, int tid) {
        const int lane = tid & 63, w = tid >> 6;
        const Op *wqp = reinterpret_cast<const Op *>(pkg + p.L.wq);
#pragma unroll
        for (int j = 0; j < WQB; ++j) {
            const int b = w + 4 * j;
            if (b < NRT * KSK) wq[j].load(wqp + (static_cast<size_t>(b) * 64 + lane) * 8);
        }
        const Op *ktp = reinterpret_cast<const Op *>(pkg + p.L.kt);
#pragma unroll
        for (int j = 0; j < KTB; ++j) {
            const int b = w + 4 * j;
            if (b < NTK * KSC) kt[j].load(ktp + (static_cast<size_t>(b) * 64 + lane) * 8);
        }
#pragma unroll
        for (int j = 0; j < GLE; ++j) {
            const int x = tid + kBwdThreads * j;
            gl[j] = x < D ? reinterpret_cast<const float *>(pkg + p.L.gl)[x] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < DOE; ++j) {
            const int x = tid + kBwdThreads * j, i = x / 16, jj = x % 16;
            dO[j] = (x < C * 16 && i < nvalid) ? p.d_o[((row0 + i) * p.H + h) * D + 16 * ct + jj] : 0.f;
        }
    }

    // scatter into the [token][channel] fp32 LDS copies
    template <int GS, int SS>
    __device__ __forceinline__ void store(float (*sW)[GS], float (*sQ)[GS], float (*sKt)[GS], float *sGL,
                                          float (*sdO)[SS], int tid) const {
        const int lane = tid & 63, w = tid >> 6, l16 = lane & 15, kg = lane >> 4;
#pragma unroll
        for (int j = 0; j < WQB; ++j) {
            const int b = w + 4 * j;
            if (b < NRT * KSK) {
                const int rt = b / KSK, ks = b % KSK, i = 16 * (rt % NT16) + l16;
                float(*dst)[GS] = rt < NT16 ? sW : sQ;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ch = 32 * ks + (e < 4 ? 4 * kg + e : 16 + 4 * kg + e - 4);
                    if (ch < D) dst[i][ch] = wq[j].at(e);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < KTB; ++j) {
            const int b = w + 4 * j;
            if (b < NTK * KSC) {
                const int tk = b / KSC, ks = b % KSC;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int i = 32 * ks + 8 * kg + e;
                    if (i < C) sKt[i][16 * tk + l16] = kt[j].at(e);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < GLE; ++j) {
            const int x = tid + kBwdThreads * j;
            if (x < D) sGL[x] = gl[j];
        }
#pragma unroll
        for (int j = 0; j < DOE; ++j) {
            const int x = tid + kBwdThreads * j;
            if (x < C * 16) sdO[x / 16][x % 16] = dO[j];
        }
    }

    // The 16-bit path's LDS copies, laid out as the fp16 matrix-core operands
    // want them (8 consecutive k per lane): W^T and Q'^T [channel][token], Kt
    // [token][channel] (the package's fp16 values as they are), and dO as an
    // fp16 hi + lo pair [column][token].
    template <int TS, int CS>
    __device__ __forceinline__ void store16(_Float16 (*sWT)[TS], _Float16 (*sQT)[TS], _Float16 (*sKt)[CS], float *sGL,
                                            _Float16 (*sdOh)[TS], _Float16 (*sdOl)[TS], int tid) const {
        static_assert(BF, "the fp16 layout holds the 16-bit path's operands");
        const int lane = tid & 63, w = tid >> 6, l16 = lane & 15, kg = lane >> 4;
#pragma unroll
        for (int j = 0; j < WQB; ++j) {
            const int b = w + 4 * j;
            if (b < NRT * KSK) {
                const int rt = b / KSK, ks = b % KSK, i = 16 * (rt % NT16) + l16;
                _Float16(*dst)[TS] = rt < NT16 ? sWT : sQT;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ch = 32 * ks + (e < 4 ? 4 * kg + e : 16 + 4 * kg + e - 4);
                    if (ch < D) dst[ch][i] = wq[j].v[e];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < KTB; ++j) {
            const int b = w + 4 * j;
            if (b < NTK * KSC) {
                const int tk = b / KSC, ks = b % KSC;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int i = 32 * ks + 8 * kg + e;
                    if (i < C) sKt[i][16 * tk + l16] = kt[j].v[e];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < GLE; ++j) {
            const int x = tid + kBwdThreads * j;
            if (x < D) sGL[x] = gl[j];
        }
#pragma unroll
        for (int j = 0; j < DOE; ++j) {
            const int x = tid + kBwdThreads * j;
            if (x < C * 16) {
                const _Float16 hi = static_cast<_Float16>(dO[j]);
                sdOh[x % 16][x / 16] = hi;
                sdOl[x % 16][x / 16] = static_cast<_Float16>(dO[j] - static_cast<float>(hi));
            }
        }
    }
};

template <int C, int D, bool BF>
__global__ void __launch_bounds__(kBwdThreads) bwd_state_kernel(BwdStateParams p) {
    using Frags = BwdFrags<C, D, BF>;
    constexpr int NT16 = C / 16, NTK = D / 16;
    constexpr int GS = D + 1, SS = 17;
    __shared__ float sW[C][GS], sQ[C][GS], sKt[C][GS];
    __shared__ float sdO[C][SS], sdS[D][SS], sX[C][SS];
    __shared__ float sGL[D];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    const int H = p.H;
    int n, h, ct;
    if (!state_unit<D / 16>(p.N, H, n, h, ct)) return;
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
    // this launch's chunks of the sequence: [cb, ce), walked backwards
    const int64_t cb = p.s0 > slot_base ? p.s0 - slot_base : 0;
    const int64_t ce = p.s1 - slot_base < nchunks ? p.s1 - slot_base : nchunks;
    if (nchunks == 0 ? !p.do_empty : cb >= ce) return;
    const int col = 16 * ct + l16;
    const size_t sbase = (static_cast<size_t>(n) * H + h) * D * D;
    auto pkg_of = [&](int64_t c) {
        return p.ws + (static_cast<size_t>(slot_base + c - p.s0) * H + h) * p.pkg_bytes;
    };
    auto nvalid_of = [&](int64_t c) { return static_cast<int>(L - c * C < C ? L - c * C : C); };

    // dS slab: wave w owns the 16-channel tiles tk = w, w + 4, ...; it starts
    // as the gradient of the state leaving chunk ce - 1 (the final state's, or
    // the one carried in from the slots after s1)
    const float *ds_in = ce == nchunks ? (p.d_final ? p.d_final + sbase : nullptr)
                                       : p.dcarry_in + static_cast<size_t>(h) * D * D;
    constexpr int SPW = (NTK + 3) / 4;
    f32x4 dS[SPW];
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl) {
        const int tk = w + 4 * sl;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dS[sl][r] = (tk < NTK && ds_in) ? ds_in[static_cast<size_t>(16 * tk + 4 * kg + r) * D + col] : 0.f;
    }

    Frags cur, nxt;
    if (ce > cb) cur.load(p, pkg_of(ce - 1), tok_base + (ce - 1) * C, nvalid_of(ce - 1), ct, h, tid);
    for (int64_t c = ce - 1; c >= cb; --c) {
        // dS1 of this chunk: to the chunk-state buffer and to LDS
        float *cds = p.chunk_dstates + (static_cast<size_t>(slot_base + c - p.s0) * H + h) * D * D;
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk < NTK) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * tk + 4 * kg + r;
                    cds[static_cast<size_t>(row) * D + col] = dS[sl][r];
                    sdS[row][l16] = dS[sl][r];
                }
            }
        }
        cur.template store<GS, SS>(sW, sQ, sKt, sGL, sdO, tid);
        if (c > cb) nxt.load(p, pkg_of(c - 1), tok_base + (c - 1) * C, nvalid_of(c - 1), ct, h, tid);
        __syncthreads();
        // X = Kt dS1 (C x 16), one 16-token tile per wave
        if (w < NT16) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mm_f32<D>(acc, [&](int r, int k) { return sKt[16 * w + r][k]; }, [&](int k, int nn) { return sdS[k][nn]; },
                      lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) sX[16 * w + 4 * kg + r][l16] = acc[r];
        }
        __syncthreads();
        // dS0 = Diag(Gamma_C) dS1 + Q'^T dO - W^T X
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk < NTK) {
                f32x4 acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = sGL[16 * tk + 4 * kg + r] * dS[sl][r];
                mm_f32<C>(acc, [&](int r, int k) { return sQ[k][16 * tk + r]; }, [&](int k, int nn) { return sdO[k][nn]; },
                          lane);
                mm_f32<C>(acc, [&](int r, int k) { return -sW[k][16 * tk + r]; }, [&](int k, int nn) { return sX[k][nn]; },
                          lane);
                dS[sl] = acc;
            }
        }
        __syncthreads();  // LDS is refilled by the next (earlier) chunk
        cur = nxt;
    }
    // the gradient of the state entering chunk cb: of the initial state, or
    // carried out to the slots before s0
    float *ds_out = cb == 0 ? (p.d_init ? p.d_init + sbase : nullptr)
                            : (p.dcarry_out ? p.dcarry_out + static_cast<size_t>(h) * D * D : nullptr);
    if (ds_out) {
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk < NTK) {
#pragma unroll
                for (int r = 0; r < 4; ++r) ds_out[static_cast<size_t>(16 * tk + 4 * kg + r) * D + col] = dS[sl][r];
            }
        }
    }
}

// The same reverse state pass on the 16-bit path with fp16 matrix cores: the
// package's W, Q' and Kt are fp16 values already, and each fp32 right-hand
// operand (dS1, dO, X) enters as an fp16 hi + lo pair, two products per K step
// of 32 instead of eight fp32 ones per 4.  Channel and token dimensions below
// 32 are padded with zeros to one K step.
template <int C, int D>
__global__ void __launch_bounds__(kBwdThreads) bwd_state_f16_kernel(BwdStateParams p) {
    using Frags = BwdFrags<C, D, true>;
    constexpr int NT16 = C / 16, NTK = D / 16;
    constexpr int CP = C < 32 ? 32 : C, DP = D < 32 ? 32 : D;
    constexpr int TS = CP + 8, CS = DP + 8;  // LDS row strides (fp16 elements)
    __shared__ __align__(16) _Float16 sWT[DP][TS], sQT[DP][TS];  // [channel][token]
    __shared__ __align__(16) _Float16 sKt[CP][CS];               // [token][channel]
    __shared__ __align__(16) _Float16 sdSh[16][CS], sdSl[16][CS];  // dS1 [column][channel]
    __shared__ __align__(16) _Float16 sdOh[16][TS], sdOl[16][TS];  // dO [column][token]
    __shared__ __align__(16) _Float16 sXh[16][TS], sXl[16][TS];    // -X [column][token]
    __shared__ float sGL[D];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;
    const int H = p.H;
    int n, h, ct;
    if (!state_unit<D / 16>(p.N, H, n, h, ct)) return;
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
    const int64_t cb = p.s0 > slot_base ? p.s0 - slot_base : 0;
    const int64_t ce = p.s1 - slot_base < nchunks ? p.s1 - slot_base : nchunks;
    if (nchunks == 0 ? !p.do_empty : cb >= ce) return;
    const int col = 16 * ct + l16;
    const size_t sbase = (static_cast<size_t>(n) * H + h) * D * D;
    auto pkg_of = [&](int64_t c) {
        return p.ws + (static_cast<size_t>(slot_base + c - p.s0) * H + h) * p.pkg_bytes;
    };
    auto nvalid_of = [&](int64_t c) { return static_cast<int>(L - c * C < C ? L - c * C : C); };

    // the padding (channels >= D, tokens >= C) stays zero; the rest is
    // rewritten every chunk
    for (int x = tid; x < DP * TS; x += kBwdThreads) {
        (&sWT[0][0])[x] = _Float16(0.f);
        (&sQT[0][0])[x] = _Float16(0.f);
    }
    for (int x = tid; x < CP * CS; x += kBwdThreads) (&sKt[0][0])[x] = _Float16(0.f);
    for (int x = tid; x < 16 * CS; x += kBwdThreads) (&sdSh[0][0])[x] = (&sdSl[0][0])[x] = _Float16(0.f);
    for (int x = tid; x < 16 * TS; x += kBwdThreads) {
        (&sdOh[0][0])[x] = (&sdOl[0][0])[x] = _Float16(0.f);
        (&sXh[0][0])[x] = (&sXl[0][0])[x] = _Float16(0.f);
    }

    const float *ds_in = ce == nchunks ? (p.d_final ? p.d_final + sbase : nullptr)
                                       : p.dcarry_in + static_cast<size_t>(h) * D * D;
    constexpr int SPW = (NTK + 3) / 4;
    f32x4 dS[SPW];
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl) {
        const int tk = w + 4 * sl;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dS[sl][r] = (tk < NTK && ds_in) ? ds_in[static_cast<size_t>(16 * tk + 4 * kg + r) * D + col] : 0.f;
    }
    __syncthreads();  // the zero fill is done before any chunk's writes

    Frags cur, nxt;
    if (ce > cb) cur.load(p, pkg_of(ce - 1), tok_base + (ce - 1) * C, nvalid_of(ce - 1), ct, h, tid);
    for (int64_t c = ce - 1; c >= cb; --c) {
        // dS1 of this chunk: to the chunk-state buffer and, as hi + lo, to LDS
        float *cds = p.chunk_dstates + (static_cast<size_t>(slot_base + c - p.s0) * H + h) * D * D;
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk < NTK) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * tk + 4 * kg + r;
                    cds[static_cast<size_t>(row) * D + col] = dS[sl][r];
                    const _Float16 hi = static_cast<_Float16>(dS[sl][r]);
                    sdSh[l16][row] = hi;
                    sdSl[l16][row] = static_cast<_Float16>(dS[sl][r] - static_cast<float>(hi));
                }
            }
        }
        cur.template store16<TS, CS>(sWT, sQT, sKt, sGL, sdOh, sdOl, tid);
        if (c > cb) nxt.load(p, pkg_of(c - 1), tok_base + (c - 1) * C, nvalid_of(c - 1), ct, h, tid);
        __syncthreads();
        // -X = -(Kt dS1) (C x 16), one 16-token tile per wave, into LDS as hi + lo
        if (w < NT16) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DP / 32; ++ks) {
                const f16x8 a = *reinterpret_cast<const f16x8 *>(&sKt[16 * w + l16][32 * ks + 8 * kg]);
                const f16x8 bh = *reinterpret_cast<const f16x8 *>(&sdSh[l16][32 * ks + 8 * kg]);
                const f16x8 bl = *reinterpret_cast<const f16x8 *>(&sdSl[l16][32 * ks + 8 * kg]);
                acc = mfma_f16(a, bl, acc);
                acc = mfma_f16(a, bh, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = -acc[r];
                const _Float16 hi = static_cast<_Float16>(x);
                sXh[l16][16 * w + 4 * kg + r] = hi;
                sXl[l16][16 * w + 4 * kg + r] = static_cast<_Float16>(x - static_cast<float>(hi));
            }
        }
        __syncthreads();
        // dS0 = Diag(Gamma_C) dS1 + Q'^T dO + W^T (-X)
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk < NTK) {
                f32x4 acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = sGL[16 * tk + 4 * kg + r] * dS[sl][r];
#pragma unroll
                for (int ks = 0; ks < CP / 32; ++ks) {
                    const f16x8 aq = *reinterpret_cast<const f16x8 *>(&sQT[16 * tk + l16][32 * ks + 8 * kg]);
                    const f16x8 aw = *reinterpret_cast<const f16x8 *>(&sWT[16 * tk + l16][32 * ks + 8 * kg]);
                    acc = mfma_f16(aq, *reinterpret_cast<const f16x8 *>(&sdOl[l16][32 * ks + 8 * kg]), acc);
                    acc = mfma_f16(aw, *reinterpret_cast<const f16x8 *>(&sXl[l16][32 * ks + 8 * kg]), acc);
                    acc = mfma_f16(aq, *reinterpret_cast<const f16x8 *>(&sdOh[l16][32 * ks + 8 * kg]), acc);
                    acc = mfma_f16(aw, *reinterpret_cast<const f16x8 *>(&sXh[l16][32 * ks + 8 * kg]), acc);
                }
                dS[sl] = acc;
            }
        }
        __syncthreads();  // LDS is refilled by the next (earlier) chunk
        cur = nxt;
    }
    float *ds_out = cb == 0 ? (p.d_init ? p.d_init + sbase : nullptr)
                            : (p.dcarry_out ? p.dcarry_out + static_cast<size_t>(h) * D * D : nullptr);
    if (ds_out) {
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int tk = w + 4 * sl;
            if (tk < NTK) {
#pragma unroll
                for (int r = 0; r < 4; ++r) ds_out[static_cast<size_t>(16 * tk + 4 * kg + r) * D + col] = dS[sl][r];
            }
        }
    }
}

// -----------------------------------------------------------------------------
// gradients of one (chunk, head) at a time; persistent workgroups
// -----------------------------------------------------------------------------
// Per-workgroup fp32 [C][D] scratch matrices in the workspace.
enum Scratch { kKG, kKT, kR, kU, kDU, kDR, kNumScratch };
static_assert(kNumScratch == kBwdScratchMats, "scratch matrices per workgroup");

constexpr int kBwdIntraThreads = 512;  // 8 waves: two per SIMD hide the products' memory latency
// On a diagonal 16-token block the decay-weighted products go through the
// matrix cores with the block's token 7 as the reference: a channel whose
// cumulative log-decay spans more than this on either side of it (factors up
// to e^40) takes the exact per-pair path instead.
constexpr float kDiagSpan = 40.0f;
constexpr int kIW = kBwdIntraThreads / 64;

template <int C, int D, bool BF>
__global__ void __launch_bounds__(kBwdIntraThreads) intra_bwd_kernel(BwdIntraParams p, int64_t n_items) {
    using In = std::conditional_t<BF, uint16_t, float>;
    // The cumulative decay G is held in fp64 on the fp32-input path: every decay
    // factor is e^(G_i - G_j), and G_i, G_j of a chunk reach |G| ~ 10^2, so their
    // fp32 roundings would put ~|G| 2^-24 into each factor (and the reverse sum
    // of dG cancels); the difference is formed in fp64, the exponential in fp32.
    using GT = std::conditional_t<BF, float, double>;
    constexpr int GS = D + 1, MS = C + 1, NTI = C / 16, NTD = D / 16, NBI = C / 4;
    constexpr int NBLK = NBI * (NBI + 1) / 2;
    static_assert(NBLK <= kBwdIntraThreads, "one 4x4 block of the Gram matrices per thread");
    __shared__ GT sG[C][GS];
    __shared__ In sK[C][GS], sQ[C][GS];
    __shared__ float sM[4][C][MS];  // Abar; P -> dT -> dAbar; T; Y -> dP
    __shared__ float sBeta[C];
    __shared__ int sCnt[C], sNotRst[C];
    __shared__ float sGC[D];
    __shared__ float sPart[C][NTD], sPart2[C][NTI];
    __shared__ int sFirst, sLast;
    __shared__ uint8_t sNegInf[C][D];  // log_alpha is -inf here (its gradient is 0)
    // the cumulative decay and the reverse cumulative sum of dG run in NSEG
    // segments of RPS tokens per channel
    constexpr int NSEG = kBwdIntraThreads / D < C / 4 ? kBwdIntraThreads / D : C / 4, RPS = C / NSEG;
    __shared__ GT sSegG[NSEG][D];
    static_assert(NSEG * D <= kBwdIntraThreads && RPS <= 16, "cumulative sum layout");
    static_assert(NSEG * D * sizeof(GT) <= 4 * C * MS * sizeof(float), "segment sums fit in sM");

    const int H = p.H;
    float *scr = p.scratch + static_cast<size_t>(blockIdx.x) * kNumScratch * C * D;
    auto S_ = [&](int m) { return scr + static_cast<size_t>(m) * C * D; };
    float *KG = S_(kKG), *KT = S_(kKT), *R = S_(kR), *U = S_(kU), *DU = S_(kDU), *DR = S_(kDR);
    auto toF = [](In x) {
        if constexpr (BF) return bf16_bits_to_f32(x);
        else return x;
    };

    for (int64_t item = p.item0 + blockIdx.x; item < n_items; item += gridDim.x) {
        // lane-dependent addresses are recomputed per item: hoisted out of the
        // loop they would be held in registers across all of it
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int l16 = lane & 15, kg = lane >> 4;
        int64_t slot, hh;
        divmod_nonneg(item, H, slot, hh);
        const int h = static_cast<int>(hh);
        int64_t tok0;
        int nvalid;
        if (!locate_chunk(slot, C, p.T, p.N, p.cu_seqlens, p.chunk_offsets, tok0, nvalid)) break;
        const float *S0 = p.chunk_states + (static_cast<size_t>(slot - p.s0) * H + h) * D * D;
        const float *dS1 = p.chunk_dstates + (static_cast<size_t>(slot - p.s0) * H + h) * D * D;
        auto row_of = [&](int i) { return (tok0 + i) * H + h; };
        // loads of token i's inputs are unconditional, from a row inside the chunk,
        // and the value selected after them (a load under a branch waits before
        // the branch rejoins, which serialises a batch of them)
        auto rowc = [&](int i) { return row_of(i < nvalid ? i : nvalid - 1); };
        auto dO_at = [&](int i, int col) {
            const float x = p.d_o[rowc(i) * D + col];
            return i < nvalid ? x : 0.f;
        };
        auto dO4 = [&](int i, int col) {
            const f32x4 x = ld4(p.d_o + rowc(i) * D + col);
            return i < nvalid ? x : f32x4{0.f, 0.f, 0.f, 0.f};
        };

        // ---- inputs, resets, cumulative decay (natural-log units)
#pragma unroll
        for (int x = tid; x < C * D; x += kBwdIntraThreads) {
            const int i = x / D, c = x % D;
            const bool ok = i < nvalid;
            const int64_t o = row_of(ok ? i : 0) * D + c;
            sK[i][c] = ok ? static_cast<const In *>(p.k)[o] : In(0);
            sQ[i][c] = ok ? static_cast<const In *>(p.q)[o] : In(0);
            sG[i][c] = ok ? static_cast<GT>(p.log_alpha[o]) : GT(0);
        }
        for (int i = tid; i < C; i += kBwdIntraThreads) {
            sBeta[i] = i < nvalid ? p.beta[row_of(i)] : 0.f;
            sNotRst[i] = i < nvalid ? 0 : 1;
        }
        for (int x = tid; x < C * 4 * MS; x += kBwdIntraThreads) (&sM[0][0][0])[x] = 0.f;
        __syncthreads();
        for (int x = tid; x < C * D; x += kBwdIntraThreads) {
            const int i = x / D, c = x % D;
            const bool ninf = i < nvalid && sG[i][c] == static_cast<GT>(kNegInf);
            if (i < nvalid && !ninf) sNotRst[i] = 1;
            sNegInf[i][c] = ninf ? 1 : 0;
        }
        __syncthreads();
        // cumulative decay: NSEG segments of RPS tokens per channel, then each
        // segment adds the totals before it; reset counts by one wave-wide ballot
        {
            const int c = tid % D, sg = tid / D;
            if (sg < NSEG) {
                GT acc = 0;
                for (int x = 0; x < RPS; ++x) {
                    const int i = sg * RPS + x;
                    acc += sNotRst[i] ? (sG[i][c] > GT(kGFloor) ? sG[i][c] : GT(kGFloor)) : GT(0);
                    sG[i][c] = acc;
                }
                sSegG[sg][c] = acc;
            }
            if (w == kIW - 1) {
                const unsigned long long rm = __ballot(lane < C && !sNotRst[lane]);
                if (lane < C) sCnt[lane] = __popcll(rm & ((2ull << lane) - 1ull));
                if (lane == 0) {
                    sFirst = rm ? __ffsll(static_cast<long long>(rm)) - 1 : C;
                    sLast = rm ? 63 - __clzll(rm) : -1;
                }
            }
            __syncthreads();
            if (sg > 0 && sg < NSEG) {
                GT off = 0;
                for (int q = 0; q < sg; ++q) off += sSegG[q][c];
                for (int x = 0; x < RPS; ++x) sG[sg * RPS + x][c] += off;
            }
        }
        __syncthreads();
        const int first_rst = sFirst, last_rst = sLast;

        // ---- K*Gamma and Kt (scratch: left operands of the products below); Gamma_C
        for (int x = tid; x < C * D; x += kBwdIntraThreads) {
            const int i = x / D, c = x % D;
            const GT G = sG[i][c];
            const float kv = toF(sK[i][c]);
            const float eg = i < first_rst ? __expf(static_cast<float>(G)) : 0.f;
            KG[x] = kv * eg;
            KT[x] = i >= last_rst ? kv * __expf(static_cast<float>(sG[C - 1][c] - G)) : 0.f;
        }
        for (int c = tid; c < D; c += kBwdIntraThreads)
            sGC[c] = last_rst >= 0 ? 0.f : __expf(static_cast<float>(sG[C - 1][c]));

        // ---- Abar (strictly lower) and P (lower).  Blocks below the diagonal on
        //      the fp32 matrix cores, one 16x16 block pair per wave: with m = the
        //      last token of block J, Abar_IJ = (e^{G_I - G_m} * K_I)(e^{G_m - G_J} * K_J)^T
        //      and P_IJ the same with Q_I, both factors <= 1.  The diagonal blocks'
        //      pairs with the exact exponential per term: one 4x4 sub-block per
        //      thread, its channels in four quarters whose sums meet in LDS (over
        //      sM[2] and sM[3], not yet in use) and are added in a fixed order.
        {
            constexpr int NPAIR = NTI * (NTI - 1) / 2;
            auto pair_job = [&](int pr) {
                int I = 1, J = pr;
                while (J >= I) { J -= I; ++I; }
                const int m = 16 * J + 15, i = 16 * I + l16, j = 16 * J + l16;
                f32x4 acA = {0.f, 0.f, 0.f, 0.f}, acP = acA;
#pragma unroll 4
                for (int s4 = 0; s4 < D / 4; ++s4) {
                    const int c = 4 * s4 + kg;
                    const GT Gm = sG[m][c];
                    const float fa = __expf(static_cast<float>(sG[i][c] - Gm));
                    const float fb = __expf(static_cast<float>(Gm - sG[j][c])) * toF(sK[j][c]);
                    acA = __builtin_amdgcn_mfma_f32_16x16x4f32(fa * toF(sK[i][c]), fb, acA, 0, 0, 0);
                    acP = __builtin_amdgcn_mfma_f32_16x16x4f32(fa * toF(sQ[i][c]), fb, acP, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ii = 16 * I + 4 * kg + r;
                    const bool nores = sCnt[ii] == sCnt[j];
                    sM[0][ii][j] = nores ? acA[r] : 0.f;
                    sM[1][ii][j] = nores ? acP[r] : 0.f;
                }
            };
            if constexpr (BF) {
            // 16-bit path: the diagonal blocks on the matrix cores too, with the
            // block's token 7 as the reference (factors up to e^kDiagSpan); a
            // channel spanning more on either side of it is left out of the
            // products and added with the exact exponential of every pair.  Jobs:
            // the NPAIR blocks below the diagonal, then the NTI diagonal ones.
            for (int jb = w; jb < NPAIR + NTI; jb += kIW) {
                if (jb < NPAIR) {
                    pair_job(jb);
                    continue;
                }
                const int J = jb - NPAIR, m = 16 * J + 7, j = 16 * J + l16;
                f32x4 acA = {0.f, 0.f, 0.f, 0.f}, acP = acA;
                constexpr int NWD = (D + 31) / 32, SPW = D / 4 < 8 ? D / 4 : 8;  // words, 4-channel steps per word
                uint32_t uns[NWD];  // bit c % 32 of word c / 32: channel c left out
#pragma unroll
                for (int wd = 0; wd < NWD; ++wd) {
                    uint32_t bits = 0u;
#pragma unroll 4
                    for (int s8 = 0; s8 < SPW; ++s8) {
                        const int c = 32 * wd + 4 * s8 + kg;
                        const GT Gm = sG[m][c];
                        const bool safe = sG[16 * J][c] - Gm <= GT(kDiagSpan) && Gm - sG[16 * J + 15][c] <= GT(kDiagSpan);
                        const float fa = safe ? __expf(static_cast<float>(sG[j][c] - Gm)) : 0.f;
                        const float fb = safe ? __expf(static_cast<float>(Gm - sG[j][c])) * toF(sK[j][c]) : 0.f;
                        acA = __builtin_amdgcn_mfma_f32_16x16x4f32(fa * toF(sK[j][c]), fb, acA, 0, 0, 0);
                        acP = __builtin_amdgcn_mfma_f32_16x16x4f32(fa * toF(sQ[j][c]), fb, acP, 0, 0, 0);
                        const uint64_t ub = __ballot(!safe);  // lane 16 g: channel 32 wd + 4 s8 + g
                        const uint32_t nib = static_cast<uint32_t>((ub & 1u) | ((ub >> 15) & 2u) | ((ub >> 30) & 4u) |
                                                                   ((ub >> 45) & 8u));
                        bits |= nib << (4 * s8);
                    }
                    uns[wd] = bits;
                }
#pragma unroll
                for (int wd = 0; wd < NWD; ++wd) {
                    uint32_t bits = uns[wd];
                    while (bits) {  // rare
                        const int ch = 32 * wd + __builtin_ctz(bits);
                        bits &= bits - 1u;
                        const GT Gj = sG[j][ch];
                        const float kj = toF(sK[j][ch]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int ii = 16 * J + 4 * kg + r;
                            const float e = __expf(fminf(static_cast<float>(sG[ii][ch] - Gj), 0.f)) * kj;
                            acA[r] += toF(sK[ii][ch]) * e;
                            acP[r] += toF(sQ[ii][ch]) * e;
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ii = 16 * J + 4 * kg + r;
                    const bool nores = sCnt[ii] == sCnt[j];
                    sM[0][ii][j] = (j < ii && nores) ? acA[r] : 0.f;
                    sM[1][ii][j] = (j <= ii && nores) ? acP[r] : 0.f;
                }
            }
            } else {
            for (int pr = w; pr < NPAIR; pr += kIW) pair_job(pr);
            constexpr int NSB = NTI * 10;
            constexpr int NQ = (4 * NSB <= kBwdIntraThreads && 3 * NSB * 32 <= 2 * C * MS) ? 4
                             : (2 * NSB <= kBwdIntraThreads && NSB * 32 <= 2 * C * MS) ? 2 : 1;
            constexpr int CQ = D / NQ, NP = NQ > 1 ? NQ - 1 : 1;
            static_assert(NSB * NP * 32 <= 2 * C * MS, "the partial sums fit in two C x C buffers");
            float(*part)[NP][32] = reinterpret_cast<float(*)[NP][32]>(&sM[2][0][0]);
            const int sb = tid % NSB, qt = tid / NSB;
            int li = 0, lj = sb % 10;  // sub-block (li, lj), li >= lj, of diagonal block sb / 10
            while (lj > li) { lj -= li + 1; ++li; }
            const int bi = 4 * (sb / 10) + li, bj = 4 * (sb / 10) + lj;
            float a[4][4] = {}, pp[4][4] = {};
            if (tid < NQ * NSB) {
#pragma unroll 4
                for (int c = qt * CQ; c < (qt + 1) * CQ; ++c) {
                    GT gi[4], gj[4];
                    float ki[4], kj[4], qi[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        gi[x] = sG[4 * bi + x][c];
                        gj[x] = sG[4 * bj + x][c];
                        ki[x] = toF(sK[4 * bi + x][c]);
                        kj[x] = toF(sK[4 * bj + x][c]);
                        qi[x] = toF(sQ[4 * bi + x][c]);
                    }
#pragma unroll
                    for (int x = 0; x < 4; ++x)
#pragma unroll
                        for (int y = 0; y < 4; ++y) {
                            const float e = __expf(fminf(static_cast<float>(gi[x] - gj[y]), 0.f)) * kj[y];
                            a[x][y] += ki[x] * e;
                            pp[x][y] += qi[x] * e;
                        }
                }
                if (qt > 0) {
#pragma unroll
                    for (int x = 0; x < 4; ++x)
#pragma unroll
                        for (int y = 0; y < 4; ++y) {
                            part[sb][qt - 1][4 * x + y] = a[x][y];
                            part[sb][qt - 1][16 + 4 * x + y] = pp[x][y];
                        }
                }
            }
            __syncthreads();
            if (tid < NSB) {
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int y = 0; y < 4; ++y) {
#pragma unroll
                        for (int q = 1; q < NQ; ++q) {
                            a[x][y] += part[sb][q - 1][4 * x + y];
                            pp[x][y] += part[sb][q - 1][16 + 4 * x + y];
                        }
                        const int i = 4 * bi + x, j = 4 * bj + y;
                        const bool nores = sCnt[i] == sCnt[j];
                        sM[0][i][j] = (j < i && nores) ? a[x][y] : 0.f;
                        sM[1][i][j] = (j <= i && nores) ? pp[x][y] : 0.f;
                    }
            }
            }
        }
        __syncthreads();

        // ---- T = (I + A)^-1 with A = Diag(beta) Abar, in place in sM[2]: the
        //      16x16 diagonal blocks by forward substitution (one wave each, one
        //      column per lane), then T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ on
        //      the fp32 matrix cores, one block row at a time
        for (int x = tid; x < C * C; x += kBwdIntraThreads) {
            const int i = x / C, j = x % C;
            sM[2][i][j] = sBeta[i] * sM[0][i][j];
        }
        __syncthreads();
        if (w < NTI && lane < 16) {
            const int base = 16 * w, col = lane;
            float tv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float val = (i == col) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) val -= sM[2][base + i][base + j] * tv[j];
                tv[i] = val;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sM[2][base + i][base + col] = i >= col ? tv[i] : 0.f;
        }
        __syncthreads();
        for (int I = 1; I < NTI; ++I) {
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            const int J = w;
            if (J < I) {
                f32x4 xv = {0.f, 0.f, 0.f, 0.f};
                for (int K = J; K < I; ++K)
                    mm_f32<16>(xv, [&](int r, int k) { return sM[2][16 * I + r][16 * K + k]; },
                               [&](int k, int nn) { return sM[2][16 * K + k][16 * J + nn]; }, lane);
                // y = T_II xv: xv's rows come back through LDS-free lane exchange
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[2][16 * I + l16][16 * I + 4 * kg + r], xv[r], y, 0, 0, 0);
            }
            __syncthreads();
            if (J < I) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sM[2][16 * I + 4 * kg + r][16 * J + l16] = -y[r];
            }
            __syncthreads();
        }  // also: K*Gamma, Kt written

        // ---- R = V - (K*Gamma) S0
                // (the column tile of every tile a wave takes, t = w + 8 m, is w % NTD: NTD
        //  divides 8, so each wave loads its right-hand operand once per product)
        static_assert(kIW % NTD == 0 && kIW % NTI == 0, "column tiles divide the waves");
        const Frag<D> bS0 = frag_of<D>([&](int k0, int nn) {
            const float *b = S0 + static_cast<size_t>(k0) * D + 16 * (w % NTD) + nn;
            return f32x4{b[0], b[D], b[2 * D], b[3 * D]};
        }, lane);
        tiles_vb<D>(w, NTI * NTD, kIW,
            [&](int t, int r, int k0) { return ld4(KG + (16 * (t / NTD) + r) * D + k0); }, bS0,
            [&](int t) {
                f32x4 vv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * (t / NTD) + 4 * kg + r, cc = 16 * (t % NTD) + l16;
                    const float x = toF(static_cast<const In *>(p.v)[rowc(i) * D + cc]);
                    vv[r] = i < nvalid ? x : 0.f;
                }
                return vv;
            },
            [&](int t, const f32x4 &acc, const f32x4 &vv) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * (t / NTD) + 4 * kg + r, cc = 16 * (t % NTD) + l16;
                    R[i * D + cc] = vv[r] - acc[r];
                }
            }, lane);
        __syncthreads();
        // ---- U = T Diag(beta) R;  dU = P^T dO + Kt dS1
                {
            const int tdw = w % NTD;
            const Frag<C> bX = frag_of<C>([&](int k0, int nn) {
                const float *b = R + k0 * D + 16 * tdw + nn;
                return f32x4{sBeta[k0] * b[0], sBeta[k0 + 1] * b[D], sBeta[k0 + 2] * b[2 * D], sBeta[k0 + 3] * b[3 * D]};
            }, lane);
            const Frag<C> bO = frag_of<C>([&](int k0, int nn) {
                return f32x4{dO_at(k0, 16 * tdw + nn), dO_at(k0 + 1, 16 * tdw + nn), dO_at(k0 + 2, 16 * tdw + nn),
                             dO_at(k0 + 3, 16 * tdw + nn)};
            }, lane);
            const Frag<D> bS1 = frag_of<D>([&](int k0, int nn) {
                const float *b = dS1 + static_cast<size_t>(k0) * D + 16 * tdw + nn;
                return f32x4{b[0], b[D], b[2 * D], b[3 * D]};
            }, lane);
#pragma unroll 1
        for (int t = w; t < NTI * NTD; t += kIW) {
            const int ti = t / NTD, td = t % NTD;
            f32x4 u = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
            mm_f32_vb<C>(u, [&](int r, int k0) {
                const float *a = &sM[2][16 * ti + r][k0];
                return f32x4{a[0], a[1], a[2], a[3]};
            }, bX, lane);
            mm_f32_vb<C>(du, [&](int r, int k0) {
                return f32x4{sM[1][k0][16 * ti + r], sM[1][k0 + 1][16 * ti + r], sM[1][k0 + 2][16 * ti + r],
                             sM[1][k0 + 3][16 * ti + r]};
            }, bO, lane);
            mm_f32_vb<D>(du, [&](int r, int k0) { return ld4(KT + (16 * ti + r) * D + k0); }, bS1, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ti + 4 * kg + r, cc = 16 * td + l16;
                U[i * D + cc] = u[r];
                DU[i * D + cc] = du[r];
            }
        }
        }
        __syncthreads();
        // ---- dX = T^T dU;  dR = dV = Diag(beta) dX;  dbeta (value part)
                const Frag<C> bDU = frag_of<C>([&](int k0, int nn) {
            const float *b = DU + k0 * D + 16 * (w % NTD) + nn;
            return f32x4{b[0], b[D], b[2 * D], b[3 * D]};
        }, lane);
#pragma unroll 1
        for (int t = w; t < NTI * NTD; t += kIW) {
            const int ti = t / NTD, td = t % NTD;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mm_f32_vb<C>(acc, [&](int r, int k0) {
                return f32x4{sM[2][k0][16 * ti + r], sM[2][k0 + 1][16 * ti + r], sM[2][k0 + 2][16 * ti + r],
                             sM[2][k0 + 3][16 * ti + r]};
            }, bDU, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ti + 4 * kg + r, cc = 16 * td + l16;
                const float dr = sBeta[i] * acc[r];
                DR[i * D + cc] = dr;
                if (i < nvalid) p.dv[row_of(i) * D + cc] = dr;
                const float part = sum16(R[i * D + cc] * acc[r]);
                if (l16 == 0) sPart[i][td] = part;
            }
        }
        // ---- dT = dU X^T (into P's buffer: P is no longer needed)
                const Frag<D> bXT = frag_of<D>([&](int k0, int nn) {
            const int j = 16 * (w % NTI) + nn;
            return sBeta[j] * ld4(R + j * D + k0);
        }, lane);
        tiles_vb<D>(w, NTI * NTI, kIW,
            [&](int t, int r, int k0) { return ld4(DU + (16 * (t / NTI) + r) * D + k0); }, bXT,
            [&](int) { return f32x4{0.f, 0.f, 0.f, 0.f}; },
            [&](int t, const f32x4 &acc, const f32x4 &) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sM[3][16 * (t / NTI) + 4 * kg + r][16 * (t % NTI) + l16] = acc[r];
            }, lane);
        __syncthreads();
        // Y = dT T^T  (dT in sM[3] for now, Y into sM[1])
        #pragma unroll 1
        for (int t = w; t < NTI * NTI; t += kIW) {
            const int ti = t / NTI, tj = t % NTI;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mm_f32<C>(acc, [&](int r, int k) { return sM[3][16 * ti + r][k]; },
                      [&](int k, int nn) { return sM[2][16 * tj + nn][k]; }, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) sM[1][16 * ti + 4 * kg + r][16 * tj + l16] = acc[r];
        }
        __syncthreads();
        // dA = -T^T Y (strictly lower, no reset in (j, i]) into sM[3]; dbeta (gate
        // part) = sum_j dA_ij Abar_ij; then dAbar = Diag(beta) dA in place
        #pragma unroll 1
        for (int t = w; t < NTI * NTI; t += kIW) {
            const int ti = t / NTI, tj = t % NTI;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mm_f32<C>(acc, [&](int r, int k) { return sM[2][k][16 * ti + r]; },
                      [&](int k, int nn) { return sM[1][k][16 * tj + nn]; }, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ti + 4 * kg + r, j = 16 * tj + l16;
                const float da = (j < i && sCnt[i] == sCnt[j]) ? -acc[r] : 0.f;
                const float part = sum16(da * sM[0][i][j]);
                if (l16 == 0) sPart2[i][tj] = part;
                sM[3][i][j] = sBeta[i] * da;
            }
        }
        __syncthreads();
        // ---- dP = dO U^T (lower, no reset in (j, i]) into sM[1]
                const Frag<D> bUT = frag_of<D>([&](int k0, int nn) { return ld4(U + (16 * (w % NTI) + nn) * D + k0); }, lane);
        tiles_vb<D>(w, NTI * NTI, kIW,
            [&](int t, int r, int k0) { return dO4(16 * (t / NTI) + r, k0); }, bUT,
            [&](int) { return f32x4{0.f, 0.f, 0.f, 0.f}; },
            [&](int t, const f32x4 &acc, const f32x4 &) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * (t / NTI) + 4 * kg + r, j = 16 * (t % NTI) + l16;
                    sM[1][i][j] = (j <= i && sCnt[i] == sCnt[j]) ? acc[r] : 0.f;
                }
            }, lane);
        // From here to dlog_alpha, wave w < NTD owns the 16-channel column tile w
        // for every token and keeps dq, dk and dG of its tile in registers:
        // element r of tile I is token 16 I + 4 (lane / 16) + r, channel
        // 16 w + lane % 16 (the matrix cores' output layout).
        f32x4 DQr[NTI], DKr[NTI], DGr[NTI];
        // dG of the chunk's last token at this lane's channel (wave w < NTD):
        // dGamma_C = rowsum(S0 * dS1) times Gamma_C, plus the dKt terms
        float dgl = 0.f;
        // ---- d(Q*Gamma) = dO S0^T, d(K*Gamma) = -dR S0^T, dKt = U dS1^T and
        //      their Gamma terms
        if (w < NTD) {
            const int c = 16 * w + l16;  // this lane's channel
            const Frag<D> bS0T = frag_of<D>([&](int k0, int nn) {
                return ld4(S0 + static_cast<size_t>(16 * w + nn) * D + k0);
            }, lane);
            const Frag<D> bS1T = frag_of<D>([&](int k0, int nn) {
                return ld4(dS1 + static_cast<size_t>(16 * w + nn) * D + k0);
            }, lane);
            // row c of S0 and dS1 are in the two fragments already: this lane holds
            // columns 16 t + 4 (lane / 16) + j, the four lanes of row c all of them
            {
                float rs = 0.f;
#pragma unroll
                for (int t = 0; t < D / 16; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) rs += bS0T.v[t][j] * bS1T.v[t][j];
                rs += __shfl_xor(rs, 16);
                rs += __shfl_xor(rs, 32);
                dgl = rs * sGC[c];
            }
            // the 3 NTI products dO_I S0^T, dR_I S0^T, U_I dS1^T in that order, each
            // one's left-hand rows loaded while the product before it runs
            constexpr int NKT = D / 16;
            f32x4 Ab[2][NKT];
            auto lda = [&](int pidx, f32x4 (&a)[NKT]) {
                const int ti = pidx / 3, which = pidx % 3, row = 16 * ti + l16;
#pragma unroll
                for (int t = 0; t < NKT; ++t) {
                    const int k0 = 16 * t + 4 * kg;
                    if (which == 0) a[t] = dO4(row, k0);
                    else a[t] = ld4((which == 1 ? DR : U) + row * D + k0);
                }
            };
            auto mma_pre = [&](f32x4 &acc, const f32x4 (&a)[NKT], const Frag<D> &bf) {
#pragma unroll
                for (int t = 0; t < NKT; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t][j], bf.v[t][j], acc, 0, 0, 0);
            };
            lda(0, Ab[0]);
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti) {
                f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = aq, at = aq;
                const int p0 = 3 * ti;
                lda(p0 + 1, Ab[(p0 + 1) & 1]);
                mma_pre(aq, Ab[p0 & 1], bS0T);
                lda(p0 + 2, Ab[(p0 + 2) & 1]);
                mma_pre(ak, Ab[(p0 + 1) & 1], bS0T);
                if (ti + 1 < NTI) lda(p0 + 3, Ab[(p0 + 3) & 1]);
                mma_pre(at, Ab[(p0 + 2) & 1], bS1T);
                float colsum = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * ti + 4 * kg + r;
                    // Q*Gamma, K*Gamma and Kt at (i, c), formed from LDS
                    const float eg = i < first_rst ? __expf(static_cast<float>(sG[i][c])) : 0.f;
                    const float et = i >= last_rst ? __expf(static_cast<float>(sG[C - 1][c] - sG[i][c])) : 0.f;
                    const float kv = toF(sK[i][c]);
                    const float qg = i < first_rst ? toF(sQ[i][c]) * eg : 0.f, kgm = i < first_rst ? kv * eg : 0.f;
                    const float ktv = i >= last_rst ? kv * et : 0.f;
                    DQr[ti][r] = aq[r] * eg;
                    DKr[ti][r] = -ak[r] * eg + at[r] * et;
                    DGr[ti][r] = aq[r] * qg - ak[r] * kgm - at[r] * ktv;
                    colsum += at[r] * ktv;
                }
                colsum += __shfl_xor(colsum, 16);
                colsum += __shfl_xor(colsum, 32);
                dgl += colsum;
            }
        }
        __syncthreads();  // dP complete
        // ---- the decay-weighted products e^{G_i - G_j} of dP (with q_i, k_j) and
        //      dAbar (with k_i, k_j), on the fp32 matrix cores, one 16-token block
        //      pair (I >= J) at a time.  With a reference token m,
        //      e^{G_i - G_j} = e^{G_i - G_m} e^{G_m - G_j}, so (dM = dP with X = Q,
        //      dM = dAbar with X = K)
        //        row sums of block I    += e^{G_I - G_m} * (dM_IJ (e^{G_m - G_J} * K_J))
        //        column sums of block J += e^{G_m - G_J} * (dM_IJ^T (e^{G_I - G_m} * X_I)).
        //      Below the diagonal m is the last token of J and both factors are
        //      <= 1.  On the diagonal m is the block's token 7 and the factors
        //      are bounded by e^{half-span}; a channel whose half-span there
        //      exceeds kDiagSpan takes the exact exponential of every pair
        //      instead (its matrix-core operands are zero), and so does every
        //      channel on the fp32-input path, where the two-factor form's extra
        //      rounding would be a visible part of the tighter bound.
        if (w < NTD) {
            const int c = 16 * w + l16;  // this lane's channel
            f32x4 rP[NTI], rA[NTI], cS[NTI];  // row sums of dP, dAbar; column sums of both
#pragma unroll
            for (int I = 0; I < NTI; ++I) rP[I] = rA[I] = cS[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int J = 0; J < NTI; ++J) {
                // diagonal block J
                {
                    const int m = 16 * J + 7;
                    const GT Gm = sG[m][c];
                    const bool safe = BF && sG[16 * J][c] - Gm <= GT(kDiagSpan) && Gm - sG[16 * J + 15][c] <= GT(kDiagSpan);
                    float ys[4], xq[4], xk[4];
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        const int j = 16 * J + 4 * s4 + kg;
                        const float kj = toF(sK[j][c]);
                        const float fb = safe ? __expf(static_cast<float>(Gm - sG[j][c])) : 0.f;
                        const float fa = safe ? __expf(static_cast<float>(sG[j][c] - Gm)) : 0.f;
                        ys[s4] = fb * kj;
                        xq[s4] = fa * toF(sQ[j][c]);
                        xk[s4] = fa * kj;
                    }
                    f32x4 zp = {0.f, 0.f, 0.f, 0.f}, za = zp, wp = zp, wa = zp;
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        zp = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[1][16 * J + l16][16 * J + 4 * s4 + kg], ys[s4], zp, 0, 0, 0);
                        za = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[3][16 * J + l16][16 * J + 4 * s4 + kg], ys[s4], za, 0, 0, 0);
                        wp = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[1][16 * J + 4 * s4 + kg][16 * J + l16], xq[s4], wp, 0, 0, 0);
                        wa = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[3][16 * J + 4 * s4 + kg][16 * J + l16], xk[s4], wa, 0, 0, 0);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * J + 4 * kg + r;
                        const float ei = safe ? __expf(static_cast<float>(sG[i][c] - Gm)) : 0.f;
                        const float ej = safe ? __expf(static_cast<float>(Gm - sG[i][c])) : 0.f;
                        rP[J][r] += ei * zp[r];
                        rA[J][r] += ei * za[r];
                        cS[J][r] += ej * (wp[r] + wa[r]);
                    }
                    if (!safe) {  // rare: every pair of the block with its exact decay
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int i = 16 * J + 4 * kg + r, i0 = 16 * J;
                            const GT Gi = sG[i][c];
                            float rowP = 0.f, rowA = 0.f, col = 0.f;
                            for (int j = i0; j <= i; ++j) {
                                const float e = __expf(static_cast<float>(Gi - sG[j][c])) * toF(sK[j][c]);
                                rowP += sM[1][i][j] * e;
                                rowA += sM[3][i][j] * e;
                            }
                            for (int mm = i; mm < i0 + 16; ++mm) {
                                const float e = __expf(static_cast<float>(sG[mm][c] - Gi));
                                col += sM[1][mm][i] * e * toF(sQ[mm][c]) + sM[3][mm][i] * e * toF(sK[mm][c]);
                            }
                            rP[J][r] += rowP;
                            rA[J][r] += rowA;
                            cS[J][r] += col;
                        }
                    }
                }
                // the blocks below it
                if (J + 1 < NTI) {
                    const int m = 16 * J + 15;
                    const GT Gm = sG[m][c];
                    float ys[4];  // e^{G_m - G_j} k_j at j = 16 J + 4 s + lane / 16
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        const int j = 16 * J + 4 * s4 + kg;
                        ys[s4] = __expf(static_cast<float>(Gm - sG[j][c])) * toF(sK[j][c]);
                    }
#pragma unroll
                    for (int I = J + 1; I < NTI; ++I) {
                        f32x4 zp = {0.f, 0.f, 0.f, 0.f}, za = zp, wp = zp, wa = zp;
                        float xq[4], xk[4];  // e^{G_i - G_m} q_i, k_i at i = 16 I + 4 s + lane / 16
#pragma unroll
                        for (int s4 = 0; s4 < 4; ++s4) {
                            const int i = 16 * I + 4 * s4 + kg;
                            const float f = __expf(static_cast<float>(sG[i][c] - Gm));
                            xq[s4] = f * toF(sQ[i][c]);
                            xk[s4] = f * toF(sK[i][c]);
                        }
#pragma unroll
                        for (int s4 = 0; s4 < 4; ++s4) {
                            zp = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[1][16 * I + l16][16 * J + 4 * s4 + kg], ys[s4], zp, 0, 0, 0);
                            za = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[3][16 * I + l16][16 * J + 4 * s4 + kg], ys[s4], za, 0, 0, 0);
                            wp = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[1][16 * I + 4 * s4 + kg][16 * J + l16], xq[s4], wp, 0, 0, 0);
                            wa = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[3][16 * I + 4 * s4 + kg][16 * J + l16], xk[s4], wa, 0, 0, 0);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float ei = __expf(static_cast<float>(sG[16 * I + 4 * kg + r][c] - Gm));
                            const float ej = __expf(static_cast<float>(Gm - sG[16 * J + 4 * kg + r][c]));
                            rP[I][r] += ei * zp[r];
                            rA[I][r] += ei * za[r];
                            cS[J][r] += ej * (wp[r] + wa[r]);
                        }
                    }
                }
            }
            // dq, dk out; dG
#pragma unroll
            for (int I = 0; I < NTI; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * kg + r;
                    const float kv = toF(sK[i][c]), qv = toF(sQ[i][c]);
                    const float dq = DQr[I][r] + rP[I][r], dk = DKr[I][r] + rA[I][r] + cS[I][r];
                    DGr[I][r] += qv * rP[I][r] + kv * rA[I][r] - kv * cS[I][r];
                    if (i < nvalid) {
                        p.dq[row_of(i) * D + c] = dq;
                        p.dk[row_of(i) * D + c] = dk;
                    }
                }
            // ---- dlog_alpha = reverse cumulative sum of dG over the chunk, from
            //      the last token's dG term (dgl): within each lane's four tokens
            //      of a block, then over the four lanes of the channel (lane / 16),
            //      then over the blocks, last first
            GT after_blocks = dgl;
#pragma unroll
            for (int I = NTI - 1; I >= 0; --I) {
                GT suf[4];
                suf[3] = DGr[I][3];
#pragma unroll
                for (int r = 2; r >= 0; --r) suf[r] = suf[r + 1] + GT(DGr[I][r]);
                const GT tot = suf[0];
                const GT t1 = __shfl_down(tot, 16), t2 = __shfl_down(tot, 32), t3 = __shfl_down(tot, 48);
                const GT after_lanes = (kg < 3 ? t1 : GT(0)) + (kg < 2 ? t2 : GT(0)) + (kg < 1 ? t3 : GT(0));
                GT block = tot + __shfl_xor(tot, 16);
                block += __shfl_xor(block, 32);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * kg + r;
                    const GT acc = after_blocks + after_lanes + suf[r];
                    if (i < nvalid)
                        p.dlog_alpha[row_of(i) * D + c] = (sNotRst[i] && !sNegInf[i][c]) ? static_cast<float>(acc) : 0.f;
                }
                after_blocks += block;
            }
        }
        for (int i = tid; i < nvalid; i += kBwdIntraThreads) {
            float s = 0.f;
            for (int td = 0; td < NTD; ++td) s += sPart[i][td];
            for (int tj = 0; tj < NTI; ++tj) s += sPart2[i][tj];
            p.dbeta[row_of(i)] = s;
        }
        __syncthreads();  // LDS and scratch are reused by the next item
    }
}

// The chunk slots are taken in segments of a.seg_slots.  First the forward
// runs over segments 0 .. n_seg - 2 keeping only the state entering each next
// segment (a checkpoint); then, from the last segment to the first, each
// segment's forward is recomputed from its checkpoint (packages and the state
// entering each chunk), the state gradients walk it backwards from the
// gradient carried in from the segment after it, and the gradient kernel
// takes its (chunk, head) items.
template <int C, int D, bool BF>
hipError_t launch_bwd_t(const BackwardArgs &a, hipStream_t stream) {
    PrefillArgs f = a.fwd;
    f.o = nullptr;
    f.final_state = nullptr;
    const int64_t K = a.seg_slots, slots = f.n_slots;
    const int64_t nseg = slots > 0 ? (slots + K - 1) / K : 1;
    const size_t hd2 = static_cast<size_t>(f.H) * D * D;
    auto ckpt = [&](int64_t g) { return g > 0 ? a.checkpoints + static_cast<size_t>(g - 1) * hd2 : nullptr; };
    hipError_t e = hipSuccess;
    for (int64_t g = 0; g + 1 < nseg; ++g) {
        const FwdSegment fs{g * K, (g + 1) * K, f.workspace, true, g == 0, false, ckpt(g), ckpt(g + 1), nullptr};
        e = launch_forward_segment<C, D, D, BF>(f, fs, stream);
        if (e != hipSuccess) return e;
    }
    const PackageLayout L = package_layout(C, D, D, BF);
    for (int64_t g = nseg - 1; g >= 0; --g) {
        const int64_t s0 = g * K, s1 = std::min(slots, s0 + K);
        const FwdSegment fs{s0, s1, f.workspace, true, nseg == 1, false, ckpt(g), nullptr, a.chunk_states};
        e = launch_forward_segment<C, D, D, BF>(f, fs, stream);
        if (e != hipSuccess) return e;
        BwdStateParams sp{f.cu_seqlens, f.chunk_offsets, f.T, f.H, f.N, f.workspace, f.pkg_bytes, L,
                          a.d_o, a.d_final_state, a.chunk_dstates, a.d_init_state,
                          s0, s1, a.dcarry + ((g + 1) & 1) * hd2, a.dcarry + (g & 1) * hd2, g == 0};
        dim3 sgrid;
        if (!state_grid(f.N, f.H, D, sgrid)) return hipErrorInvalidValue;
        if constexpr (BF)
            hipLaunchKernelGGL((bwd_state_f16_kernel<C, D>), sgrid, dim3(kBwdThreads), 0, stream, sp);
        else
            hipLaunchKernelGGL((bwd_state_kernel<C, D, BF>), sgrid, dim3(kBwdThreads), 0, stream, sp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t n_items = (s1 - s0) * f.H;
        if (n_items <= 0) continue;
        const int64_t grid = std::min<int64_t>(n_items, std::min<int64_t>(kBwdMaxGroups, device_cu_count()));
        BwdIntraParams ip{f.q, f.k, f.v, f.log_alpha, f.beta, f.cu_seqlens, f.chunk_offsets, f.T, f.H, f.N,
                          a.d_o, a.chunk_states, a.chunk_dstates, a.scratch,
                          a.dq, a.dk, a.dv, a.dlog_alpha, a.dbeta, s0 * f.H, s0};
        hipLaunchKernelGGL((intra_bwd_kernel<C, D, BF>), dim3(static_cast<unsigned>(grid)), dim3(kBwdIntraThreads), 0,
                           stream, ip, s1 * f.H);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int C, bool BF>
hipError_t dispatch_bwd_d(const BackwardArgs &a, hipStream_t s) {
    switch (a.fwd.Dk) {
        case 16: return launch_bwd_t<C, 16, BF>(a, s);
        case 32: return launch_bwd_t<C, 32, BF>(a, s);
        case 64: return launch_bwd_t<C, 64, BF>(a, s);
        case 128:
            if constexpr (BF || C <= 32) return launch_bwd_t<C, 128, BF>(a, s);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_backward(const BackwardArgs &a, hipStream_t stream) {
    if (a.fwd.N == 0) return hipSuccess;
    const bool bf = a.fwd.bf16;
    switch (a.fwd.C) {
        case 16: return bf ? dispatch_bwd_d<16, true>(a, stream) : dispatch_bwd_d<16, false>(a, stream);
        case 32: return bf ? dispatch_bwd_d<32, true>(a, stream) : dispatch_bwd_d<32, false>(a, stream);
        case 64: return bf ? dispatch_bwd_d<64, true>(a, stream) : dispatch_bwd_d<64, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
