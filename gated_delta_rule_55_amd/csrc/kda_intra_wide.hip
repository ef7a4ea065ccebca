// kda_intra_wide.hip -- intra-chunk package for 64-token chunks at
// d_k = d_v = 128 with bf16 inputs, computed with the chunk held in registers.
//
// It writes the same package, bit layout for bit layout, as intra_kernel in
// kda_prefill.hip (the WY/UT quantities of the chunked form in the section
// "Kimi Delta Attention (KDA)" of the page "Kimi Linear 高效注意力架构": W,
// Q' = Q*Gamma - P W, Kt, U' and O_intra).  What differs is the work split:
// intra_kernel stages k, q, v and the fp32 cumulative decay G of the whole
// chunk in LDS (about 124 KB, one workgroup per compute unit), while here
// wave w of the four owns key channels 32w .. 32w + 31 (and value columns
// 32w .. 32w + 31) and keeps them in registers:
//
//   lane l holds, for each 16-token tile t (token 16 t + l%16), the channels
//       ch(e) = 32 w + 16 (e / 4) + 4 (l / 16) + e % 4,   e = 0 .. 7,
//   of k, q, v (bf16 bits) and of G (fp32).
//
// That is the k-slot layout of the 16x16x32 bf16 / fp16 matrix instructions
// for the Gram tiles (a sum over channels may take them in any order as long
// as both operands agree; diagonal tiles with operands split in bf16 hi/lo,
// three products, for the fp32 exponent range their midpoint factors need;
// tiles below the diagonal, whose factors are all <= 1, with plain fp16
// operands, one product), so every wave forms its channels' share of all ten
// Gram tiles without touching LDS.  It is also the row layout of the [W; Q']
// fragments, so Q*Gamma adds into Q' in place.  The cumulative decay is a scan
// over the 16 lanes of a row (DPP) plus a carry over the four tiles.  The four
// shares of each Gram tile are summed in a fixed order through LDS, then T, R
// and M = [T'; -R] are formed as in intra_kernel.  About 74 KB of LDS in all,
// so two workgroups share a compute unit.
#include <algorithm>
#include <type_traits>

#include "kda_prefill.h"

namespace kda {
namespace {

constexpr int kWC = 64;                           // chunk
constexpr int kWD = 128;                          // d_k = d_v
constexpr int kAS = kWC + 8;                      // fp32 row stride of A/T and P/R; bf16 stride of M
constexpr int kXS = kWC + 8;                      // 16-bit row stride of a wave's transpose buffer
constexpr int kApBytes = 2 * kWC * kAS * 4;       // A and P (fp32), later M (bf16 hi/lo)
constexpr int kXBytes = 2 * 32 * kXS * 2;         // one wave's transpose buffer
constexpr int kSmemBytes = kApBytes + 4 * kXBytes;
constexpr int kRedBytes = 20 * 3 * 64 * 16;       // Gram shares in flight
static_assert(2 * 2 * kWC * kAS * 2 == kApBytes, "M overlays A and P");
static_assert(kRedBytes <= kSmemBytes, "Gram shares overlay A, P and the transpose buffers");

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf,
                                                                 true));
}
// inclusive prefix sum over the 16 lanes of each row
__device__ __forceinline__ float row_scan(float x) {
    x += dpp_f<0x111>(x);  // row_shr:1
    x += dpp_f<0x112>(x);  // row_shr:2
    x += dpp_f<0x114>(x);  // row_shr:4
    x += dpp_f<0x118>(x);  // row_shr:8
    return x;
}
// value of lane N of each row of 16 lanes
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return dpp_f<0x150 + N>(x);  // row_newbcast:N
}

// element e of 8 packed bf16 values
__device__ __forceinline__ float bf_at(const uint32_t (&u)[4], int e) {
    const uint32_t w = u[e >> 1];
    return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
}
__device__ __forceinline__ uint16_t bf_bits(const uint32_t (&u)[4], int e) {
    const uint32_t w = u[e >> 1];
    return static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xffffu));
}

// orders this wave's LDS accesses around a change of a buffer's role
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bits of tokens (j, i] of a 64-bit token mask (empty when j >= i).
__device__ __forceinline__ uint64_t tokens_between(int j, int i) {
    if (j >= i) return 0;
    const uint64_t upto_i = i >= 63 ? ~uint64_t(0) : ((uint64_t(1) << (i + 1)) - 1);
    const uint64_t upto_j = (uint64_t(1) << (j + 1)) - 1;  // j < i <= 63
    return upto_i & ~upto_j;
}

// f(std::integral_constant<int, B>{}), ..., f(std::integral_constant<int, E - 1>{})
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// (I, J) of lower-triangular 16x16 tile index ti = I (I + 1) / 2 + J
__host__ __device__ constexpr int tile_i(int ti) { return ti < 1 ? 0 : ti < 3 ? 1 : ti < 6 ? 2 : 3; }
__host__ __device__ constexpr int tile_j(int ti) { return ti - tile_i(ti) * (tile_i(ti) + 1) / 2; }

// One wave's share of a 16x16 Gram tile over its 32 channels: x (8 channels
// of this lane's row token) against y (split as yh + yl) with bf16 hi/lo
// operands, three 16x16x32 products (the lo x lo term is below fp32 rounding).
__device__ __forceinline__ f32x4 gram_bf16x3(const float (&x)[8], const bf16x8 &yh, const bf16x8 &yl) {
    bf16x8 xh, xl;
    split_bf16(x, xh, xl);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma_bf16(xl, yh, acc);
    acc = mfma_bf16(xh, yl, acc);
    return mfma_bf16(xh, yh, acc);
}

// One work item's raw inputs as this lane holds them (layout above).  Rows
// past the chunk's end are loaded from its last token (always in bounds) and
// zeroed when the item is unpacked, so no wait sits between the loads.
struct WideRaw {
    uint32_t k[4][4], q[4][4], v[4][4];
    float la[4][8];     // log_alpha (gate modes 0 and 1)
    float beta;         // beta of token l (lane l; gate modes 0 and 1)
    uint32_t xa[4][4];  // gate mode 2: x_alpha, bf16 bits
    uint16_t xb;        // gate mode 2: x_beta of token l, bf16 bits
};

// Gate modes of the kernel:
//   0  KDA: log_alpha [.., Dk] fp32 per key channel, beta fp32
//   1  Gated DeltaNet: one log_alpha per (token, head), broadcast to every channel
//   2  KDA layer: q and k arrive unnormalised and are L2-normalised here; the
//      decay gate log_alpha = -softplus(x_alpha) and beta = sigmoid(x_beta) are
//      formed from bf16 projections (the KDA-layer item of the page's
//      model-architecture list: L2Norm on q/k, low-rank channel-wise decay gate)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each 16-bit input arrives as one 16-byte load per lane of 8 consecutive
// channels, at 16 (kg & 1) + 8 (kg >> 1) within the wave's 32 (so the four
// lanes of a token cover them once).  Swapping halves with the lane 16 away
// (rows of 16 lanes: even rows keep their first half and take the odd
// neighbour's first half as their second; odd rows take the even neighbour's
// second half as their first) leaves lane l with channels 4 (l / 16) + 0..3
// and 16 + 4 (l / 16) + 0..3, the layout above.
__device__ __forceinline__ int64_t load16_channel(int kg) { return 16 * (kg & 1) + 8 * (kg >> 1); }
__device__ __forceinline__ void halves_to_layout(uint32_t (&u)[4]) {
    const auto a = __builtin_amdgcn_permlane16_swap(u[0], u[2], false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(u[1], u[3], false, false);
    u[0] = a[0];
    u[2] = a[1];
    u[1] = b[0];
    u[3] = b[1];
}
__device__ __forceinline__ void put4(uint32_t (&d)[4], const u32x4 &x) {
    d[0] = x[0];
    d[1] = x[1];
    d[2] = x[2];
    d[3] = x[3];
}

// Loads one work item's inputs (raw 16-bit words still in load order: the
// unpack puts them in the register layout once they have arrived).  Lane l
// of wave 0 also loads the beta of token l; the other waves, which do not use
// it, all read token 0's (one cache line instead of one per token).
template <int GM>
__device__ __forceinline__ void fetch_item(const IntraParams &p, int64_t tok0, int nvalid, int h, int w, int t16,
                                           int kg, WideRaw &r) {
    const int H = p.H;
    {
        const int l = w == 0 ? 16 * kg + t16 : 0;
        const int64_t row = (tok0 + (l < nvalid ? l : nvalid - 1)) * H + h;
        if constexpr (GM == 2) r.xb = p.x_beta[row];
        else r.beta = p.beta[row];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i = 16 * t + t16;
        const int64_t row = (tok0 + (i < nvalid ? i : nvalid - 1)) * H + h;
        const int64_t off = row * kWD + 32 * w + 4 * kg;
        const int64_t off16 = row * kWD + 32 * w + load16_channel(kg);
        put4(r.k[t], *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.k) + off16));
        put4(r.q[t], *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.q) + off16));
        put4(r.v[t], *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.v) + off16));
        if constexpr (GM == 2) {
            put4(r.xa[t], *reinterpret_cast<const u32x4 *>(p.x_alpha + off16));
        } else if constexpr (GM == 1) {
            const float g = p.log_alpha[row];
#pragma unroll
            for (int e = 0; e < 8; ++e) r.la[t][e] = g;
        } else {
            const f32x4 l0 = *reinterpret_cast<const f32x4 *>(p.log_alpha + off);
            const f32x4 l1 = *reinterpret_cast<const f32x4 *>(p.log_alpha + off + 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r.la[t][e] = l0[e];
                r.la[t][4 + e] = l1[e];
            }
        }
    }
}

template <int GM>
__global__ void __launch_bounds__(kIntraThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
intra_wide_kernel(IntraParams p, int64_t n_items) {
    constexpr int C = kWC, NT16 = 4, PARTS = 2, MS = kAS;
    __shared__ __align__(16) unsigned char smem[kSmemBytes];
    __shared__ float sBeta[C];
    __shared__ uint64_t sRst[4];
    __shared__ float sNrm[GM == 2 ? 4 : 1][2][GM == 2 ? C : 1];  // per-wave sums of k^2, q^2 per token
    __shared__ float sGs[GM == 1 ? C : 1];  // scalar gate: cumulative log2-decay per token

    float(*sA)[kAS] = reinterpret_cast<float(*)[kAS]>(smem);
    float(*sP)[kAS] = reinterpret_cast<float(*)[kAS]>(smem + kWC * kAS * 4);
    __bf16 *Mp = reinterpret_cast<__bf16 *>(smem);  // [PARTS][2C][MS]
    f32x4 *red = reinterpret_cast<f32x4 *>(smem);   // [20 tile matrices][3 senders][64 lanes]
    const int H = p.H;

    // work items are visited in order; varlen grids end with empty slots, so
    // the first empty slot ends the walk
    int64_t item = p.item0 + blockIdx.x;
    int64_t tok0;
    int nvalid;
    int64_t slot, h0;
    divmod_nonneg(item, H, slot, h0);
    if (item >= n_items || !locate_chunk(slot, C, p.T, p.N, p.cu_seqlens, p.chunk_offsets, tok0, nvalid)) return;
    WideRaw raw;
    {
        const int tid = threadIdx.x;
        fetch_item<GM>(p, tok0, nvalid, static_cast<int>(h0), tid >> 6, tid & 15, (tid & 63) >> 4, raw);
    }
    for (;;) {
        // Lane-dependent addresses and masks are recomputed per item: hoisted out
        // of the loop they would outnumber the registers two workgroups leave.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int t16 = lane & 15, kg = lane >> 4;
        uint16_t *xb = reinterpret_cast<uint16_t *>(smem + kApBytes + w * kXBytes);  // [2][32][kXS]
        char *pkg = p.ws + static_cast<size_t>(item - p.item0) * p.pkg_bytes;

        // ---- unpack this lane's tokens and channels (tokens >= nvalid are zeros)
        uint32_t kr[4][4], qr[4][4], vr[4][4];
        float G[4][8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int i = 16 * t + t16;
            const bool ok = i < nvalid;
            const uint32_t m = ok ? 0xffffffffu : 0u;
            halves_to_layout(raw.k[t]);
            halves_to_layout(raw.q[t]);
            halves_to_layout(raw.v[t]);
            if constexpr (GM == 2) halves_to_layout(raw.xa[t]);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                kr[t][x] = raw.k[t][x] & m;
                qr[t][x] = raw.q[t][x] & m;
                vr[t][x] = raw.v[t][x] & m;
            }
            if constexpr (GM == 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) G[t][e] = ok ? neg_softplus(bf_at(raw.xa[t], e)) : 0.f;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) G[t][e] = ok ? raw.la[t][e] : 0.f;
            }
        }
        if (w == 0) {  // beta of token l from lane l
            const bool ok = lane < nvalid;
            if constexpr (GM == 2)
                sBeta[lane] = ok ? sigmoid_f(__builtin_bit_cast(float, static_cast<uint32_t>(raw.xb) << 16)) : 0.f;
            else
                sBeta[lane] = ok ? raw.beta : 0.f;
        }
        if constexpr (GM == 2) {
            // this wave's share of |k|^2 and |q|^2 per token: 8 channels per lane,
            // summed over the four lane groups of the wave, then across waves in LDS
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float sk = 0.f, sq = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sk += bf_at(kr[t], e) * bf_at(kr[t], e);
                    sq += bf_at(qr[t], e) * bf_at(qr[t], e);
                }
                sk += __shfl_xor(sk, 16);
                sq += __shfl_xor(sq, 16);
                sk += __shfl_xor(sk, 32);
                sq += __shfl_xor(sq, 32);
                if (kg == 0) {
                    sNrm[w][0][16 * t + t16] = sk;
                    sNrm[w][1][16 * t + t16] = sq;
                }
            }
        }
        // gate mode 2: 1 / |k|, 1 / |q| of this lane's four tokens, applied at every
        // use in fp32 (rounding the normalised vectors back to bf16 would cost
        // ~1e-2 of the output's RMS); 1 otherwise
        float nk[4] = {1.f, 1.f, 1.f, 1.f}, nq[4] = {1.f, 1.f, 1.f, 1.f};
        auto Kf = [&](int t, int e) { return bf_at(kr[t], e) * nk[t]; };
        auto Qf = [&](int t, int e) { return bf_at(qr[t], e) * nq[t]; };

        // ---- resets: tokens whose log_alpha is -inf on all channels
        {
            uint64_t mine = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                bool all = 16 * t + t16 < nvalid;
#pragma unroll
                for (int e = 0; e < 8; ++e) all = all && G[t][e] == kNegInf;
                const uint64_t m = __ballot(all);
                mine |= ((m & (m >> 16) & (m >> 32) & (m >> 48)) & 0xffffu) << (16 * t);
            }
            if (lane == 0) sRst[w] = mine;
        }
        __syncthreads();  // also: every wave is done with the previous item's LDS
        if constexpr (GM == 2) {
            // 1 / sqrt(|x|^2 + eps) per token; padding rows are zeros already and
            // keep a zero scale whatever eps is
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int i = 16 * t + t16;
                const bool ok = i < nvalid;
                nk[t] = ok ? 1.f / sqrtf(sNrm[0][0][i] + sNrm[1][0][i] + sNrm[2][0][i] + sNrm[3][0][i] + p.l2_eps)
                           : 0.f;
                nq[t] = ok ? 1.f / sqrtf(sNrm[0][1][i] + sNrm[1][1][i] + sNrm[2][1][i] + sNrm[3][1][i] + p.l2_eps)
                           : 0.f;
            }
        }
        const uint64_t rst = sRst[0] & sRst[1] & sRst[2] & sRst[3];
        const int first_rst = rst ? __builtin_ctzll(rst) : C;  // tokens before it see the incoming state
        const int last_rst = rst ? 63 - __builtin_clzll(rst) : -1;

        // ---- cumulative log2-decay: scan within each 16-token tile, then carry
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool r = (rst >> (16 * t + t16)) & 1;
#pragma unroll
            for (int e = 0; e < 8; ++e) G[t][e] = row_scan(r ? 0.f : fmaxf(G[t][e], kGFloor) * kLog2e);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float carry = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float tot = row_bcast<15>(G[t][e]);
                G[t][e] += carry;
                carry += tot;
            }
        }

        if constexpr (GM == 1) {
            if (w == 0 && kg == 0) {
#pragma unroll
                for (int t = 0; t < 4; ++t) sGs[16 * t + t16] = G[t][0];
            }
        }

        // ---- this wave's share of the Gram tiles A' (k k) and P (q k), factored
        //      exponents.  Tile matrix tm (A tiles 0..9, P tiles 10..19) belongs to
        //      wave tm % 4; the other waves leave their shares in LDS for it.
        f32x4 fin[5];
        auto emit = [&](auto tmc, const f32x4 &v) {
            constexpr int tm = decltype(tmc)::value, owner = tm & 3;
            if (owner == w) fin[tm >> 2] = v;
            else red[(tm * 3 + ((w - owner + 3) & 3)) * 64 + lane] = v;
        };
        // Scalar gate (GDN): the decay e^{G_i - G_j} is one number per token pair,
        // so the tiles are plain K K^T and Q K^T on the bf16 inputs (exact
        // products, fp32 sums) and the decay is applied per element when the
        // shares are summed.
        auto bits8 = [](const uint32_t (&u)[4]) {
            typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
            return __builtin_bit_cast(bf16x8, u32x4_t{u[0], u[1], u[2], u[3]});
        };
        if constexpr (GM == 1) {
            static_for<0, 4>([&](auto Jc) {
                constexpr int J = decltype(Jc)::value;
                const bf16x8 kj = bits8(kr[J]);
                static_for<J, 4>([&](auto Ic) {
                    constexpr int I = decltype(Ic)::value;
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    emit(std::integral_constant<int, I * (I + 1) / 2 + J>{}, mfma_bf16(bits8(kr[I]), kj, z));
                    emit(std::integral_constant<int, 10 + I * (I + 1) / 2 + J>{}, mfma_bf16(bits8(qr[I]), kj, z));
                });
            });
        } else
        static_for<0, 4>([&](auto Jc) {
            constexpr int J = decltype(Jc)::value;
            float gm[8];  // G at token 16 J + 15
#pragma unroll
            for (int e = 0; e < 8; ++e) gm[e] = row_bcast<15>(G[J][e]);
            if constexpr (J < 3) {
                // tiles below the diagonal, reference = last token of column tile
                // J: both factors are <= 1 and |k|, |q| <= 1, so every operand
                // lies in [-1, 1] and plain fp16 operands (11-bit significands,
                // one product per tile) keep the parity error where bf16 hi/lo
                // splits put it; bf16 alone would not
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = Kf(J, e) * fast_exp2(gm[e] - G[J][e]);
                const f16x8 y16 = pack_f16(y);
                static_for<J + 1, 4>([&](auto Ic) {
                    constexpr int I = decltype(Ic)::value;
                    float xk[8], xq[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float fa = fast_exp2(G[I][e] - gm[e]);
                        xk[e] = Kf(I, e) * fa;
                        xq[e] = Qf(I, e) * fa;
                    }
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    emit(std::integral_constant<int, I * (I + 1) / 2 + J>{}, mfma_f16(pack_f16(xk), y16, z));
                    emit(std::integral_constant<int, 10 + I * (I + 1) / 2 + J>{}, mfma_f16(pack_f16(xq), y16, z));
                });
            }
            // diagonal tile, reference = token 16 J + 7; a channel whose half-span
            // there exceeds the safe range is left out and added exactly below
            uint32_t unsafe = 0;  // bit 16 (e / 4) + 4 kg + e % 4 of this wave's channels
            float xk[8], xq[8], kb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float g7 = row_bcast<7>(G[J][e]);
                const float g0 = row_bcast<0>(G[J][e]);
                const bool uns = !(fmaxf(g0 - g7, g7 - gm[e]) <= kSafeSpan2);
                const float d = G[J][e] - g7;
                const float fa = uns ? 0.f : fast_exp2(d);
                const float fb = uns ? 0.f : fast_exp2(-d);
                kb[e] = Kf(J, e) * fb;
                xk[e] = Kf(J, e) * fa;
                xq[e] = Qf(J, e) * fa;
                const uint64_t b = __ballot(uns);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if ((b >> (16 * r)) & 1) unsafe |= 1u << (16 * (e >> 2) + 4 * r + (e & 3));
            }
            bf16x8 kbh, kbl;
            split_bf16(kb, kbh, kbl);
            f32x4 a = gram_bf16x3(xk, kbh, kbl), pq = gram_bf16x3(xq, kbh, kbl);
            if (unsafe) {
                // rare: exact terms of the channels left out, with the tile's values
                // of channel (e, row kgs) fetched from lanes 16 kgs + token
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t ub = (unsafe >> (16 * (e >> 2) + (e & 3))) & 0x1111u;
                    if (!ub) continue;
                    const float kv = Kf(J, e), qv = Qf(J, e), gv = G[J][e];
                    for (int kgs = 0; kgs < 4; ++kgs) {
                        if (!((ub >> (4 * kgs)) & 1)) continue;
                        const float kj = __shfl(kv, 16 * kgs + t16), gj = __shfl(gv, 16 * kgs + t16);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int src = 16 * kgs + 4 * kg + r;
                            const float ki = __shfl(kv, src), qi = __shfl(qv, src), gi = __shfl(gv, src);
                            const float ex = fast_exp2(fminf(gi - gj, 0.f));
                            a[r] += ki * kj * ex;
                            pq[r] += qi * kj * ex;
                        }
                    }
                }
            }
            emit(std::integral_constant<int, J * (J + 1) / 2 + J>{}, a);
            emit(std::integral_constant<int, 10 + J * (J + 1) / 2 + J>{}, pq);
        });

        // ---- the next item (located now, fetched once this one's stores are issued)
        const int64_t next = item + gridDim.x;
        int64_t slot_n, h_n;
        divmod_nonneg(next, H, slot_n, h_n);
        int64_t tok0_n = 0;
        int nvalid_n = 0;
        const bool more =
            next < n_items && locate_chunk(slot_n, C, p.T, p.N, p.cu_seqlens, p.chunk_offsets, tok0_n, nvalid_n);

        // ---- sum the shares in a fixed order; apply masks and beta
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            const int tm = 4 * k + w;
#pragma unroll
            for (int j = 0; j < 3; ++j) fin[k] += red[(tm * 3 + j) * 64 + lane];
        }
        __syncthreads();  // the shares overlay A and P
        auto finalize = [&](auto masked_tag) {
            constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
            for (int k = 0; k < 5; ++k) {
                const int tm = 4 * k + w;
                const int ti = tm < 10 ? tm : tm - 10;
                const int I = tile_i(ti), J = tile_j(ti);
                const int j = 16 * J + t16;
                float(*dst)[kAS] = tm < 10 ? sA : sP;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * kg + r;
                    bool keep = tm < 10 ? j < i : j <= i;
                    if constexpr (kMasked) keep = keep && (rst & tokens_between(j, i)) == 0;  // no reset in (j, i]
                    float val = (tm < 10 ? sBeta[i] : 1.f) * fin[k][r];
                    if constexpr (GM == 1) val *= fast_exp2(sGs[i] - sGs[j]);  // i >= j: at most 1
                    dst[i][j] = keep ? val : 0.f;
                }
            }
        };
        if (rst == 0) finalize(std::false_type{});  // most chunks have no reset
        else finalize(std::true_type{});
        __syncthreads();

        // ---- Kt = K e^{G_last - G} (fp16) and Gamma_last, stored now; K Gamma
        //      (bf16 hi/lo) parked in this wave's transpose buffer; Q Gamma kept in
        //      registers.  Transposes go through the buffer: row = channel, k = token.
        {
            using Op = _Float16;
            Op *kt = reinterpret_cast<Op *>(pkg + p.L.kt);
            float gl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gl[e] = row_bcast<15>(G[3][e]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int lc = 16 * (e >> 2) + 4 * kg + (e & 3);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int i = 16 * t + t16;
                    const float v = i >= last_rst ? Kf(t, e) * fast_exp2(gl[e] - G[t][e]) : 0.f;
                    xb[lc * kXS + i] = __builtin_bit_cast(uint16_t, static_cast<Op>(v));
                }
            }
            wave_sync();
#pragma unroll
            for (int hc = 0; hc < 2; ++hc)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int ct = 2 * w + hc;
                    const f16x8 v = *reinterpret_cast<const f16x8 *>(&xb[(16 * hc + t16) * kXS + 32 * s + 8 * kg]);
                    *reinterpret_cast<f16x8 *>(kt + ((static_cast<size_t>(ct) * 2 + s) * 64 + lane) * 8) = v;
                }
            wave_sync();
            if (t16 == 0) {
                float *glp = reinterpret_cast<float *>(pkg + p.L.gl);
                f32x4 g0, g1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    g0[r] = last_rst >= 0 ? 0.f : fast_exp2(gl[r]);
                    g1[r] = last_rst >= 0 ? 0.f : fast_exp2(gl[4 + r]);
                }
                *reinterpret_cast<f32x4 *>(glp + 32 * w + 4 * kg) = g0;
                *reinterpret_cast<f32x4 *>(glp + 32 * w + 16 + 4 * kg) = g1;
            }
        }
        float qg[4][8];  // Q Gamma (0 from the first reset on)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int i = 16 * t + t16;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int lc = 16 * (e >> 2) + 4 * kg + (e & 3);
                const float eg = fast_exp2(G[t][e]);
                const float v = i < first_rst ? Kf(t, e) * eg : 0.f;
                qg[t][e] = i < first_rst ? Qf(t, e) * eg : 0.f;
                const __bf16 hi = static_cast<__bf16>(v);
                const __bf16 lo = static_cast<__bf16>(v - static_cast<float>(hi));
                xb[(0 * 32 + lc) * kXS + i] = __builtin_bit_cast(uint16_t, hi);
                xb[(1 * 32 + lc) * kXS + i] = __builtin_bit_cast(uint16_t, lo);
            }
        }

        // ---- T = (I + A)^-1 (unit lower triangular), in place over A
        if (lane < 16) {
            const int base = 16 * w, col = lane;
            float tv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float val = (i == col) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) val -= sA[base + i][base + j] * tv[j];
                tv[i] = val;
                __builtin_amdgcn_sched_barrier(0);  // keep the row loads from piling up
            }
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i >= col) sA[base + i][base + col] = tv[i];
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
                        xv = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[16 * I + t16][16 * K + kk],
                                                                   sA[16 * K + kk][16 * J + t16], xv, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[16 * I + t16][16 * I + 4 * kg + r], xv[r], y, 0,
                                                              0, 0);
            }
            __syncthreads();
            if (J < I) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sA[16 * I + 4 * kg + r][16 * J + t16] = -y[r];
            }
            __syncthreads();
        }

        // ---- R = P T' and M = [T'; -R] (T' = T Diag(beta)) as bf16 hi/lo operands
        {
            constexpr int NB = NT16 * (NT16 + 1) / 2;
            constexpr int BPW = (NB + 3) / 4;
            f32x4 tv[BPW], rv[BPW];
#pragma unroll
            for (int b = 0; b < BPW; ++b) {
                const int t = w + 4 * b;
                tv[b] = rv[b] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (t < NB) {
                    int I = 0, J = t;
                    while (J > I) { J -= I + 1; ++I; }
                    const float bj = sBeta[16 * J + t16];
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    for (int K = J; K <= I; ++K) {
#pragma unroll
                        for (int s4 = 0; s4 < 4; ++s4) {
                            const int kk = 4 * s4 + kg;
                            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sP[16 * I + t16][16 * K + kk],
                                                                        sA[16 * K + kk][16 * J + t16], acc, 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        rv[b][r] = -acc[r] * bj;
                        tv[b][r] = sA[16 * I + 4 * kg + r][16 * J + t16] * bj;
                    }
                }
            }
            __syncthreads();  // every fp32 read of A/T and P is done: M overlays them
            for (int idx = tid; idx < PARTS * 2 * C * MS * 2 / 16; idx += kIntraThreads)
                reinterpret_cast<f32x4 *>(Mp)[idx] = f32x4{0.f, 0.f, 0.f, 0.f};
            __syncthreads();
#pragma unroll
            for (int b = 0; b < BPW; ++b) {
                const int t = w + 4 * b;
                if (t < NB) {
                    int I = 0, J = t;
                    while (J > I) { J -= I + 1; ++I; }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * I + 4 * kg + r, col = 16 * J + t16;
                        const float vals[2] = {tv[b][r], rv[b][r]};
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const size_t o = static_cast<size_t>(hh * C + row) * MS + col;
                            const __bf16 hi = static_cast<__bf16>(vals[hh]);
                            Mp[o] = hi;
                            Mp[static_cast<size_t>(2 * C) * MS + o] = static_cast<__bf16>(vals[hh] - static_cast<float>(hi));
                        }
                    }
                }
            }
        }
        __syncthreads();

        // ---- [W; Q'] = [0; Q Gamma] + M (K Gamma) (computed transposed: rows =
        //      channels) and [U'; -O_intra] = M V, for this wave's 32 channels
        auto m_frag = [&](int rt, int s, bf16x8 &hi, bf16x8 &lo) {  // B operand: row 16 rt + l%16 of M
            const size_t o = static_cast<size_t>(16 * rt + t16) * MS + 32 * s + 8 * kg;
            hi = *reinterpret_cast<const bf16x8 *>(Mp + o);
            lo = *reinterpret_cast<const bf16x8 *>(Mp + static_cast<size_t>(2 * C) * MS + o);
        };
        bf16x8 ka_hi[2][2], ka_lo[2][2], vb[2][2];
#pragma unroll
        for (int hc = 0; hc < 2; ++hc)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                ka_hi[hc][s] = *reinterpret_cast<const bf16x8 *>(&xb[(0 * 32 + 16 * hc + t16) * kXS + 32 * s + 8 * kg]);
                ka_lo[hc][s] = *reinterpret_cast<const bf16x8 *>(&xb[(1 * 32 + 16 * hc + t16) * kXS + 32 * s + 8 * kg]);
            }
        wave_sync();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int i = 16 * t + t16;
#pragma unroll
            for (int e = 0; e < 8; ++e) xb[(16 * (e >> 2) + 4 * kg + (e & 3)) * kXS + i] = bf_bits(vr[t], e);
        }
        wave_sync();
#pragma unroll
        for (int hc = 0; hc < 2; ++hc)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                vb[hc][s] = *reinterpret_cast<const bf16x8 *>(&xb[(16 * hc + t16) * kXS + 32 * s + 8 * kg]);
        {
            _Float16 *wq = reinterpret_cast<_Float16 *>(pkg + p.L.wq);
            f32x4 *up = reinterpret_cast<f32x4 *>(pkg + p.L.up);
            f32x4 *oi = reinterpret_cast<f32x4 *>(pkg + p.L.oi);
#pragma unroll
            for (int I = 0; I < NT16; ++I) {
                constexpr int kMaxS = 2;
                const int nks = I >= 2 ? 2 : 1;  // token steps with nonzeros
#pragma unroll
                for (int half = 0; half < 2; ++half) {  // W / U' rows, then Q' / -O_intra rows
                    const int rt = I + NT16 * half;
                    f32x4 aw[2], au[2];
#pragma unroll
                    for (int hc = 0; hc < 2; ++hc) {
                        au[hc] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int r = 0; r < 4; ++r) aw[hc][r] = half ? qg[I][4 * hc + r] : 0.f;
                    }
#pragma unroll
                    for (int s = 0; s < kMaxS; ++s) {
                        if (s >= nks) break;
                        bf16x8 mh, ml;
                        m_frag(rt, s, mh, ml);
#pragma unroll
                        for (int hc = 0; hc < 2; ++hc) {
                            aw[hc] = mfma_bf16(ka_lo[hc][s], mh, aw[hc]);
                            aw[hc] = mfma_bf16(ka_hi[hc][s], ml, aw[hc]);
                            aw[hc] = mfma_bf16(ka_hi[hc][s], mh, aw[hc]);
                            au[hc] = mfma_bf16(ml, vb[hc][s], au[hc]);
                            au[hc] = mfma_bf16(mh, vb[hc][s], au[hc]);
                        }
                    }
                    float v8[8];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        v8[r] = aw[0][r];
                        v8[4 + r] = aw[1][r];
                    }
                    store8(wq + ((static_cast<size_t>(rt) * 4 + w) * 64 + lane) * 8, v8);
#pragma unroll
                    for (int hc = 0; hc < 2; ++hc) {
                        const size_t o = (static_cast<size_t>(2 * w + hc) * NT16 + I) * 64 + lane;
                        if (half == 0) up[o] = au[hc];
                        else oi[o] = -au[hc];
                    }
                }
            }
        }
        if (!more) break;
        item = next;
        tok0 = tok0_n;
        nvalid = nvalid_n;
        fetch_item<GM>(p, tok0, nvalid, static_cast<int>(h_n), w, t16, kg, raw);
    }
}

}  // namespace

template <int GM>
static hipError_t launch_intra_wide_t(const IntraParams &p, int64_t n_items, hipStream_t stream) {
    static thread_local int per_cu = 0;
    if (per_cu == 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, intra_wide_kernel<GM>, kIntraThreads, 0) !=
                hipSuccess ||
            nb <= 0)
            nb = 1;
        per_cu = nb;
    }
    const int64_t grid = std::min<int64_t>(n_items - p.item0, static_cast<int64_t>(device_cu_count()) * per_cu);
    hipLaunchKernelGGL(intra_wide_kernel<GM>, dim3(static_cast<unsigned>(grid)), dim3(kIntraThreads), 0, stream,
                       p, n_items);
    return hipGetLastError();
}

hipError_t launch_intra_wide(const IntraParams &p, int64_t n_items, hipStream_t stream) {
    if (n_items <= p.item0) return hipSuccess;
    switch (p.gate_mode) {
        case 0: return launch_intra_wide_t<0>(p, n_items, stream);
        case 1: return launch_intra_wide_t<1>(p, n_items, stream);
        case 2: return launch_intra_wide_t<2>(p, n_items, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
