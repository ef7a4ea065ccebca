// kda_state_head.hip -- the sequential state pass of the chunked prefill with
// one workgroup per (sequence, head) holding the whole 128 x 128 state, for
// 64-token chunks at d_k = d_v = 128 on the bf16 path.
//
// Per chunk (the chunked form of the recurrence in the section "Kimi Delta
// Attention (KDA)" of the page "Kimi Linear 高效注意力架构"; the package holds
// W, the folded readout operator Q' = Q*Gamma - P W, Kt = K e^{G_last - G},
// U', O_intra = P U' and Gamma_last, see kda_prefill.hip):
//
//   U = U' - W S,   O = O_intra + Q' S,   S <- Diag(Gamma_last) S + Kt^T U
//
// The column-slab state pass (state_kernel) splits S into eight 16-column
// slabs, one workgroup each, so every slab workgroup loads the whole W and Q'
// of every chunk: eight loads of the same 32 KiB per chunk and head.  Here the
// four waves of one workgroup (one per SIMD, so each may hold 512 registers)
// share the chunk instead:
//   wave w holds the rows of tokens 16 w .. 16 w + 15 of W and of Q' against
//     all eight 16-column tiles of S (every B fragment read from LDS feeds two
//     matrix products), and channel tiles w and w + 4 of the state (all 128
//     columns) in registers, with the next chunk's package in flight;
//   S is mirrored in LDS as fp16 (the B operand of [W; Q'] S) and U as fp16
//     hi/lo (the B operand of Kt^T U), the same operand precision as the slab
//     pass, so the two passes give the same results up to the order of fp32
//     sums.
// Each chunk's package is read once (112.5 KiB), against 8 x 56 KiB by the
// slab pass, and the output rows are written 512 bytes at a time.
//
// The kernel walks chunks [c_begin, c_end) of each sequence (the whole
// sequence, or one segment of it when the prefill is pipelined over segments:
// the state then enters from init_state and leaves through final_state, which
// may be the same buffer).
#include <mutex>

#include "kda_prefill.h"
#include "kda_state_head.h"

namespace kda {
namespace {

constexpr int kHC = 64;                // chunk
constexpr int kHD = 128;               // d_k = d_v
constexpr int kSS = kHD + 8;           // fp16 row stride of the LDS state (row = column of S)
constexpr int kUS = kHC + 8;           // fp16 row stride of the LDS U (row = column of S)

// One chunk's package as one wave consumes it (layouts in kda_internal.h).
// The workgroup owns the 64 state columns 16 ct0 .. 16 ct0 + 63; wave w takes
// row tile w of [W; Q'] (tokens 16 (w % 4) .., W rows for w < 4, Q' rows for
// w >= 4) against those four column tiles, and the state's channel tile w.
struct HeadFrags {
    f16x8 wq[4];     // row tile w of [W; Q'], channel steps 0..3
    f32x4 uo[4];     // U' (w < 4) or O_intra (w >= 4) of row tile w % 4
    f16x8 kt[2];     // channel tile w of Kt, token steps 0..1
    f32x4 gl;        // Gamma_last of channels 16 w + 4 (lane / 16) + r

    __device__ __forceinline__ void load(const char *pkg, const PackageLayout &L, int w, int lane, int ct0) {
        const _Float16 *wqp = reinterpret_cast<const _Float16 *>(pkg + L.wq);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            wq[ks] = *reinterpret_cast<const f16x8 *>(wqp + ((static_cast<size_t>(w) * 4 + ks) * 64 + lane) * 8);
        const f32x4 *uop = reinterpret_cast<const f32x4 *>(pkg + (w < 4 ? L.up : L.oi));
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) uo[ct] = uop[(static_cast<size_t>(ct0 + ct) * 4 + (w & 3)) * 64 + lane];
        const _Float16 *ktp = reinterpret_cast<const _Float16 *>(pkg + L.kt);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            kt[ks] = *reinterpret_cast<const f16x8 *>(ktp + ((static_cast<size_t>(w) * 2 + ks) * 64 + lane) * 8);
        // loaded with the rest of the package: a load issued later would make
        // the wait for it also wait for every prefetch issued before it
        gl = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(pkg + L.gl) + 16 * w + 4 * (lane >> 4));
    }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
    const _Float16 ha = static_cast<_Float16>(a), hb = static_cast<_Float16>(b);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ha)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hb)) << 16);
}

// Two workgroups per (sequence, head), each 64 columns of the state;
// workgroups b and b + 8 take the two halves of one unit (same XCD, so the
// W, Q' and Kt lines they both read are fetched from HBM once).
__global__ void __launch_bounds__(kHeadThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
state_head_kernel(StateHeadParams p) {
    constexpr int NCT = 4, NCOL = 64;
    __shared__ __align__(16) _Float16 sS[NCOL][kSS];      // S as a B operand: [column][channel position]
    __shared__ __align__(16) _Float16 sU[2][NCOL][kUS];   // U hi, lo as a B operand: [column][token]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, kg = lane >> 4;
    const int b = blockIdx.x;
    const int unit = (b & 7) + 8 * (b >> 4);
    const int ct0 = NCT * ((b >> 3) & 1);
    if (unit >= p.N * p.H) return;
    const int n = unit / p.H, h = unit % p.H;
    const int H = p.H;

    int64_t tok_base, L, slot_base;
    if (p.cu_seqlens) {
        tok_base = p.cu_seqlens[n];
        L = p.cu_seqlens[n + 1] - tok_base;
        slot_base = p.chunk_offsets[n];
    } else {
        tok_base = static_cast<int64_t>(n) * p.T;
        L = p.T;
        slot_base = static_cast<int64_t>(n) * ((p.T + kHC - 1) / kHC);
    }
    const int64_t nchunks = (L + kHC - 1) / kHC;
    const int64_t c_begin = p.c_begin < nchunks ? p.c_begin : nchunks;
    const int64_t c_end = p.c_end < nchunks ? p.c_end : nchunks;
    const int64_t c_full = (L / kHC) < c_end ? L / kHC : c_end;  // chunks below hold 64 tokens
    auto pkg_of = [&](int64_t c) {
        return p.ws + (static_cast<size_t>(slot_base + c) * H + h) * p.pkg_bytes;
    };

    // this wave's channel tile of the state: channels 16 w + 4 kg + r, column 16 (ct0 + ct) + l16
    const size_t sbase = (static_cast<size_t>(n) * H + h) * kHD * kHD;
    f32x4 S[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[ct][r] = p.init_state ? p.init_state[sbase + static_cast<size_t>(16 * w + 4 * kg + r) * kHD +
                                                   16 * (ct0 + ct) + l16]
                                    : 0.f;
    // fp16 copy for the B operand, channels in the order of the WQ fragments:
    // within each 32-channel step, position 8 g + 4 half + r holds channel
    // 16 half + 4 g + r (so channel tile w lands at 32 (w / 2) + 8 kg + 4 (w % 2))
    const int spos = 32 * (w >> 1) + 8 * kg + 4 * (w & 1);
    auto put_state = [&]() {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const u32x2 v = {pack_half2(S[ct][0], S[ct][1]), pack_half2(S[ct][2], S[ct][3])};
            *reinterpret_cast<u32x2 *>(&sS[16 * ct + l16][spos]) = v;
        }
    };
    put_state();

    // One chunk.  The package's U' / O_intra registers serve as the
    // accumulators of [W; Q'] S: W rows accumulate -U' + W S = -U, Q' rows
    // O_intra + Q' S = O.  kPartial: the sequence's last chunk has fewer
    // than 64 tokens, so its o stores are masked (full chunks store without
    // a condition).
    auto step = [&](HeadFrags &f, int64_t c, auto partial_tag) {
        constexpr bool kPartial = decltype(partial_tag)::value;
        if (w < 4) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) f.uo[ct] = -f.uo[ct];
        }
        __syncthreads();  // sS holds this chunk's incoming state; the last step's sU reads are done

#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const f16x8 bs = *reinterpret_cast<const f16x8 *>(&sS[16 * ct + l16][32 * ks + 8 * kg]);
                f.uo[ct] = mfma_f16(f.wq[ks], bs, f.uo[ct]);
            }
        if (w < 4) {
            const int j = 16 * w + 4 * kg;  // tokens j .. j + 3
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f32x4 u = -f.uo[ct];
                float hi[4], lo[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hi[r] = static_cast<float>(static_cast<_Float16>(u[r]));
                    lo[r] = u[r] - hi[r];
                }
                const u32x2 vh = {pack_half2(hi[0], hi[1]), pack_half2(hi[2], hi[3])};
                const u32x2 vl = {pack_half2(lo[0], lo[1]), pack_half2(lo[2], lo[3])};
                *reinterpret_cast<u32x2 *>(&sU[0][16 * ct + l16][j]) = vh;
                *reinterpret_cast<u32x2 *>(&sU[1][16 * ct + l16][j]) = vl;
            }
        } else {
            const int i0 = 16 * (w - 4) + 4 * kg;  // tokens i0 .. i0 + 3 of the chunk
            float *orow = p.o + ((tok_base + c * kHC + i0) * H + h) * kHD + 16 * ct0 + l16;
            if constexpr (!kPartial) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) orow[static_cast<size_t>(r) * H * kHD + 16 * ct] = f.uo[ct][r];
            } else {
                const int64_t rem = L - c * kHC;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (i0 + r < rem) {
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) orow[static_cast<size_t>(r) * H * kHD + 16 * ct] = f.uo[ct][r];
                    }
            }
        }
        __syncthreads();  // sU complete; every read of sS is done

        // S <- Diag(Gamma_last) S + Kt^T U for channel tile w, this workgroup's columns
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 a = f.gl * S[ct];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f16x8 bh = *reinterpret_cast<const f16x8 *>(&sU[0][16 * ct + l16][32 * ks + 8 * kg]);
                const f16x8 bl = *reinterpret_cast<const f16x8 *>(&sU[1][16 * ct + l16][32 * ks + 8 * kg]);
                a = mfma_f16(f.kt[ks], bl, a);
                a = mfma_f16(f.kt[ks], bh, a);
            }
            S[ct] = a;
        }
        put_state();
    };

    // software pipeline, three packages deep: chunk c + 2 loads while chunk c
    // computes; the main loop's loads are unconditional (a conditional load
    // would make every later wait assume it was not issued)
    using Full = std::false_type;
    using Part = std::true_type;
    HeadFrags f0, f1, f2;
    auto load = [&](HeadFrags &f, int64_t cc) { f.load(pkg_of(cc), p.L, w, lane, ct0); };
    int64_t c = c_begin;
    if (c < c_end) load(f0, c);
    if (c + 1 < c_end) load(f1, c + 1);
    for (; c + 4 < c_full; c += 3) {  // chunks c .. c + 2 are full; c + 3 and c + 4 exist
        load(f2, c + 2);
        step(f0, c, Full{});
        load(f0, c + 3);
        step(f1, c + 1, Full{});
        load(f1, c + 4);
        step(f2, c + 2, Full{});
    }
    // tail: f0 holds chunk c and f1 chunk c + 1 (when it exists)
    for (; c < c_end; ++c) {
        if (c + 2 < c_end) load(f2, c + 2);
        if (c < c_full) step(f0, c, Full{});
        else step(f0, c, Part{});
        f0 = f1;
        f1 = f2;
    }

    if (p.final_state) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p.final_state[sbase + static_cast<size_t>(16 * w + 4 * kg + r) * kHD + 16 * (ct0 + ct) + l16] = S[ct][r];
    }
}

// ---------------------------------------------------------------------------
// Pipelined prefill of one long sequence: the intra-chunk pass of segment s + 1
// runs on most compute units while the state pass of segment s runs on the
// rest (one unit per head), through two CU-masked streams ordered by events.
// The intra pass is bound by VALU issue, the state pass by its chunk-serial
// chain and package reads, so they overlap instead of taking turns.
// ---------------------------------------------------------------------------
constexpr int64_t kSegChunks = 512;   // 32768 tokens per segment
constexpr int kMaxDev = 64;

struct Pipe {
    bool tried = false, ok = false;
    hipStream_t intra = nullptr, state = nullptr;
    hipEvent_t fork = nullptr, seg = nullptr, join = nullptr;
    int intra_cus = 0;
};

std::mutex g_pipe_mu;
Pipe g_pipe[kMaxDev][8];   // [device][state units / 8 - 1]

// Bit i of a stream's CU mask selects a compute unit of XCD i % 8 (the
// dispatcher's order on MI355X), so the first n bits give n / 8 units on every
// XCD: state_cus bits for the state stream, all others for the intra stream.
bool pipe_setup(Pipe &P, int state_cus) {
    P.tried = true;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    if (cus < 4 * state_cus || cus > 1024) return false;
    uint32_t mi[32] = {0}, ms[32] = {0};
    const int words = (cus + 31) / 32;
    for (int i = 0; i < cus; ++i) {
        if (i < state_cus) ms[i / 32] |= 1u << (i % 32);
        else mi[i / 32] |= 1u << (i % 32);
    }
    // the size argument counts 32-bit words of the mask
    if (hipExtStreamCreateWithCUMask(&P.intra, words, mi) != hipSuccess) return false;
    if (hipExtStreamCreateWithCUMask(&P.state, words, ms) != hipSuccess) return false;
    if (hipEventCreateWithFlags(&P.fork, hipEventDisableTiming) != hipSuccess) return false;
    if (hipEventCreateWithFlags(&P.seg, hipEventDisableTiming) != hipSuccess) return false;
    if (hipEventCreateWithFlags(&P.join, hipEventDisableTiming) != hipSuccess) return false;
    P.intra_cus = cus - state_cus;
    P.ok = true;
    return true;
}

IntraParams intra_params(const PrefillArgs &a) {
    IntraParams ip{a.q, a.k, a.v, a.log_alpha, a.beta, a.cu_seqlens, a.chunk_offsets,
                   a.T, a.H, a.N, a.workspace, a.pkg_bytes, package_layout(kHC, kHD, kHD, true),
                   a.gate_mode == 1 ? 1 : kHD, a.gate_mode == 1 ? 0 : 1,
                   a.gate_mode, a.x_alpha, a.x_beta, a.l2_eps};
    return ip;
}

StateHeadParams state_params(const PrefillArgs &a) {
    StateHeadParams sp{};
    sp.init_state = a.init_state;
    sp.cu_seqlens = a.cu_seqlens;
    sp.chunk_offsets = a.chunk_offsets;
    sp.o = a.o;
    sp.final_state = a.final_state;
    sp.T = a.T;
    sp.H = a.H;
    sp.N = a.N;
    sp.ws = a.workspace;
    sp.pkg_bytes = a.pkg_bytes;
    sp.L = package_layout(kHC, kHD, kHD, true);
    sp.c_begin = 0;
    sp.c_end = INT64_MAX;
    return sp;
}

// Enqueues the segments; returns hipErrorNotSupported (nothing enqueued) when
// the CU-masked streams are unavailable.
hipError_t pipelined(const PrefillArgs &a, hipStream_t stream) {
    const int state_cus = ((2 * a.H + 7) / 8) * 8;  // two workgroups (column halves) per head
    if (state_cus > 64) return hipErrorNotSupported;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return hipErrorNotSupported;
    std::lock_guard<std::mutex> lock(g_pipe_mu);
    Pipe &P = g_pipe[dev][state_cus / 8 - 1];
    if (!P.tried) pipe_setup(P, state_cus);
    if (!P.ok) return hipErrorNotSupported;
    const int64_t nchunks = (a.T + kHC - 1) / kHC;
    hipError_t e;
    if ((e = hipEventRecord(P.fork, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(P.intra, P.fork, 0)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(P.state, P.fork, 0)) != hipSuccess) return e;
    IntraParams ip = intra_params(a);
    ip.grid_cus = P.intra_cus;
    StateHeadParams sp = state_params(a);
    for (int64_t c0 = 0; c0 < nchunks; c0 += kSegChunks) {
        const int64_t c1 = c0 + kSegChunks < nchunks ? c0 + kSegChunks : nchunks;
        ip.item0 = c0 * a.H;
        if ((e = launch_intra_wide(ip, c1 * a.H, P.intra)) != hipSuccess) return e;
        if ((e = hipEventRecord(P.seg, P.intra)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(P.state, P.seg, 0)) != hipSuccess) return e;
        sp.c_begin = c0;
        sp.c_end = c1;
        sp.init_state = c0 == 0 ? a.init_state : a.state_carry;
        sp.final_state = c1 == nchunks ? a.final_state : a.state_carry;
        if ((e = launch_state_head(sp, P.state)) != hipSuccess) return e;
    }
    if ((e = hipEventRecord(P.join, P.state)) != hipSuccess) return e;
    return hipStreamWaitEvent(stream, P.join, 0);
}

}  // namespace

hipError_t launch_prefill_pipelined(const PrefillArgs &a, hipStream_t stream) {
    const int64_t nchunks = (a.T + kHC - 1) / kHC;
    const bool eligible = a.cu_seqlens == nullptr && a.N == 1 && a.H <= 32 && a.state_carry != nullptr &&
                          nchunks >= 2 * kSegChunks;
    if (!eligible) return hipErrorNotSupported;
    const hipError_t e = pipelined(a, stream);
    if (e != hipSuccess) return e;
    if (a.gate_mode == 2)
        return launch_layer_epilogue(a.o, a.out_gate, a.norm_weight, static_cast<int64_t>(a.B) * a.T * a.H,
                                     a.norm_eps, stream);
    return hipSuccess;
}

hipError_t launch_state_head(const StateHeadParams &p, hipStream_t stream) {
    if (p.N <= 0) return hipSuccess;
    const int64_t units = static_cast<int64_t>(p.N) * p.H;
    if (units > 0x3fffffff) return hipErrorInvalidValue;
    // two workgroups per unit (column halves), b and b + 8 on one XCD
    const int64_t grid = 16 * ((units + 7) / 8);
    hipLaunchKernelGGL(state_head_kernel, dim3(static_cast<unsigned>(grid)), dim3(kHeadThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda
