// kda_prefill.h -- declarations shared by the prefill kernels (intra-chunk
// kernels and the sequential state pass).  Internal; not installed.
#pragma once

#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"
#include "kda_mma.h"

namespace kda {

constexpr float kGFloor = -88.0f;               // clamp for partial -inf decays
constexpr float kSafeSpan2 = 110.0f;            // max |exponent| (log2) of a factor
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kIntraThreads = 256;               // 4 waves

struct IntraParams {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    const int32_t *cu_seqlens, *chunk_offsets;  // varlen only
    int64_t T;
    int32_t H, N;
    char *ws;
    size_t pkg_bytes;
    PackageLayout L;
    // log_alpha element of (token-head row r, key channel c) is
    // log_alpha[r * g_row + c * g_ch]: (Dk, 1) per-channel gates (KDA),
    // (1, 0) one scalar gate per token and head (GDN)
    int32_t g_row, g_ch;
    // 0 KDA, 1 GDN, 2 KDA layer (raw q, k; bf16 x_alpha [.., Dk], x_beta [..])
    int32_t gate_mode;
    const uint16_t *x_alpha, *x_beta;
    float l2_eps;
    // the kernels walk items [item0, n_items) (item = slot * H + head) and
    // write item's package at ws + (item - item0) * pkg_bytes
    int64_t item0 = 0;
};

struct StateParams {
    const float *init_state;
    const int32_t *cu_seqlens, *chunk_offsets;
    float *o, *final_state;
    float *chunk_states;  // saving variant: the state entering each chunk, [slots, H, Dk, Dv]
    int64_t T;
    int32_t H, N;
    const char *ws;
    size_t pkg_bytes;
    PackageLayout L;
    // Chunk slots [s0, s1) only (the backward's segments; the prefill takes
    // them all).  Slot X's package is at ws + ((X - s0) H + h) pkg_bytes and its
    // saved state at chunk_states + ((X - s0) H + h) Dk Dv.  A sequence that
    // begins before s0 starts from carry_in[h]; one that goes on past s1 leaves
    // the state entering slot s1 in carry_out[h] (nullable).  A sequence with
    // no tokens is handled only where do_empty is set.
    int64_t s0 = 0, s1 = INT64_MAX;
    const float *carry_in = nullptr;
    float *carry_out = nullptr;
    bool do_empty = true;
    // The KDA layer's epilogue (layer_state_kernel): out = o / sqrt(mean o^2 +
    // norm_eps) * norm_weight * sigmoid(out_gate) per (token, head) row.
    const uint16_t *out_gate = nullptr;
    const float *norm_weight = nullptr;
    float norm_eps = 0.f;
    uint32_t layer_tag = 0;
    uint64_t *norm_xchg = nullptr;  // [slots][H][Dv / 16][CP] words (norm_xchg_bytes each (slot, head))
};

// Grid of the sequential state passes (forward and reverse): one-dimensional,
// with NS = DV / 16 column slabs per (sequence, head) unit, block 8 (NS g + ct)
// + x is slab ct of unit 8 g + x.  Blocks go to the eight XCDs round-robin, so
// the NS slabs of a unit run on one XCD, one after another in its dispatch
// order: they are resident together and share the unit's packages in that
// XCD's L2 whatever the number of units.  false when the grid exceeds the
// one-dimensional limit.
inline bool state_grid(int32_t N, int32_t H, int DV, dim3 &grid) {
    const int64_t units = static_cast<int64_t>(N) * H;
    const int64_t blocks = (units + 7) / 8 * 8 * (DV / 16);
    if (blocks <= 0 || blocks > 0x7fffffff) return false;
    grid = dim3(static_cast<unsigned>(blocks));
    return true;
}

// (sequence n, head h, slab ct) of this block of a state_grid launch; false for
// the blocks past the last unit.
template <int NS>
__device__ __forceinline__ bool state_unit(int32_t N, int32_t H, int &n, int &h, int &ct) {
    const int blk = blockIdx.x, q8 = blk >> 3;
    ct = q8 % NS;
    const int unit = 8 * (q8 / NS) + (blk & 7);
    if (unit >= N * H) return false;
    n = unit / H;
    h = unit - n * H;
    return true;
}

struct BwdStateParams {
    const int32_t *cu_seqlens, *chunk_offsets;
    int64_t T;
    int32_t H, N;
    const char *ws;
    size_t pkg_bytes;
    PackageLayout L;
    const float *d_o, *d_final;  // d_final nullable
    float *chunk_dstates;
    float *d_init;               // nullable
    // chunk slots [s0, s1), as in StateParams, walked backwards: a sequence
    // that goes on past s1 starts from dcarry_in[h] (the gradient of the state
    // entering slot s1); one that begins before s0 leaves the gradient of the
    // state entering slot s0 in dcarry_out[h]
    int64_t s0 = 0, s1 = INT64_MAX;
    const float *dcarry_in = nullptr;
    float *dcarry_out = nullptr;
    bool do_empty = true;
};

struct BwdIntraParams {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    const int32_t *cu_seqlens, *chunk_offsets;
    int64_t T;
    int32_t H, N;
    const float *d_o, *chunk_states, *chunk_dstates;
    float *scratch;
    float *dq, *dk, *dv, *dlog_alpha, *dbeta;
    // items [item0, n_items); the states of item's chunk slot X at
    // chunk_states + ((X - s0) H + h) D D (and chunk_dstates alike)
    int64_t item0 = 0, s0 = 0;
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
// q = a / b, r = a % b for a >= 0, b > 0; 32-bit division when both fit
// (int64 division is a long software sequence on the GPU).
__device__ __forceinline__ void divmod_nonneg(int64_t a, int64_t b, int64_t &q, int64_t &r) {
    if (((a | b) >> 32) == 0) {
        const uint32_t a32 = static_cast<uint32_t>(a), b32 = static_cast<uint32_t>(b);
        const uint32_t q32 = a32 / b32;
        q = q32;
        r = a32 - q32 * b32;
    } else {
        q = a / b;
        r = a - q * b;
    }
}

__device__ __forceinline__ bool locate_chunk(int64_t x, int C, int64_t T, int32_t N,
                                             const int32_t *cu, const int32_t *off,
                                             int64_t &tok0, int &nvalid) {
    if (cu == nullptr) {
        const int64_t cps = (T + C - 1) / C;
        int64_t n, c;
        divmod_nonneg(x, cps, n, c);
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


// Reads one 32-bit word of each 128-byte line of the next work item's q, k,
// v and log_alpha rows, so that those lines are in L2 when the item starts.
// Returns the sum of the words (only to keep the loads alive).
template <int C, int DK, int DV, bool BF>
__device__ __forceinline__ float touch_next_item(const IntraParams &p, int64_t item, int64_t n_items,
                                                 int tid) {
    using In = typename Cfg<C, DK, DV, BF>::In;
    if (item >= n_items) return 0.f;
    const int H = p.H;
    int64_t tok0;
    int nvalid;
    if (!locate_chunk(item / H, C, p.T, p.N, p.cu_seqlens, p.chunk_offsets, tok0, nvalid)) return 0.f;
    const int h = static_cast<int>(item % H);
    constexpr int LK = DK * sizeof(In) / 128 > 0 ? DK * sizeof(In) / 128 : 1;  // lines per q/k row
    constexpr int LV = DV * sizeof(In) / 128 > 0 ? DV * sizeof(In) / 128 : 1;
    constexpr int LG = DK * 4 / 128 > 0 ? DK * 4 / 128 : 1;
    constexpr int PER_ROW = 2 * LK + LV + LG;
    float acc = 0.f;
    for (int idx = tid; idx < nvalid * PER_ROW; idx += kIntraThreads) {
        const int i = idx / PER_ROW, l = idx % PER_ROW;
        const int64_t row = (tok0 + i) * H + h;
        const float *src;
        if (l < LK) src = reinterpret_cast<const float *>(static_cast<const In *>(p.q) + row * DK) + l * 32;
        else if (l < 2 * LK) src = reinterpret_cast<const float *>(static_cast<const In *>(p.k) + row * DK) + (l - LK) * 32;
        else if (l < 2 * LK + LV) src = reinterpret_cast<const float *>(static_cast<const In *>(p.v) + row * DV) + (l - 2 * LK) * 32;
        else  // the gate row: Dk values (KDA) or one value (g_ch = 0, scalar gate)
            src = p.log_alpha + row * p.g_row + (p.g_ch ? (l - 2 * LK - LV) * 32 : 0);
        acc += *src;
    }
    return acc;
}

// Compute units of the current device (queried once per device).
inline int device_cu_count() {
    static thread_local int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Launches the register-resident intra-chunk kernel for 64-token chunks at
// d_k = d_v = 128 with bf16 inputs (kda_intra_wide.hip).
hipError_t launch_intra_wide(const IntraParams &p, int64_t n_items, hipStream_t stream);

// One segment of the backward's forward pass: chunk slots [s0, s1) of every
// sequence.  With intra set, their packages are made first (into pkgs, slot
// s0's first; plan: also the varlen plan); then the state pass in its saving
// variant walks them, writing the state entering each chunk to chunk_states
// ([s1 - s0, H, DK, DV] fp32, nullable) and no output.  carry_in / carry_out
// hold, per head, the state entering slot s0 / s1 of a sequence that crosses
// that boundary (see StateParams).  kda_prefill.hip; instantiated for the
// shapes the backward supports.
struct FwdSegment {
    int64_t s0, s1;
    char *pkgs;
    bool intra, plan, do_empty;
    const float *carry_in;
    float *carry_out;
    float *chunk_states;
};
template <int C, int DK, int DV, bool BF>
hipError_t launch_forward_segment(const PrefillArgs &a, const FwdSegment &g, hipStream_t stream);

// chunk_offsets[n] = sum_{m<n} ceil(len_m / C) for varlen batches, on the device
hipError_t launch_plan(const int32_t *cu_seqlens, int32_t N, int C, int32_t *chunk_offsets, hipStream_t stream);

// The DPLR form's state pass over packages already in sp.ws (kda_prefill.hip;
// d_k = d_v = D).
template <int C, int D, bool BF>
hipError_t launch_dplr_state(const StateParams &sp, hipStream_t stream);

}  // namespace kda
