// kda_internal.h -- launcher interface between the C-ABI host code and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    float *state, *o;
    int32_t N, H, Dk, Dv;
    bool bf16;
    int32_t gate_mode;  // 0 KDA, 1 GDN (log_alpha [N, H]), 2 KDA layer (below), 3 DPLR
    // gate mode 2: q, k unnormalised; bf16 x_alpha [N, H, Dk], x_beta [N, H],
    // output gate [N, H, Dv]; RMSNorm weight [Dv]
    const uint16_t *x_alpha, *x_beta, *out_gate;
    const float *norm_weight;
    float l2_eps, norm_eps;
    const void *lr_a, *lr_b;  // gate mode 3: low-rank vectors a, b [N, H, Dk] in_dtype (no beta)
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace kda

namespace kda {

// Byte layout of one intra-chunk package (one chunk of one head) in the
// prefill workspace.  Sections are 256-byte aligned.  Fragment layouts are the
// register layouts the state pass feeds to the matrix cores, so its loads are
// contiguous 1 KB (16-bit operands) or 2 KB (fp32 operands) per wave:
//   WQ  A operand of [W; Q'] S: rows 2C (W then Q'), K = Dk.
//       block (row tile rt, k-step ks) = 64 lanes x 8 values, lane l holding
//       row 16 rt + l%16, k = 32 ks + 8 (l/16) + e; order [rt][ks][lane][8].
//   KT  A operand of Ktilde^T U: rows Dk (channels), K = C tokens (padded to
//       32); order [ct][ks][lane][8] (fp16 on the 16-bit path, fp32 otherwise).
//   UP  U' in accumulator layout: tile (col tile ct, row tile rt), lane l
//       holding rows 4 (l/16) + r of the tile, column 16 ct + l%16;
//       order [ct][rt][lane][4] fp32.
//   OI  the intra-chunk output P U', same layout as UP.
//   GL  Gamma of the chunk's last token per key channel, fp32 [Dk].
struct PackageLayout {
    size_t wq, kt, up, oi, gl, bytes;  // offsets of sections and total size
    size_t vx;                         // DPLR only: the chunk's V in the UP layout
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline PackageLayout package_layout(int C, int Dk, int Dv, bool bf16) {
    const size_t osz = bf16 ? 2 : 4;                   // matrix-core operand bytes
    const size_t dkp = Dk < 32 ? 32 : Dk;              // K padded to a 32-wide step
    const size_t cp = C < 32 ? 32 : C;
    PackageLayout L;
    size_t off = 0;
    L.wq = off; off += align256(2 * (size_t)C * dkp * osz);
    L.kt = off; off += align256((size_t)Dk * cp * osz);
    L.up = off; off += align256((size_t)C * Dv * 4);
    L.oi = off; off += align256((size_t)C * Dv * 4);
    L.gl = off; off += align256((size_t)Dk * 4);
    L.bytes = off;
    L.vx = 0;  // no V section
    return L;
}

// The DPLR form's package (kda_dplr.hip): WQ, UP, OI and GL as above with W
// stored negated and UP holding U' = T Abk V; KT holds 2 CP tokens, the
// decayed low-rank vectors A-tilde (k-steps 0 .. CP/32 - 1) then the decayed
// keys K-tilde; VX holds the chunk's V (fp32, zero past its last token) in the
// UP layout.
__host__ __device__ inline PackageLayout dplr_package_layout(int C, int Dk, int Dv, bool bf16) {
    const size_t osz = bf16 ? 2 : 4;
    const size_t dkp = Dk < 32 ? 32 : Dk;
    const size_t cp = C < 32 ? 32 : C;
    PackageLayout L;
    size_t off = 0;
    L.wq = off; off += align256(2 * (size_t)C * dkp * osz);
    L.kt = off; off += align256((size_t)Dk * 2 * cp * osz);
    L.up = off; off += align256((size_t)C * Dv * 4);
    L.oi = off; off += align256((size_t)C * Dv * 4);
    L.gl = off; off += align256((size_t)Dk * 4);
    L.vx = off; off += align256((size_t)C * Dv * (bf16 ? 2 : 4));  // V rows: bf16 as given, or fp32
    L.bytes = off;
    return L;
}

struct PrefillArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta, *init_state;
    const int32_t *cu_seqlens;  // nullable
    int32_t B, H, Dk, Dv, N, C;
    int64_t T;
    bool bf16;
    int32_t gate_mode;          // 0 KDA, 1 GDN (log_alpha [B, T, H]), 2 KDA layer (below), 3 DPLR
    const void *lr_a, *lr_b;    // gate mode 3: low-rank vectors a, b [B, T, H, Dk] in_dtype (no beta)
    // gate mode 2: q, k unnormalised; bf16 x_alpha [B, T, H, Dk], x_beta [B, T, H],
    // output gate [B, T, H, Dv]; RMSNorm weight [Dv]
    const uint16_t *x_alpha, *x_beta, *out_gate;
    const float *norm_weight;
    float l2_eps, norm_eps;
    float *o, *final_state;     // final_state nullable
    uint32_t layer_tag;         // gate mode 2: this call's nonzero tag for the norm exchange
    char *norm_xchg;            // gate mode 2: the row-norm exchange in the workspace
    char *workspace;
    int64_t n_slots;            // chunk slots in the workspace
    size_t pkg_bytes;
    int32_t *chunk_offsets;     // varlen: [N + 1] in the workspace
};

// The KDA layer's row-norm exchange, after the packages (and the varlen plan)
// in the prefill workspace: per (chunk slot, head), 64-bit words [Dv / 16][CP],
// word (slab s, token i) = (call tag << 32) | bits of the sum of o^2 over the
// 16 columns of slab s for token i, written by that slab's state-pass
// workgroup and read by the other slabs of the head.
__host__ __device__ inline size_t norm_xchg_bytes(int C, int Dv) {
    return align256((size_t)(Dv < 16 ? 1 : Dv / 16) * (C < 32 ? 32 : C) * 8);
}

// Chunk slots the workspace reserves: every chunk of every sequence.
inline int64_t prefill_slots(int32_t B, int64_t T, int32_t N, int32_t C, bool varlen) {
    const int64_t per = (T + C - 1) / C;
    return varlen ? per + N : per * B;
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

// The DPLR form's prefill (gate mode 3; Dk = Dv, packages of dplr_package_layout).
hipError_t launch_dplr(const PrefillArgs &a, hipStream_t stream);

// Backward of the prefill: fwd describes the forward call (its o and
// final_state are unused; its workspace holds the packages and, for varlen,
// the chunk plan).  chunk_states / chunk_dstates: [slots, H, Dk, Dv] fp32, the
// state entering each chunk and the gradient with respect to the state leaving
// it; scratch: kBwdMaxGroups * kBwdScratchMats * C * Dk fp32.
// The backward walks the chunk slots in segments of seg_slots (the last one
// first), recomputing each segment's forward from the state that enters it:
// fwd.workspace holds one segment's packages, chunk_states / chunk_dstates
// one segment's states and state gradients ([seg_slots, H, D, D] fp32 each),
// checkpoints the state entering segments 1, 2, ... ([n_seg - 1, H, D, D]),
// dcarry two [H, D, D] buffers for the state gradient crossing a segment
// boundary.
struct BackwardArgs {
    PrefillArgs fwd;
    const float *d_o, *d_final_state;  // d_final_state nullable (zero)
    float *dq, *dk, *dv, *dlog_alpha, *dbeta;
    float *d_init_state;               // nullable
    float *chunk_states, *chunk_dstates, *scratch;
    float *checkpoints, *dcarry;
    int64_t seg_slots;
};
constexpr int kBwdMaxGroups = 1024;    // persistent workgroups of the gradient kernel
constexpr int kBwdScratchMats = 6;     // fp32 [C][D] scratch matrices per workgroup
// (chunk, head) items per backward segment: 16384 keeps every pass of a
// segment wide enough to fill the chip (64 items per compute unit) while the
// segment's buffers stay a few GB at d = 128
constexpr int64_t kBwdSegmentItems = 16384;
inline int64_t bwd_segment_slots(int32_t H) { return (kBwdSegmentItems + H - 1) / H; }

hipError_t launch_backward(const BackwardArgs &a, hipStream_t stream);

// kda_chunk_fwd_noalloc takes its workspace from a static device array of
// this many bytes (one copy per device, held until the process ends).
constexpr size_t kNoallocScratchBytes = size_t(256) << 20;

// Device address of the current device's copy of that array, looked up with
// hipGetSymbolAddress on the first call on each device and kept.
hipError_t noalloc_scratch(void **ptr);

// Chunk size the kernels use for a requested one (the fp32 path at d = 128 is
// limited to 32 tokens by LDS capacity).  Results do not depend on it beyond
// rounding.
inline int prefill_effective_chunk(int C, int Dk, int Dv, bool bf16) {
    if (!bf16 && (Dk > 64 || Dv > 64) && C > 32) return 32;
    return C;
}

}  // namespace kda
