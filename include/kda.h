/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library.
 *
 * The operator is the gated delta-rule recurrence of the section
 * "Kimi Delta Attention (KDA)" on the page "Kimi Linear 高效注意力架构":
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *
 * with one state S of d_k x d_v per (sequence, head), a channel-wise decay
 * alpha_t in [0,1]^{d_k} (bullet on channel-wise decay, same section) passed
 * as log_alpha = log(alpha) (-inf encodes alpha = 0), a scalar beta_t per
 * (token, head), and the output o_t = S_t^T q_t read after the token's write
 * (the page prints no readout; this is the operator's defined output, with no
 * 1/sqrt(d_k) scale -- callers may pre-scale q).  The chunked prefill follows
 * the bullet on the hardware-efficient chunked algorithm (DPLR with a = b = k)
 * and the complexity table O(T d_k d_v + T C d_h + T C^2) of the comparison
 * table on the same page; the decode step keeps the fixed-size d_k x d_v state
 * of the linear-complexity bullet.
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers (hipMalloc'd memory of the current device)
 *     unless stated otherwise, 16-byte aligned except beta and cu_seqlens
 *     (4-byte aligned).  Every tensor is dense and row-major in the layout
 *     below: a range of tokens of a B = 1 tensor is dense and may be passed
 *     directly; a subset of heads is not (its rows lie H * D elements apart)
 *     and must be copied into a dense tensor first.
 *   - Layouts: q, k, log_alpha [B, T, H, Dk]; v, o [B, T, H, Dv];
 *     beta [B, T, H]; states [N, H, Dk, Dv] (row c of a head's state is key
 *     channel c).  bf16 inputs are raw IEEE bfloat16 bit patterns.
 *   - Accumulation and states are fp32; o is always fp32.
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     device memory, keeps no pointer after returning, and never
 *     synchronises: work is enqueued on `stream` and runs asynchronously.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued (no HIP call, no pointer dereference); on any error nothing is
 *     written and a status other than KDA_OK is returned, with a detail
 *     message in kda_last_error().  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - Determinism: identical inputs give bit-identical outputs on one device.
 *   - Thread safety: no global mutable state except the thread-local error
 *     message; calls on different streams may overlap if they share no
 *     output or workspace buffer.
 *   - Numerical preconditions: log_alpha <= 0 (alpha in [0,1]); q and k are
 *     expected L2-normalised as the KDA layer produces them (not checked);
 *     NaN inputs propagate.  On the bf16 path the state and the per-chunk
 *     innovation U = beta (v - ...) are fed to fp16 matrix cores: above 65504
 *     in magnitude they overflow (the output is not finite), and where the
 *     whole state is below about 1e-4 they lose precision to fp16's subnormal
 *     range.  On the tested workloads (unit q and k, v ~ N(0, 1) times s,
 *     slow decay) the stated accuracy holds for s from 2^-10 to 2^14 and
 *     s = 2^15 overflows.  The fp32-input path has
 *     fp32's range.  A log_alpha of -inf on every channel of a
 *     token is an exact state reset; -inf on only some channels is taken as
 *     -88 (alpha ~ 6e-39).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION 150 /* 1.5.0: adds kda_layer_chunk_fwd_workspace_size (the layer prefill's
                            workspace now holds its row-norm exchange); 1.4.0:
                            kda_chunk_fwd_noalloc; 1.3.0: kda_dplr_chunk_fwd and
                            kda_dplr_decode_step; 1.2.0: kda_chunk_bwd; 1.1.0: the gdn_* and
                            kda_layer_* entry points */

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, aliasing   */
    KDA_ERR_UNSUPPORTED = 2, /* Dk/Dv outside {16,32,64,128}, chunk size,
                                dtype; the layer prefill: sizes other than
                                Dk = Dv = 128                                 */
    KDA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
    KDA_ERR_HIP = 4          /* a kernel launch failed (hipGetLastError)      */
} kda_status;

typedef enum {
    KDA_BF16 = 0, /* q, k, v are bfloat16                              */
    KDA_F32 = 1   /* q, k, v are float32 (fp32 matrix-core path)       */
} kda_dtype;

/*
 * kda_chunk_fwd_workspace_size -- bytes of device workspace kda_chunk_fwd
 * needs for these sizes (host only, pure; 0 for invalid arguments).  The
 * workspace holds one intra-chunk package per (chunk, head): the WY factors
 * W, the folded readout operator Q' = Q*Gamma - P W, the decayed keys, U' and
 * the intra-chunk output, all computed from the chunk alone.
 */
size_t kda_chunk_fwd_workspace_size(int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv,
                                    int32_t n_seqs, kda_dtype in_dtype, int32_t chunk_size);

/*
 * kda_chunk_fwd -- chunked prefill over whole sequences.
 *
 *   q, k        [B, T, H, Dk] in_dtype           queries / keys
 *   v           [B, T, H, Dv] in_dtype           values
 *   log_alpha   [B, T, H, Dk] fp32               per-channel log decay (<= 0)
 *   beta        [B, T, H]     fp32               write strength
 *   init_state  [N, H, Dk, Dv] fp32, nullable    incoming state (NULL: zeros)
 *   cu_seqlens  [N + 1] int32, nullable          packed sequence offsets (device)
 *   B, T, H, Dk, Dv                              sizes; Dk, Dv each in {16, 32, 64, 128}
 *   n_seqs      N when cu_seqlens is given (then B must be 1), else ignored (N = B)
 *   in_dtype    KDA_BF16 or KDA_F32
 *   chunk_size  16, 32 or 64 (0 selects 64); results do not depend on it
 *               beyond rounding (the fp32 path at d = 128 uses at most 32,
 *               which kda_chunk_fwd_workspace_size accounts for)
 *   o           [B, T, H, Dv] fp32 output; must not overlap any input
 *   final_state [N, H, Dk, Dv] fp32, nullable; may alias init_state
 *   workspace   device scratch of at least kda_chunk_fwd_workspace_size()
 *               bytes (256-byte aligned); contents on entry are ignored.  At
 *               T = 0 (every sequence empty) it is not used and may be NULL:
 *               the call then only writes final_state = init_state (or zeros)
 *   stream      HIP stream the kernels are enqueued on
 *
 * cu_seqlens must satisfy cu[0] = 0, cu[N] = T and be non-decreasing (the
 * device-side contents are the caller's contract and are not read by the
 * host).  Zero-length sequences keep their initial state.  Chunks restart at
 * each sequence start; the last chunk of a sequence may be partial.
 */
kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, const float *init_state, const int32_t *cu_seqlens,
                         int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                         kda_dtype in_dtype, int32_t chunk_size, float *o, float *final_state,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and bit-identical results.  The workspace is the library's own
 * static device array of kda_chunk_fwd_noalloc_max_workspace() bytes
 * (256 MiB): one copy per GPU, set up on the first call on that device and
 * held until the process ends.  The call itself allocates nothing and calls
 * no allocating routine.
 *
 * Sizes whose kda_chunk_fwd_workspace_size() exceeds that limit return
 * KDA_ERR_WORKSPACE before anything is enqueued (at Dk = Dv = 128, bf16,
 * 64-token chunks that is T * H above about 149,000 token-heads of a dense
 * batch; e.g. T = 4096 with H = 32 fits).  Every call on one GPU shares that
 * GPU's array: calls that overlap on one device (other streams, other host
 * threads) race on it and must be serialised by the caller.  Its contents on
 * entry are ignored.  A failure to look up the array's device address
 * returns KDA_ERR_HIP.
 */
kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *log_alpha,
                                 const float *beta, const float *init_state, const int32_t *cu_seqlens,
                                 int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                                 kda_dtype in_dtype, int32_t chunk_size, float *o, float *final_state,
                                 hipStream_t stream);

/* Bytes of the static scratch behind kda_chunk_fwd_noalloc (host only, pure). */
size_t kda_chunk_fwd_noalloc_max_workspace(void);

/*
 * kda_chunk_bwd_workspace_size -- bytes of device workspace kda_chunk_bwd
 * needs (host only, pure; 0 for invalid or unsupported arguments).  The
 * backward takes the chunk slots in segments of ceil(16384 / H) chunks and
 * recomputes each segment's forward from the state entering it, so the
 * workspace holds one segment's packages and its states and state gradients
 * ([segment chunks, H, Dk, Dv] fp32 each), one [H, Dk, Dv] fp32 checkpoint per
 * segment boundary, two [H, Dk, Dv] fp32 carries and a fixed scratch of
 * 1024 x 6 x C x Dk fp32: about 4.3 GB at T = 1M, H = 32, d = 128.
 */
size_t kda_chunk_bwd_workspace_size(int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv,
                                    int32_t n_seqs, kda_dtype in_dtype, int32_t chunk_size);

/*
 * kda_chunk_bwd -- gradients of kda_chunk_fwd (the training workload of the
 * page "Kimi Linear 高效注意力架构"; the recurrence of its section "Kimi Delta
 * Attention (KDA)", differentiated through the same chunked form).
 *
 *   q .. chunk_size     the forward's inputs, as in kda_chunk_fwd (the forward
 *                       is recomputed; its outputs are not needed)
 *   d_o           [B, T, H, Dv] fp32     gradient of the loss w.r.t. o
 *   d_final_state [N, H, Dk, Dv] fp32, nullable (zero)   w.r.t. final_state
 *   dq, dk        [B, T, H, Dk] fp32 out
 *   dv            [B, T, H, Dv] fp32 out
 *   dlog_alpha    [B, T, H, Dk] fp32 out (0 where log_alpha is -inf)
 *   dbeta         [B, T, H]     fp32 out
 *   d_init_state  [N, H, Dk, Dv] fp32 out, nullable      w.r.t. init_state
 *   workspace     at least kda_chunk_bwd_workspace_size() bytes, 256-byte aligned
 *
 * Dk must equal Dv (KDA_ERR_UNSUPPORTED otherwise).  Outputs must not overlap
 * each other, any input or the workspace; all pointers 16-byte aligned except
 * beta, dbeta and cu_seqlens (4).  Arithmetic after the forward's packages is
 * fp32; the result is bitwise deterministic.
 */
kda_status kda_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, const float *init_state, const int32_t *cu_seqlens,
                         int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                         kda_dtype in_dtype, int32_t chunk_size, const float *d_o,
                         const float *d_final_state, float *dq, float *dk, float *dv, float *dlog_alpha,
                         float *dbeta, float *d_init_state, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * kda_decode_step -- one token for each of N independent sequences, the state
 * updated in place (the fixed d_k x d_v per-head state of the linear-complexity
 * bullet of the same section).
 *
 *   q, k        [N, H, Dk] in_dtype
 *   v           [N, H, Dv] in_dtype
 *   log_alpha   [N, H, Dk] fp32
 *   beta        [N, H]     fp32
 *   state       [N, H, Dk, Dv] fp32, read and written in place
 *   o           [N, H, Dv] fp32 output; must not overlap any input or state
 *
 * Each state is streamed from HBM once and written back once; the arithmetic
 * is fp32 throughout.
 */
kda_status kda_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, float *state, int32_t N, int32_t H, int32_t Dk,
                           int32_t Dv, kda_dtype in_dtype, float *o, hipStream_t stream);

/*
 * Gated DeltaNet (GDN): the scalar-gate recurrence the same page sets KDA
 * against (bullet on channel-wise decay in the KDA section: GDN's forget gate
 * alpha_t is one head-wise scalar; list of related work: GDN is DeltaNet with
 * a scalar forget gate):
 *
 *     S_t = (I - beta_t k_t k_t^T) alpha_t S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 *
 * i.e. KDA with Diag(alpha_t) = alpha_t I.  The two entry points below run the
 * KDA kernels with that gate read once per (token, head) and applied to every
 * key channel; everything not stated here (layouts of q, k, v, beta, states,
 * o, workspace, cu_seqlens, chunk sizes, dtypes, ownership, errors,
 * determinism, preconditions) is exactly as for kda_chunk_fwd and
 * kda_decode_step.
 *
 * gdn_chunk_fwd -- chunked prefill; log_alpha is [B, T, H] fp32 (one log gate
 * <= 0 per token and head, 4-byte aligned; -inf resets the state).  The
 * workspace is kda_chunk_fwd_workspace_size() bytes for the same sizes.
 */
kda_status gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, const float *init_state, const int32_t *cu_seqlens,
                         int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                         kda_dtype in_dtype, int32_t chunk_size, float *o, float *final_state,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The general diagonal-plus-low-rank (DPLR) transition that the same section
 * contrasts KDA with (its bullet on the hardware-efficient chunked algorithm:
 * KDA ties both low-rank vectors to the key, which removes work; the
 * related-work list places GLA and RWKV7 on the general form), read with two
 * free per-token vectors a_t, b_t and an unscaled write:
 *
 *     S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
 *
 * (KDA is a_t = -beta_t k_t, b_t = alpha_t * k_t with v_t scaled by beta_t).
 *
 * kda_dplr_chunk_fwd_workspace_size -- bytes of device workspace
 * kda_dplr_chunk_fwd needs (host only, pure; 0 for invalid arguments).
 *
 * kda_dplr_chunk_fwd -- chunked prefill of that recurrence; d_k = d_v = D.
 *   q, k, a, b  [B, T, H, D] in_dtype, 16-byte aligned
 *   v           [B, T, H, D] in_dtype
 *   log_alpha   [B, T, H, D] fp32 (<= 0; a token whose log_alpha is -inf on
 *               every channel keeps only the low-rank and write terms)
 *   everything else (init_state, cu_seqlens, B, T, H, n_seqs, in_dtype,
 *   chunk_size, o, final_state, workspace, stream, ownership, aliasing rules,
 *   errors) as for kda_chunk_fwd with Dk = Dv = D; there is no beta.
 * The arithmetic of the intra-chunk pass is fp32 on every path; the state
 * pass uses the precision scheme of kda_chunk_fwd.
 */
size_t kda_dplr_chunk_fwd_workspace_size(int32_t B, int64_t T, int32_t H, int32_t D, int32_t n_seqs,
                                         kda_dtype in_dtype, int32_t chunk_size);

kda_status kda_dplr_chunk_fwd(const void *q, const void *k, const void *v, const void *a, const void *b,
                              const float *log_alpha, const float *init_state, const int32_t *cu_seqlens,
                              int32_t B, int64_t T, int32_t H, int32_t D, int32_t n_seqs, kda_dtype in_dtype,
                              int32_t chunk_size, float *o, float *final_state, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * kda_dplr_decode_step -- one token of the DPLR recurrence above for each of N
 * independent sequences, the state updated in place (e = b^T S_{t-1} is taken
 * before the decay).
 *   q, k, a, b  [N, H, D] in_dtype, 16-byte aligned
 *   v           [N, H, D] in_dtype
 *   log_alpha   [N, H, D] fp32
 *   state, o, N, H, in_dtype, stream and errors as for kda_decode_step with
 *   Dk = Dv = D; there is no beta.
 */
kda_status kda_dplr_decode_step(const void *q, const void *k, const void *v, const void *a, const void *b,
                                const float *log_alpha, float *state, int32_t N, int32_t H, int32_t D,
                                kda_dtype in_dtype, float *o, hipStream_t stream);

/*
 * gdn_decode_step -- one GDN token for each of N independent sequences, the
 * state updated in place; log_alpha is [N, H] fp32 (4-byte aligned).
 */
kda_status gdn_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, float *state, int32_t N, int32_t H, int32_t Dk,
                           int32_t Dv, kda_dtype in_dtype, float *o, hipStream_t stream);

/*
 * The KDA layer around the operator (the KDA-layer item of the page's
 * model-architecture list: L2Norm on q/k, a low-rank channel-wise decay gate,
 * a sigmoid output gate with RMSNorm), fused into the operator's kernels.  The
 * caller passes the raw bf16 projections; per (token, head) the library forms
 *
 *     q = q_raw / sqrt(|q_raw|^2 + l2_eps),  k likewise       (L2Norm)
 *     log_alpha = -softplus(x_alpha) = -log(1 + exp(x_alpha))  (decay gate)
 *     beta = sigmoid(x_beta)
 *
 * runs the KDA recurrence and readout o_t = S_t^T q_t, and returns
 *
 *     out = o / sqrt(mean_j o_j^2 + norm_eps) * norm_weight * sigmoid(out_gate)
 *
 * (RMSNorm over the head's Dv values, then the output gate).  The low-rank
 * projection producing x_alpha (and any bias) is the caller's GEMM; the page
 * does not name the gate's activation, -softplus is the one taken.  x_alpha =
 * +inf on every channel of a token resets the state.  The norms are formed in
 * fp32 and 1/|q|, 1/|k| are applied to the bf16 inputs at every use, so the
 * normalised vectors are never rounded.  l2_eps = 0 with an all-zero q or k row, or
 * norm_eps = 0 with an all-zero output row, gives NaN, as the formulas do.
 *
 *   q, k        [B, T, H, Dk] bf16   unnormalised queries / keys
 *   v           [B, T, H, Dv] bf16
 *   x_alpha     [B, T, H, Dk] bf16   decay-gate pre-activation (16-byte aligned)
 *   x_beta      [B, T, H]     bf16   beta pre-activation (2-byte aligned)
 *   out_gate    [B, T, H, Dv] bf16   output-gate pre-activation (16-byte aligned)
 *   norm_weight [Dv]          fp32   RMSNorm weight shared by all heads
 *   l2_eps, norm_eps                 finite, >= 0 (else KDA_ERR_INVALID_ARG)
 *   o           [B, T, H, Dv] fp32   the layer's output before its output projection
 *
 * kda_layer_chunk_fwd -- prefill at Dk = Dv = 128 with 64-token chunks (other
 * sizes return KDA_ERR_UNSUPPORTED).  init_state, cu_seqlens, n_seqs,
 * final_state, workspace (kda_layer_chunk_fwd_workspace_size(B, T, H, n_seqs)
 * bytes), stream and every convention not stated here are as for
 * kda_chunk_fwd.  The RMSNorm and output gate run inside the state pass: the
 * eight workgroups that each produce 16 of a row's 128 outputs exchange their
 * per-row sums of squares through the workspace (64-bit words tagged with a
 * per-call number), each waiting a bounded time for the others'.  They are
 * launched so that the eight are resident together; should a wait still run
 * out, the rows that wave of the workgroup writes from then on are NaN rather
 * than wrong.
 *
 * kda_layer_chunk_fwd_workspace_size -- bytes of device workspace
 * kda_layer_chunk_fwd needs: kda_chunk_fwd_workspace_size(B, T, H, 128, 128,
 * n_seqs, KDA_BF16, 64) plus 4 KiB per (chunk, head) for the row-norm
 * exchange.  0 for invalid sizes.
 */
size_t kda_layer_chunk_fwd_workspace_size(int32_t B, int64_t T, int32_t H, int32_t n_seqs);

kda_status kda_layer_chunk_fwd(const void *q, const void *k, const void *v, const void *x_alpha,
                               const void *x_beta, const void *out_gate, const float *norm_weight,
                               float l2_eps, float norm_eps, const float *init_state,
                               const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t Dk,
                               int32_t Dv, int32_t n_seqs, float *o, float *final_state, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * kda_layer_decode_step -- one layer token for each of N sequences, the state
 * updated in place; shapes as above without T ([N, H, ...]; x_beta [N, H],
 * 2-byte aligned), Dk, Dv in {16, 32, 64, 128}, everything else as for
 * kda_decode_step.
 */
kda_status kda_layer_decode_step(const void *q, const void *k, const void *v, const void *x_alpha,
                                 const void *x_beta, const void *out_gate, const float *norm_weight,
                                 float l2_eps, float norm_eps, float *state, int32_t N, int32_t H,
                                 int32_t Dk, int32_t Dv, float *o, hipStream_t stream);

/* Static name of a status code ("KDA_OK", ...). */
const char *kda_status_string(kda_status status);

/* Detail message of the last failing call on this host thread ("" if none). */
const char *kda_last_error(void);

/* KDA_VERSION of the built library. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
