/*
 * kda_oracle.c -- plain fp64 CPU oracle for the Kimi Delta Attention (KDA)
 * recurrence.  TEST INFRASTRUCTURE ONLY: nothing in the product path links,
 * loads or calls this file.  It shares no code, header, table or constant with
 * the HIP kernels or the C-ABI library.
 *
 * What it computes (per sequence n, per head h, tokens t of that sequence in
 * order), following the state-update equation in the section "Kimi Delta
 * Attention (KDA)" of the page "Kimi Linear 高效注意力架构" (chenshi221 wiki):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *
 * with the channel-wise decay alpha_t in [0,1]^{d_k} of the bullet on
 * channel-wise decay in the same section (alpha_t = exp(log_alpha_t); a
 * log_alpha of -inf is alpha = 0 exactly), and the readout o_t = S_t^T q_t
 * taken after the token's own write (the pages print no readout; this is the
 * operator's defined output).
 *
 * The product (I - b k k^T) Diag(a) S is expanded once, in the order the
 * equation writes it: first the decay Diag(a) S, then the erase/write
 *     S <- S' - b k (k^T S') + b k v^T  =  S' + b k (v - S'^T k)^T.
 * Nothing else is reordered, blocked or fused.  All arithmetic is IEEE fp64
 * with libm exp; build without -ffast-math.
 *
 * Layouts (dense, row-major, element strides):
 *   q, k       [B, T, H, Dk]     v, o  [B, T, H, Dv]
 *   log_alpha  [B, T, H, Dk]     beta  [B, T, H]
 *   states     [N, H, Dk, Dv]    (row c of a head's state is key channel c)
 * With cu_seqlens (int32 [N+1], host memory) the batch is one packed row
 * (B == 1) and sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]).
 * Without it there are N = B sequences of T tokens each.
 *
 * Gated DeltaNet (GDN), the scalar-gate recurrence the same page sets KDA
 * against (bullet on channel-wise decay in the KDA section: GDN has one
 * head-wise scalar alpha_t; the list of related work: GDN is DeltaNet with a
 * scalar forget gate; KDA's positioning: KDA turns that scalar into a
 * per-channel diagonal), is computed by gdn_token_update below from its own
 * equation, with alpha_t = exp(log_alpha_t) one number per (token, head):
 *
 *     S_t = (I - beta_t k_t k_t^T) alpha_t S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 *
 * and log_alpha laid out [B, T, H] (prefill) or [N, H] (decode).  It shares no
 * arithmetic with token_update, so the two can be checked against each other.
 *
 * The general diagonal-plus-low-rank (DPLR) transition that the same section
 * contrasts KDA with (its bullet on the hardware-efficient chunked algorithm:
 * KDA ties both low-rank vectors to the key; the related-work list: GLA and
 * RWKV7 use the general form), read with two free per-token vectors a_t and
 * b_t and an unscaled write, is computed by dplr_token_update:
 *
 *     S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t.
 *
 * KDA is the case a_t = -beta_t k_t, b_t = alpha_t * k_t with v_t scaled by
 * beta_t.  Both terms of the transition act on S_{t-1} as it was before the
 * token: e = b^T S_{t-1} first, then S = Diag(alpha) S_{t-1} + a e + k v^T.
 *
 * kda_oracle_backward is reverse-mode differentiation of the KDA token loop
 * above, one token at a time in reverse order (the gradients the training
 * workload of the pages needs: of q, k, v, log_alpha, beta and the initial
 * state, given the gradients of o and of the final state).  Written out for
 * one token, with S' = Diag(alpha) S_prev, p = S'^T k, u = beta (v - p),
 * S = S' + k u^T and o = S^T q, and dS the gradient of the loss with respect
 * to S from everything after the token:
 *
 *     dS += q do^T            dq = S do
 *     du  = dS^T k            dk = dS u + S' dp,   dp = -beta du
 *     dv  = beta du           dbeta = du . (v - p)
 *     dS' = dS + k dp^T       dlog_alpha_c = alpha_c sum_j S_prev[c][j] dS'[c][j]
 *     dS_prev = Diag(alpha) dS'
 *
 * (dlog_alpha is 0 where log_alpha = -inf: alpha = 0 there.)  The states the
 * reverse sweep needs are recomputed from checkpoints every 64 tokens.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *log_alpha, *beta, *init_state;
    const double *a, *b;    /* DPLR low-rank vectors [B, T, H, Dk] (mode 2 only) */
    const int32_t *cu_seqlens;
    int64_t B, T, H, Dk, Dv, N;
    int scalar_gate;        /* 0: KDA, log_alpha [.., Dk]; 1: GDN, log_alpha [..]; 2: DPLR */
    double *o, *final_state;
    /* native-typed inputs (kda_oracle_forward_native only): q, k, v as bf16
       bit patterns or fp32, log_alpha and beta fp32, read for the heads
       [h_lo, h_lo + Hs) of H; o, init_state and final_state then hold those
       Hs heads only ([B, T, Hs, Dv] and [N, Hs, Dk, Dv]). */
    const void *nq, *nk, *nv;
    const float *nla, *nbeta;
    int native, native_bf16;
    int64_t h_lo, Hs;
    int64_t next_unit;      /* work counter, guarded by lock */
    pthread_mutex_t lock;
} oracle_job;

/* Element i of a native-typed array, widened exactly to fp64 (a bf16 bit
 * pattern is the high half of an fp32 word). */
static double widen(const void *base, int bf16, size_t i)
{
    if (bf16) {
        const uint32_t w = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &w, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[i];
}

/* One token of the recurrence on one head's state S [Dk x Dv] (fp64).
 * p is caller scratch of length Dv.  Writes o_t (length Dv). */
static void token_update(double *S, int64_t Dk, int64_t Dv,
                         const double *q, const double *k, const double *v,
                         const double *log_alpha, double beta,
                         double *p, double *o_t)
{
    /* Diag(alpha_t) S_{t-1}: row c scaled by alpha_c = exp(log_alpha_c). */
    for (int64_t c = 0; c < Dk; ++c) {
        double a = exp(log_alpha[c]);
        for (int64_t j = 0; j < Dv; ++j) S[c * Dv + j] *= a;
    }
    /* p = S'^T k  (what the decayed memory returns for key k). */
    for (int64_t j = 0; j < Dv; ++j) p[j] = 0.0;
    for (int64_t c = 0; c < Dk; ++c)
        for (int64_t j = 0; j < Dv; ++j) p[j] += S[c * Dv + j] * k[c];
    /* S = S' + beta k (v - p)^T  ==  (I - beta k k^T) S' + beta k v^T. */
    for (int64_t c = 0; c < Dk; ++c) {
        double bk = beta * k[c];
        for (int64_t j = 0; j < Dv; ++j) S[c * Dv + j] += bk * (v[j] - p[j]);
    }
    /* o_t = S_t^T q_t. */
    for (int64_t j = 0; j < Dv; ++j) o_t[j] = 0.0;
    for (int64_t c = 0; c < Dk; ++c)
        for (int64_t j = 0; j < Dv; ++j) o_t[j] += S[c * Dv + j] * q[c];
}

/* One token of the GDN recurrence: the whole state is scaled by the head's
 * scalar alpha_t, then the same delta-rule erase/write, then the readout.
 * The rank-1 terms are formed explicitly from (I - beta k k^T) S':
 * e = k^T S' (a row vector), S = S' - beta k e + beta k v^T. */
static void gdn_token_update(double *S, int64_t Dk, int64_t Dv,
                             const double *q, const double *k, const double *v,
                             double log_alpha, double beta, double *e, double *o_t)
{
    const double a = exp(log_alpha);
    for (int64_t i = 0; i < Dk * Dv; ++i) S[i] = a * S[i];
    for (int64_t j = 0; j < Dv; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < Dk; ++c) acc += k[c] * S[c * Dv + j];
        e[j] = acc;
    }
    for (int64_t c = 0; c < Dk; ++c)
        for (int64_t j = 0; j < Dv; ++j)
            S[c * Dv + j] = S[c * Dv + j] - beta * k[c] * e[j] + beta * k[c] * v[j];
    for (int64_t j = 0; j < Dv; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < Dk; ++c) acc += q[c] * S[c * Dv + j];
        o_t[j] = acc;
    }
}

/* One token of the DPLR recurrence.  e (caller scratch, length Dv) is
 * b^T S_{t-1}, taken before S changes; then every row c of the state becomes
 * alpha_c S_{t-1}[c] + a_c e + k_c v^T; then the readout. */
static void dplr_token_update(double *S, int64_t Dk, int64_t Dv,
                              const double *q, const double *k, const double *v,
                              const double *a, const double *b, const double *log_alpha,
                              double *e, double *o_t)
{
    for (int64_t j = 0; j < Dv; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < Dk; ++c) acc += b[c] * S[c * Dv + j];
        e[j] = acc;
    }
    for (int64_t c = 0; c < Dk; ++c) {
        const double al = exp(log_alpha[c]);
        for (int64_t j = 0; j < Dv; ++j)
            S[c * Dv + j] = al * S[c * Dv + j] + a[c] * e[j] + k[c] * v[j];
    }
    for (int64_t j = 0; j < Dv; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < Dk; ++c) acc += q[c] * S[c * Dv + j];
        o_t[j] = acc;
    }
}

/* The token loop of one (sequence n, head h) unit on native-typed inputs:
 * each token's q, k, v, log_alpha and beta are widened to fp64 (exactly) into
 * the caller's buffers x (2 Dk + Dv + Dk), then token_update runs as in
 * run_unit below. */
static void run_unit_native(const oracle_job *J, int64_t n, int64_t h, double *S, double *p, double *x)
{
    const int64_t Dk = J->Dk, Dv = J->Dv, H = J->H, hs = h - J->h_lo;
    double *qb = x, *kb = qb + Dk, *vb = kb + Dk, *lab = vb + Dv;
    int64_t b, t0, t1;
    if (J->cu_seqlens) { b = 0; t0 = J->cu_seqlens[n]; t1 = J->cu_seqlens[n + 1]; }
    else               { b = n; t0 = 0;               t1 = J->T; }

    const size_t sidx = (size_t)(n * J->Hs + hs) * (size_t)(Dk * Dv);
    if (J->init_state) memcpy(S, J->init_state + sidx, sizeof(double) * (size_t)(Dk * Dv));
    else               memset(S, 0, sizeof(double) * (size_t)(Dk * Dv));

    for (int64_t t = t0; t < t1; ++t) {
        const size_t row = (size_t)((b * J->T + t) * H + h);
        for (int64_t c = 0; c < Dk; ++c) {
            qb[c] = widen(J->nq, J->native_bf16, row * (size_t)Dk + (size_t)c);
            kb[c] = widen(J->nk, J->native_bf16, row * (size_t)Dk + (size_t)c);
            lab[c] = (double)J->nla[row * (size_t)Dk + (size_t)c];
        }
        for (int64_t j = 0; j < Dv; ++j) vb[j] = widen(J->nv, J->native_bf16, row * (size_t)Dv + (size_t)j);
        const size_t orow = (size_t)((b * J->T + t) * J->Hs + hs);
        token_update(S, Dk, Dv, qb, kb, vb, lab, (double)J->nbeta[row], p, J->o + orow * (size_t)Dv);
    }
    if (J->final_state) memcpy(J->final_state + sidx, S, sizeof(double) * (size_t)(Dk * Dv));
}

/* Runs the whole token loop of one (sequence n, head h) unit. */
static void run_unit(const oracle_job *J, int64_t n, int64_t h, double *S, double *p)
{
    const int64_t Dk = J->Dk, Dv = J->Dv, H = J->H;
    int64_t b, t0, t1;
    if (J->cu_seqlens) { b = 0; t0 = J->cu_seqlens[n]; t1 = J->cu_seqlens[n + 1]; }
    else               { b = n; t0 = 0;               t1 = J->T; }

    const size_t sidx = (size_t)(n * H + h) * (size_t)(Dk * Dv);
    if (J->init_state) memcpy(S, J->init_state + sidx, sizeof(double) * (size_t)(Dk * Dv));
    else               memset(S, 0, sizeof(double) * (size_t)(Dk * Dv));

    for (int64_t t = t0; t < t1; ++t) {
        const size_t row = (size_t)((b * J->T + t) * H + h);
        if (J->scalar_gate == 2)
            dplr_token_update(S, Dk, Dv,
                              J->q + row * (size_t)Dk, J->k + row * (size_t)Dk,
                              J->v + row * (size_t)Dv, J->a + row * (size_t)Dk,
                              J->b + row * (size_t)Dk, J->log_alpha + row * (size_t)Dk,
                              p, J->o + row * (size_t)Dv);
        else if (J->scalar_gate)
            gdn_token_update(S, Dk, Dv,
                             J->q + row * (size_t)Dk, J->k + row * (size_t)Dk,
                             J->v + row * (size_t)Dv, J->log_alpha[row],
                             J->beta[row], p, J->o + row * (size_t)Dv);
        else
            token_update(S, Dk, Dv,
                         J->q + row * (size_t)Dk, J->k + row * (size_t)Dk,
                         J->v + row * (size_t)Dv, J->log_alpha + row * (size_t)Dk,
                         J->beta[row], p, J->o + row * (size_t)Dv);
    }
    if (J->final_state) memcpy(J->final_state + sidx, S, sizeof(double) * (size_t)(Dk * Dv));
}

static void *worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)(J->Dk * J->Dv));
    double *p = (double *)malloc(sizeof(double) * (size_t)J->Dv);
    double *x = (double *)malloc(sizeof(double) * (size_t)(3 * J->Dk + J->Dv));
    if (!S || !p || !x) { free(S); free(p); free(x); return (void *)1; }
    const int64_t hs = J->native ? J->Hs : J->H;
    const int64_t units = J->N * hs;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (u >= units) break;
        if (J->native) run_unit_native(J, u / hs, J->h_lo + u % hs, S, p, x);
        else           run_unit(J, u / hs, u % hs, S, p);
    }
    free(S);
    free(p);
    free(x);
    return NULL;
}

/* Spreads the job's (sequence, head) units over n_threads POSIX threads. */
static int run_job(oracle_job *J, int n_threads)
{
    const int64_t units = J->N * (J->native ? J->Hs : J->H);
    pthread_mutex_init(&J->lock, NULL);
    if (n_threads < 1) n_threads = 1;
    if ((int64_t)n_threads > units) n_threads = (int)(units > 0 ? units : 1);
    int rc = 0;
    pthread_t *tid = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    int started = 0;
    if (!tid) rc = -2;
    for (int i = 0; i < n_threads && rc == 0; ++i) {
        if (pthread_create(&tid[i], NULL, worker, J) != 0) rc = -2;
        else ++started;
    }
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(tid[i], &ret);
        if (ret) rc = -2;
    }
    free(tid);
    pthread_mutex_destroy(&J->lock);
    return rc;
}

/*
 * kda_oracle_forward: the recurrence over every (sequence, head) unit.
 * All pointers are host memory.  init_state and final_state may be NULL
 * (zeros in / no state out); cu_seqlens may be NULL (dense batch).  Units are
 * independent and are spread over n_threads POSIX threads (<= 0 means 1);
 * each unit is computed by exactly one thread in token order, so results do
 * not depend on n_threads.  Returns 0 on success, -1 on a bad argument,
 * -2 when a thread or allocation fails.
 */
static int forward_impl(const double *q, const double *k, const double *v,
                        const double *log_alpha, const double *beta,
                        const double *init_state, const int32_t *cu_seqlens,
                        int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                        int64_t n_seqs, double *o, double *final_state, int n_threads,
                        int scalar_gate, const double *a, const double *b)
{
    if (!q || !k || !v || !log_alpha || !o) return -1;
    if (scalar_gate == 2 ? (!a || !b) : !beta) return -1;
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return -1;
    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.scalar_gate = scalar_gate;
    J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta;
    J.a = a; J.b = b;
    J.init_state = init_state; J.cu_seqlens = cu_seqlens;
    J.B = B; J.T = T; J.H = H; J.Dk = Dk; J.Dv = Dv;
    J.o = o; J.final_state = final_state;
    if (cu_seqlens) {
        if (B != 1 || n_seqs < 1) return -1;
        if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != T) return -1;
        for (int64_t n = 0; n < n_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
        J.N = n_seqs;
    } else {
        J.N = B;
    }
    return run_job(&J, n_threads);
}

int kda_oracle_forward(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *beta,
                       const double *init_state, const int32_t *cu_seqlens,
                       int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                       int64_t n_seqs, double *o, double *final_state, int n_threads)
{
    return forward_impl(q, k, v, log_alpha, beta, init_state, cu_seqlens, B, T, H, Dk, Dv,
                        n_seqs, o, final_state, n_threads, 0, NULL, NULL);
}

/*
 * kda_oracle_forward_native: kda_oracle_forward on inputs in the types the
 * GPU path receives, for the heads [h_lo, h_hi) of H only.  q, k
 * [B, T, H, Dk] and v [B, T, H, Dv] are bf16 bit patterns (in_bf16 = 1) or
 * fp32 (in_bf16 = 0); log_alpha [B, T, H, Dk] and beta [B, T, H] are fp32.
 * Each token's values are widened exactly to fp64 and the same token_update
 * runs, so the result equals kda_oracle_forward on the widened arrays.
 * init_state (nullable), o and final_state (nullable) are fp64 and hold the
 * selected heads only: [N, h_hi - h_lo, Dk, Dv] and [B, T, h_hi - h_lo, Dv].
 * cu_seqlens, threads and return codes as in kda_oracle_forward.
 */
int kda_oracle_forward_native(const void *q, const void *k, const void *v, int in_bf16,
                              const float *log_alpha, const float *beta,
                              const double *init_state, const int32_t *cu_seqlens,
                              int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                              int64_t n_seqs, int64_t h_lo, int64_t h_hi,
                              double *o, double *final_state, int n_threads)
{
    if (!q || !k || !v || !log_alpha || !beta || !o) return -1;
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return -1;
    if (h_lo < 0 || h_hi > H || h_lo >= h_hi) return -1;
    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.native = 1;
    J.native_bf16 = in_bf16 ? 1 : 0;
    J.nq = q; J.nk = k; J.nv = v; J.nla = log_alpha; J.nbeta = beta;
    J.h_lo = h_lo; J.Hs = h_hi - h_lo;
    J.init_state = init_state; J.cu_seqlens = cu_seqlens;
    J.B = B; J.T = T; J.H = H; J.Dk = Dk; J.Dv = Dv;
    J.o = o; J.final_state = final_state;
    if (cu_seqlens) {
        if (B != 1 || n_seqs < 1) return -1;
        if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != T) return -1;
        for (int64_t n = 0; n < n_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
        J.N = n_seqs;
    } else {
        J.N = B;
    }
    return run_job(&J, n_threads);
}

/*
 * gdn_oracle_forward: the GDN recurrence over every (sequence, head) unit,
 * with log_alpha [B, T, H] (one scalar per token and head).  Everything else
 * (layouts, cu_seqlens, threads, return codes) is as in kda_oracle_forward.
 */
int gdn_oracle_forward(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *beta,
                       const double *init_state, const int32_t *cu_seqlens,
                       int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                       int64_t n_seqs, double *o, double *final_state, int n_threads)
{
    return forward_impl(q, k, v, log_alpha, beta, init_state, cu_seqlens, B, T, H, Dk, Dv,
                        n_seqs, o, final_state, n_threads, 1, NULL, NULL);
}

/*
 * dplr_oracle_forward: the DPLR recurrence over every (sequence, head) unit,
 * with a, b [B, T, H, Dk] beside q and k and no beta.  Everything else
 * (layouts, cu_seqlens, threads, return codes) is as in kda_oracle_forward.
 */
int dplr_oracle_forward(const double *q, const double *k, const double *v,
                        const double *a, const double *b, const double *log_alpha,
                        const double *init_state, const int32_t *cu_seqlens,
                        int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                        int64_t n_seqs, double *o, double *final_state, int n_threads)
{
    return forward_impl(q, k, v, log_alpha, NULL, init_state, cu_seqlens, B, T, H, Dk, Dv,
                        n_seqs, o, final_state, n_threads, 2, a, b);
}

/*
 * kda_oracle_decode_step: one token for each of N independent states, the
 * state updated in place.  q, k [N, H, Dk]; v, o [N, H, Dv];
 * log_alpha [N, H, Dk]; beta [N, H]; state [N, H, Dk, Dv].  This is the same
 * token_update as above, applied once per (n, h).
 */
int kda_oracle_decode_step(const double *q, const double *k, const double *v,
                           const double *log_alpha, const double *beta,
                           double *state, int64_t N, int64_t H, int64_t Dk,
                           int64_t Dv, double *o)
{
    if (!q || !k || !v || !log_alpha || !beta || !state || !o) return -1;
    if (N < 1 || H < 1 || Dk < 1 || Dv < 1) return -1;
    double *p = (double *)malloc(sizeof(double) * (size_t)Dv);
    if (!p) return -2;
    for (int64_t u = 0; u < N * H; ++u)
        token_update(state + (size_t)u * (size_t)(Dk * Dv), Dk, Dv,
                     q + (size_t)u * (size_t)Dk, k + (size_t)u * (size_t)Dk,
                     v + (size_t)u * (size_t)Dv, log_alpha + (size_t)u * (size_t)Dk,
                     beta[u], p, o + (size_t)u * (size_t)Dv);
    free(p);
    return 0;
}

/*
 * gdn_oracle_decode_step: one GDN token for each of N independent states, the
 * state updated in place; log_alpha [N, H], the other layouts as in
 * kda_oracle_decode_step.
 */
int gdn_oracle_decode_step(const double *q, const double *k, const double *v,
                           const double *log_alpha, const double *beta,
                           double *state, int64_t N, int64_t H, int64_t Dk,
                           int64_t Dv, double *o)
{
    if (!q || !k || !v || !log_alpha || !beta || !state || !o) return -1;
    if (N < 1 || H < 1 || Dk < 1 || Dv < 1) return -1;
    double *e = (double *)malloc(sizeof(double) * (size_t)Dv);
    if (!e) return -2;
    for (int64_t u = 0; u < N * H; ++u)
        gdn_token_update(state + (size_t)u * (size_t)(Dk * Dv), Dk, Dv,
                         q + (size_t)u * (size_t)Dk, k + (size_t)u * (size_t)Dk,
                         v + (size_t)u * (size_t)Dv, log_alpha[u],
                         beta[u], e, o + (size_t)u * (size_t)Dv);
    free(e);
    return 0;
}

/*
 * dplr_oracle_decode_step: one DPLR token for each of N independent states,
 * the state updated in place; q, k, a, b, log_alpha [N, H, Dk], v, o
 * [N, H, Dv].  This is dplr_token_update applied once per (n, h).
 */
int dplr_oracle_decode_step(const double *q, const double *k, const double *v,
                            const double *a, const double *b, const double *log_alpha,
                            double *state, int64_t N, int64_t H, int64_t Dk,
                            int64_t Dv, double *o)
{
    if (!q || !k || !v || !a || !b || !log_alpha || !state || !o) return -1;
    if (N < 1 || H < 1 || Dk < 1 || Dv < 1) return -1;
    double *e = (double *)malloc(sizeof(double) * (size_t)Dv);
    if (!e) return -2;
    for (int64_t u = 0; u < N * H; ++u)
        dplr_token_update(state + (size_t)u * (size_t)(Dk * Dv), Dk, Dv,
                          q + (size_t)u * (size_t)Dk, k + (size_t)u * (size_t)Dk,
                          v + (size_t)u * (size_t)Dv, a + (size_t)u * (size_t)Dk,
                          b + (size_t)u * (size_t)Dk, log_alpha + (size_t)u * (size_t)Dk,
                          e, o + (size_t)u * (size_t)Dv);
    free(e);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Backward (reverse mode) of the KDA token loop.                            */
/* ------------------------------------------------------------------------- */
#define BWD_SEG 64

typedef struct {
    const double *q, *k, *v, *log_alpha, *beta, *init_state, *d_o, *d_final;
    const int32_t *cu_seqlens;
    int64_t B, T, H, Dk, Dv, N;
    double *dq, *dk, *dv, *dlog_alpha, *dbeta, *d_init;
    int64_t next_unit;
    pthread_mutex_t lock;
} bwd_job;

/* Reverse step of one token.  S_prev: state before the token, S: after it,
 * dS: in = gradient with respect to S from later tokens and the final state;
 * out = gradient with respect to S_prev.  Scratch: Sd (Dk*Dv), p, u, du, dp (Dv). */
static void token_backward(int64_t Dk, int64_t Dv, const double *S_prev, const double *S,
                           const double *q, const double *k, const double *v,
                           const double *log_alpha, double beta, const double *d_o,
                           double *dS, double *Sd, double *p, double *u, double *du, double *dp,
                           double *dq, double *dk, double *dv, double *dla, double *dbeta)
{
    /* the forward quantities of the token: S' (Sd), p, u */
    for (int64_t c = 0; c < Dk; ++c) {
        const double a = exp(log_alpha[c]);
        for (int64_t j = 0; j < Dv; ++j) Sd[c * Dv + j] = a * S_prev[c * Dv + j];
    }
    for (int64_t j = 0; j < Dv; ++j) p[j] = 0.0;
    for (int64_t c = 0; c < Dk; ++c)
        for (int64_t j = 0; j < Dv; ++j) p[j] += Sd[c * Dv + j] * k[c];
    for (int64_t j = 0; j < Dv; ++j) u[j] = beta * (v[j] - p[j]);

    /* readout o = S^T q */
    for (int64_t c = 0; c < Dk; ++c)
        for (int64_t j = 0; j < Dv; ++j) dS[c * Dv + j] += q[c] * d_o[j];
    for (int64_t c = 0; c < Dk; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < Dv; ++j) acc += S[c * Dv + j] * d_o[j];
        dq[c] = acc;
    }
    /* S = S' + k u^T */
    for (int64_t j = 0; j < Dv; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < Dk; ++c) acc += dS[c * Dv + j] * k[c];
        du[j] = acc;
    }
    for (int64_t c = 0; c < Dk; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < Dv; ++j) acc += dS[c * Dv + j] * u[j];
        dk[c] = acc;
    }
    /* u = beta (v - p) */
    double db = 0.0;
    for (int64_t j = 0; j < Dv; ++j) {
        db += du[j] * (v[j] - p[j]);
        dv[j] = beta * du[j];
        dp[j] = -beta * du[j];
    }
    *dbeta = db;
    /* p = S'^T k: dS' = dS + k dp^T, dk += S' dp */
    for (int64_t c = 0; c < Dk; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < Dv; ++j) acc += Sd[c * Dv + j] * dp[j];
        dk[c] += acc;
        for (int64_t j = 0; j < Dv; ++j) dS[c * Dv + j] += k[c] * dp[j];
    }
    /* S' = Diag(alpha) S_prev */
    for (int64_t c = 0; c < Dk; ++c) {
        const double a = exp(log_alpha[c]);
        double acc = 0.0;
        for (int64_t j = 0; j < Dv; ++j) acc += S_prev[c * Dv + j] * dS[c * Dv + j];
        dla[c] = a * acc;
        for (int64_t j = 0; j < Dv; ++j) dS[c * Dv + j] *= a;
    }
}

static int run_bwd_unit(const bwd_job *J, int64_t n, int64_t h, double *ckpt, double *seg,
                        double *dS, double *scratch)
{
    const int64_t Dk = J->Dk, Dv = J->Dv, H = J->H, DD = Dk * Dv;
    int64_t b, t0, t1;
    if (J->cu_seqlens) { b = 0; t0 = J->cu_seqlens[n]; t1 = J->cu_seqlens[n + 1]; }
    else               { b = n; t0 = 0;               t1 = J->T; }
    const int64_t L = t1 - t0, nseg = (L + BWD_SEG - 1) / BWD_SEG;
    const size_t sidx = (size_t)(n * H + h) * (size_t)DD;
    double *Sd = scratch, *p = Sd + DD, *o_t = p + Dv, *u = o_t + Dv, *du = u + Dv, *dp = du + Dv;

    /* forward: checkpoint the state at the start of every segment */
    double *S = seg;  /* running state (seg[0]) */
    if (J->init_state) memcpy(S, J->init_state + sidx, sizeof(double) * (size_t)DD);
    else               memset(S, 0, sizeof(double) * (size_t)DD);
    for (int64_t t = t0; t < t1; ++t) {
        if ((t - t0) % BWD_SEG == 0)
            memcpy(ckpt + (size_t)((t - t0) / BWD_SEG) * (size_t)DD, S, sizeof(double) * (size_t)DD);
        const size_t row = (size_t)((b * J->T + t) * H + h);
        token_update(S, Dk, Dv, J->q + row * (size_t)Dk, J->k + row * (size_t)Dk, J->v + row * (size_t)Dv,
                     J->log_alpha + row * (size_t)Dk, J->beta[row], p, o_t);
    }
    /* reverse sweep */
    if (J->d_final) memcpy(dS, J->d_final + sidx, sizeof(double) * (size_t)DD);
    else            memset(dS, 0, sizeof(double) * (size_t)DD);
    for (int64_t m = nseg - 1; m >= 0; --m) {
        const int64_t s0 = t0 + m * BWD_SEG, s1 = (s0 + BWD_SEG < t1) ? s0 + BWD_SEG : t1;
        /* seg[i] = state before token s0 + i; seg[s1 - s0] = state after the last */
        memcpy(seg, ckpt + (size_t)m * (size_t)DD, sizeof(double) * (size_t)DD);
        for (int64_t t = s0; t < s1; ++t) {
            double *nxt = seg + (size_t)(t - s0 + 1) * (size_t)DD;
            memcpy(nxt, seg + (size_t)(t - s0) * (size_t)DD, sizeof(double) * (size_t)DD);
            const size_t row = (size_t)((b * J->T + t) * H + h);
            token_update(nxt, Dk, Dv, J->q + row * (size_t)Dk, J->k + row * (size_t)Dk,
                         J->v + row * (size_t)Dv, J->log_alpha + row * (size_t)Dk, J->beta[row], p, o_t);
        }
        for (int64_t t = s1 - 1; t >= s0; --t) {
            const size_t row = (size_t)((b * J->T + t) * H + h);
            token_backward(Dk, Dv, seg + (size_t)(t - s0) * (size_t)DD, seg + (size_t)(t - s0 + 1) * (size_t)DD,
                           J->q + row * (size_t)Dk, J->k + row * (size_t)Dk, J->v + row * (size_t)Dv,
                           J->log_alpha + row * (size_t)Dk, J->beta[row], J->d_o + row * (size_t)Dv,
                           dS, Sd, p, u, du, dp,
                           J->dq + row * (size_t)Dk, J->dk + row * (size_t)Dk, J->dv + row * (size_t)Dv,
                           J->dlog_alpha + row * (size_t)Dk, J->dbeta + row);
        }
    }
    if (J->d_init) memcpy(J->d_init + sidx, dS, sizeof(double) * (size_t)DD);
    return 0;
}

static void *bwd_worker(void *arg)
{
    bwd_job *J = (bwd_job *)arg;
    const int64_t DD = J->Dk * J->Dv;
    int64_t maxL = J->T;  /* the longest sequence bounds the checkpoints */
    const int64_t nck = (maxL + BWD_SEG - 1) / BWD_SEG + 1;
    double *ckpt = (double *)malloc(sizeof(double) * (size_t)(nck * DD));
    double *seg = (double *)malloc(sizeof(double) * (size_t)((BWD_SEG + 1) * DD));
    double *dS = (double *)malloc(sizeof(double) * (size_t)DD);
    double *scratch = (double *)malloc(sizeof(double) * (size_t)(DD + 5 * J->Dv));
    if (!ckpt || !seg || !dS || !scratch) { free(ckpt); free(seg); free(dS); free(scratch); return (void *)1; }
    const int64_t units = J->N * J->H;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t un = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (un >= units) break;
        run_bwd_unit(J, un / J->H, un % J->H, ckpt, seg, dS, scratch);
    }
    free(ckpt); free(seg); free(dS); free(scratch);
    return NULL;
}

/*
 * kda_oracle_backward: gradients of the KDA forward (kda_oracle_forward, same
 * layouts and cu_seqlens rules) given d_o [B, T, H, Dv] and d_final
 * [N, H, Dk, Dv] (NULL: zero).  Writes dq, dk, dlog_alpha [B, T, H, Dk],
 * dv [B, T, H, Dv], dbeta [B, T, H] and d_init [N, H, Dk, Dv] (NULL: not
 * written).  Tokens of no sequence are left untouched.  Threads and return
 * codes as in kda_oracle_forward.
 */
int kda_oracle_backward(const double *q, const double *k, const double *v,
                        const double *log_alpha, const double *beta,
                        const double *init_state, const int32_t *cu_seqlens,
                        int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t n_seqs,
                        const double *d_o, const double *d_final,
                        double *dq, double *dk, double *dv, double *dlog_alpha, double *dbeta,
                        double *d_init, int n_threads)
{
    if (!q || !k || !v || !log_alpha || !beta || !d_o || !dq || !dk || !dv || !dlog_alpha || !dbeta) return -1;
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return -1;
    bwd_job J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta;
    J.init_state = init_state; J.d_o = d_o; J.d_final = d_final; J.cu_seqlens = cu_seqlens;
    J.B = B; J.T = T; J.H = H; J.Dk = Dk; J.Dv = Dv;
    J.dq = dq; J.dk = dk; J.dv = dv; J.dlog_alpha = dlog_alpha; J.dbeta = dbeta; J.d_init = d_init;
    if (cu_seqlens) {
        if (B != 1 || n_seqs < 1) return -1;
        if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != T) return -1;
        for (int64_t n = 0; n < n_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
        J.N = n_seqs;
    } else {
        J.N = B;
    }
    pthread_mutex_init(&J.lock, NULL);
    if (n_threads < 1) n_threads = 1;
    if ((int64_t)n_threads > J.N * H) n_threads = (int)(J.N * H);
    int rc = 0, started = 0;
    pthread_t *tid = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!tid) rc = -2;
    for (int i = 0; i < n_threads && rc == 0; ++i) {
        if (pthread_create(&tid[i], NULL, bwd_worker, &J) != 0) rc = -2;
        else ++started;
    }
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(tid[i], &ret);
        if (ret) rc = -2;
    }
    free(tid);
    pthread_mutex_destroy(&J.lock);
    return rc;
}
