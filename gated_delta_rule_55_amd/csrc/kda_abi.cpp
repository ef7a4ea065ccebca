// kda_abi.cpp -- the extern "C" entry points of libkda.so: host-only argument
// validation, workspace sizing and dispatch to the gfx950 kernels.  Nothing
// here dereferences a device pointer or calls HIP before validation passes.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_err[512] = "";

kda_status fail(kda_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

bool supported_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// A nonzero tag per layer prefill call: the state pass marks its row-norm
// partial sums with it, so words left in a reused workspace by an earlier call
// never pass for this call's.
uint32_t next_layer_tag() {
    static std::atomic<uint32_t> counter{0};
    uint32_t t;
    do {
        t = counter.fetch_add(1, std::memory_order_relaxed) + 1;
    } while (t == 0);
    return t;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void *p, size_t bytes) {
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// Multiplies non-negative sizes, reporting overflow of size_t.
bool mul_ok(size_t &acc, uint64_t f) {
    if (f != 0 && acc > SIZE_MAX / f) return false;
    acc *= f;
    return true;
}

bool bytes_of(size_t &out, std::initializer_list<uint64_t> dims, size_t elem) {
    size_t acc = elem;
    for (uint64_t d : dims)
        if (!mul_ok(acc, d)) return false;
    out = acc;
    return true;
}

// One device buffer the call reads: its bytes and the alignment its loads need.
struct Input {
    const void *p;
    const char *name;
    size_t bytes;
    unsigned align;
    bool required;
};

bool aligned(const void *p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The KDA layer's extra arguments (gate mode 2).
struct LayerIn {
    const void *x_alpha, *x_beta, *out_gate;
    const float *norm_weight;
    float l2_eps, norm_eps;
};

bool eps_ok(float e) { return e >= 0.f && e <= 3.0e38f; }  // rejects NaN, inf and negatives

}  // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

const char *kda_last_error(void) { return g_err; }

int kda_version(void) { return KDA_VERSION; }

static kda_status decode_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                              const float *beta, float *state, int32_t N, int32_t H, int32_t Dk,
                              int32_t Dv, kda_dtype in_dtype, float *o, hipStream_t stream,
                              int gate_mode, const LayerIn *L, const void *lr_a = nullptr,
                              const void *lr_b = nullptr) {
    g_err[0] = '\0';
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype %d is not KDA_BF16 or KDA_F32", (int)in_dtype);
    if (gate_mode == 2 && in_dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "the layer entry points take bf16 inputs");
    if (!supported_dim(Dk) || !supported_dim(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "Dk=%d Dv=%d: each must be 16, 32, 64 or 128", Dk, Dv);
    if (N < 0 || H < 1) return fail(KDA_ERR_INVALID_ARG, "N=%d H=%d: need N >= 0, H >= 1", N, H);
    if ((int64_t)N * H > 0x7fffffff)
        return fail(KDA_ERR_INVALID_ARG, "N*H=%lld exceeds the grid limit", (long long)N * H);
    if (gate_mode == 2 && (!eps_ok(L->l2_eps) || !eps_ok(L->norm_eps)))
        return fail(KDA_ERR_INVALID_ARG, "l2_eps and norm_eps must be finite and >= 0");
    if (N == 0) return KDA_OK;
    const size_t esz = in_dtype == KDA_BF16 ? 2 : 4;
    size_t bq, bv, bg, bb, bs, bo, bxa, bxb, bog;
    if (!bytes_of(bq, {(uint64_t)N, (uint64_t)H, (uint64_t)Dk}, esz) ||
        !bytes_of(bv, {(uint64_t)N, (uint64_t)H, (uint64_t)Dv}, esz) ||
        !bytes_of(bg, {(uint64_t)N, (uint64_t)H, gate_mode == 1 ? 1u : (uint64_t)Dk}, 4) ||
        !bytes_of(bb, {(uint64_t)N, (uint64_t)H}, 4) ||
        !bytes_of(bs, {(uint64_t)N, (uint64_t)H, (uint64_t)Dk, (uint64_t)Dv}, 4) ||
        !bytes_of(bo, {(uint64_t)N, (uint64_t)H, (uint64_t)Dv}, 4) ||
        !bytes_of(bxa, {(uint64_t)N, (uint64_t)H, (uint64_t)Dk}, 2) ||
        !bytes_of(bxb, {(uint64_t)N, (uint64_t)H}, 2) ||
        !bytes_of(bog, {(uint64_t)N, (uint64_t)H, (uint64_t)Dv}, 2))
        return fail(KDA_ERR_INVALID_ARG, "tensor sizes overflow size_t");
    Input in[8];
    int n_in = 0;
    in[n_in++] = {q, "q", bq, 16, true};
    in[n_in++] = {k, "k", bq, 16, true};
    in[n_in++] = {v, "v", bv, 16, true};
    if (gate_mode == 2) {
        in[n_in++] = {L->x_alpha, "x_alpha", bxa, 2, true};
        in[n_in++] = {L->x_beta, "x_beta", bxb, 2, true};
        in[n_in++] = {L->out_gate, "out_gate", bog, 2, true};
        in[n_in++] = {L->norm_weight, "norm_weight", (size_t)Dv * 4, 16, true};
    } else if (gate_mode == 3) {
        in[n_in++] = {lr_a, "a", bq, 16, true};
        in[n_in++] = {lr_b, "b", bq, 16, true};
        in[n_in++] = {log_alpha, "log_alpha", bg, 16, true};
    } else {
        // a per-channel gate is read in 16-byte vectors; a scalar gate and beta one by one
        in[n_in++] = {log_alpha, "log_alpha", bg, gate_mode == 1 ? 4u : 16u, true};
        in[n_in++] = {beta, "beta", bb, 4, true};
    }
    for (int i = 0; i < n_in; ++i) {
        if (!in[i].p) return fail(KDA_ERR_INVALID_ARG, "%s is NULL", in[i].name);
        if (!aligned(in[i].p, in[i].align))
            return fail(KDA_ERR_INVALID_ARG, "%s is not %u-byte aligned", in[i].name, in[i].align);
    }
    if (!state) return fail(KDA_ERR_INVALID_ARG, "state is NULL");
    if (!aligned16(state)) return fail(KDA_ERR_INVALID_ARG, "state is not 16-byte aligned");
    if (!o) return fail(KDA_ERR_INVALID_ARG, "o is NULL");
    if (!aligned16(o)) return fail(KDA_ERR_INVALID_ARG, "o is not 16-byte aligned");
    const Range ro = span(o, bo), rs = span(state, bs);
    for (int i = 0; i < n_in; ++i) {
        const Range ri = span(in[i].p, in[i].bytes);
        if (overlap(ro, ri)) return fail(KDA_ERR_INVALID_ARG, "o overlaps %s", in[i].name);
        if (overlap(rs, ri)) return fail(KDA_ERR_INVALID_ARG, "state overlaps %s", in[i].name);
    }
    if (overlap(ro, rs)) return fail(KDA_ERR_INVALID_ARG, "o overlaps state");

    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.state = state; a.o = o;
    a.N = N; a.H = H; a.Dk = Dk; a.Dv = Dv; a.bf16 = in_dtype == KDA_BF16; a.gate_mode = gate_mode;
    if (gate_mode == 2) {
        a.x_alpha = static_cast<const uint16_t *>(L->x_alpha);
        a.x_beta = static_cast<const uint16_t *>(L->x_beta);
        a.out_gate = static_cast<const uint16_t *>(L->out_gate);
        a.norm_weight = L->norm_weight;
        a.l2_eps = L->l2_eps;
        a.norm_eps = L->norm_eps;
    }
    a.lr_a = lr_a; a.lr_b = lr_b;
    hipError_t e = kda::launch_decode(a, stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

kda_status kda_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, float *state, int32_t N, int32_t H, int32_t Dk,
                           int32_t Dv, kda_dtype in_dtype, float *o, hipStream_t stream) {
    return decode_impl(q, k, v, log_alpha, beta, state, N, H, Dk, Dv, in_dtype, o, stream, 0, nullptr);
}

kda_status kda_dplr_decode_step(const void *q, const void *k, const void *v, const void *a, const void *b,
                                const float *log_alpha, float *state, int32_t N, int32_t H, int32_t D,
                                kda_dtype in_dtype, float *o, hipStream_t stream) {
    return decode_impl(q, k, v, log_alpha, nullptr, state, N, H, D, D, in_dtype, o, stream, 3, nullptr, a, b);
}

kda_status gdn_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, float *state, int32_t N, int32_t H, int32_t Dk,
                           int32_t Dv, kda_dtype in_dtype, float *o, hipStream_t stream) {
    return decode_impl(q, k, v, log_alpha, beta, state, N, H, Dk, Dv, in_dtype, o, stream, 1, nullptr);
}

static bool workspace_bytes(int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                            bool varlen, bool bf16, int32_t C, size_t &out, size_t &pkg,
                            int64_t &slots, bool dplr = false, bool layer = false) {
    const kda::PackageLayout L = dplr ? kda::dplr_package_layout(C, Dk, Dv, bf16)
                                      : kda::package_layout(C, Dk, Dv, bf16);
    pkg = L.bytes;
    slots = kda::prefill_slots(B, T, N, C, varlen);
    size_t total = pkg;
    if (!mul_ok(total, (uint64_t)slots) || !mul_ok(total, (uint64_t)H)) return false;
    if (varlen) {
        const size_t plan = kda::align256(((size_t)N + 1) * sizeof(int32_t));
        if (total > SIZE_MAX - plan) return false;
        total += plan;
    }
    if (layer) {  // the KDA layer's row-norm exchange
        size_t x = kda::norm_xchg_bytes(C, Dv);
        if (!mul_ok(x, (uint64_t)slots) || !mul_ok(x, (uint64_t)H) || total > SIZE_MAX - x) return false;
        total += x;
    }
    out = total;
    return true;
}

size_t kda_chunk_fwd_workspace_size(int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv,
                                    int32_t n_seqs, kda_dtype in_dtype, int32_t chunk_size) {
    if (chunk_size == 0) chunk_size = 64;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return 0;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return 0;
    if (B < 1 || T < 0 || H < 1 || n_seqs < 0) return 0;
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32) return 0;
    chunk_size = kda::prefill_effective_chunk(chunk_size, Dk, Dv, in_dtype == KDA_BF16);
    const bool varlen = n_seqs > 0 && B == 1;
    size_t out = 0, pkg = 0;
    int64_t slots = 0;
    if (!workspace_bytes(B, T, H, Dk, Dv, varlen ? n_seqs : B, varlen, in_dtype == KDA_BF16,
                         chunk_size, out, pkg, slots))
        return 0;
    return out;
}

size_t kda_layer_chunk_fwd_workspace_size(int32_t B, int64_t T, int32_t H, int32_t n_seqs) {
    if (B < 1 || T < 0 || H < 1 || n_seqs < 0) return 0;
    const bool varlen = n_seqs > 0 && B == 1;
    size_t out = 0, pkg = 0;
    int64_t slots = 0;
    if (!workspace_bytes(B, T, H, 128, 128, varlen ? n_seqs : B, varlen, true, 64, out, pkg, slots, false, true))
        return 0;
    return out;
}

static kda_status chunk_fwd_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                                 const float *beta, const float *init_state, const int32_t *cu_seqlens,
                                 int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                                 kda_dtype in_dtype, int32_t chunk_size, float *o, float *final_state,
                                 void *workspace, size_t ws_bytes, hipStream_t stream, int gate_mode,
                                 const LayerIn *L, const void *lr_a = nullptr, const void *lr_b = nullptr,
                                 bool static_ws = false) {
    g_err[0] = '\0';
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype %d is not KDA_BF16 or KDA_F32", (int)in_dtype);
    if (!supported_dim(Dk) || !supported_dim(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "Dk=%d Dv=%d: each must be 16, 32, 64 or 128", Dk, Dv);
    if (chunk_size == 0) chunk_size = 64;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size %d: must be 16, 32 or 64", chunk_size);
    chunk_size = kda::prefill_effective_chunk(chunk_size, Dk, Dv, in_dtype == KDA_BF16);
    if (gate_mode == 3 && Dk != Dv)
        return fail(KDA_ERR_UNSUPPORTED, "the DPLR prefill needs Dk == Dv (got %d, %d)", Dk, Dv);
    if (gate_mode == 2 && (in_dtype != KDA_BF16 || Dk != 128 || chunk_size != 64))
        return fail(KDA_ERR_UNSUPPORTED, "the layer prefill runs bf16 inputs at Dk = Dv = 128 in 64-token chunks");
    if (B < 1 || T < 0 || H < 1)
        return fail(KDA_ERR_INVALID_ARG, "B=%d T=%lld H=%d: need B >= 1, T >= 0, H >= 1", B,
                    (long long)T, H);
    const bool varlen = cu_seqlens != nullptr;
    if (varlen && B != 1) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens given but B=%d != 1", B);
    if (varlen && n_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens given but n_seqs=%d", n_seqs);
    if (!varlen && n_seqs != 0 && n_seqs != B)
        return fail(KDA_ERR_INVALID_ARG, "n_seqs=%d without cu_seqlens (must be 0 or B)", n_seqs);
    const int32_t N = varlen ? n_seqs : B;
    if ((int64_t)N * H > 0x7fffffff || T > ((int64_t)1 << 40))
        return fail(KDA_ERR_INVALID_ARG, "sizes exceed the supported range");
    // the state pass runs Dv / 16 workgroups per (sequence, head) on a one-dimensional grid
    if (((int64_t)N * H + 7) / 8 * 8 * (Dv / 16) > 0x7fffffff)
        return fail(KDA_ERR_INVALID_ARG, "N*H=%lld (sequence, head) units: more than the state pass's grid takes",
                    (long long)N * H);
    if (gate_mode == 2 && (!eps_ok(L->l2_eps) || !eps_ok(L->norm_eps)))
        return fail(KDA_ERR_INVALID_ARG, "l2_eps and norm_eps must be finite and >= 0");
    if (N == 0) return KDA_OK;
    const bool bf16 = in_dtype == KDA_BF16;
    const size_t esz = bf16 ? 2 : 4;
    size_t bq, bv, bg, bb, bs, bo, bc, bxa, bxb, bog;
    if (!bytes_of(bq, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dk}, esz) ||
        !bytes_of(bv, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dv}, esz) ||
        !bytes_of(bg, {(uint64_t)B, (uint64_t)T, (uint64_t)H, gate_mode == 1 ? 1u : (uint64_t)Dk}, 4) ||
        !bytes_of(bb, {(uint64_t)B, (uint64_t)T, (uint64_t)H}, 4) ||
        !bytes_of(bs, {(uint64_t)N, (uint64_t)H, (uint64_t)Dk, (uint64_t)Dv}, 4) ||
        !bytes_of(bo, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dv}, 4) ||
        !bytes_of(bxa, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dk}, 2) ||
        !bytes_of(bxb, {(uint64_t)B, (uint64_t)T, (uint64_t)H}, 2) ||
        !bytes_of(bog, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dv}, 2))
        return fail(KDA_ERR_INVALID_ARG, "tensor sizes overflow size_t");
    bc = varlen ? ((size_t)N + 1) * 4 : 0;
    // inputs in checking order; init_state stays last (final_state may alias it)
    Input in[10];
    int n_in = 0;
    in[n_in++] = {q, "q", bq, 16, true};
    in[n_in++] = {k, "k", bq, 16, true};
    in[n_in++] = {v, "v", bv, 16, true};
    if (gate_mode == 2) {
        in[n_in++] = {L->x_alpha, "x_alpha", bxa, 16, true};
        in[n_in++] = {L->x_beta, "x_beta", bxb, 2, true};
        in[n_in++] = {L->out_gate, "out_gate", bog, 16, true};
        in[n_in++] = {L->norm_weight, "norm_weight", (size_t)Dv * 4, 16, true};
    } else if (gate_mode == 3) {
        in[n_in++] = {lr_a, "a", bq, 16, true};
        in[n_in++] = {lr_b, "b", bq, 16, true};
        in[n_in++] = {log_alpha, "log_alpha", bg, 16u, true};
    } else {
        // a per-channel gate is read in 16-byte vectors; a scalar gate and beta one by one
        in[n_in++] = {log_alpha, "log_alpha", bg, gate_mode == 1 ? 4u : 16u, true};
        in[n_in++] = {beta, "beta", bb, 4, true};
    }
    in[n_in++] = {cu_seqlens, "cu_seqlens", bc, 4, false};
    in[n_in++] = {init_state, "init_state", init_state ? bs : 0, 16, false};
    for (int i = 0; i < n_in; ++i) {
        if (in[i].required && !in[i].p && T > 0) return fail(KDA_ERR_INVALID_ARG, "%s is NULL", in[i].name);
        if (in[i].p && !aligned(in[i].p, in[i].align))
            return fail(KDA_ERR_INVALID_ARG, "%s is not %u-byte aligned", in[i].name, in[i].align);
    }
    if (!o && T > 0) return fail(KDA_ERR_INVALID_ARG, "o is NULL");
    if (o && !aligned16(o)) return fail(KDA_ERR_INVALID_ARG, "o is not 16-byte aligned");
    if (final_state && !aligned16(final_state))
        return fail(KDA_ERR_INVALID_ARG, "final_state is not 16-byte aligned");
    size_t need_ws = 0, pkg = 0;
    int64_t slots = 0;
    if (!workspace_bytes(B, T, H, Dk, Dv, N, varlen, bf16, chunk_size, need_ws, pkg, slots, gate_mode == 3,
                         gate_mode == 2))
        return fail(KDA_ERR_INVALID_ARG, "workspace size overflows size_t");
    if (static_ws) {
        // the library's own device array stands in for the workspace; it is
        // looked up only once every argument has passed validation
        if (need_ws > kda::kNoallocScratchBytes)
            return fail(KDA_ERR_WORKSPACE,
                        "these sizes need %zu bytes of workspace; the static scratch of "
                        "kda_chunk_fwd_noalloc holds %zu (use kda_chunk_fwd with a caller workspace)",
                        need_ws, kda::kNoallocScratchBytes);
        workspace = nullptr;
        ws_bytes = 0;
    } else {
        if (T > 0 && (!workspace || ws_bytes < need_ws))
            return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu needed", ws_bytes,
                        workspace, need_ws);
        if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
            return fail(KDA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    }
    // at T = 0 the workspace is not used (see below), so it can overlap nothing;
    // neither can the static scratch, a buffer of the library's own
    const Range ro = span(o, bo), rws = span(workspace, T > 0 && !static_ws ? need_ws : 0);
    const Range rfs = span(final_state, final_state ? bs : 0);
    const Range rinit = span(init_state, init_state ? bs : 0);
    for (int i = 0; i < n_in; ++i) {
        const Range ri = span(in[i].p, in[i].bytes);
        if (overlap(ro, ri)) return fail(KDA_ERR_INVALID_ARG, "o overlaps %s", in[i].name);
        if (overlap(rws, ri)) return fail(KDA_ERR_INVALID_ARG, "workspace overlaps %s", in[i].name);
        // final_state may alias init_state exactly (continuing a sequence), nothing else
        if (in[i].p != init_state && overlap(rfs, ri))
            return fail(KDA_ERR_INVALID_ARG, "final_state overlaps %s", in[i].name);
    }
    if (final_state && init_state && overlap(rfs, rinit) && final_state != init_state)
        return fail(KDA_ERR_INVALID_ARG, "final_state partially overlaps init_state");
    if (overlap(ro, rws) || overlap(ro, rfs) || overlap(rws, rfs))
        return fail(KDA_ERR_INVALID_ARG, "o, final_state and workspace must not overlap");
    if (static_ws && T > 0) {
        const hipError_t e = kda::noalloc_scratch(&workspace);
        if (e != hipSuccess)
            return fail(KDA_ERR_HIP, "device address of the static scratch: %s", hipGetErrorString(e));
        ws_bytes = kda::kNoallocScratchBytes;
    }

    kda::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
    a.init_state = init_state; a.cu_seqlens = cu_seqlens;
    a.B = B; a.H = H; a.Dk = Dk; a.Dv = Dv; a.N = N; a.C = chunk_size; a.T = T;
    a.bf16 = bf16; a.gate_mode = gate_mode; a.o = o; a.final_state = final_state;
    if (gate_mode == 2) {
        a.x_alpha = static_cast<const uint16_t *>(L->x_alpha);
        a.x_beta = static_cast<const uint16_t *>(L->x_beta);
        a.out_gate = static_cast<const uint16_t *>(L->out_gate);
        a.norm_weight = L->norm_weight;
        a.l2_eps = L->l2_eps;
        a.norm_eps = L->norm_eps;
        a.layer_tag = next_layer_tag();
    }
    a.workspace = static_cast<char *>(workspace);
    a.n_slots = slots; a.pkg_bytes = pkg;
    a.chunk_offsets = varlen && T > 0 ? reinterpret_cast<int32_t *>(a.workspace + pkg * (size_t)slots * (size_t)H)
                                      : nullptr;
    if (gate_mode == 2 && T > 0)  // after the packages and the plan: the last bytes of the workspace
        a.norm_xchg = a.workspace + need_ws - kda::norm_xchg_bytes(chunk_size, Dv) * (size_t)slots * (size_t)H;
    if (T == 0) {
        // Every sequence is empty (cu[N] = T = 0): only final_state <- init_state
        // remains.  Run it as a dense batch of N empty sequences so that neither
        // the varlen plan nor the workspace (which may be NULL here) is touched.
        a.cu_seqlens = nullptr;
        a.B = N;
        a.n_slots = 0;
        a.workspace = nullptr;
        a.norm_xchg = nullptr;
        a.chunk_offsets = nullptr;
    }
    a.lr_a = lr_a; a.lr_b = lr_b;
    hipError_t e = gate_mode == 3 ? kda::launch_dplr(a, stream) : kda::launch_prefill(a, stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, const float *init_state, const int32_t *cu_seqlens,
                         int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                         kda_dtype in_dtype, int32_t chunk_size, float *o, float *final_state,
                         void *workspace, size_t ws_bytes, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, init_state, cu_seqlens, B, T, H, Dk, Dv, n_seqs,
                          in_dtype, chunk_size, o, final_state, workspace, ws_bytes, stream, 0, nullptr);
}

kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *log_alpha,
                                 const float *beta, const float *init_state, const int32_t *cu_seqlens,
                                 int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                                 kda_dtype in_dtype, int32_t chunk_size, float *o, float *final_state,
                                 hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, init_state, cu_seqlens, B, T, H, Dk, Dv, n_seqs,
                          in_dtype, chunk_size, o, final_state, nullptr, 0, stream, 0, nullptr, nullptr,
                          nullptr, true);
}

size_t kda_chunk_fwd_noalloc_max_workspace(void) { return kda::kNoallocScratchBytes; }

size_t kda_dplr_chunk_fwd_workspace_size(int32_t B, int64_t T, int32_t H, int32_t D, int32_t n_seqs,
                                         kda_dtype in_dtype, int32_t chunk_size) {
    if (chunk_size == 0) chunk_size = 64;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return 0;
    if (!supported_dim(D)) return 0;
    if (B < 1 || T < 0 || H < 1 || n_seqs < 0) return 0;
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32) return 0;
    chunk_size = kda::prefill_effective_chunk(chunk_size, D, D, in_dtype == KDA_BF16);
    const bool varlen = n_seqs > 0 && B == 1;
    size_t out = 0, pkg = 0;
    int64_t slots = 0;
    if (!workspace_bytes(B, T, H, D, D, varlen ? n_seqs : B, varlen, in_dtype == KDA_BF16, chunk_size, out, pkg,
                         slots, true))
        return 0;
    return out;
}

kda_status kda_dplr_chunk_fwd(const void *q, const void *k, const void *v, const void *a, const void *b,
                              const float *log_alpha, const float *init_state, const int32_t *cu_seqlens,
                              int32_t B, int64_t T, int32_t H, int32_t D, int32_t n_seqs, kda_dtype in_dtype,
                              int32_t chunk_size, float *o, float *final_state, void *workspace,
                              size_t ws_bytes, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, nullptr, init_state, cu_seqlens, B, T, H, D, D, n_seqs, in_dtype,
                          chunk_size, o, final_state, workspace, ws_bytes, stream, 3, nullptr, a, b);
}

kda_status gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, const float *init_state, const int32_t *cu_seqlens,
                         int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                         kda_dtype in_dtype, int32_t chunk_size, float *o, float *final_state,
                         void *workspace, size_t ws_bytes, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, init_state, cu_seqlens, B, T, H, Dk, Dv, n_seqs,
                          in_dtype, chunk_size, o, final_state, workspace, ws_bytes, stream, 1, nullptr);
}

kda_status kda_layer_chunk_fwd(const void *q, const void *k, const void *v, const void *x_alpha,
                               const void *x_beta, const void *out_gate, const float *norm_weight,
                               float l2_eps, float norm_eps, const float *init_state,
                               const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t Dk,
                               int32_t Dv, int32_t n_seqs, float *o, float *final_state, void *workspace,
                               size_t ws_bytes, hipStream_t stream) {
    const LayerIn L{x_alpha, x_beta, out_gate, norm_weight, l2_eps, norm_eps};
    return chunk_fwd_impl(q, k, v, nullptr, nullptr, init_state, cu_seqlens, B, T, H, Dk, Dv, n_seqs,
                          KDA_BF16, 64, o, final_state, workspace, ws_bytes, stream, 2, &L);
}

// Backward workspace, sections 256-byte aligned: one segment's packages, the
// varlen plan, the checkpoints (the state entering segments 1, 2, ...), the
// two state-gradient carries, one segment's states and state gradients, and
// the gradient kernel's per-workgroup scratch.
struct BwdLayout {
    size_t pkg;                // bytes of one (chunk, head) package
    int64_t slots, seg, nseg;  // chunk slots (a bound for varlen), per segment, segments
    size_t plan, ckpt, dcarry, states, dstates, scratch, total;  // section offsets; total size
};

static bool bwd_layout(int32_t B, int64_t T, int32_t H, int32_t D, int32_t N, bool varlen, bool bf16, int32_t C,
                       BwdLayout &o) {
    const kda::PackageLayout L = kda::package_layout(C, D, D, bf16);
    o.pkg = L.bytes;
    o.slots = kda::prefill_slots(B, T, N, C, varlen);
    const int64_t K = kda::bwd_segment_slots(H);
    o.seg = o.slots < K ? o.slots : K;
    o.nseg = o.slots > 0 ? (o.slots + K - 1) / K : 1;
    const size_t state = (size_t)H * D * D * 4;  // one [H, D, D] fp32 state per head; T-independent
    size_t pk = o.pkg, st = state, ck = state;
    if (!mul_ok(pk, (uint64_t)o.seg) || !mul_ok(pk, (uint64_t)H) || !mul_ok(st, (uint64_t)o.seg) ||
        !mul_ok(ck, (uint64_t)(o.nseg - 1)))
        return false;
    const size_t sizes[] = {
        pk,                                                   // packages
        varlen ? ((size_t)N + 1) * sizeof(int32_t) : 0,       // plan
        ck,                                                   // checkpoints
        o.nseg > 1 ? 2 * state : 0,                           // dcarry
        st, st,                                               // states, dstates
        (size_t)kda::kBwdMaxGroups * kda::kBwdScratchMats * (size_t)C * (size_t)D * 4,
    };
    size_t off[7], at = 0;
    for (int i = 0; i < 7; ++i) {
        off[i] = at;
        const size_t a = kda::align256(sizes[i]);
        if (a < sizes[i] || at > SIZE_MAX - a) return false;
        at += a;
    }
    o.plan = off[1]; o.ckpt = off[2]; o.dcarry = off[3]; o.states = off[4]; o.dstates = off[5]; o.scratch = off[6];
    o.total = at;
    return true;
}

size_t kda_chunk_bwd_workspace_size(int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                                    kda_dtype in_dtype, int32_t chunk_size) {
    if (chunk_size == 0) chunk_size = 64;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return 0;
    if (!supported_dim(Dk) || Dk != Dv) return 0;
    if (B < 1 || T < 0 || H < 1 || n_seqs < 0) return 0;
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32) return 0;
    chunk_size = kda::prefill_effective_chunk(chunk_size, Dk, Dv, in_dtype == KDA_BF16);
    const bool varlen = n_seqs > 0 && B == 1;
    BwdLayout lay{};
    if (!bwd_layout(B, T, H, Dk, varlen ? n_seqs : B, varlen, in_dtype == KDA_BF16, chunk_size, lay)) return 0;
    return lay.total;
}

kda_status kda_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha, const float *beta,
                         const float *init_state, const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t H,
                         int32_t Dk, int32_t Dv, int32_t n_seqs, kda_dtype in_dtype, int32_t chunk_size,
                         const float *d_o, const float *d_final_state, float *dq, float *dk, float *dv,
                         float *dlog_alpha, float *dbeta, float *d_init_state, void *workspace, size_t ws_bytes,
                         hipStream_t stream) {
    g_err[0] = '\0';
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype %d is not KDA_BF16 or KDA_F32", (int)in_dtype);
    if (!supported_dim(Dk) || Dk != Dv)
        return fail(KDA_ERR_UNSUPPORTED, "Dk=%d Dv=%d: the backward needs Dk = Dv in {16, 32, 64, 128}", Dk, Dv);
    if (chunk_size == 0) chunk_size = 64;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size %d: must be 16, 32 or 64", chunk_size);
    chunk_size = kda::prefill_effective_chunk(chunk_size, Dk, Dv, in_dtype == KDA_BF16);
    if (B < 1 || T < 0 || H < 1)
        return fail(KDA_ERR_INVALID_ARG, "B=%d T=%lld H=%d: need B >= 1, T >= 0, H >= 1", B, (long long)T, H);
    const bool varlen = cu_seqlens != nullptr;
    if (varlen && B != 1) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens given but B=%d != 1", B);
    if (varlen && n_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens given but n_seqs=%d", n_seqs);
    if (!varlen && n_seqs != 0 && n_seqs != B)
        return fail(KDA_ERR_INVALID_ARG, "n_seqs=%d without cu_seqlens (must be 0 or B)", n_seqs);
    const int32_t N = varlen ? n_seqs : B;
    if ((int64_t)N * H > 0x7fffffff || T > ((int64_t)1 << 40))
        return fail(KDA_ERR_INVALID_ARG, "sizes exceed the supported range");
    // the state pass runs Dv / 16 workgroups per (sequence, head) on a one-dimensional grid
    if (((int64_t)N * H + 7) / 8 * 8 * (Dv / 16) > 0x7fffffff)
        return fail(KDA_ERR_INVALID_ARG, "N*H=%lld (sequence, head) units: more than the state pass's grid takes",
                    (long long)N * H);
    if (N == 0) return KDA_OK;
    const bool bf16 = in_dtype == KDA_BF16;
    const size_t esz = bf16 ? 2 : 4;
    size_t bq, bg, bb, bs, bf;
    if (!bytes_of(bq, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dk}, esz) ||
        !bytes_of(bg, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dk}, 4) ||
        !bytes_of(bb, {(uint64_t)B, (uint64_t)T, (uint64_t)H}, 4) ||
        !bytes_of(bs, {(uint64_t)N, (uint64_t)H, (uint64_t)Dk, (uint64_t)Dv}, 4) ||
        !bytes_of(bf, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dk}, 4))
        return fail(KDA_ERR_INVALID_ARG, "tensor sizes overflow size_t");
    const size_t bc = varlen ? ((size_t)N + 1) * 4 : 0;
    // Dk = Dv: q, k, v share a size, and so do the fp32 [B, T, H, D] tensors
    const Input in[] = {
        {q, "q", bq, 16, true},           {k, "k", bq, 16, true},
        {v, "v", bq, 16, true},           {log_alpha, "log_alpha", bg, 16, true},
        {beta, "beta", bb, 4, true},      {d_o, "d_o", bf, 16, true},
        {cu_seqlens, "cu_seqlens", bc, 4, false},
        {init_state, "init_state", init_state ? bs : 0, 16, false},
        {d_final_state, "d_final_state", d_final_state ? bs : 0, 16, false},
    };
    const Input out[] = {
        {dq, "dq", bf, 16, true},         {dk, "dk", bf, 16, true},
        {dv, "dv", bf, 16, true},         {dlog_alpha, "dlog_alpha", bf, 16, true},
        {dbeta, "dbeta", bb, 4, true},    {d_init_state, "d_init_state", d_init_state ? bs : 0, 16, false},
    };
    for (const Input &x : in) {
        if (x.required && !x.p && T > 0) return fail(KDA_ERR_INVALID_ARG, "%s is NULL", x.name);
        if (x.p && !aligned(x.p, x.align)) return fail(KDA_ERR_INVALID_ARG, "%s is not %u-byte aligned", x.name, x.align);
    }
    for (const Input &x : out) {
        if (x.required && !x.p && T > 0) return fail(KDA_ERR_INVALID_ARG, "%s is NULL", x.name);
        if (x.p && !aligned(x.p, x.align)) return fail(KDA_ERR_INVALID_ARG, "%s is not %u-byte aligned", x.name, x.align);
    }
    BwdLayout lay{};
    if (!bwd_layout(B, T, H, Dk, N, varlen, bf16, chunk_size, lay))
        return fail(KDA_ERR_INVALID_ARG, "workspace size overflows size_t");
    const size_t need_ws = lay.total;
    if (!workspace || ws_bytes < need_ws)
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu needed", ws_bytes, workspace, need_ws);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(KDA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    const Range rws = span(workspace, need_ws);
    for (size_t i = 0; i < sizeof(out) / sizeof(out[0]); ++i) {
        const Range ro = span(out[i].p, out[i].bytes);
        if (overlap(ro, rws)) return fail(KDA_ERR_INVALID_ARG, "%s overlaps the workspace", out[i].name);
        for (const Input &x : in)
            if (overlap(ro, span(x.p, x.bytes))) return fail(KDA_ERR_INVALID_ARG, "%s overlaps %s", out[i].name, x.name);
        for (size_t j = 0; j < i; ++j)
            if (overlap(ro, span(out[j].p, out[j].bytes)))
                return fail(KDA_ERR_INVALID_ARG, "%s overlaps %s", out[i].name, out[j].name);
    }
    for (const Input &x : in)
        if (overlap(rws, span(x.p, x.bytes))) return fail(KDA_ERR_INVALID_ARG, "workspace overlaps %s", x.name);

    kda::BackwardArgs a{};
    kda::PrefillArgs &f = a.fwd;
    f.q = q; f.k = k; f.v = v; f.log_alpha = log_alpha; f.beta = beta;
    f.init_state = init_state; f.cu_seqlens = cu_seqlens;
    f.B = B; f.H = H; f.Dk = Dk; f.Dv = Dv; f.N = N; f.C = chunk_size; f.T = T;
    f.bf16 = bf16; f.gate_mode = 0;
    f.workspace = static_cast<char *>(workspace);
    f.n_slots = lay.slots; f.pkg_bytes = lay.pkg;
    f.chunk_offsets = varlen ? reinterpret_cast<int32_t *>(f.workspace + lay.plan) : nullptr;
    a.d_o = d_o; a.d_final_state = d_final_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dlog_alpha = dlog_alpha; a.dbeta = dbeta; a.d_init_state = d_init_state;
    a.checkpoints = reinterpret_cast<float *>(f.workspace + lay.ckpt);
    a.dcarry = reinterpret_cast<float *>(f.workspace + lay.dcarry);
    a.chunk_states = reinterpret_cast<float *>(f.workspace + lay.states);
    a.chunk_dstates = reinterpret_cast<float *>(f.workspace + lay.dstates);
    a.scratch = reinterpret_cast<float *>(f.workspace + lay.scratch);
    a.seg_slots = lay.seg > 0 ? lay.seg : 1;
    hipError_t e = kda::launch_backward(a, stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

kda_status kda_layer_decode_step(const void *q, const void *k, const void *v, const void *x_alpha,
                                 const void *x_beta, const void *out_gate, const float *norm_weight,
                                 float l2_eps, float norm_eps, float *state, int32_t N, int32_t H,
                                 int32_t Dk, int32_t Dv, float *o, hipStream_t stream) {
    const LayerIn L{x_alpha, x_beta, out_gate, norm_weight, l2_eps, norm_eps};
    return decode_impl(q, k, v, nullptr, nullptr, state, N, H, Dk, Dv, KDA_BF16, o, stream, 2, &L);
}

}  // extern "C"
