// kda_abi.cpp -- the extern "C" entry points of libkda.so: host-only argument
// validation, workspace sizing and dispatch to the gfx950 kernels.  Nothing
// here dereferences a device pointer or calls HIP before validation passes.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

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

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

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
                              bool scalar_gate) {
    g_err[0] = '\0';
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype %d is not KDA_BF16 or KDA_F32", (int)in_dtype);
    if (!supported_dim(Dk) || !supported_dim(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "Dk=%d Dv=%d: each must be 16, 32, 64 or 128", Dk, Dv);
    if (N < 0 || H < 1) return fail(KDA_ERR_INVALID_ARG, "N=%d H=%d: need N >= 0, H >= 1", N, H);
    if ((int64_t)N * H > 0x7fffffff)
        return fail(KDA_ERR_INVALID_ARG, "N*H=%lld exceeds the grid limit", (long long)N * H);
    if (N == 0) return KDA_OK;
    const void *ptrs[] = {q, k, v, log_alpha, beta, state, o};
    const char *names[] = {"q", "k", "v", "log_alpha", "beta", "state", "o"};
    for (int i = 0; i < 7; ++i) {
        if (!ptrs[i]) return fail(KDA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        // beta and a scalar gate are read element by element
        const bool scalar = i == 4 || (i == 3 && scalar_gate);
        if (scalar ? !aligned4(ptrs[i]) : !aligned16(ptrs[i]))
            return fail(KDA_ERR_INVALID_ARG, "%s is not %d-byte aligned", names[i], scalar ? 4 : 16);
    }
    const size_t esz = in_dtype == KDA_BF16 ? 2 : 4;
    size_t bq, bv, bg, bb, bs, bo;
    if (!bytes_of(bq, {(uint64_t)N, (uint64_t)H, (uint64_t)Dk}, esz) ||
        !bytes_of(bv, {(uint64_t)N, (uint64_t)H, (uint64_t)Dv}, esz) ||
        !bytes_of(bg, {(uint64_t)N, (uint64_t)H, scalar_gate ? 1u : (uint64_t)Dk}, 4) ||
        !bytes_of(bb, {(uint64_t)N, (uint64_t)H}, 4) ||
        !bytes_of(bs, {(uint64_t)N, (uint64_t)H, (uint64_t)Dk, (uint64_t)Dv}, 4) ||
        !bytes_of(bo, {(uint64_t)N, (uint64_t)H, (uint64_t)Dv}, 4))
        return fail(KDA_ERR_INVALID_ARG, "tensor sizes overflow size_t");
    const Range ro = span(o, bo), rs = span(state, bs);
    const Range ins[] = {span(q, bq), span(k, bq), span(v, bv), span(log_alpha, bg), span(beta, bb)};
    const char *in_names[] = {"q", "k", "v", "log_alpha", "beta"};
    for (int i = 0; i < 5; ++i) {
        if (overlap(ro, ins[i])) return fail(KDA_ERR_INVALID_ARG, "o overlaps %s", in_names[i]);
        if (overlap(rs, ins[i])) return fail(KDA_ERR_INVALID_ARG, "state overlaps %s", in_names[i]);
    }
    if (overlap(ro, rs)) return fail(KDA_ERR_INVALID_ARG, "o overlaps state");

    kda::DecodeArgs a{q, k, v, log_alpha, beta, state, o, N, H, Dk, Dv, in_dtype == KDA_BF16, scalar_gate};
    hipError_t e = kda::launch_decode(a, stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

kda_status kda_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, float *state, int32_t N, int32_t H, int32_t Dk,
                           int32_t Dv, kda_dtype in_dtype, float *o, hipStream_t stream) {
    return decode_impl(q, k, v, log_alpha, beta, state, N, H, Dk, Dv, in_dtype, o, stream, false);
}

kda_status gdn_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, float *state, int32_t N, int32_t H, int32_t Dk,
                           int32_t Dv, kda_dtype in_dtype, float *o, hipStream_t stream) {
    return decode_impl(q, k, v, log_alpha, beta, state, N, H, Dk, Dv, in_dtype, o, stream, true);
}

static bool workspace_bytes(int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                            bool varlen, bool bf16, int32_t C, size_t &out, size_t &pkg,
                            int64_t &slots) {
    const kda::PackageLayout L = kda::package_layout(C, Dk, Dv, bf16);
    pkg = L.bytes;
    slots = kda::prefill_slots(B, T, N, C, varlen);
    size_t total = pkg;
    if (!mul_ok(total, (uint64_t)slots) || !mul_ok(total, (uint64_t)H)) return false;
    if (varlen) {
        const size_t plan = kda::align256(((size_t)N + 1) * sizeof(int32_t));
        if (total > SIZE_MAX - plan) return false;
        total += plan;
    }
    out = total;
    return true;
}

size_t kda_chunk_fwd_workspace_size(int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv,
                                    int32_t n_seqs, kda_dtype in_dtype, int32_t chunk_size) {
    if (chunk_size == 0) chunk_size = 64;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return 0;
    if (!supported_dim(Dk) || !supported_dim(Dv) || Dk != Dv) return 0;
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

static kda_status chunk_fwd_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                                 const float *beta, const float *init_state, const int32_t *cu_seqlens,
                                 int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                                 kda_dtype in_dtype, int32_t chunk_size, float *o, float *final_state,
                                 void *workspace, size_t ws_bytes, hipStream_t stream, bool scalar_gate) {
    g_err[0] = '\0';
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype %d is not KDA_BF16 or KDA_F32", (int)in_dtype);
    if (!supported_dim(Dk) || !supported_dim(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "Dk=%d Dv=%d: each must be 16, 32, 64 or 128", Dk, Dv);
    if (Dk != Dv) return fail(KDA_ERR_UNSUPPORTED, "prefill needs Dk == Dv (got %d, %d)", Dk, Dv);
    if (chunk_size == 0) chunk_size = 64;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size %d: must be 16, 32 or 64", chunk_size);
    chunk_size = kda::prefill_effective_chunk(chunk_size, Dk, Dv, in_dtype == KDA_BF16);
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
    if (N == 0) return KDA_OK;
    const void *need[] = {q, k, v, log_alpha, beta, o};
    const char *nn[] = {"q", "k", "v", "log_alpha", "beta", "o"};
    for (int i = 0; i < 6; ++i) {
        if (!need[i] && T > 0) return fail(KDA_ERR_INVALID_ARG, "%s is NULL", nn[i]);
        // beta and a scalar gate are read element by element
        const bool scalar = i == 4 || (i == 3 && scalar_gate);
        if (need[i] && (scalar ? !aligned4(need[i]) : !aligned16(need[i])))
            return fail(KDA_ERR_INVALID_ARG, "%s is not %d-byte aligned", nn[i], scalar ? 4 : 16);
    }
    const void *opt[] = {init_state, cu_seqlens, final_state};
    const char *on[] = {"init_state", "cu_seqlens", "final_state"};
    for (int i = 0; i < 3; ++i) {
        const bool scalar = i == 1;  // cu_seqlens: int32 offsets
        if (opt[i] && (scalar ? !aligned4(opt[i]) : !aligned16(opt[i])))
            return fail(KDA_ERR_INVALID_ARG, "%s is not %d-byte aligned", on[i], scalar ? 4 : 16);
    }
    const bool bf16 = in_dtype == KDA_BF16;
    size_t need_ws = 0, pkg = 0;
    int64_t slots = 0;
    if (!workspace_bytes(B, T, H, Dk, Dv, N, varlen, bf16, chunk_size, need_ws, pkg, slots))
        return fail(KDA_ERR_INVALID_ARG, "workspace size overflows size_t");
    if (T > 0 && (!workspace || ws_bytes < need_ws))
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu needed", ws_bytes,
                    workspace, need_ws);
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(KDA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    const size_t esz = bf16 ? 2 : 4;
    size_t bq, bv, bg, bb, bs, bo, bc;
    if (!bytes_of(bq, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dk}, esz) ||
        !bytes_of(bv, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dv}, esz) ||
        !bytes_of(bg, {(uint64_t)B, (uint64_t)T, (uint64_t)H, scalar_gate ? 1u : (uint64_t)Dk}, 4) ||
        !bytes_of(bb, {(uint64_t)B, (uint64_t)T, (uint64_t)H}, 4) ||
        !bytes_of(bs, {(uint64_t)N, (uint64_t)H, (uint64_t)Dk, (uint64_t)Dv}, 4) ||
        !bytes_of(bo, {(uint64_t)B, (uint64_t)T, (uint64_t)H, (uint64_t)Dv}, 4))
        return fail(KDA_ERR_INVALID_ARG, "tensor sizes overflow size_t");
    bc = varlen ? ((size_t)N + 1) * 4 : 0;
    const Range ro = span(o, bo), rws = span(workspace, need_ws);
    const Range rin[] = {span(q, bq), span(k, bq), span(v, bv), span(log_alpha, bg),
                         span(beta, bb), span(init_state, init_state ? bs : 0),
                         span(cu_seqlens, bc)};
    const char *in_n[] = {"q", "k", "v", "log_alpha", "beta", "init_state", "cu_seqlens"};
    const Range rfs = span(final_state, final_state ? bs : 0);
    for (int i = 0; i < 7; ++i) {
        if (overlap(ro, rin[i])) return fail(KDA_ERR_INVALID_ARG, "o overlaps %s", in_n[i]);
        if (overlap(rws, rin[i])) return fail(KDA_ERR_INVALID_ARG, "workspace overlaps %s", in_n[i]);
        // final_state may alias init_state exactly (continuing a sequence), nothing else
        if (i != 5 && overlap(rfs, rin[i]))
            return fail(KDA_ERR_INVALID_ARG, "final_state overlaps %s", in_n[i]);
    }
    if (final_state && init_state && overlap(rfs, rin[5]) && final_state != init_state)
        return fail(KDA_ERR_INVALID_ARG, "final_state partially overlaps init_state");
    if (overlap(ro, rws) || overlap(ro, rfs) || overlap(rws, rfs))
        return fail(KDA_ERR_INVALID_ARG, "o, final_state and workspace must not overlap");

    kda::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
    a.init_state = init_state; a.cu_seqlens = cu_seqlens;
    a.B = B; a.H = H; a.Dk = Dk; a.Dv = Dv; a.N = N; a.C = chunk_size; a.T = T;
    a.bf16 = bf16; a.scalar_gate = scalar_gate; a.o = o; a.final_state = final_state;
    a.workspace = static_cast<char *>(workspace);
    a.n_slots = slots; a.pkg_bytes = pkg;
    a.chunk_offsets = varlen ? reinterpret_cast<int32_t *>(a.workspace + pkg * (size_t)slots * (size_t)H)
                             : nullptr;
    hipError_t e = kda::launch_prefill(a, stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, const float *init_state, const int32_t *cu_seqlens,
                         int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                         kda_dtype in_dtype, int32_t chunk_size, float *o, float *final_state,
                         void *workspace, size_t ws_bytes, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, init_state, cu_seqlens, B, T, H, Dk, Dv, n_seqs,
                          in_dtype, chunk_size, o, final_state, workspace, ws_bytes, stream, false);
}

kda_status gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, const float *init_state, const int32_t *cu_seqlens,
                         int32_t B, int64_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t n_seqs,
                         kda_dtype in_dtype, int32_t chunk_size, float *o, float *final_state,
                         void *workspace, size_t ws_bytes, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, init_state, cu_seqlens, B, T, H, Dk, Dv, n_seqs,
                          in_dtype, chunk_size, o, final_state, workspace, ws_bytes, stream, true);
}

}  // extern "C"
