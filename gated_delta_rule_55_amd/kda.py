"""Python binding of libkda.so (ctypes).

Argument marshalling only: every step of the operator runs in the library's
HIP kernels.  torch provides device memory (tensors, ``data_ptr()``) and the
current HIP stream; there is no fallback path -- if the library is missing or
a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY names another build of the library to load instead of the
# in-tree one (e.g. a host-only build of the argument checks under the
# sanitizers)
LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(_HERE, "libkda.so")

KDA_BF16, KDA_F32 = 0, 1
_lib = None


class KdaError(RuntimeError):
    pass


def load():
    """Loads libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KdaError(f"{LIB_PATH} is missing: build it with gated_delta_rule_55_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, ctypes.c_int, i32]
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_layer_chunk_fwd_workspace_size.argtypes = [i32, i64, i32, i32]
    lib.kda_layer_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i64, i32, i32, i32, i32,
                                  ctypes.c_int, i32, fp, fp, vp, sz, vp]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i64, i32, i32, i32, i32,
                                          ctypes.c_int, i32, fp, fp, vp]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc_max_workspace.argtypes = []
    lib.kda_chunk_fwd_noalloc_max_workspace.restype = sz
    lib.kda_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, i32, i32, i32, i32, ctypes.c_int, fp, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = lib.kda_chunk_fwd.argtypes
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = lib.kda_decode_step.argtypes
    lib.gdn_decode_step.restype = ctypes.c_int
    f32 = ctypes.c_float
    lib.kda_layer_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, fp, f32, f32, fp, ip, i32, i64, i32, i32,
                                        i32, i32, fp, fp, vp, sz, vp]
    lib.kda_layer_chunk_fwd.restype = ctypes.c_int
    lib.kda_layer_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, fp, f32, f32, fp, i32, i32, i32, i32,
                                          fp, vp]
    lib.kda_layer_decode_step.restype = ctypes.c_int
    lib.kda_chunk_bwd_workspace_size.argtypes = lib.kda_chunk_fwd_workspace_size.argtypes
    lib.kda_chunk_bwd_workspace_size.restype = sz
    lib.kda_chunk_bwd.argtypes = [vp, vp, vp, fp, fp, fp, ip, i32, i64, i32, i32, i32, i32, ctypes.c_int, i32,
                                  fp, fp, fp, fp, fp, fp, fp, fp, vp, sz, vp]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_dplr_chunk_fwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, ctypes.c_int, i32]
    lib.kda_dplr_chunk_fwd_workspace_size.restype = sz
    lib.kda_dplr_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, fp, fp, ip, i32, i64, i32, i32, i32, ctypes.c_int, i32,
                                       fp, fp, vp, sz, vp]
    lib.kda_dplr_chunk_fwd.restype = ctypes.c_int
    lib.kda_dplr_decode_step.argtypes = [vp, vp, vp, vp, vp, fp, fp, i32, i32, i32, ctypes.c_int, fp, vp]
    lib.kda_dplr_decode_step.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        lib = load()
        raise KdaError(f"{lib.kda_status_string(rc).decode()}: {lib.kda_last_error().decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise KdaError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_F32 = (torch.float32,)
_IN = (torch.bfloat16, torch.float32)
_BF16 = (torch.bfloat16,)


def _validate(specs, devices=True):
    """Checks every tensor argument before anything is launched.

    specs: (name, tensor, expected shape, allowed dtypes, required) tuples; a
    shape entry of None matches any size.  The library sizes every buffer from
    q's dtype and the dimensions it is given and reads dense row-major memory,
    so a wrong dtype, a non-contiguous view (a head slice of a [B, T, H, D]
    tensor, for instance), a CPU tensor or a tensor on another device would be
    read out of bounds or with the wrong stride; each raises KdaError here.
    Structure (dtype, shape, layout) is checked first, then (unless devices is
    False) that every tensor sits on the CUDA device of the first one.
    """
    present = []
    for name, t, shape, dtypes, required in specs:
        if t is None:
            if required:
                raise KdaError(f"{name} is required")
            continue
        if not isinstance(t, torch.Tensor):
            raise KdaError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
        if t.dtype not in dtypes:
            raise KdaError(f"{name} has dtype {t.dtype}; expected {' or '.join(str(d) for d in dtypes)}")
        if shape is not None:
            if t.dim() != len(shape) or any(e is not None and int(n) != int(e) for n, e in zip(t.shape, shape)):
                want = "[" + ", ".join("*" if e is None else str(int(e)) for e in shape) + "]"
                raise KdaError(f"{name} has shape {list(t.shape)}; expected {want}")
        if not t.is_contiguous():
            raise KdaError(f"{name} is not contiguous (the kernels read dense row-major memory; "
                           f"copy it with .contiguous() first)")
        present.append((name, t))
    if not devices:
        return
    ref_name, ref = present[0]
    if ref.device.type != "cuda":
        raise KdaError(f"{ref_name} is on {ref.device}; the library runs on a CUDA (HIP) device")
    for name, t in present:
        if t.device != ref.device:
            raise KdaError(f"{name} is on {t.device}, {ref_name} on {ref.device}: all tensors must share one device")


def _seq_count(B, cu_seqlens):
    """(n_seqs for the ABI, N) with a 1-D int32 cu_seqlens of N + 1 entries."""
    if cu_seqlens is None:
        return 0, B
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise KdaError("cu_seqlens must be a 1-D tensor of N + 1 >= 2 offsets")
    if cu_seqlens.dtype != torch.int32:
        raise KdaError(f"cu_seqlens has dtype {cu_seqlens.dtype}; expected torch.int32")
    n = cu_seqlens.numel() - 1
    return n, n


def _workspace_spec(workspace):
    return ("workspace", workspace, (None,), (torch.uint8,), False)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace_size(B, T, H, Dk, Dv, n_seqs=0, dtype=torch.bfloat16, chunk_size=64) -> int:
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load().kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, n_seqs, code, chunk_size))


def layer_workspace_size(B, T, H, n_seqs=0) -> int:
    """Workspace bytes of layer_chunk_fwd (Dk = Dv = 128, bf16, 64-token chunks)."""
    return int(load().kda_layer_chunk_fwd_workspace_size(B, T, H, n_seqs))


def chunk_fwd(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, chunk_size=64,
              out=None, final_state=None, output_final_state=True, workspace=None, stream=None):
    """KDA chunked prefill.  q, k [B,T,H,Dk]; v [B,T,H,Dv]; log_alpha [B,T,H,Dk] fp32;
    beta [B,T,H] fp32; init_state [N,H,Dk,Dv] fp32 or None; cu_seqlens int32 [N+1]
    (device) or None.  Returns (o [B,T,H,Dv] fp32, final_state [N,H,Dk,Dv] or None)."""
    return _chunk_fwd(load().kda_chunk_fwd, q, k, v, log_alpha, beta, init_state, cu_seqlens,
                      chunk_size, out, final_state, output_final_state, workspace, stream)


def gdn_chunk_fwd(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, chunk_size=64,
                  out=None, final_state=None, output_final_state=True, workspace=None, stream=None):
    """Gated DeltaNet chunked prefill: as ``chunk_fwd`` with log_alpha [B,T,H] fp32
    (one scalar gate per token and head)."""
    return _chunk_fwd(load().gdn_chunk_fwd, q, k, v, log_alpha, beta, init_state, cu_seqlens,
                      chunk_size, out, final_state, output_final_state, workspace, stream, scalar_gate=True)


def _chunk_fwd(fn, q, k, v, log_alpha, beta, init_state, cu_seqlens, chunk_size, out,
               final_state, output_final_state, workspace, stream, scalar_gate=False):
    _validate([("q", q, (None,) * 4, _IN, True)], devices=False)  # q fixes the sizes below
    B, T, H, Dk = q.shape
    Dv = v.shape[-1] if isinstance(v, torch.Tensor) and v.dim() == 4 else None
    n_seqs, N = _seq_count(B, cu_seqlens)
    _validate([("q", q, (B, T, H, Dk), _IN, True), ("k", k, (B, T, H, Dk), (q.dtype,), True),
               ("v", v, (B, T, H, Dv), (q.dtype,), True),
               ("log_alpha", log_alpha, (B, T, H) if scalar_gate else (B, T, H, Dk), _F32, True),
               ("beta", beta, (B, T, H), _F32, True),
               ("init_state", init_state, (N, H, Dk, Dv), _F32, False),
               ("cu_seqlens", cu_seqlens, (N + 1,), (torch.int32,), False),
               ("out", out, (B, T, H, Dv), _F32, False),
               ("final_state", final_state, (N, H, Dk, Dv), _F32, False), _workspace_spec(workspace)])
    lib = load()
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    code = _dtype_code(q)
    ws_bytes = int(lib.kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, n_seqs, code, chunk_size))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
              _ptr(init_state), _ptr(cu_seqlens), B, T, H, Dk, Dv, n_seqs, code,
              chunk_size, _ptr(out), _ptr(final_state), _ptr(workspace),
              workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, final_state


def chunk_fwd_noalloc(q, k, v, log_alpha, beta, out, init_state=None, cu_seqlens=None, chunk_size=64,
                      final_state=None, stream=None):
    """``chunk_fwd`` through kda_chunk_fwd_noalloc: no workspace and nothing
    allocated here or in the library (the caller supplies ``out`` and, if
    wanted, ``final_state``); the library's static device scratch stands in
    for the workspace, so the sizes are limited (KdaError beyond them) and
    calls that overlap on one GPU race.  Returns (out, final_state)."""
    _validate([("q", q, (None,) * 4, _IN, True)], devices=False)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1] if isinstance(v, torch.Tensor) and v.dim() == 4 else None
    n_seqs, N = _seq_count(B, cu_seqlens)
    _validate([("q", q, (B, T, H, Dk), _IN, True), ("k", k, (B, T, H, Dk), (q.dtype,), True),
               ("v", v, (B, T, H, Dv), (q.dtype,), True), ("log_alpha", log_alpha, (B, T, H, Dk), _F32, True),
               ("beta", beta, (B, T, H), _F32, True), ("out", out, (B, T, H, Dv), _F32, True),
               ("init_state", init_state, (N, H, Dk, Dv), _F32, False),
               ("cu_seqlens", cu_seqlens, (N + 1,), (torch.int32,), False),
               ("final_state", final_state, (N, H, Dk, Dv), _F32, False)])
    _check(load().kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                        _ptr(init_state), _ptr(cu_seqlens), B, T, H, Dk, Dv, n_seqs,
                                        _dtype_code(q), chunk_size, _ptr(out), _ptr(final_state),
                                        _stream(stream)))
    return out, final_state


def noalloc_max_workspace() -> int:
    """Bytes of the static scratch behind ``chunk_fwd_noalloc``."""
    return int(load().kda_chunk_fwd_noalloc_max_workspace())


def dplr_workspace_size(B, T, H, D, n_seqs=0, dtype=torch.bfloat16, chunk_size=64) -> int:
    """Bytes of workspace ``dplr_chunk_fwd`` needs (0 for unsupported sizes)."""
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load().kda_dplr_chunk_fwd_workspace_size(B, T, H, D, n_seqs, code, chunk_size))


def dplr_chunk_fwd(q, k, v, a, b, log_alpha, init_state=None, cu_seqlens=None, chunk_size=64,
                   out=None, final_state=None, output_final_state=True, workspace=None, stream=None):
    """Chunked prefill of the general DPLR recurrence
    S_t = (Diag(exp(log_alpha_t)) + a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t.
    q, k, v, a, b [B,T,H,D] (one dtype); log_alpha [B,T,H,D] fp32; the rest as
    ``chunk_fwd``.  Returns (o [B,T,H,D] fp32, final_state [N,H,D,D] or None)."""
    _validate([("q", q, (None,) * 4, _IN, True)], devices=False)
    B, T, H, D = q.shape
    n_seqs, N = _seq_count(B, cu_seqlens)
    x4 = (B, T, H, D)
    _validate([("q", q, x4, _IN, True), ("k", k, x4, (q.dtype,), True), ("v", v, x4, (q.dtype,), True),
               ("a", a, x4, (q.dtype,), True), ("b", b, x4, (q.dtype,), True),
               ("log_alpha", log_alpha, x4, _F32, True),
               ("init_state", init_state, (N, H, D, D), _F32, False),
               ("cu_seqlens", cu_seqlens, (N + 1,), (torch.int32,), False),
               ("out", out, x4, _F32, False), ("final_state", final_state, (N, H, D, D), _F32, False),
               _workspace_spec(workspace)])
    lib = load()
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    code = _dtype_code(q)
    ws_bytes = int(lib.kda_dplr_chunk_fwd_workspace_size(B, T, H, D, n_seqs, code, chunk_size))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.kda_dplr_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha),
                                  _ptr(init_state), _ptr(cu_seqlens), B, T, H, D, n_seqs, code, chunk_size,
                                  _ptr(out), _ptr(final_state), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, final_state


def bwd_workspace_size(B, T, H, D, n_seqs=0, dtype=torch.bfloat16, chunk_size=64) -> int:
    """Bytes of workspace ``chunk_bwd`` needs (0 for unsupported sizes)."""
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load().kda_chunk_bwd_workspace_size(B, T, H, D, D, n_seqs, code, chunk_size))


def chunk_bwd(q, k, v, log_alpha, beta, d_o, init_state=None, cu_seqlens=None, d_final_state=None,
              chunk_size=64, grads=None, output_d_init_state=True, workspace=None, stream=None):
    """Gradients of ``chunk_fwd``: given d_o [B,T,H,Dv] fp32 (and optionally
    d_final_state [N,H,Dk,Dv]), returns (dq, dk, dv, dlog_alpha, dbeta,
    d_init_state) in fp32, d_init_state None unless requested.  Dk must equal Dv.
    ``grads`` may supply the six output tensors."""
    _validate([("q", q, (None,) * 4, _IN, True)], devices=False)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1] if isinstance(v, torch.Tensor) and v.dim() == 4 else None
    n_seqs, N = _seq_count(B, cu_seqlens)
    specs = [("q", q, (B, T, H, Dk), _IN, True), ("k", k, (B, T, H, Dk), (q.dtype,), True),
             ("v", v, (B, T, H, Dv), (q.dtype,), True), ("log_alpha", log_alpha, (B, T, H, Dk), _F32, True),
             ("beta", beta, (B, T, H), _F32, True), ("d_o", d_o, (B, T, H, Dv), _F32, True),
             ("init_state", init_state, (N, H, Dk, Dv), _F32, False),
             ("cu_seqlens", cu_seqlens, (N + 1,), (torch.int32,), False),
             ("d_final_state", d_final_state, (N, H, Dk, Dv), _F32, False), _workspace_spec(workspace)]
    if grads is not None:
        if len(grads) != 6:
            raise KdaError("grads must hold (dq, dk, dv, dlog_alpha, dbeta, d_init_state)")
        for name, t, shape in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "d_init_state"), grads,
                                  ((B, T, H, Dk), (B, T, H, Dk), (B, T, H, Dv), (B, T, H, Dk), (B, T, H),
                                   (N, H, Dk, Dv))):
            specs.append((name, t, shape, _F32, name != "d_init_state"))
    _validate(specs)
    lib = load()
    dev = q.device
    if grads is None:
        f32 = dict(dtype=torch.float32, device=dev)
        grads = (torch.empty((B, T, H, Dk), **f32), torch.empty((B, T, H, Dk), **f32),
                 torch.empty((B, T, H, Dv), **f32), torch.empty((B, T, H, Dk), **f32),
                 torch.empty((B, T, H), **f32),
                 torch.empty((N, H, Dk, Dv), **f32) if output_d_init_state else None)
    dq, dk, dv, dla, dbeta, ds0 = grads
    code = _dtype_code(q)
    ws_bytes = int(lib.kda_chunk_bwd_workspace_size(B, T, H, Dk, Dv, n_seqs, code, chunk_size))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state),
                             _ptr(cu_seqlens), B, T, H, Dk, Dv, n_seqs, code, chunk_size, _ptr(d_o),
                             _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dla), _ptr(dbeta),
                             _ptr(ds0), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream)))
    return dq, dk, dv, dla, dbeta, ds0


def decode_step(q, k, v, log_alpha, beta, state, out=None, stream=None):
    """One KDA step per (n, h); log_alpha [N,H,Dk]; state [N,H,Dk,Dv] fp32 is
    updated in place.  Returns o [N,H,Dv] fp32."""
    return _decode(load().kda_decode_step, q, k, v, log_alpha, beta, state, out, stream)


def gdn_decode_step(q, k, v, log_alpha, beta, state, out=None, stream=None):
    """One Gated DeltaNet step per (n, h): as ``decode_step`` with log_alpha [N,H]."""
    return _decode(load().gdn_decode_step, q, k, v, log_alpha, beta, state, out, stream, scalar_gate=True)


def dplr_decode_step(q, k, v, a, b, log_alpha, state, out=None, stream=None):
    """One step of the general DPLR recurrence per (n, h): q, k, v, a, b [N,H,D]
    (one dtype), log_alpha [N,H,D] fp32; state [N,H,D,D] fp32 updated in place.
    Returns o [N,H,D] fp32."""
    _validate([("q", q, (None,) * 3, _IN, True)], devices=False)
    N, H, D = q.shape
    x3 = (N, H, D)
    _validate([("q", q, x3, _IN, True), ("k", k, x3, (q.dtype,), True), ("v", v, x3, (q.dtype,), True),
               ("a", a, x3, (q.dtype,), True), ("b", b, x3, (q.dtype,), True),
               ("log_alpha", log_alpha, x3, _F32, True), ("state", state, (N, H, D, D), _F32, True),
               ("out", out, x3, _F32, False)])
    if out is None:
        out = torch.empty((N, H, D), dtype=torch.float32, device=q.device)
    _check(load().kda_dplr_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha),
                                       _ptr(state), N, H, D, _dtype_code(q), _ptr(out), _stream(stream)))
    return out


def _decode(fn, q, k, v, log_alpha, beta, state, out, stream, scalar_gate=False):
    _validate([("q", q, (None,) * 3, _IN, True)], devices=False)
    N, H, Dk = q.shape
    Dv = v.shape[-1] if isinstance(v, torch.Tensor) and v.dim() == 3 else None
    _validate([("q", q, (N, H, Dk), _IN, True), ("k", k, (N, H, Dk), (q.dtype,), True),
               ("v", v, (N, H, Dv), (q.dtype,), True),
               ("log_alpha", log_alpha, (N, H) if scalar_gate else (N, H, Dk), _F32, True),
               ("beta", beta, (N, H), _F32, True), ("state", state, (N, H, Dk, Dv), _F32, True),
               ("out", out, (N, H, Dv), _F32, False)])
    if out is None:
        out = torch.empty((N, H, Dv), dtype=torch.float32, device=q.device)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
              _ptr(state), N, H, Dk, Dv, _dtype_code(q), _ptr(out), _stream(stream)))
    return out


def layer_chunk_fwd(q, k, v, x_alpha, x_beta, out_gate, norm_weight, l2_eps=1e-6, norm_eps=1e-5,
                    init_state=None, cu_seqlens=None, out=None, final_state=None,
                    output_final_state=True, workspace=None, stream=None):
    """The KDA layer's prefill: L2Norm(q, k), log_alpha = -softplus(x_alpha),
    beta = sigmoid(x_beta), the recurrence, then RMSNorm(o) * norm_weight *
    sigmoid(out_gate).  q, k, x_alpha [B,T,H,128], v, out_gate [B,T,H,128],
    x_beta [B,T,H], all bf16; norm_weight [128] fp32.  Returns (out fp32, final_state)."""
    _validate([("q", q, (None,) * 4, _BF16, True)], devices=False)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1] if isinstance(v, torch.Tensor) and v.dim() == 4 else None
    n_seqs, N = _seq_count(B, cu_seqlens)
    _validate([("q", q, (B, T, H, Dk), _BF16, True), ("k", k, (B, T, H, Dk), _BF16, True),
               ("v", v, (B, T, H, Dv), _BF16, True), ("x_alpha", x_alpha, (B, T, H, Dk), _BF16, True),
               ("x_beta", x_beta, (B, T, H), _BF16, True), ("out_gate", out_gate, (B, T, H, Dv), _BF16, True),
               ("norm_weight", norm_weight, (Dv,), _F32, True),
               ("init_state", init_state, (N, H, Dk, Dv), _F32, False),
               ("cu_seqlens", cu_seqlens, (N + 1,), (torch.int32,), False),
               ("out", out, (B, T, H, Dv), _F32, False),
               ("final_state", final_state, (N, H, Dk, Dv), _F32, False), _workspace_spec(workspace)])
    lib = load()
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    ws_bytes = int(lib.kda_layer_chunk_fwd_workspace_size(B, T, H, n_seqs))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.kda_layer_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(x_alpha), _ptr(x_beta),
                                   _ptr(out_gate), _ptr(norm_weight), float(l2_eps), float(norm_eps),
                                   _ptr(init_state), _ptr(cu_seqlens), B, T, H, Dk, Dv, n_seqs,
                                   _ptr(out), _ptr(final_state), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, final_state


def layer_decode_step(q, k, v, x_alpha, x_beta, out_gate, norm_weight, state, l2_eps=1e-6,
                      norm_eps=1e-5, out=None, stream=None):
    """One KDA-layer token per (n, h); bf16 q, k, x_alpha [N,H,Dk], v, out_gate
    [N,H,Dv], x_beta [N,H]; state [N,H,Dk,Dv] fp32 updated in place.  Returns out fp32."""
    _validate([("q", q, (None,) * 3, _BF16, True)], devices=False)
    N, H, Dk = q.shape
    Dv = v.shape[-1] if isinstance(v, torch.Tensor) and v.dim() == 3 else None
    _validate([("q", q, (N, H, Dk), _BF16, True), ("k", k, (N, H, Dk), _BF16, True),
               ("v", v, (N, H, Dv), _BF16, True), ("x_alpha", x_alpha, (N, H, Dk), _BF16, True),
               ("x_beta", x_beta, (N, H), _BF16, True), ("out_gate", out_gate, (N, H, Dv), _BF16, True),
               ("norm_weight", norm_weight, (Dv,), _F32, True), ("state", state, (N, H, Dk, Dv), _F32, True),
               ("out", out, (N, H, Dv), _F32, False)])
    if out is None:
        out = torch.empty((N, H, Dv), dtype=torch.float32, device=q.device)
    _check(load().kda_layer_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(x_alpha), _ptr(x_beta),
                                        _ptr(out_gate), _ptr(norm_weight), float(l2_eps),
                                        float(norm_eps), _ptr(state), N, H, Dk, Dv, _ptr(out),
                                        _stream(stream)))
    return out
