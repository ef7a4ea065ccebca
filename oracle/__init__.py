"""fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package; the product path (the HIP library and
its binding) never does, and this package imports nothing from it.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, libm ``exp``); this
module only builds it with gcc, converts arrays to contiguous fp64 and calls
it through ctypes.  It follows the state-update equation of the section
"Kimi Delta Attention (KDA)" on the page "Kimi Linear 高效注意力架构":
``S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T`` with
``alpha_t = exp(log_alpha_t)`` per key channel, and the readout
``o_t = S_t^T q_t`` after the token's write.

``gdn_forward`` and ``gdn_decode_step`` run Gated DeltaNet (GDN), the
scalar-gate recurrence the same page sets KDA against (one head-wise
``alpha_t``; KDA replaces it by a per-channel diagonal):
``S_t = (I - beta_t k_t k_t^T) alpha_t S_{t-1} + beta_t k_t v_t^T``, with
``log_alpha`` of shape [B, T, H] (prefill) or [N, H] (decode).  Its C update
shares no arithmetic with the KDA one.

``dplr_forward`` runs the general diagonal-plus-low-rank recurrence that the
page contrasts KDA with (KDA ties both low-rank vectors to the key), read with
free per-token vectors a_t, b_t and an unscaled write:
``S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T``, ``o_t = S_t^T q_t``.

``forward_native`` and ``decode_step_native`` run the same KDA token update on
inputs in the types the GPU path receives (bf16 or fp32 q, k, v; fp32 gates),
for a range of heads, widening each token's values to fp64 in C: the check of
a 1M-token, 32-head output then needs no fp64 copy of whole inputs, and the
decode step is threaded over its states.

``backward`` differentiates the KDA token loop in reverse mode, one token at
a time (the gradients with respect to q, k, v, log_alpha, beta and the initial
state, given those of o and of the final state).

``layer_forward`` and ``layer_decode_step`` (``layer.py``) add the KDA
layer's prologue (L2Norm of q and k, the -softplus decay gate, the sigmoid
beta) and epilogue (RMSNorm and the sigmoid output gate) around ``forward`` /
``decode_step``.

Every function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_pins_gdn.py``, ``tests/test_oracle_pins_layer.py`` and
``tests/test_oracle_pins_bwd.py`` (finite differences of ``forward``) and
``tests/test_oracle_pins_dplr.py``
against closed forms, special cases, invariants, exact rational arithmetic and
explicit-matrix brute force; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
# KDA_ORACLE_LIBRARY: another build of kda_oracle.c to load (the sanitizer test)
_LIB = os.environ.get("KDA_ORACLE_LIBRARY") or os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compiles kda_oracle.c with gcc -O2 (no fast-math) into libkda_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.kda_oracle_forward.argtypes = [
            dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32),
            i64, i64, i64, i64, i64, i64, dp, dp, ctypes.c_int]
        lib.kda_oracle_forward.restype = ctypes.c_int
        vp = ctypes.c_void_p
        fp32p = ctypes.POINTER(ctypes.c_float)
        lib.kda_oracle_forward_native.argtypes = [
            vp, vp, vp, ctypes.c_int, fp32p, fp32p, dp, ctypes.POINTER(ctypes.c_int32),
            i64, i64, i64, i64, i64, i64, i64, i64, dp, dp, ctypes.c_int]
        lib.kda_oracle_forward_native.restype = ctypes.c_int
        lib.gdn_oracle_forward.argtypes = lib.kda_oracle_forward.argtypes
        lib.gdn_oracle_forward.restype = ctypes.c_int
        lib.dplr_oracle_forward.argtypes = [
            dp, dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32),
            i64, i64, i64, i64, i64, i64, dp, dp, ctypes.c_int]
        lib.dplr_oracle_forward.restype = ctypes.c_int
        lib.kda_oracle_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, dp]
        lib.kda_oracle_decode_step.restype = ctypes.c_int
        lib.dplr_oracle_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, dp]
        lib.dplr_oracle_decode_step.restype = ctypes.c_int
        lib.gdn_oracle_decode_step.argtypes = lib.kda_oracle_decode_step.argtypes
        lib.gdn_oracle_decode_step.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [
            dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32),
            i64, i64, i64, i64, i64, i64, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    """Contiguous fp64 numpy copy/view of an array-like (torch tensors included)."""
    if hasattr(x, "detach"):  # torch tensor: widen exactly on the host
        x = x.detach().to("cpu")
        if x.dtype != __import__("torch").float64:
            x = x.double()
        x = x.numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def forward(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, n_threads=None):
    """Runs the KDA recurrence token by token in fp64.

    q, k, log_alpha: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H];
    init_state: [N, H, Dk, Dv] or None (zeros); cu_seqlens: int [N+1] or None.
    Returns (o [B, T, H, Dv], final_state [N, H, Dk, Dv]) as fp64 numpy arrays.
    """
    return _forward(False, q, k, v, log_alpha, beta, init_state, cu_seqlens, n_threads)


def _host_native(x, want):
    """A contiguous host copy of a torch tensor in one of the dtypes ``want``."""
    import torch
    x = x.detach()
    if x.dtype not in want:
        raise TypeError(f"dtype {x.dtype} is not one of {want}")
    return x.to("cpu").contiguous()


def forward_native(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, heads=None,
                   n_threads=None):
    """``forward`` for the heads ``heads = (h_lo, h_hi)`` (default: all) of
    inputs in the types the GPU path receives: q, k, v torch bfloat16 or
    float32, log_alpha and beta float32 (CPU or CUDA tensors; copied to host
    memory as they are).  Each token's values are widened exactly to fp64 in
    C, so the result equals ``forward`` on the widened arrays, without the
    fp64 copies of whole inputs that a 1M-token check would need.

    init_state: [N, h_hi - h_lo, Dk, Dv] (any float dtype; widened) or None.
    Returns (o [B, T, h_hi - h_lo, Dv], final_state [N, h_hi - h_lo, Dk, Dv]), fp64.
    """
    import torch
    qh, kh, vh = (_host_native(x, (torch.bfloat16, torch.float32)) for x in (q, k, v))
    if not (qh.dtype == kh.dtype == vh.dtype):
        raise TypeError("q, k and v must share one dtype")
    lah, beh = (_host_native(x, (torch.float32,)) for x in (log_alpha, beta))
    B, T, H, Dk = qh.shape
    Dv = vh.shape[3]
    assert kh.shape == qh.shape and lah.shape == qh.shape
    assert vh.shape == (B, T, H, Dv) and beh.shape == (B, T, H)
    h_lo, h_hi = (0, H) if heads is None else (int(heads[0]), int(heads[1]))
    Hs = h_hi - h_lo
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens), dtype=np.int32)
        N = cu.size - 1
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        cu, N, cu_p = None, B, None
    s0 = None if init_state is None else _f64(init_state)
    if s0 is not None:
        assert s0.shape == (N, Hs, Dk, Dv)
    o = np.zeros((B, T, Hs, Dv), dtype=np.float64)
    fs = np.zeros((N, Hs, Dk, Dv), dtype=np.float64)
    if n_threads is None:
        n_threads = os.cpu_count() or 1
    fptr = lambda t: ctypes.cast(ctypes.c_void_p(t.data_ptr()), ctypes.POINTER(ctypes.c_float))
    rc = _load().kda_oracle_forward_native(
        ctypes.c_void_p(qh.data_ptr()), ctypes.c_void_p(kh.data_ptr()), ctypes.c_void_p(vh.data_ptr()),
        1 if qh.dtype == torch.bfloat16 else 0, fptr(lah), fptr(beh), _ptr(s0), cu_p,
        B, T, H, Dk, Dv, N, h_lo, h_hi, _ptr(o), _ptr(fs), int(n_threads))
    if rc != 0:
        raise ValueError(f"kda_oracle_forward_native failed with code {rc}")
    return o, fs


def decode_step_native(q, k, v, log_alpha, beta, state, n_threads=None):
    """``decode_step`` on native-typed inputs (q, k, v [N, H, Dk|Dv] bfloat16
    or float32, log_alpha [N, H, Dk] and beta [N, H] float32), threaded over
    the N * H states: one token of ``forward_native`` per state, which is the
    same token update.  state: [N, H, Dk, Dv] (fp64 numpy, or any float tensor).
    Returns (o [N, H, Dv], new_state), fp64."""
    N, H, Dk = q.shape
    r = lambda x: x.reshape(N, 1, *x.shape[1:])
    o, st = forward_native(r(q), r(k), r(v), r(log_alpha), beta.reshape(N, 1, H), state,
                           n_threads=n_threads)
    return o[:, 0], st


def gdn_forward(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, n_threads=None):
    """Runs the GDN (scalar-gate) recurrence token by token in fp64.

    As ``forward`` except log_alpha: [B, T, H] (one gate per token and head).
    """
    return _forward(True, q, k, v, log_alpha, beta, init_state, cu_seqlens, n_threads)


def _forward(scalar_gate, q, k, v, log_alpha, beta, init_state, cu_seqlens, n_threads):
    q, k, v, la, be = (_f64(a) for a in (q, k, v, log_alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    assert k.shape == q.shape
    assert la.shape == ((B, T, H) if scalar_gate else q.shape)
    assert v.shape == (B, T, H, Dv) and be.shape == (B, T, H)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens), dtype=np.int32)
        N = cu.size - 1
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        cu, N, cu_p = None, B, None
    s0 = None if init_state is None else _f64(init_state)
    if s0 is not None:
        assert s0.shape == (N, H, Dk, Dv)
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    fs = np.zeros((N, H, Dk, Dv), dtype=np.float64)
    if n_threads is None:
        n_threads = os.cpu_count() or 1
    lib = _load()
    fn = lib.gdn_oracle_forward if scalar_gate else lib.kda_oracle_forward
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(s0),
            cu_p, B, T, H, Dk, Dv, N, _ptr(o), _ptr(fs), int(n_threads))
    if rc != 0:
        raise ValueError(f"{'gdn' if scalar_gate else 'kda'}_oracle_forward failed with code {rc}")
    return o, fs


def dplr_forward(q, k, v, a, b, log_alpha, init_state=None, cu_seqlens=None, n_threads=None):
    """Runs the DPLR recurrence token by token in fp64.

    q, k, a, b, log_alpha: [B, T, H, Dk]; v: [B, T, H, Dv]; init_state:
    [N, H, Dk, Dv] or None (zeros); cu_seqlens: int [N+1] or None.
    Returns (o [B, T, H, Dv], final_state [N, H, Dk, Dv]) as fp64 numpy arrays.
    """
    q, k, v, a, b, la = (_f64(x) for x in (q, k, v, a, b, log_alpha))
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    assert k.shape == q.shape and a.shape == q.shape and b.shape == q.shape and la.shape == q.shape
    assert v.shape == (B, T, H, Dv)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens), dtype=np.int32)
        N = cu.size - 1
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        cu, N, cu_p = None, B, None
    s0 = None if init_state is None else _f64(init_state)
    if s0 is not None:
        assert s0.shape == (N, H, Dk, Dv)
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    fs = np.zeros((N, H, Dk, Dv), dtype=np.float64)
    if n_threads is None:
        n_threads = os.cpu_count() or 1
    rc = _load().dplr_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(la), _ptr(s0),
                                     cu_p, B, T, H, Dk, Dv, N, _ptr(o), _ptr(fs), int(n_threads))
    if rc != 0:
        raise ValueError(f"dplr_oracle_forward failed with code {rc}")
    return o, fs


def backward(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, d_o=None, d_final_state=None,
             n_threads=None):
    """Gradients of ``forward`` in fp64, by reverse mode over the token loop.

    d_o: [B, T, H, Dv] (required); d_final_state: [N, H, Dk, Dv] or None (zero).
    Returns (dq, dk, dv, dlog_alpha, dbeta, d_init_state) as fp64 numpy arrays;
    dlog_alpha is 0 where log_alpha is -inf.
    """
    q, k, v, la, be, do = (_f64(a) for a in (q, k, v, log_alpha, beta, d_o))
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    assert k.shape == q.shape and la.shape == q.shape
    assert v.shape == (B, T, H, Dv) and be.shape == (B, T, H) and do.shape == v.shape
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens), dtype=np.int32)
        N = cu.size - 1
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        cu, N, cu_p = None, B, None
    s0 = None if init_state is None else _f64(init_state)
    dsf = None if d_final_state is None else _f64(d_final_state)
    for a in (s0, dsf):
        if a is not None:
            assert a.shape == (N, H, Dk, Dv)
    dq = np.zeros((B, T, H, Dk))
    dk = np.zeros((B, T, H, Dk))
    dv = np.zeros((B, T, H, Dv))
    dla = np.zeros((B, T, H, Dk))
    dbeta = np.zeros((B, T, H))
    ds0 = np.zeros((N, H, Dk, Dv))
    if n_threads is None:
        n_threads = os.cpu_count() or 1
    rc = _load().kda_oracle_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(s0), cu_p, B, T, H, Dk, Dv, N,
        _ptr(do), _ptr(dsf), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dla), _ptr(dbeta), _ptr(ds0), int(n_threads))
    if rc != 0:
        raise ValueError(f"kda_oracle_backward failed with code {rc}")
    return dq, dk, dv, dla, dbeta, ds0


def decode_step(q, k, v, log_alpha, beta, state):
    """One KDA step per (n, h); q, k, log_alpha [N,H,Dk], v [N,H,Dv],
    beta [N,H], state [N,H,Dk,Dv].  Returns (o [N,H,Dv], new_state), fp64."""
    return _decode(False, q, k, v, log_alpha, beta, state)


def dplr_decode_step(q, k, v, a, b, log_alpha, state):
    """One DPLR step per (n, h); q, k, a, b, log_alpha [N,H,Dk], v [N,H,Dv],
    state [N,H,Dk,Dv].  Returns (o [N,H,Dv], new_state), fp64."""
    q, k, v, a, b, la = (_f64(x) for x in (q, k, v, a, b, log_alpha))
    st = _f64(state).copy()
    N, H, Dk = q.shape
    Dv = v.shape[2]
    assert k.shape == q.shape and a.shape == q.shape and b.shape == q.shape and la.shape == q.shape
    assert v.shape == (N, H, Dv) and st.shape == (N, H, Dk, Dv)
    o = np.zeros((N, H, Dv))
    rc = _load().dplr_oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(la), _ptr(st),
                                         N, H, Dk, Dv, _ptr(o))
    if rc != 0:
        raise ValueError(f"dplr_oracle_decode_step failed with code {rc}")
    return o, st


def gdn_decode_step(q, k, v, log_alpha, beta, state):
    """One GDN step per (n, h); as ``decode_step`` except log_alpha [N,H]."""
    return _decode(True, q, k, v, log_alpha, beta, state)


def _decode(scalar_gate, q, k, v, log_alpha, beta, state):
    q, k, v, la, be = (_f64(a) for a in (q, k, v, log_alpha, beta))
    st = _f64(state).copy()
    N, H, Dk = q.shape
    Dv = v.shape[2]
    assert st.shape == (N, H, Dk, Dv)
    assert la.shape == ((N, H) if scalar_gate else (N, H, Dk))
    o = np.zeros((N, H, Dv), dtype=np.float64)
    lib = _load()
    fn = lib.gdn_oracle_decode_step if scalar_gate else lib.kda_oracle_decode_step
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(st), N, H, Dk, Dv, _ptr(o))
    if rc != 0:
        raise ValueError(f"{'gdn' if scalar_gate else 'kda'}_oracle_decode_step failed with code {rc}")
    return o, st


from .layer import layer_decode_step, layer_forward  # noqa: E402  (the layer around the operator)
