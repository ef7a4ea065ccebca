"""Seeded synthetic inputs for the KDA operator.

This module only draws random tensors; it holds none of the operator's
arithmetic, imports neither the HIP binding nor the oracle, and serves both
(the tests hand the same tensors to each side).

Recipes (per named workload; tensors are drawn in the order listed, from one
``torch.Generator`` seeded with ``seed`` on the device the tensors are made on;
the varlen lengths come from a separate CPU generator so they do not depend on
the device):

* q, k ~ N(0, 1) in fp32, L2-normalised per (token, head) in fp32 -- the
  normalisation the KDA layer applies upstream of the operator (page "Kimi
  Linear 高效注意力架构", section on the model architecture: L2Norm on q/k) --
  then cast to the input dtype with round-to-nearest-even.
* v ~ N(0, 1), cast to the input dtype.
* log_alpha = -softplus(x + shift), x ~ N(0, 1), fp32, one value per key
  channel (channel-wise decay in [0, 1], section "Kimi Delta Attention (KDA)").
* beta = sigmoid(x), x ~ N(0, 1), fp32, one value per (token, head).
* initial states ~ N(0, 0.02^2) in fp32 where the workload has one.
* gate="scalar" (Gated DeltaNet): log_alpha = -softplus(x + shift) with one
  x ~ N(0, 1) per (token, head) instead of per key channel.
* KDA layer (make_layer_prefill / make_layer_decode): the layer's raw bf16
  projections instead -- q, k ~ 3 N(0, 1) unnormalised, v ~ N(0, 1),
  x_alpha ~ N(0, 1) + shift (so -softplus(x_alpha) has the workload's gate
  law), x_beta ~ N(0, 1), output gate ~ N(0, 1) -- plus an RMSNorm weight
  ~ U[0.5, 1.5] [Dv] fp32; resets set x_alpha = +inf.
* varlen: lengths uniform on [1, 16384], redrawn while a multiple of 64;
  a Bernoulli(0.05) draw per packed token marks a state reset, which sets
  log_alpha = -inf (alpha = 0) on every head and channel of that token.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch
import torch.nn.functional as F


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    Dk: int
    Dv: int
    chunk: int
    dtype: str            # "f32" or "bf16": dtype of q, k, v
    shift: float          # log_alpha = -softplus(N(0,1) + shift)
    init: str             # "zeros" or "normal": initial state
    varlen: int = 0       # number of packed sequences (0: dense batch)
    max_len: int = 0      # varlen: lengths drawn from [1, max_len]
    reset_p: float = 0.0  # varlen: probability of a full-token reset
    steps: int = 0        # decode: consecutive single-token steps
    N: int = 0            # decode: independent sequences


# The five synthetic workloads: a tiny fp32 case, a 4k-token prefill, a packed
# varlen prefill, the 1M-token prefill and a 256x32-state decode.
WORKLOADS = {
    "tiny": Workload("tiny", B=1, T=64, H=1, Dk=16, Dv=16, chunk=16, dtype="f32",
                     shift=0.0, init="zeros"),
    "prefill": Workload("prefill", B=1, T=4096, H=32, Dk=128, Dv=128, chunk=64, dtype="bf16",
                        shift=2.0, init="normal"),
    "varlen": Workload("varlen", B=1, T=0, H=32, Dk=128, Dv=128, chunk=64, dtype="bf16",
                       shift=0.0, init="zeros", varlen=16, max_len=16384, reset_p=0.05),
    "long": Workload("long", B=1, T=1 << 20, H=32, Dk=128, Dv=128, chunk=64, dtype="bf16",
                     shift=3.0, init="zeros"),
    "decode": Workload("decode", B=0, T=0, H=32, Dk=128, Dv=128, chunk=0, dtype="bf16",
                       shift=3.0, init="normal", steps=64, N=256),
}

STATE_STD = 0.02


def _tdtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit_rows(shape, g, device, dtype):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
    return x.to(dtype)


def varlen_lengths(n: int, max_len: int, chunk: int, seed: int) -> list:
    """Sequence lengths uniform on [1, max_len], none a multiple of ``chunk``."""
    g = _gen("cpu", seed)
    out = []
    while len(out) < n:
        L = int(torch.randint(1, max_len + 1, (1,), generator=g).item())
        if L % chunk != 0:
            out.append(L)
    return out


def make_prefill(name: str = "prefill", device="cpu", seed: int = 0, *, T: Optional[int] = None,
                 H: Optional[int] = None, dtype: Optional[str] = None, shift: Optional[float] = None,
                 lengths: Optional[list] = None, init: Optional[str] = None,
                 reset_p: Optional[float] = None, gate: str = "channel") -> dict:
    """Inputs of a prefill workload; keyword overrides give scaled-down variants.

    Returns a dict with q, k, v, log_alpha, beta, init_state (or None),
    cu_seqlens (int32 on ``device``, or None), chunk and the workload record.
    """
    w = WORKLOADS[name]
    H = w.H if H is None else H
    dt = _tdtype(w.dtype if dtype is None else dtype)
    shift = w.shift if shift is None else shift
    init = w.init if init is None else init
    reset_p = w.reset_p if reset_p is None else reset_p
    cu = None
    if w.varlen or lengths is not None:
        if lengths is None:
            lengths = varlen_lengths(w.varlen, w.max_len, w.chunk, seed)
        offs = [0]
        for L in lengths:
            offs.append(offs[-1] + int(L))
        T = offs[-1]
        cu = torch.tensor(offs, dtype=torch.int32, device=device)
        N = len(lengths)
    else:
        T = w.T if T is None else T
        N = w.B
    B = 1 if cu is not None else w.B
    g = _gen(device, seed)
    q = _unit_rows((B, T, H, w.Dk), g, device, dt)
    k = _unit_rows((B, T, H, w.Dk), g, device, dt)
    v = torch.randn((B, T, H, w.Dv), generator=g, device=device, dtype=torch.float32).to(dt)
    gshape = (B, T, H) if gate == "scalar" else (B, T, H, w.Dk)
    x = torch.randn(gshape, generator=g, device=device, dtype=torch.float32)
    log_alpha = -F.softplus(x + shift)
    del x
    beta = torch.sigmoid(torch.randn((B, T, H), generator=g, device=device, dtype=torch.float32))
    s0 = None
    if init == "normal":
        s0 = STATE_STD * torch.randn((N, H, w.Dk, w.Dv), generator=g, device=device,
                                     dtype=torch.float32)
    if reset_p > 0.0:
        mask = torch.rand((T,), generator=g, device=device) < reset_p
        log_alpha[:, mask] = float("-inf")
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, init_state=s0, cu_seqlens=cu,
                chunk=w.chunk, workload=w, T=T, N=N, H=H)


def dplr_vectors(inp: dict, seed: int = 0, gate_b: bool = True):
    """Low-rank vectors (a, b) of the general DPLR transition Diag(alpha) + a b^T
    for a prefill workload's inputs: a = -beta * u, b = alpha * u' (or u' alone
    when ``gate_b`` is False), u the workload's unit key rows and u' unit rows
    of u + 0.5 N(0, 1), both in the workload's dtype.  With u' = u this is the
    KDA transition; u' != u makes a and b independent vectors."""
    k = inp["k"]
    g = _gen(k.device, seed)
    u = k.float()
    u2 = u + 0.5 * torch.randn(u.shape, generator=g, device=k.device, dtype=torch.float32)
    u2 = u2 / torch.linalg.vector_norm(u2, dim=-1, keepdim=True)
    a = (-inp["beta"][..., None] * u).to(k.dtype)
    b = (torch.exp(inp["log_alpha"]) * u2 if gate_b else u2).to(k.dtype)
    return a, b


def scalar_log_alpha(shape, shift: float, device="cpu", seed: int = 0) -> torch.Tensor:
    """Gated DeltaNet gates of any shape: -softplus(x + shift), x ~ N(0, 1), fp32,
    from a generator of their own seeded with ``seed``."""
    g = _gen(device, seed)
    return -F.softplus(torch.randn(shape, generator=g, device=device, dtype=torch.float32) + shift)


def make_decode(name: str = "decode", device="cpu", seed: int = 0, *, N: Optional[int] = None,
                H: Optional[int] = None, steps: Optional[int] = None,
                dtype: Optional[str] = None, D: Optional[int] = None,
                gate: str = "channel") -> dict:
    """Initial state [N, H, Dk, Dv] and per-step inputs of the decode workload.

    Returns a dict with ``state`` and lists q, k, v, log_alpha, beta (one
    [N, H, ...] tensor per step), drawn state first, then step by step.
    """
    w = WORKLOADS[name]
    N = w.N if N is None else N
    H = w.H if H is None else H
    steps = w.steps if steps is None else steps
    Dk = Dv = (w.Dk if D is None else D)
    dt = _tdtype(w.dtype if dtype is None else dtype)
    g = _gen(device, seed)
    state = STATE_STD * torch.randn((N, H, Dk, Dv), generator=g, device=device, dtype=torch.float32)
    out = dict(state=state, q=[], k=[], v=[], log_alpha=[], beta=[], workload=w, N=N, H=H,
               steps=steps)
    for _ in range(steps):
        out["q"].append(_unit_rows((N, H, Dk), g, device, dt))
        out["k"].append(_unit_rows((N, H, Dk), g, device, dt))
        out["v"].append(torch.randn((N, H, Dv), generator=g, device=device).to(dt))
        x = torch.randn((N, H) if gate == "scalar" else (N, H, Dk), generator=g, device=device)
        out["log_alpha"].append(-F.softplus(x + w.shift))
        out["beta"].append(torch.sigmoid(torch.randn((N, H), generator=g, device=device)))
    return out


def _bf16_normal(shape, g, device, scale=1.0, shift=0.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (scale * x + shift).to(torch.bfloat16)


def make_layer_prefill(name: str = "prefill", device="cpu", seed: int = 0, *, T: Optional[int] = None,
                       H: Optional[int] = None, shift: Optional[float] = None,
                       lengths: Optional[list] = None, init: Optional[str] = None,
                       reset_p: Optional[float] = None) -> dict:
    """Raw bf16 projections of the KDA layer for a prefill workload's shapes
    (d = 128).  Returns q, k, v, x_alpha, x_beta, out_gate, norm_weight,
    init_state, cu_seqlens, T, N, H."""
    w = WORKLOADS[name]
    H = w.H if H is None else H
    shift = w.shift if shift is None else shift
    init = w.init if init is None else init
    reset_p = w.reset_p if reset_p is None else reset_p
    cu = None
    if w.varlen or lengths is not None:
        if lengths is None:
            lengths = varlen_lengths(w.varlen, w.max_len, w.chunk, seed)
        offs = [0]
        for L in lengths:
            offs.append(offs[-1] + int(L))
        T = offs[-1]
        cu = torch.tensor(offs, dtype=torch.int32, device=device)
        N = len(lengths)
    else:
        T = w.T if T is None else T
        N = w.B
    B = 1 if cu is not None else w.B
    g = _gen(device, seed)
    q = _bf16_normal((B, T, H, w.Dk), g, device, scale=3.0)
    k = _bf16_normal((B, T, H, w.Dk), g, device, scale=3.0)
    v = _bf16_normal((B, T, H, w.Dv), g, device)
    x_alpha = _bf16_normal((B, T, H, w.Dk), g, device, shift=shift)
    x_beta = _bf16_normal((B, T, H), g, device)
    out_gate = _bf16_normal((B, T, H, w.Dv), g, device)
    norm_weight = 0.5 + torch.rand((w.Dv,), generator=g, device=device, dtype=torch.float32)
    s0 = None
    if init == "normal":
        s0 = STATE_STD * torch.randn((N, H, w.Dk, w.Dv), generator=g, device=device,
                                     dtype=torch.float32)
    if reset_p > 0.0:
        mask = torch.rand((T,), generator=g, device=device) < reset_p
        x_alpha[:, mask] = float("inf")
    return dict(q=q, k=k, v=v, x_alpha=x_alpha, x_beta=x_beta, out_gate=out_gate,
                norm_weight=norm_weight, init_state=s0, cu_seqlens=cu, T=T, N=N, H=H, workload=w)


def make_layer_decode(name: str = "decode", device="cpu", seed: int = 0, *, N: Optional[int] = None,
                      H: Optional[int] = None, steps: Optional[int] = None,
                      D: Optional[int] = None) -> dict:
    """Initial state and per-step raw bf16 projections of the KDA layer for the
    decode workload's shapes."""
    w = WORKLOADS[name]
    N = w.N if N is None else N
    H = w.H if H is None else H
    steps = w.steps if steps is None else steps
    Dk = Dv = (w.Dk if D is None else D)
    g = _gen(device, seed)
    state = STATE_STD * torch.randn((N, H, Dk, Dv), generator=g, device=device, dtype=torch.float32)
    norm_weight = 0.5 + torch.rand((Dv,), generator=g, device=device, dtype=torch.float32)
    out = dict(state=state, norm_weight=norm_weight, q=[], k=[], v=[], x_alpha=[], x_beta=[],
               out_gate=[], N=N, H=H, steps=steps, workload=w)
    for _ in range(steps):
        out["q"].append(_bf16_normal((N, H, Dk), g, device, scale=3.0))
        out["k"].append(_bf16_normal((N, H, Dk), g, device, scale=3.0))
        out["v"].append(_bf16_normal((N, H, Dv), g, device))
        out["x_alpha"].append(_bf16_normal((N, H, Dk), g, device, shift=w.shift))
        out["x_beta"].append(_bf16_normal((N, H), g, device))
        out["out_gate"].append(_bf16_normal((N, H, Dv), g, device))
    return out
