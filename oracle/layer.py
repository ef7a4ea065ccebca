"""fp64 oracle of the KDA layer around the operator: the prologue and epilogue
of the list item describing the KDA layer in the model-architecture list of
the page "Kimi Linear 高效注意力架构" (L2Norm on q/k, a channel-wise decay
gate from a low-rank projection, a sigmoid output gate with RMSNorm).

TEST INFRASTRUCTURE ONLY, like the rest of this package.  The recurrence
itself is the pinned C oracle (``oracle.forward`` / ``oracle.decode_step``);
this module adds the steps on either side in plain numpy fp64, in the order
the layer applies them:

  1. q = q_raw / sqrt(sum q_raw^2 + l2_eps), likewise k      (L2Norm per token, head)
  2. log_alpha = -softplus(x_alpha) = -log(1 + exp(x_alpha))  (decay gate; the
     low-rank projection producing x_alpha is the caller's GEMM, and the page
     leaves the activation unstated -- the workloads' -softplus is taken)
  3. beta = sigmoid(x_beta)
  4. the KDA recurrence and readout o_t = S_t^T q_t
  5. out = o / sqrt(mean_j o_j^2 + norm_eps) * w * sigmoid(g)  (RMSNorm over the
     head's d_v channels with a per-channel weight w shared by all heads, then
     the sigmoid output gate)

Shapes: q_raw, k_raw, x_alpha [B, T, H, Dk]; v, g [B, T, H, Dv];
x_beta [B, T, H]; w [Dv]; states [N, H, Dk, Dv] (decode: drop T).
"""
from __future__ import annotations

import numpy as np

from . import _f64, decode_step, forward


def l2norm(x, eps):
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def softplus(x):
    """log(1 + exp(x)), evaluated without overflow (+inf -> +inf)."""
    return np.logaddexp(0.0, x)


def sigmoid(x):
    """1 / (1 + exp(-x)) without overflow for either sign."""
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def rmsnorm_gate(o, g, w, eps):
    """RMSNorm over the last axis with weight w, times sigmoid(g)."""
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * w * sigmoid(g)


def prologue(q_raw, k_raw, x_alpha, x_beta, l2_eps):
    q = l2norm(_f64(q_raw), l2_eps)
    k = l2norm(_f64(k_raw), l2_eps)
    return q, k, -softplus(_f64(x_alpha)), sigmoid(_f64(x_beta))


def layer_forward(q_raw, k_raw, v, x_alpha, x_beta, g, w, l2_eps, norm_eps,
                  init_state=None, cu_seqlens=None, n_threads=None):
    """Steps 1-5 over whole sequences.  Returns (out [B,T,H,Dv], final_state), fp64."""
    q, k, la, beta = prologue(q_raw, k_raw, x_alpha, x_beta, l2_eps)
    o, fs = forward(q, k, v, la, beta, init_state, cu_seqlens, n_threads=n_threads)
    return rmsnorm_gate(o, _f64(g), _f64(w), norm_eps), fs


def layer_decode_step(q_raw, k_raw, v, x_alpha, x_beta, g, w, l2_eps, norm_eps, state):
    """One token per (n, h).  Returns (out [N,H,Dv], new_state), fp64."""
    q, k, la, beta = prologue(q_raw, k_raw, x_alpha, x_beta, l2_eps)
    o, st = decode_step(q, k, v, la, beta, state)
    return rmsnorm_gate(o, _f64(g), _f64(w), norm_eps), st
