"""CPU model of the chunked KDA algorithm that the HIP prefill kernels implement.

Not the oracle: this is the kernel's arithmetic written in numpy so that the
derivation (WY/UT form, sub-block exponent references, reset masks) can be
checked against the oracle on the CPU, and so that operand rounding of every
matrix product can be emulated (``rnd`` hooks) to choose the MFMA operand
precision.  It imports nothing from the oracle or from the HIP binding.

Derivation (the state-update equation of the section "Kimi Delta Attention
(KDA)" on the page "Kimi Linear 高效注意力架构", unrolled over a chunk; the
chunkwise form with the DPLR constraint a = b = k is what the page's bullet on
the hardware-efficient chunked algorithm refers to):

  within a chunk (local tokens i = 0..C-1, incoming state S0, per-channel
  cumulative log-decay G_i = sum_{m<=i} g_m):
    (I + A) U = Diag(beta) (V - (K*Gamma) S0),  A_ij = beta_i sum_c k_ic k_jc e^{G_ic-G_jc}, j<i
    T = (I + A)^-1,  W = T Diag(beta) (K*Gamma),  U' = T Diag(beta) V,  U = U' - W S0
    O = (Q*Gamma) S0 + P U,                       P_ij = sum_c q_ic k_jc e^{G_ic-G_jc}, j<=i
    S_C = Diag(Gamma_{C-1}) S0 + (K * e^{G_{C-1}-G})^T U

  exponent references (every factor stays representable in fp32):
    off-diagonal 16x16 tiles (row tile I > column tile J): reference = last
      token of tile J; both factors e^{G_i-G_m}, e^{G_m-G_j} are <= 1.
    diagonal tiles: reference = the tile's middle token (index 7 of 16); factors
      are bounded by e^{half-span}.  Channels whose half-span exceeds SAFE_SPAN
      are taken out of the factored product and added exactly, per element.
  resets: a token whose log_alpha is -inf on every channel is a reset; its g is
    replaced by 0 in all exponent arithmetic, A and P entries (i, j) with a
    reset in (j, i] are zeroed, rows of Q*Gamma and K*Gamma at or after the
    chunk's first reset are zeroed, rows of the K-tilde tile before the chunk's
    last reset are zeroed and Gamma_{C-1} is zeroed.  Other -inf entries are
    clamped to G_FLOOR (e^-88 ~ 6e-39: zero at fp32 resolution).
"""
from __future__ import annotations

import numpy as np

TILE = 16
SAFE_SPAN = 80.0
G_FLOOR = -88.0


def _ident(x):
    return x


def chunk_forward(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, chunk=64,
                  rnd=None, fold=False):
    """Chunked forward over [B,T,H,D] inputs (numpy); returns (o, final_state).

    ``rnd`` maps a product-group name to a function (X, Y) -> X @ Y that
    emulates the operand precision of that product; groups: 'AP' (Gram tiles;
    'APo' / 'APd' override it for the tiles below / on the diagonal), 'WU',
    'WS', 'QS', 'PU', 'KU', 'QW'.  Default: exact (fp64) products.  ``fold`` selects
    the form the HIP state pass uses, O = (Qg - P W) S0 + P U'.
    """
    q, k, v, la, be = (np.asarray(a, dtype=np.float64) for a in (q, k, v, log_alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        seqs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    else:
        seqs = [(b, 0, T) for b in range(B)]
    N = len(seqs)
    mm = {} if rnd is None else dict(rnd)
    for g in ("AP", "WU", "WS", "QS", "PU", "KU", "QW"):
        mm.setdefault(g, lambda X, Y: X @ Y)
    mm.setdefault("APo", mm["AP"])
    mm.setdefault("APd", mm["AP"])
    o = np.zeros((B, T, H, Dv))
    fs = np.zeros((N, H, Dk, Dv))
    for n, (b, t0, t1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if init_state is None else np.array(init_state[n, h], np.float64)
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                S, oc = _one_chunk(q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h],
                                   la[b, c0:c1, h], be[b, c0:c1, h], S, chunk, mm, fold)
                o[b, c0:c1, h] = oc
            fs[n, h] = S
    return o, fs


def _one_chunk(q, k, v, la, be, S0, C, mm, fold):
    n = q.shape[0]
    Dk, Dv = q.shape[1], v.shape[1]
    # pad a partial chunk with identity tokens: k = q = v = 0, beta = 0, g = 0
    pad = C - n
    if pad:
        z = lambda x: np.concatenate([x, np.zeros((pad,) + x.shape[1:])])
        q, k, v, la, be = z(q), z(k), z(v), z(la), z(be)
    reset = np.all(np.isneginf(la), axis=1)
    g = np.where(reset[:, None], 0.0, np.maximum(la, G_FLOOR))
    G = np.cumsum(g, axis=0)                               # [C, Dk]
    idx = np.arange(C)
    last_reset_upto = np.maximum.accumulate(np.where(reset, idx, -1))
    # M_ij = 1 when no reset lies in (j, i]
    M = (last_reset_upto[:, None] <= idx[None, :]).astype(np.float64)
    alive_from_start = (last_reset_upto < 0).astype(np.float64)        # no reset in [0, i]
    any_reset = bool(reset.any())
    last_reset = int(last_reset_upto[-1])
    ktil_alive = (idx >= last_reset).astype(np.float64) if any_reset else np.ones(C)

    Aprime = np.zeros((C, C))
    P = np.zeros((C, C))
    nt = C // TILE
    for I in range(nt):
        ri = slice(I * TILE, (I + 1) * TILE)
        for J in range(I + 1):
            rj = slice(J * TILE, (J + 1) * TILE)
            if J < I:
                m = (J + 1) * TILE - 1
                Xq = q[ri] * np.exp(G[ri] - G[m])
                Xk = k[ri] * np.exp(G[ri] - G[m])
                Y = k[rj] * np.exp(G[m] - G[rj])
                Aprime[ri, rj] = mm["APo"](Xk, Y.T)
                P[ri, rj] = mm["APo"](Xq, Y.T)
            else:
                m = I * TILE + TILE // 2 - 1
                span = np.maximum(G[I * TILE] - G[m], G[m] - G[(I + 1) * TILE - 1])
                safe = span <= SAFE_SPAN
                Xq = np.where(safe, q[ri] * np.exp(np.where(safe, G[ri] - G[m], 0.0)), 0.0)
                Xk = np.where(safe, k[ri] * np.exp(np.where(safe, G[ri] - G[m], 0.0)), 0.0)
                Y = np.where(safe, k[rj] * np.exp(np.where(safe, G[m] - G[rj], 0.0)), 0.0)
                Ad = mm["APd"](Xk, Y.T)
                Pd = mm["APd"](Xq, Y.T)
                for c in np.nonzero(~safe)[0]:       # exact per-element path
                    E = np.exp(np.minimum(G[ri, c][:, None] - G[rj, c][None, :], 0.0))
                    Ad += np.outer(k[ri, c], k[rj, c]) * E
                    Pd += np.outer(q[ri, c], k[rj, c]) * E
                Aprime[ri, rj] = Ad
                P[ri, rj] = Pd
    A = np.tril(be[:, None] * Aprime * M, -1)
    P = np.tril(P * M)
    Tm = np.linalg.inv(np.eye(C) + A)                      # unit lower-triangular
    Gam = np.exp(G) * alive_from_start[:, None]
    Kg = k * Gam
    Qg = q * Gam
    Ktil = k * np.exp(G[-1] - G) * ktil_alive[:, None]
    gam_last = np.exp(G[-1]) * (0.0 if any_reset else 1.0)
    W = mm["WU"](Tm, be[:, None] * Kg)
    Up = mm["WU"](Tm, be[:, None] * v)
    if fold:
        # O = Qg S0 + P (U' - W S0) = (Qg - P W) S0 + P U': the state pass then
        # needs only [W; Q'] S0, U' and O_intra = P U'.
        Qp = Qg - mm["QW"](P, W)
        Oi = mm["QW"](P, Up)
        U = Up - mm["WS"](W, S0)
        O = mm["QS"](Qp, S0) + Oi
    else:
        U = Up - mm["WS"](W, S0)
        O = mm["QS"](Qg, S0) + mm["PU"](P, U)
    S1 = gam_last[:, None] * S0 + mm["KU"](Ktil.T, U)
    return S1, O[:n]


# ---- operand-precision emulation -------------------------------------------------

def to_bf16(x):
    """Round fp64 -> fp32 -> bf16 (round to nearest even), returned as fp64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isfinite(f), out, f.astype(np.float64))


def to_f16(x):
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)


def to_f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def product(kind):
    """(X, Y) -> X @ Y with operands in a given precision, fp32 result.

    kind: 'f64', 'f32', 'bf16', 'f16', 'bf16x3' (hi/lo split of both operands,
    three products), 'f16x3'.
    """
    def split(r):
        def f(X, Y):
            Xh, Yh = r(X), r(Y)
            Xl, Yl = r(X - Xh), r(Y - Yh)
            return to_f32(Xh @ Yh + (Xh @ Yl + Xl @ Yh))
        return f
    table = {
        "f64": lambda X, Y: X @ Y,
        "f32": lambda X, Y: to_f32(to_f32(X) @ to_f32(Y)),
        "bf16": lambda X, Y: to_f32(to_bf16(X) @ to_bf16(Y)),
        "f16": lambda X, Y: to_f32(to_f16(X) @ to_f16(Y)),
        "bf16x3": split(to_bf16),
        "f16x3": split(to_f16),
        # split only one operand (two products): 'L' the left, 'R' the right
        "f16x2L": lambda X, Y: to_f32(to_f16(X) @ to_f16(Y) + to_f16(X - to_f16(X)) @ to_f16(Y)),
        "f16x2R": lambda X, Y: to_f32(to_f16(X) @ to_f16(Y) + to_f16(X) @ to_f16(Y - to_f16(Y))),
    }
    return table[kind]
