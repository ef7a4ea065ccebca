"""Pins the fp64 GDN (scalar-gate) oracle to things other than itself.

Gated DeltaNet is the recurrence the page "Kimi Linear 高效注意力架构" sets KDA
against: one head-wise scalar forget gate alpha_t (bullet on channel-wise decay
in the section "Kimi Delta Attention (KDA)"; list of related work: GDN adds a
scalar forget gate to DeltaNet), i.e.

    S_t = (I - beta_t k_t k_t^T) alpha_t S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.

Mistakes each pin is meant to catch:
  hand example / exact rationals  -> everything, incl. a gate applied after the write
  brute force (explicit M_t)      -> association order, dropped terms, index errors
  KDA with a broadcast gate       -> gate read from the wrong token or head
  decay-only closed form          -> exp vs log mix-ups, gate applied twice
  retrieval after write           -> misplaced beta, wrong sign of the erase
  reset (alpha = 0)               -> NaN from exp(-inf), history leaking through a reset
  DeltaNet (alpha = 1), orthonormal keys -> the erase term
  split, varlen, prefill == decode -> state carry-over and bookkeeping errors
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rand(rng, T, H, Dk, Dv, B=1, with_state=True):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    la = -np.log1p(np.exp(rng.standard_normal((B, T, H))))  # -softplus, one per token-head
    be = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = 0.5 * rng.standard_normal((B, H, Dk, Dv)) if with_state else None
    return q, k, v, la, be, s0


def test_hand_example():
    """d_k = 2, d_v = 1, worked by hand.
    Token 1: alpha = 1/2, beta = 1/2, k = (1, 0), v = 2, q = (1, 1), S_0 = (1, 0)^T:
      alpha S_0 = (0.5, 0); k^T(alpha S_0) = 0.5; S_1 = (0.5 - 0.25 + 1, 0) = (1.25, 0);
      o_1 = 1.25.
    Token 2: alpha = 1, beta = 1, k = (0, 1), v = -1, q = (0, 1):
      k^T S_1 = 0; S_2 = (1.25, -1); o_2 = -1."""
    q = np.array([[1.0, 1.0], [0.0, 1.0]])[None, :, None]
    k = np.array([[1.0, 0.0], [0.0, 1.0]])[None, :, None]
    v = np.array([[2.0], [-1.0]])[None, :, None]
    la = np.array([math.log(0.5), 0.0])[None, :, None]
    be = np.array([0.5, 1.0])[None, :, None]
    s0 = np.array([[1.0], [0.0]])[None, None]
    o, fs = oracle.gdn_forward(q, k, v, la, be, s0)
    np.testing.assert_allclose(o[0, :, 0, 0], [1.25, -1.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(fs[0, 0, :, 0], [1.25, -1.0], rtol=0, atol=1e-15)


def _exact_literal(S0, alphas, betas, ks, vs, qs):
    """Exact rationals: S_t = alpha (I - b k k^T) S_{t-1} + b k v^T with an explicit
    d_k x d_k matrix, then o_t = S_t^T q_t."""
    Dk, Dv = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for a, b, kk, vv, qq in zip(alphas, betas, ks, vs, qs):
        M = [[a * (Fraction(int(i == j)) - b * kk[i] * kk[j]) for j in range(Dk)] for i in range(Dk)]
        S = [[sum(M[i][c] * S[c][j] for c in range(Dk)) + b * kk[i] * vv[j] for j in range(Dv)]
             for i in range(Dk)]
        outs.append([sum(S[c][j] * qq[c] for c in range(Dk)) for j in range(Dv)])
    return outs, S


def test_exact_rational_brute_force():
    rng = np.random.default_rng(21)
    T, Dk, Dv = 7, 3, 4

    def fr(lo, hi, den):
        return Fraction(int(rng.integers(lo * den, hi * den + 1)), den)

    S0 = [[fr(-2, 2, 8) for _ in range(Dv)] for _ in range(Dk)]
    # alpha = 2^-e or 0 so that exp(log(alpha)) is exact in binary floating point
    alphas = [Fraction(1, 2 ** int(rng.integers(0, 4))) if rng.random() > 0.15 else Fraction(0)
              for _ in range(T)]
    betas = [fr(0, 1, 16) for _ in range(T)]
    ks = [[fr(-1, 1, 8) for _ in range(Dk)] for _ in range(T)]
    vs = [[fr(-3, 3, 4) for _ in range(Dv)] for _ in range(T)]
    qs = [[fr(-1, 1, 8) for _ in range(Dk)] for _ in range(T)]
    outs, S = _exact_literal(S0, alphas, betas, ks, vs, qs)

    f = lambda rows: np.array([[float(x) for x in r] for r in rows])
    la = np.array([math.log(float(a)) if a > 0 else -math.inf for a in alphas])
    o, fs = oracle.gdn_forward(f(qs)[None, :, None], f(ks)[None, :, None], f(vs)[None, :, None],
                               la[None, :, None], np.array([float(b) for b in betas])[None, :, None],
                               f(S0)[None, None])
    np.testing.assert_allclose(o[0, :, 0], f(outs), rtol=0, atol=1e-12)
    np.testing.assert_allclose(fs[0, 0], f(S), rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_brute_force_matrix_expansion(T):
    """S_t = (M_t...M_1) S_0 + sum_j (M_t...M_{j+1}) b_j k_j v_j^T,
    M_m = alpha_m (I - b_m k_m k_m^T), explicit matrices."""
    rng = np.random.default_rng(200 + T)
    Dk, Dv = 5, 3
    q, k, v, la, be, s0 = _rand(rng, T, 1, Dk, Dv)
    M = [np.exp(la[0, m, 0]) * (np.eye(Dk) - be[0, m, 0] * np.outer(k[0, m, 0], k[0, m, 0]))
         for m in range(T)]
    o_bf = []
    for t in range(T):
        prod = np.eye(Dk)
        for m in range(t, -1, -1):
            prod = prod @ M[m]
        S = prod @ s0[0, 0]
        for j in range(t + 1):
            P = np.eye(Dk)
            for m in range(t, j, -1):
                P = P @ M[m]
            S = S + P @ (be[0, j, 0] * np.outer(k[0, j, 0], v[0, j, 0]))
        o_bf.append(S.T @ q[0, t, 0])
    o, fs = oracle.gdn_forward(q, k, v, la, be, s0)
    np.testing.assert_allclose(o[0, :, 0], np.array(o_bf), rtol=0, atol=1e-13)
    np.testing.assert_allclose(fs[0, 0], S, rtol=0, atol=1e-13)


def test_equals_kda_with_broadcast_gate():
    """Diag(alpha 1) = alpha I: GDN is KDA with the same gate on every channel
    (the KDA oracle is pinned on its own in test_oracle_pins.py)."""
    rng = np.random.default_rng(22)
    lens = [9, 0, 31, 4]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, Dk, Dv = int(cu[-1]), 3, 6, 5
    q, k, v, la, be, _ = _rand(rng, T, H, Dk, Dv)
    s0 = 0.3 * rng.standard_normal((len(lens), H, Dk, Dv))
    la[0, 7, 1] = -np.inf
    o, fs = oracle.gdn_forward(q, k, v, la, be, s0, cu_seqlens=cu)
    la_b = np.repeat(la[..., None], Dk, axis=-1)
    o_k, fs_k = oracle.forward(q, k, v, la_b, be, s0, cu_seqlens=cu)
    np.testing.assert_allclose(o, o_k, rtol=0, atol=1e-13)
    np.testing.assert_allclose(fs, fs_k, rtol=0, atol=1e-13)


def test_decay_only_closed_form():
    rng = np.random.default_rng(23)
    q, k, v, la, be, s0 = _rand(rng, 30, 2, 6, 4)
    be[:] = 0.0
    o, fs = oracle.gdn_forward(q, k, v, la, be, s0)
    G = np.cumsum(la[0], axis=0)  # [T, H]
    np.testing.assert_allclose(fs[0], np.exp(G[-1])[:, None, None] * s0[0], rtol=1e-13, atol=0)
    for t in (0, 13, 29):
        ref = np.exp(G[t])[:, None] * np.einsum("hc,hcj->hj", q[0, t], s0[0])
        np.testing.assert_allclose(o[0, t], ref, rtol=0, atol=1e-14)


def test_retrieval_after_write_any_gate():
    """Unit-norm k, beta = 1: S_t^T k_t = v_t whatever alpha_t is."""
    rng = np.random.default_rng(24)
    q, k, v, la, be, s0 = _rand(rng, 40, 3, 6, 9)
    be[:] = 1.0
    o, _ = oracle.gdn_forward(k, k, v, la, be, s0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)
    # general beta: S_t^T k_t = (1 - beta) alpha S_{t-1}^T k_t + beta v_t
    q, k, v, la, be, s0 = _rand(rng, 1, 2, 6, 9)
    o, _ = oracle.gdn_forward(k, k, v, la, be, s0)
    for h in range(2):
        ref = (1 - be[0, 0, h]) * np.exp(la[0, 0, h]) * s0[0, h].T @ k[0, 0, h] + be[0, 0, h] * v[0, 0, h]
        np.testing.assert_allclose(o[0, 0, h], ref, rtol=0, atol=1e-14)


def test_reset_alpha_zero():
    rng = np.random.default_rng(25)
    q, k, v, la, be, s0 = _rand(rng, 10, 2, 5, 7)
    r = 4
    la[0, r] = -np.inf
    o, fs = oracle.gdn_forward(q, k, v, la, be, s0)
    assert np.all(np.isfinite(o))
    for h in range(2):
        ref = be[0, r, h] * (k[0, r, h] @ q[0, r, h]) * v[0, r, h]
        np.testing.assert_allclose(o[0, r, h], ref, rtol=0, atol=1e-15)
    v2 = v.copy()
    v2[0, :r] -= 2.0
    la2 = la.copy()
    la2[0, :r] *= 0.25
    o2, fs2 = oracle.gdn_forward(q, k, v2, la2, be, -3.0 * s0)
    np.testing.assert_array_equal(o2[0, r:], o[0, r:])
    np.testing.assert_array_equal(fs2, fs)


def test_deltanet_orthonormal_keys():
    """alpha = 1 (DeltaNet) with orthonormal keys: every erase removes nothing, so
    o_t = sum_{j<=t} beta_j (k_j . q_t) v_j from a zero state."""
    rng = np.random.default_rng(26)
    T, Dk, Dv = 6, 8, 3
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm[:, :T].T[None, :, None, :].copy()
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    be = rng.uniform(0.1, 1.0, (1, T, 1))
    la = np.zeros((1, T, 1))
    o, _ = oracle.gdn_forward(q, k, v, la, be, None)
    for t in range(T):
        ref = sum(be[0, j, 0] * (k[0, j, 0] @ q[0, t, 0]) * v[0, j, 0] for j in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], ref, rtol=0, atol=1e-14)
    # same key written twice with beta = 1: the second write replaces the first
    k2 = np.concatenate([k[:, :1], k[:, :1]], axis=1)
    v2 = rng.standard_normal((1, 2, 1, Dv))
    o2, fs2 = oracle.gdn_forward(k2, k2, v2, np.zeros((1, 2, 1)), np.ones((1, 2, 1)), None)
    np.testing.assert_allclose(fs2[0, 0], np.outer(k[0, 0, 0], v2[0, 1, 0]), rtol=0, atol=1e-14)


def test_split_varlen_and_decode_agree():
    rng = np.random.default_rng(27)
    q, k, v, la, be, s0 = _rand(rng, 23, 2, 4, 6, B=2)
    o, fs = oracle.gdn_forward(q, k, v, la, be, s0)
    T1 = 10
    oa, fa = oracle.gdn_forward(q[:, :T1], k[:, :T1], v[:, :T1], la[:, :T1], be[:, :T1], s0)
    ob, fb = oracle.gdn_forward(q[:, T1:], k[:, T1:], v[:, T1:], la[:, T1:], be[:, T1:], fa)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
    np.testing.assert_array_equal(fb, fs)
    st = s0.copy()
    for t in range(q.shape[1]):
        ot, st = oracle.gdn_decode_step(q[:, t], k[:, t], v[:, t], la[:, t], be[:, t], st)
        np.testing.assert_array_equal(ot, o[:, t])
    np.testing.assert_array_equal(st, fs)
    # packed rows = the dense batch's rows one after the other
    cu = np.array([0, 23, 46], np.int32)
    cat = lambda x: np.concatenate([x[0:1], x[1:2]], axis=1)
    o_p, fs_p = oracle.gdn_forward(cat(q), cat(k), cat(v), cat(la), cat(be), s0, cu_seqlens=cu)
    np.testing.assert_array_equal(o_p[0, :23], o[0])
    np.testing.assert_array_equal(o_p[0, 23:], o[1])
    np.testing.assert_array_equal(fs_p, fs)


def test_bad_gate_shape_raises():
    rng = np.random.default_rng(28)
    q, k, v, la, be, s0 = _rand(rng, 4, 1, 2, 2)
    with pytest.raises(AssertionError):
        oracle.gdn_forward(q, k, v, np.repeat(la[..., None], 2, axis=-1), be, s0)
