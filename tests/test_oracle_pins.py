"""Pins the fp64 oracle to things other than itself.

The pages print no worked numbers for the operator, so every pin is a hand
calculation, exact rational arithmetic, a closed form, a special case, an
invariant or an explicit-matrix brute force of the state-update equation of
the section "Kimi Delta Attention (KDA)" on the page "Kimi Linear 高效注意力架构".
Shapes use d_k != d_v throughout so that a transposed state fails.

Mistakes each pin is meant to catch:
  hand example / exact rationals  -> everything, incl. decay-before-erase order
  brute force (explicit M_t)      -> association order, dropped terms, index errors
  frozen state (alpha=1, beta=0)  -> a write term that survives beta = 0
  orthonormal keys                -> misplaced beta, wrong sign of the erase
  retrieval after write           -> decay applied after the erase, readout before write
  reset (alpha = 0)               -> NaN from exp(-inf), history leaking through a reset
  decay-only closed form          -> exp vs log mix-ups, per-channel vs per-value decay
  linearity, split, varlen,
  prefill == decode               -> state carry-over and bookkeeping errors
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, T, H, Dk, Dv, B=1, unit_keys=True, with_state=True):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    la = -np.log1p(np.exp(rng.standard_normal((B, T, H, Dk))))  # -softplus
    be = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = 0.5 * rng.standard_normal((B, H, Dk, Dv)) if with_state else None
    return q, k, v, la, be, s0


def test_hand_example_golden():
    with open(os.path.join(GOLDEN, "hand_example_dk2_dv3.json")) as f:
        g = json.load(f)
    toks = g["tokens"]
    q = np.array([t["q"] for t in toks], float)[None, :, None, :]
    k = np.array([t["k"] for t in toks], float)[None, :, None, :]
    v = np.array([t["v"] for t in toks], float)[None, :, None, :]
    la = np.array([[(-math.inf if x is None else x) for x in t["log_alpha"]] for t in toks])[None, :, None, :]
    be = np.array([t["beta"] for t in toks], float)[None, :, None]
    s0 = np.array(g["S0"], float)[None, None]
    o, fs = oracle.forward(q, k, v, la, be, s0)
    np.testing.assert_allclose(o[0, :, 0], np.array(g["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(fs[0, 0], np.array(g["final_state"]), rtol=0, atol=1e-14)


def _exact_literal(S0, alphas, betas, ks, vs, qs):
    """Exact rational evaluation of S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T
    with explicit matrices, then o_t = S_t^T q_t."""
    Dk, Dv = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for a, b, kk, vv, qq in zip(alphas, betas, ks, vs, qs):
        M = [[(Fraction(int(i == j)) - b * kk[i] * kk[j]) * a[j] for j in range(Dk)] for i in range(Dk)]
        S = [[sum(M[i][c] * S[c][j] for c in range(Dk)) + b * kk[i] * vv[j] for j in range(Dv)]
             for i in range(Dk)]
        outs.append([sum(S[c][j] * qq[c] for c in range(Dk)) for j in range(Dv)])
    return outs, S


def test_exact_rational_brute_force():
    rng = np.random.default_rng(7)
    T, Dk, Dv = 6, 3, 4

    def fr(lo, hi, den):
        return Fraction(int(rng.integers(lo * den, hi * den + 1)), den)

    S0 = [[fr(-2, 2, 8) for _ in range(Dv)] for _ in range(Dk)]
    # alpha = 2^-e or 0 so that exp(log(alpha)) is exact in binary floating point
    alphas = [[Fraction(1, 2 ** int(rng.integers(0, 4))) if rng.random() > 0.15 else Fraction(0)
               for _ in range(Dk)] for _ in range(T)]
    betas = [fr(0, 1, 16) for _ in range(T)]
    ks = [[fr(-1, 1, 8) for _ in range(Dk)] for _ in range(T)]
    vs = [[fr(-3, 3, 4) for _ in range(Dv)] for _ in range(T)]
    qs = [[fr(-1, 1, 8) for _ in range(Dk)] for _ in range(T)]
    outs, S = _exact_literal(S0, alphas, betas, ks, vs, qs)

    f = lambda rows: np.array([[float(x) for x in r] for r in rows])
    la = np.array([[math.log(float(a)) if a > 0 else -math.inf for a in row] for row in alphas])
    o, fs = oracle.forward(f(qs)[None, :, None], f(ks)[None, :, None], f(vs)[None, :, None],
                           la[None, :, None], np.array([float(b) for b in betas])[None, :, None],
                           f(S0)[None, None])
    np.testing.assert_allclose(o[0, :, 0], f(outs), rtol=0, atol=1e-12)
    np.testing.assert_allclose(fs[0, 0], f(S), rtol=0, atol=1e-12)


def _brute_force_expansion(q, k, v, la, be, s0):
    """S_t = (M_t...M_1) S_0 + sum_j (M_t...M_{j+1}) b_j k_j v_j^T with explicit
    d_k x d_k matrices M_m = (I - b_m k_m k_m^T) Diag(alpha_m), one unit (b=0, h=0)."""
    T, Dk = q.shape[1], q.shape[3]
    M = [(np.eye(Dk) - be[0, m, 0] * np.outer(k[0, m, 0], k[0, m, 0])) @ np.diag(np.exp(la[0, m, 0]))
         for m in range(T)]
    outs = []
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
        outs.append(S.T @ q[0, t, 0])
    return np.array(outs), S


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_brute_force_matrix_expansion(T):
    rng = np.random.default_rng(100 + T)
    q, k, v, la, be, s0 = _rand_inputs(rng, T, 1, 5, 3)
    o_bf, s_bf = _brute_force_expansion(q, k, v, la, be, s0)
    o, fs = oracle.forward(q, k, v, la, be, s0)
    np.testing.assert_allclose(o[0, :, 0], o_bf, rtol=0, atol=1e-13)
    np.testing.assert_allclose(fs[0, 0], s_bf, rtol=0, atol=1e-13)


def test_frozen_state_alpha1_beta0():
    rng = np.random.default_rng(1)
    q, k, v, la, be, s0 = _rand_inputs(rng, 12, 2, 6, 4)
    la[:] = 0.0
    be[:] = 0.0
    o, fs = oracle.forward(q, k, v, la, be, s0)
    assert np.array_equal(fs, s0)
    np.testing.assert_array_equal(o[0], np.einsum("thc,hcj->thj", q[0], s0[0]))


def test_orthonormal_keys_reduce_to_linear_attention():
    rng = np.random.default_rng(2)
    T, Dk, Dv = 7, 8, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm[:, :T].T[None, :, None, :].copy()
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    be = rng.uniform(0.1, 1.0, (1, T, 1))
    la = np.zeros((1, T, 1, Dk))
    o, fs = oracle.forward(q, k, v, la, be, None)
    for t in range(T):
        ref = sum(be[0, j, 0] * (k[0, j, 0] @ q[0, t, 0]) * v[0, j, 0] for j in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], ref, rtol=0, atol=1e-14)
    ref_S = sum(be[0, j, 0] * np.outer(k[0, j, 0], v[0, j, 0]) for j in range(T))
    np.testing.assert_allclose(fs[0, 0], ref_S, rtol=0, atol=1e-14)


def test_retrieval_after_write_any_decay():
    """Unit-norm k, beta = 1: S_t^T k_t = v_t for any alpha.  Reading with q_t = k_t
    makes the readout o_t equal v_t."""
    rng = np.random.default_rng(3)
    q, k, v, la, be, s0 = _rand_inputs(rng, 40, 3, 6, 9)
    be[:] = 1.0
    o, _ = oracle.forward(k, k, v, la, be, s0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)
    # general beta: S_t^T k_t = (1 - beta) (D_t S_{t-1})^T k_t + beta v_t for unit k
    q, k, v, la, be, s0 = _rand_inputs(rng, 1, 2, 6, 9)
    o, _ = oracle.forward(k, k, v, la, be, s0)
    for h in range(2):
        DS = np.exp(la[0, 0, h])[:, None] * s0[0, h]
        ref = (1 - be[0, 0, h]) * DS.T @ k[0, 0, h] + be[0, 0, h] * v[0, 0, h]
        np.testing.assert_allclose(o[0, 0, h], ref, rtol=0, atol=1e-14)


def test_reset_alpha_zero():
    rng = np.random.default_rng(4)
    q, k, v, la, be, s0 = _rand_inputs(rng, 10, 2, 5, 7)
    r = 6
    la[0, r] = -np.inf
    o, _ = oracle.forward(q, k, v, la, be, s0)
    assert np.all(np.isfinite(o))
    for h in range(2):
        ref = be[0, r, h] * (k[0, r, h] @ q[0, r, h]) * v[0, r, h]
        np.testing.assert_allclose(o[0, r, h], ref, rtol=0, atol=1e-15)
    # history before the reset cannot matter: change it and compare everything from r on
    q2, k2, v2, la2 = q.copy(), k.copy(), v.copy(), la.copy()
    v2[0, :r] += 3.0
    k2[0, :r] *= -1.0
    la2[0, :r] *= 0.5
    o2, fs2 = oracle.forward(q2, k2, v2, la2, be, 7.0 * s0)
    _, fs = oracle.forward(q, k, v, la, be, s0)
    np.testing.assert_array_equal(o2[0, r:], o[0, r:])
    np.testing.assert_array_equal(fs2, fs)


def test_decay_only_closed_form():
    rng = np.random.default_rng(5)
    q, k, v, la, be, s0 = _rand_inputs(rng, 30, 2, 6, 4)
    be[:] = 0.0
    o, fs = oracle.forward(q, k, v, la, be, s0)
    G = np.cumsum(la[0], axis=0)  # [T, H, Dk]
    np.testing.assert_allclose(fs[0], np.exp(G[-1])[:, :, None] * s0[0], rtol=1e-13, atol=0)
    for t in (0, 11, 29):
        ref = np.einsum("hc,hcj->hj", q[0, t] * np.exp(G[t]), s0[0])
        np.testing.assert_allclose(o[0, t], ref, rtol=0, atol=1e-14)


def test_linearity_in_v_and_state():
    rng = np.random.default_rng(6)
    q, k, v, la, be, s0 = _rand_inputs(rng, 25, 2, 6, 5)
    v2 = rng.standard_normal(v.shape)
    s02 = rng.standard_normal(s0.shape)
    a, b = 0.7, -1.9
    o1, f1 = oracle.forward(q, k, v, la, be, s0)
    o2, f2 = oracle.forward(q, k, v2, la, be, s02)
    o3, f3 = oracle.forward(q, k, a * v + b * v2, la, be, a * s0 + b * s02)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(f3, a * f1 + b * f2, rtol=0, atol=1e-12)


def test_contraction_bound():
    """||k|| = 1, beta, alpha in [0,1]: ||S_t||_2 <= ||S_{t-1}||_2 + beta_t ||v_t||."""
    rng = np.random.default_rng(8)
    T = 24
    q, k, v, la, be, s0 = _rand_inputs(rng, T, 1, 6, 4)
    prev = np.linalg.norm(s0[0, 0], 2)
    for t in range(1, T + 1):
        _, fs = oracle.forward(q[:, :t], k[:, :t], v[:, :t], la[:, :t], be[:, :t], s0)
        cur = np.linalg.norm(fs[0, 0], 2)
        assert cur <= prev + be[0, t - 1, 0] * np.linalg.norm(v[0, t - 1, 0]) + 1e-12
        prev = cur


def test_split_resume():
    rng = np.random.default_rng(9)
    q, k, v, la, be, s0 = _rand_inputs(rng, 50, 3, 6, 5, B=2)
    o, fs = oracle.forward(q, k, v, la, be, s0)
    T1 = 19
    oa, fa = oracle.forward(q[:, :T1], k[:, :T1], v[:, :T1], la[:, :T1], be[:, :T1], s0)
    ob, fb = oracle.forward(q[:, T1:], k[:, T1:], v[:, T1:], la[:, T1:], be[:, T1:], fa)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
    np.testing.assert_array_equal(fb, fs)


def test_varlen_equals_separate_calls():
    rng = np.random.default_rng(10)
    lens = [5, 0, 1, 17, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, la, be, _ = _rand_inputs(rng, T, 2, 4, 6)
    s0 = rng.standard_normal((len(lens), 2, 4, 6))
    o, fs = oracle.forward(q, k, v, la, be, s0, cu_seqlens=cu)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        on, fn = oracle.forward(q[:, a:b], k[:, a:b], v[:, a:b], la[:, a:b], be[:, a:b], s0[n:n + 1])
        np.testing.assert_array_equal(o[:, a:b], on)
        np.testing.assert_array_equal(fs[n], fn[0])
    np.testing.assert_array_equal(fs[1], s0[1])  # length-0 sequence keeps its state


def test_prefill_equals_decode_steps():
    rng = np.random.default_rng(11)
    T, H = 9, 2
    q, k, v, la, be, s0 = _rand_inputs(rng, T, H, 5, 3, B=3)
    o, fs = oracle.forward(q, k, v, la, be, s0)
    st = s0.copy()
    for t in range(T):
        ot, st = oracle.decode_step(q[:, t], k[:, t], v[:, t], la[:, t], be[:, t], st)
        np.testing.assert_array_equal(ot, o[:, t])
    np.testing.assert_array_equal(st, fs)


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(12)
    q, k, v, la, be, s0 = _rand_inputs(rng, 33, 5, 4, 4, B=3)
    o1, f1 = oracle.forward(q, k, v, la, be, s0, n_threads=1)
    o8, f8 = oracle.forward(q, k, v, la, be, s0, n_threads=8)
    np.testing.assert_array_equal(o1, o8)
    np.testing.assert_array_equal(f1, f8)


def test_bad_arguments_raise():
    rng = np.random.default_rng(13)
    q, k, v, la, be, s0 = _rand_inputs(rng, 4, 1, 2, 2)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, la, be, None, cu_seqlens=np.array([0, 3], np.int32))  # cu[-1] != T


def test_dplr_identity():
    """(I - b k k^T) Diag(a) = Diag(a) - (b k)(a * k)^T, the diagonal-plus-low-rank
    form of the transition (KDA section: DPLR with a = b = k): the recurrence
    written as S <- Diag(a) S - (b k)((a * k)^T S) + b k v^T, with explicit
    vectors, matches the oracle (this fixes the order decay-then-erase)."""
    rng = np.random.default_rng(14)
    T, H, Dk, Dv = 11, 2, 5, 4
    q, k, v, la, be, s0 = _rand_inputs(rng, T, H, Dk, Dv)
    o, fs = oracle.forward(q, k, v, la, be, s0)
    for h in range(H):
        S = s0[0, h].copy()
        for t in range(T):
            a = np.exp(la[0, t, h])
            kk, b = k[0, t, h], be[0, t, h]
            S = a[:, None] * S - np.outer(b * kk, (a * kk) @ S) + b * np.outer(kk, v[0, t, h])
            np.testing.assert_allclose(o[0, t, h], S.T @ q[0, t, h], rtol=0, atol=1e-13)
        np.testing.assert_allclose(fs[0, h], S, rtol=0, atol=1e-13)
    # the erase after the decay is not the same operator: (I - b k k^T) then Diag(a) differs
    a = np.exp(la[0, 0, 0])
    kk, b = k[0, 0, 0], be[0, 0, 0]
    M1 = (np.eye(Dk) - b * np.outer(kk, kk)) @ np.diag(a)
    M2 = np.diag(a) @ (np.eye(Dk) - b * np.outer(kk, kk))
    assert np.max(np.abs(M1 - M2)) > 1e-3
    np.testing.assert_allclose(M1, np.diag(a) - np.outer(b * kk, a * kk), rtol=0, atol=1e-15)


def test_native_entry_equals_fp64_entry_bitwise():
    """forward_native (native-typed inputs, a range of heads, widened per token
    in C) runs the same token update as forward on the widened arrays: equal
    bit for bit, dense and varlen, with and without an initial state; and
    decode_step_native equals decode_step."""
    import torch
    g = torch.Generator().manual_seed(5)
    B, T, H, Dk, Dv = 1, 37, 5, 8, 6
    for dt in (torch.bfloat16, torch.float32):
        q = torch.randn(B, T, H, Dk, generator=g).to(dt)
        k = (torch.randn(B, T, H, Dk, generator=g) / 3).to(dt)
        v = torch.randn(B, T, H, Dv, generator=g).to(dt)
        la = -torch.nn.functional.softplus(torch.randn(B, T, H, Dk, generator=g))
        la[0, 9] = float("-inf")
        be = torch.sigmoid(torch.randn(B, T, H, generator=g))
        s0 = 0.1 * torch.randn(3, H, Dk, Dv, generator=g, dtype=torch.float64)
        cu = np.array([0, 10, 10, T], dtype=np.int32)
        o, fs = oracle.forward(q, k, v, la, be, s0, cu, n_threads=3)
        on, fn = oracle.forward_native(q, k, v, la, be, s0[:, 1:4], cu, heads=(1, 4), n_threads=2)
        assert np.array_equal(on, o[:, :, 1:4]) and np.array_equal(fn, fs[:, 1:4])
        o, fs = oracle.forward(q, k, v, la, be)
        on, fn = oracle.forward_native(q, k, v, la, be)
        assert np.array_equal(on, o) and np.array_equal(fn, fs)
        st = 0.1 * np.random.default_rng(1).standard_normal((T, H, Dk, Dv))
        od, sd = oracle.decode_step(q[0], k[0], v[0], la[0], be[0], st)
        odn, sdn = oracle.decode_step_native(q[0], k[0], v[0], la[0], be[0], st, n_threads=4)
        assert np.array_equal(od, odn) and np.array_equal(sd, sdn)
