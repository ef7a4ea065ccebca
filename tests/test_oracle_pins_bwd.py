"""Pins of the backward oracle (``oracle.backward``), none of which reuses its
arithmetic:

* central finite differences of the forward oracle, element by element, on
  small cases (one crosses the 64-token checkpoint of the reverse sweep; one
  is a varlen batch with an empty sequence, initial states, a reset token and
  a partly -inf gate);
* the adjoint identity: for fixed q, k, log_alpha, beta the forward is linear
  in (v, S_0) (the state update of the section "Kimi Delta Attention (KDA)"
  on the page "Kimi Linear 高效注意力架构" is affine in S_{t-1} with the write
  term linear in v), so <dO, O> + <dS_T, S_T> = <dV, V> + <dS_0, S_0>;
* closed forms at beta = 0, alpha = 1, where the state stays S_0;
* zero cotangents give zero gradients.
"""
import numpy as np
import pytest

import oracle



def _inputs(rng, B, T, H, Dk, Dv, N=None):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk)) / np.sqrt(Dk)
    v = rng.standard_normal((B, T, H, Dv))
    la = -np.log1p(np.exp(rng.standard_normal((B, T, H, Dk)) + 1.0))
    be = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = 0.3 * rng.standard_normal((N or B, H, Dk, Dv))
    return q, k, v, la, be, s0


def _fd_check(args, cu, do, dsf, skip=None, eps=1e-6, tol=1e-7):
    """Central differences of L = <do, o> + <dsf, S_T> for every element of
    q, k, v, log_alpha, beta and S_0 against the oracle's gradients."""
    grads = oracle.backward(*args, cu_seqlens=cu, d_o=do, d_final_state=dsf, n_threads=1)

    def loss(a):
        o, fs = oracle.forward(*a, cu_seqlens=cu, n_threads=1)
        return float((o * do).sum() + (fs * dsf).sum())

    for ai, (a, g) in enumerate(zip(args, grads)):
        scale = max(1.0, float(np.abs(g).max()))
        for idx in np.ndindex(a.shape):
            if skip is not None and skip(ai, idx):
                continue
            ap, am = a.copy(), a.copy()
            ap[idx] += eps
            am[idx] -= eps
            A = list(args)
            A[ai] = ap
            lp = loss(A)
            A[ai] = am
            lm = loss(A)
            num = (lp - lm) / (2 * eps)
            assert abs(num - g[idx]) <= tol * scale, (ai, idx, num, g[idx])
    return grads


def test_fd_dense_two_heads():
    rng = np.random.default_rng(1)
    args = _inputs(rng, 2, 6, 2, 3, 2)
    do = rng.standard_normal((2, 6, 2, 2))
    dsf = rng.standard_normal((2, 2, 3, 2))
    _fd_check(args, None, do, dsf)


def test_fd_across_the_checkpoint_segment():
    """70 tokens: the reverse sweep recomputes two segments (64 + 6 tokens)."""
    rng = np.random.default_rng(2)
    args = _inputs(rng, 1, 70, 1, 2, 2)
    do = rng.standard_normal((1, 70, 1, 2))
    dsf = rng.standard_normal((1, 1, 2, 2))
    _fd_check(args, None, do, dsf, eps=1e-6, tol=2e-7)


def test_fd_varlen_reset_and_partial_neg_inf():
    """Sequences of 3, 0 and 6 tokens with their own initial states; token 5 of
    the packed row is a reset (log_alpha = -inf on every channel), token 1 has
    one channel at -inf.  The gradient with respect to a -inf entry is 0 (alpha
    = 0 there); every finite entry is checked by finite differences."""
    rng = np.random.default_rng(3)
    cu = np.array([0, 3, 3, 9], dtype=np.int32)
    q, k, v, la, be, s0 = _inputs(rng, 1, 9, 1, 3, 2, N=3)
    la[0, 5, 0, :] = -np.inf
    la[0, 1, 0, 2] = -np.inf
    do = rng.standard_normal((1, 9, 1, 2))
    dsf = rng.standard_normal((3, 1, 3, 2))
    args = [q, k, v, la, be, s0]
    grads = _fd_check(args, cu, do, dsf, skip=lambda ai, idx: ai == 3 and np.isinf(la[idx]))
    dla = grads[3]
    assert np.all(dla[0, 5, 0] == 0.0) and dla[0, 1, 0, 2] == 0.0
    # the empty sequence passes its state gradient through unchanged
    np.testing.assert_array_equal(grads[5][1], dsf[1])


def test_adjoint_identity():
    rng = np.random.default_rng(4)
    q, k, v, la, be, s0 = _inputs(rng, 1, 200, 2, 16, 8)
    do = rng.standard_normal(v.shape)
    dsf = rng.standard_normal(s0.shape)
    o, fs = oracle.forward(q, k, v, la, be, s0)
    _, _, dv, _, _, ds0 = oracle.backward(q, k, v, la, be, s0, d_o=do, d_final_state=dsf)
    lhs = float((do * o).sum() + (dsf * fs).sum())
    rhs = float((dv * v).sum() + (ds0 * s0).sum())
    assert abs(lhs - rhs) <= 1e-11 * (abs(lhs) + 1.0)


def test_closed_form_beta_zero_alpha_one():
    """beta = 0, alpha = 1: S_t = S_0 for every t and o_t = S_0^T q_t, so with
    D_t = dS_T + sum_{s >= t} q_s do_s^T:  dq_t = S_0 do_t, dk = dv = 0,
    dS_0 = D_0, dbeta_t = k_t^T D_t (v_t - S_0^T k_t) and
    dlog_alpha_t[c] = sum_j S_0[c, j] D_t[c, j]."""
    rng = np.random.default_rng(5)
    T, Dk, Dv = 9, 4, 3
    q, k, v, _, _, s0 = _inputs(rng, 1, T, 1, Dk, Dv)
    la = np.zeros_like(q)
    be = np.zeros((1, T, 1))
    do = rng.standard_normal((1, T, 1, Dv))
    dsf = rng.standard_normal((1, 1, Dk, Dv))
    dq, dk, dv, dla, dbeta, ds0 = oracle.backward(q, k, v, la, be, s0, d_o=do, d_final_state=dsf)
    S0 = s0[0, 0]
    for t in range(T):
        D = dsf[0, 0] + sum(np.outer(q[0, s, 0], do[0, s, 0]) for s in range(t, T))
        np.testing.assert_allclose(dq[0, t, 0], S0 @ do[0, t, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dbeta[0, t, 0], k[0, t, 0] @ D @ (v[0, t, 0] - S0.T @ k[0, t, 0]),
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(dla[0, t, 0], (S0 * D).sum(axis=1), rtol=0, atol=1e-12)
    assert np.all(dk == 0) and np.all(dv == 0)
    D0 = dsf[0, 0] + sum(np.outer(q[0, s, 0], do[0, s, 0]) for s in range(T))
    np.testing.assert_allclose(ds0[0, 0], D0, rtol=0, atol=1e-12)


def test_zero_cotangents_give_zero_gradients():
    rng = np.random.default_rng(6)
    q, k, v, la, be, s0 = _inputs(rng, 1, 20, 2, 5, 4)
    grads = oracle.backward(q, k, v, la, be, s0, d_o=np.zeros(v.shape), d_final_state=None)
    for g in grads:
        assert np.all(g == 0.0)
