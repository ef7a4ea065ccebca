"""Pins of the DPLR oracle (``oracle.dplr_forward``): the general
diagonal-plus-low-rank recurrence S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T,
o_t = S_t^T q_t, which the section "Kimi Delta Attention (KDA)" of the page
"Kimi Linear 高效注意力架构" contrasts KDA with (KDA ties both low-rank vectors
to the key).  None of the checks reuses the oracle's arithmetic:

* explicit-matrix brute force: every transition built as a d_k x d_k matrix and
  the states as sums of products of those matrices (tiny T, -inf gates included);
* the KDA special case a = -beta k, b = alpha * k, v -> beta v against the
  separately pinned KDA oracle;
* the GLA case a = 0 against its closed form (per-channel decays of whole spans);
* an exact identity: alpha = 1, a = -k, b = k with unit-norm k is the delta rule
  at beta = 1, so S_t^T k_t = v_t;
* varlen packing against per-sequence dense runs.
"""
import numpy as np

import oracle


def _inputs(rng, B, T, H, Dk, Dv, N=None):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk)) / np.sqrt(Dk)
    v = rng.standard_normal((B, T, H, Dv))
    a = 0.3 * rng.standard_normal((B, T, H, Dk)) / np.sqrt(Dk)
    b = rng.standard_normal((B, T, H, Dk)) / np.sqrt(Dk)
    la = -np.log1p(np.exp(rng.standard_normal((B, T, H, Dk)) + 1.0))
    s0 = 0.3 * rng.standard_normal((N or B, H, Dk, Dv))
    return q, k, v, a, b, la, s0


def _brute(q, k, v, a, b, la, s0):
    """Dense batch: S_t = M_t ... M_1 S_0 + sum_{s<=t} M_t ... M_{s+1} k_s v_s^T with
    M_r = Diag(exp(la_r)) + a_r b_r^T as explicit matrices."""
    B, T, H, Dk = q.shape
    o = np.zeros(v.shape)
    fs = np.zeros(s0.shape)
    for n in range(B):
        for h in range(H):
            M = [np.diag(np.exp(la[n, r, h])) + np.outer(a[n, r, h], b[n, r, h]) for r in range(T)]

            def span(lo, hi):  # M_hi ... M_lo (identity when lo > hi)
                P = np.eye(Dk)
                for r in range(lo, hi + 1):
                    P = M[r] @ P
                return P
            for t in range(T):
                S = span(0, t) @ s0[n, h]
                for s in range(t + 1):
                    S = S + span(s + 1, t) @ np.outer(k[n, s, h], v[n, s, h])
                o[n, t, h] = S.T @ q[n, t, h]
                if t == T - 1:
                    fs[n, h] = S
    return o, fs


def test_brute_force_small():
    rng = np.random.default_rng(11)
    args = _inputs(rng, 2, 7, 2, 3, 2)
    o, fs = oracle.dplr_forward(*args[:6], init_state=args[6])
    bo, bfs = _brute(*args)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fs, bfs, rtol=0, atol=1e-12)


def test_brute_force_with_neg_inf_gates():
    """A token whose gate is -inf on every channel keeps only the low-rank and
    write terms (Diag(0) + a b^T); another has one channel at -inf."""
    rng = np.random.default_rng(12)
    q, k, v, a, b, la, s0 = _inputs(rng, 1, 8, 1, 4, 3)
    la[0, 3, 0, :] = -np.inf
    la[0, 5, 0, 2] = -np.inf
    o, fs = oracle.dplr_forward(q, k, v, a, b, la, init_state=s0)
    bo, bfs = _brute(q, k, v, a, b, la, s0)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fs, bfs, rtol=0, atol=1e-12)


def test_kda_special_case():
    rng = np.random.default_rng(13)
    q, k, v, _, _, la, s0 = _inputs(rng, 1, 150, 2, 8, 5)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, 150, 2))))
    a = -beta[..., None] * k
    b = np.exp(la) * k
    o, fs = oracle.dplr_forward(q, k, beta[..., None] * v, a, b, la, init_state=s0)
    ko, kfs = oracle.forward(q, k, v, la, beta, init_state=s0)
    np.testing.assert_allclose(o, ko, rtol=0, atol=1e-11)
    np.testing.assert_allclose(fs, kfs, rtol=0, atol=1e-11)


def test_gla_closed_form():
    """a = 0: o_t = sum_c q_tc (e^{L_tc} S0[c] + sum_{s<=t} e^{L_tc - L_sc} k_sc v_s),
    L the inclusive prefix sum of log_alpha."""
    rng = np.random.default_rng(14)
    q, k, v, a, b, la, s0 = _inputs(rng, 1, 40, 1, 6, 4)
    a[:] = 0.0
    o, fs = oracle.dplr_forward(q, k, v, a, b, la, init_state=s0)
    L = np.cumsum(la[0, :, 0], axis=0)
    for t in range(40):
        ref = q[0, t, 0] @ (np.exp(L[t])[:, None] * s0[0, 0])
        for s in range(t + 1):
            ref = ref + (q[0, t, 0] * np.exp(L[t] - L[s]) * k[0, s, 0]).sum() * v[0, s, 0]
        np.testing.assert_allclose(o[0, t, 0], ref, rtol=0, atol=1e-11)


def test_delta_rule_identity():
    rng = np.random.default_rng(15)
    q, k, v, a, b, la, s0 = _inputs(rng, 1, 30, 1, 5, 3)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    la[:] = 0.0
    o, _ = oracle.dplr_forward(k, k, v, -k, k, la, init_state=s0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_varlen_matches_separate_runs():
    rng = np.random.default_rng(16)
    lens = [5, 0, 9, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, a, b, la, s0 = _inputs(rng, 1, int(cu[-1]), 2, 4, 3, N=len(lens))
    o, fs = oracle.dplr_forward(q, k, v, a, b, la, init_state=s0, cu_seqlens=cu)
    for n, (t0, t1) in enumerate(zip(cu[:-1], cu[1:])):
        sl = lambda x: x[:, t0:t1]
        if t1 > t0:
            on, fn = oracle.dplr_forward(sl(q), sl(k), sl(v), sl(a), sl(b), sl(la), init_state=s0[n:n + 1])
            np.testing.assert_array_equal(o[:, t0:t1], on)
            np.testing.assert_array_equal(fs[n], fn[0])
        else:
            np.testing.assert_array_equal(fs[n], s0[n])


def test_decode_step_is_one_explicit_transition():
    """dplr_decode_step on N x H states against the explicit matrices of one
    token (brute force at T = 1), -inf gates included."""
    rng = np.random.default_rng(17)
    q, k, v, a, b, la, s0 = _inputs(rng, 3, 1, 2, 5, 4)
    la[1, 0, 1, :] = -np.inf
    la[2, 0, 0, 3] = -np.inf
    o, st = oracle.dplr_decode_step(q[:, 0], k[:, 0], v[:, 0], a[:, 0], b[:, 0], la[:, 0], s0)
    bo, bfs = _brute(q, k, v, a, b, la, s0)
    np.testing.assert_allclose(o, bo[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(st, bfs, rtol=0, atol=1e-12)
