"""Pins the fp64 oracle of the KDA layer (prologue + recurrence + epilogue) to
things other than itself: reductions to the separately pinned recurrence
oracle, closed forms of the gate activations, invariances the normalisations
imply, and edge cases.

Mistakes each pin is meant to catch:
  reduction to the KDA oracle        -> a step applied twice or not at all
  alpha = 1/2, 1/4 from x_alpha       -> sign or form of the softplus gate
  beta = 1/2 from x_beta = 0, 1/(1+e) -> sigmoid vs tanh / missing gate
  scale of q_raw, k_raw               -> a missing or partial L2Norm (e.g. one of q, k)
  scale of v and the state            -> a missing RMSNorm, norm over the wrong axis
  g and -g                            -> wrong output-gate activation, gate before the norm
  one-hot norm weight                 -> weight on the wrong axis
  zero rows                           -> eps placement (0/0)
  decode = prefill                    -> bookkeeping
"""
import math

import numpy as np
import pytest

import oracle

H, Dk, Dv = 2, 6, 5


def _raw(rng, T, B=1, scale=3.0):
    q = scale * rng.standard_normal((B, T, H, Dk))
    k = scale * rng.standard_normal((B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv))
    xa = rng.standard_normal((B, T, H, Dk)) + 1.0
    xb = rng.standard_normal((B, T, H))
    g = rng.standard_normal((B, T, H, Dv))
    w = rng.uniform(0.5, 1.5, Dv)
    s0 = 0.5 * rng.standard_normal((B, H, Dk, Dv))
    return q, k, v, xa, xb, g, w, s0


def test_reduces_to_the_recurrence_oracle():
    """Unit q, k (l2_eps = 0), x_alpha = softplus^-1(-log_alpha), x_beta = logit(beta),
    g = +40 (sigmoid = 1 in fp64), w = 1, norm_eps = 0: the layer's output is the
    recurrence's o divided by its RMS over d_v."""
    rng = np.random.default_rng(31)
    T = 13
    q = rng.standard_normal((1, T, H, Dk))
    k = rng.standard_normal((1, T, H, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, H, Dv))
    la = -np.log1p(np.exp(rng.standard_normal((1, T, H, Dk))))
    beta = rng.uniform(0.05, 0.95, (1, T, H))
    s0 = rng.standard_normal((1, H, Dk, Dv))
    xa = np.log(np.expm1(-la))           # softplus(xa) = -la
    xb = np.log(beta / (1.0 - beta))     # sigmoid(xb) = beta
    out, fs = oracle.layer_forward(q, k, v, xa, xb, np.full((1, T, H, Dv), 40.0), np.ones(Dv),
                                   0.0, 0.0, s0)
    o, fs_ref = oracle.forward(q, k, v, la, beta, s0)
    ref = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fs, fs_ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("xa,alpha", [(0.0, 0.5), (math.log(3.0), 0.25), (-math.log(3.0), 0.75)])
def test_softplus_gate_values(xa, alpha):
    """beta = 0 (x_beta = -inf): the state only decays, by exp(-softplus(x_alpha))
    = 1/(1 + e^x_alpha): x = 0 halves it, x = log 3 quarters it, x = -log 3 keeps 3/4."""
    rng = np.random.default_rng(32)
    q, k, v, _, _, g, w, s0 = _raw(rng, 1)
    x = np.full((1, 1, H, Dk), xa)
    _, fs = oracle.layer_forward(q, k, v, x, np.full((1, 1, H), -np.inf), g, w, 1e-6, 1e-6, s0)
    np.testing.assert_allclose(fs, alpha * s0, rtol=1e-15, atol=0)


def test_sigmoid_beta_values():
    """alpha = 1 (x_alpha = -inf), zero state: S_1 = beta k_hat v^T with beta = 1/2 at
    x_beta = 0 and 1/(1 + e) at x_beta = -1."""
    rng = np.random.default_rng(33)
    q, k, v, _, _, g, w, _ = _raw(rng, 1)
    xb = np.array([[[0.0, -1.0]]])
    _, fs = oracle.layer_forward(q, k, v, np.full((1, 1, H, Dk), -np.inf), xb, g, w, 0.0, 1e-6, None)
    kh = k[0, 0] / np.linalg.norm(k[0, 0], axis=-1, keepdims=True)
    for h, b in enumerate([0.5, 1.0 / (1.0 + math.e)]):
        np.testing.assert_allclose(fs[0, h], b * np.outer(kh[h], v[0, 0, h]), rtol=1e-14, atol=1e-15)


def test_invariant_to_scale_of_q_and_k():
    rng = np.random.default_rng(34)
    q, k, v, xa, xb, g, w, s0 = _raw(rng, 17)
    out, fs = oracle.layer_forward(q, k, v, xa, xb, g, w, 0.0, 1e-6, s0)
    cq = rng.uniform(0.1, 10.0, (1, 17, H, 1))
    ck = rng.uniform(0.1, 10.0, (1, 17, H, 1))
    out2, fs2 = oracle.layer_forward(cq * q, ck * k, v, xa, xb, g, w, 0.0, 1e-6, s0)
    np.testing.assert_allclose(out2, out, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(fs2, fs, rtol=1e-11, atol=1e-12)
    # and the state does depend on the direction of k
    _, fs3 = oracle.layer_forward(q, k + 0.3, v, xa, xb, g, w, 0.0, 1e-6, s0)
    assert np.max(np.abs(fs3 - fs)) > 1e-3


def test_invariant_to_scale_of_values_and_state():
    """The recurrence is linear in (v, S_0) and RMSNorm removes the scale."""
    rng = np.random.default_rng(35)
    q, k, v, xa, xb, g, w, s0 = _raw(rng, 11)
    out, fs = oracle.layer_forward(q, k, v, xa, xb, g, w, 1e-6, 0.0, s0)
    out2, fs2 = oracle.layer_forward(q, k, 7.5 * v, xa, xb, g, w, 1e-6, 0.0, 7.5 * s0)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fs2, 7.5 * fs, rtol=1e-12, atol=1e-12)


def test_output_gate_symmetry_and_weight_axis():
    """sigmoid(g) + sigmoid(-g) = 1: out(g) + out(-g) = out(g = +40), whose RMS over
    d_v divided by w is 1; a one-hot weight keeps a single channel."""
    rng = np.random.default_rng(36)
    q, k, v, xa, xb, g, w, s0 = _raw(rng, 9)
    a, _ = oracle.layer_forward(q, k, v, xa, xb, g, w, 1e-6, 0.0, s0)
    b, _ = oracle.layer_forward(q, k, v, xa, xb, -g, w, 1e-6, 0.0, s0)
    c, _ = oracle.layer_forward(q, k, v, xa, xb, np.full_like(g, 40.0), w, 1e-6, 0.0, s0)
    np.testing.assert_allclose(a + b, c, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(np.sqrt(np.mean((c / w) ** 2, axis=-1)), 1.0, rtol=1e-13)
    assert np.all(a * c > 0)  # sigmoid(g) > 0 keeps the sign of the normalised o
    e2 = np.zeros(Dv)
    e2[2] = 1.0
    d, _ = oracle.layer_forward(q, k, v, xa, xb, g, e2, 1e-6, 0.0, s0)
    assert np.all(d[..., [0, 1, 3, 4]] == 0.0)
    np.testing.assert_allclose(d[..., 2], a[..., 2] / w[2], rtol=1e-13)


def test_zero_rows_stay_finite():
    """q_raw = 0 with l2_eps > 0 reads nothing: o = 0 and the RMSNorm of a zero row
    with norm_eps > 0 is 0."""
    rng = np.random.default_rng(37)
    q, k, v, xa, xb, g, w, s0 = _raw(rng, 4)
    q[0, 2] = 0.0
    out, _ = oracle.layer_forward(q, k, v, xa, xb, g, w, 1e-6, 1e-5, s0)
    assert np.all(np.isfinite(out))
    assert np.all(out[0, 2] == 0.0)


def test_decode_steps_equal_prefill():
    rng = np.random.default_rng(38)
    q, k, v, xa, xb, g, w, _ = _raw(rng, 8, B=3)
    s0 = 0.5 * rng.standard_normal((3, H, Dk, Dv))
    out, fs = oracle.layer_forward(q, k, v, xa, xb, g, w, 1e-6, 1e-5, s0)
    st = s0.copy()
    for t in range(8):
        ot, st = oracle.layer_decode_step(q[:, t], k[:, t], v[:, t], xa[:, t], xb[:, t], g[:, t],
                                          w, 1e-6, 1e-5, st)
        np.testing.assert_allclose(ot, out[:, t], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st, fs, rtol=1e-13, atol=1e-14)


def test_reset_through_the_gate():
    """x_alpha = +inf gives alpha = 0 (log_alpha = -inf): the token resets the state."""
    rng = np.random.default_rng(39)
    q, k, v, xa, xb, g, w, s0 = _raw(rng, 6)
    xa[0, 3] = np.inf
    out, fs = oracle.layer_forward(q, k, v, xa, xb, g, w, 1e-6, 1e-5, s0)
    v2 = v.copy()
    v2[0, :3] += 1.5
    k2 = k.copy()
    k2[0, :3] *= -2.0
    out2, fs2 = oracle.layer_forward(q, k2, v2, xa, xb, g, w, 1e-6, 1e-5, -s0)
    np.testing.assert_array_equal(out2[0, 3:], out[0, 3:])
    np.testing.assert_array_equal(fs2, fs)
    assert np.all(np.isfinite(out))


def test_eps_sits_inside_the_square_roots():
    """sqrt(c^2 m + c^2 eps) = c sqrt(m + eps): scaling (v, S_0) by c and norm_eps by
    c^2 leaves the output unchanged, and so does scaling q_raw, k_raw by c with l2_eps
    by c^2 -- only if each eps is added under its square root."""
    rng = np.random.default_rng(40)
    q, k, v, xa, xb, g, w, s0 = _raw(rng, 7)
    base, _ = oracle.layer_forward(q, k, v, xa, xb, g, w, 0.3, 0.05, s0)
    c = 0.01
    a, _ = oracle.layer_forward(q, k, c * v, xa, xb, g, w, 0.3, 0.05 * c * c, c * s0)
    np.testing.assert_allclose(a, base, rtol=1e-12, atol=1e-14)
    b, _ = oracle.layer_forward(c * q, c * k, v, xa, xb, g, w, 0.3 * c * c, 0.05, s0)
    np.testing.assert_allclose(b, base, rtol=1e-11, atol=1e-13)
    # the eps values are large enough here to matter
    d, _ = oracle.layer_forward(q, k, v, xa, xb, g, w, 0.0, 0.0, s0)
    assert np.max(np.abs(d - base)) > 1e-3
