"""The chunked algorithm the HIP prefill implements, modelled in fp64 on the CPU,
against the token-loop oracle: pins the derivation (WY/UT form, sub-block
exponent references, reset masks, partial chunks) before any kernel runs."""
import numpy as np
import pytest

import oracle
from chunk_model import chunk_forward


def _inputs(rng, T, H, Dk, Dv, shift=0.0, B=1, resets=0.0, neg_inf_channels=0.0, state=True,
            gate_scale=1.0):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    la = -gate_scale * np.log1p(np.exp(rng.standard_normal((B, T, H, Dk)) + shift))
    be = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    if resets:
        la[:, rng.random(T) < resets] = -np.inf
    if neg_inf_channels:
        la[rng.random(la.shape) < neg_inf_channels] = -np.inf
    s0 = 0.02 * rng.standard_normal((B, H, Dk, Dv)) if state else None
    return q, k, v, la, be, s0


def _check(ref, got, tol=1e-11):
    o_r, s_r = ref
    o_g, s_g = got
    scale_o = np.sqrt(np.mean(o_r ** 2)) + 1e-300
    scale_s = np.sqrt(np.mean(s_r ** 2)) + 1e-300
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(s_g))
    assert np.max(np.abs(o_g - o_r)) <= tol * scale_o
    assert np.max(np.abs(s_g - s_r)) <= tol * scale_s


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("shift", [0.0, 2.0, 3.0])
@pytest.mark.parametrize("fold", [False, True])
def test_chunked_equals_token_loop(C, shift, fold):
    rng = np.random.default_rng(int(C + 10 * shift))
    args = _inputs(rng, 157, 2, 32, 24, shift=shift)
    _check(oracle.forward(*args), chunk_forward(*args, chunk=C, fold=fold))


def test_chunked_varlen_resets_partial_chunks():
    rng = np.random.default_rng(3)
    lens = [1, 64, 65, 130, 7, 0, 200]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, la, be, _ = _inputs(rng, int(cu[-1]), 2, 32, 16, resets=0.05)
    s0 = 0.02 * rng.standard_normal((len(lens), 2, 32, 16))
    args = (q, k, v, la, be, s0)
    _check(oracle.forward(*args, cu_seqlens=cu), chunk_forward(*args, cu_seqlens=cu, chunk=64, fold=True))


def test_chunked_reset_on_first_and_last_token_of_chunk():
    rng = np.random.default_rng(4)
    q, k, v, la, be, s0 = _inputs(rng, 128, 1, 16, 16)
    for t in (0, 15, 16, 63, 64, 127):
        la[0, t] = -np.inf
    _check(oracle.forward(q, k, v, la, be, s0), chunk_forward(q, k, v, la, be, s0, chunk=64, fold=True))


def test_chunked_extreme_decay_takes_exact_path():
    """Gates far below the configs' range push diagonal-tile half-spans past the
    safe bound; those channels take the per-element path."""
    rng = np.random.default_rng(5)
    args = _inputs(rng, 96, 1, 16, 8, gate_scale=12.0)
    _check(oracle.forward(*args), chunk_forward(*args, chunk=64))


def test_chunked_partial_neg_inf_channels():
    rng = np.random.default_rng(6)
    args = _inputs(rng, 100, 2, 16, 8, neg_inf_channels=0.03)
    _check(oracle.forward(*args), chunk_forward(*args, chunk=32))


def _kernel_plan():
    """The operand precision of the bf16 path's products (as the kernels do
    them): Gram tiles on the diagonal bf16 hi/lo, below it fp16; WY and fold
    products bf16 hi/lo; [W; Q'] S with an fp16 state; Kt fp16 against U as an
    fp16 hi/lo pair."""
    from chunk_model import product
    return {"APd": product("bf16x3"), "APo": product("f16"), "WU": product("bf16x3"), "QW": product("bf16x3"),
            "WS": product("f16"), "QS": product("f16"), "KU": product("f16x2R")}


@pytest.mark.parametrize("e,ok", [(-20, False), (-16, False), (-10, True), (0, True), (8, True), (14, True),
                                  (15, None)])
def test_fp16_operand_range_of_the_bf16_path(e, ok):
    """The recurrence is linear in v (and S0), so scaling v by 2^e scales o
    and S exactly and leaves the relative error unchanged -- while the fp16
    operands (the state in [W; Q'] S, U in Kt U) stay in fp16's range.  With
    v ~ N(0, 1) (max|v| ~ 4.6), slow decay: the error is that of e = 0 for
    e in [-10, 14] (max|v| up to ~7.5e4); below about e = -16 (max|v| ~ 7e-5,
    the state ~ 1e-5) the fp16 operands fall into the subnormal range and the
    error exceeds the bf16-input bound 2e-2; at e = 15 (max|v| ~ 1.5e5) U
    exceeds 65504 and the output is not finite."""
    from chunk_model import to_bf16
    rng = np.random.default_rng(0)
    T, H, d = 512, 1, 128
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = to_bf16(unit(rng.standard_normal((1, T, H, d))))
    k = to_bf16(unit(rng.standard_normal((1, T, H, d))))
    v = to_bf16(rng.standard_normal((1, T, H, d))) * 2.0 ** e  # exact in bf16: a power of two
    la = (-np.log1p(np.exp(-(rng.standard_normal((1, T, H, d)) + 2.0)))).astype(np.float32).astype(np.float64)
    be = (1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, H))))).astype(np.float32).astype(np.float64)
    o_ref, s_ref = oracle.forward(q, k, v, la, be)
    with np.errstate(all="ignore"):
        o, s = chunk_forward(q, k, v, la, be, None, None, 64, rnd=_kernel_plan(), fold=True)
    if ok is None:
        assert not np.isfinite(o).all()
        return
    rel = lambda a, b: float(np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b)))
    eo, es = rel(o, o_ref), rel(s, s_ref)
    if ok:
        assert eo < 2e-3 and es < 2e-3, (eo, es)
    else:
        assert max(eo, es) > 2e-2, (eo, es)
