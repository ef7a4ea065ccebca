"""Decode step on the GPU (through the C-ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_55_amd import kda, workloads
from kda_testlib import TAU, StreamingParity, assert_parity, host64, log, oracle_threads

pytestmark = pytest.mark.gpu


def _run_steps(inp, steps, dev="cuda"):
    state = inp["state"].clone()
    outs = []
    for t in range(steps):
        outs.append(kda.decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_alpha"][t],
                                    inp["beta"][t], state))
    torch.cuda.synchronize()
    return outs, state


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_decode_small_all_dims(dtype, D):
    log(f"decode small dtype={dtype} D={D}")
    inp = workloads.make_decode("decode", "cuda", seed=D, N=3, H=2, steps=5, dtype=dtype, D=D)
    outs, state = _run_steps(inp, 5)
    st = host64(inp["state"])
    tau = TAU[torch.bfloat16 if dtype == "bf16" else torch.float32]
    for t in range(5):
        o_ref, st = oracle.decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_alpha"][t],
                                       inp["beta"][t], st)
        # decode arithmetic is fp32 throughout: far inside the parity bar
        e = assert_parity(outs[t], o_ref, tau, f"o step {t}")
        assert e < 1e-5
    assert assert_parity(state, st, tau, "state") < 1e-5


def test_decode_reset_and_zero_beta():
    """alpha = 0 on every channel: S = beta k v^T; beta = 0 and alpha = 1: S unchanged."""
    inp = workloads.make_decode("decode", "cuda", seed=1, N=2, H=3, steps=1)
    la = inp["log_alpha"][0].clone()
    la[0] = float("-inf")
    la[1] = 0.0
    beta = inp["beta"][0].clone()
    beta[1] = 0.0
    state = inp["state"].clone()
    s0 = state.clone()
    o = kda.decode_step(inp["q"][0], inp["k"][0], inp["v"][0], la, beta, state)
    torch.cuda.synchronize()
    k = inp["k"][0].float()
    v = inp["v"][0].float()
    q = inp["q"][0].float()
    want = beta[0, :, None, None] * k[0, :, :, None] * v[0, :, None, :]
    assert torch.allclose(state[0], want, rtol=1e-6, atol=1e-7)
    assert torch.equal(state[1], s0[1])
    want_o1 = torch.einsum("hc,hcj->hj", q[1], s0[1])
    assert torch.allclose(o[1], want_o1, rtol=1e-5, atol=1e-6)
    assert torch.isfinite(o).all()


@pytest.mark.timeout(600)
def test_decode_workload_whole():
    """The full decode workload (256 sequences x 32 heads, 64 steps, 512 MiB of
    state) on the GPU; the oracle (threaded over the 8,192 states) runs the
    same 64 steps and every output of every step and every final state are
    compared, with max|err| / RMS over the whole tensors."""
    import time
    log("decode workload: 256 x 32 x 128 x 128, 64 steps")
    inp = workloads.make_decode("decode", "cuda", seed=0)
    w = inp["workload"]
    st = host64(inp["state"])
    outs, state = _run_steps(inp, w.steps)
    so = StreamingParity("o (8192 states x 64 steps)")
    t0 = time.time()
    for t in range(w.steps):
        o_ref, st = oracle.decode_step_native(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_alpha"][t],
                                              inp["beta"][t], st, n_threads=oracle_threads())
        so.add(outs[t], o_ref)
    log(f"  oracle 64 steps on {oracle_threads()} threads: {time.time() - t0:.1f} s")
    tau = TAU[torch.bfloat16]
    assert so.check(tau) < 1e-4
    sp = StreamingParity("final state (8192 states)")
    sp.add(state, st)
    assert sp.check(tau) < 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Dk,Dv", [(16, 128), (128, 16), (64, 32), (32, 64)])
def test_decode_unequal_dims(dtype, Dk, Dv):
    """d_k != d_v: the first Dk key channels (q, k re-normalised) and Dv value columns."""
    log(f"decode Dk={Dk} Dv={Dv} {dtype}")
    inp = workloads.make_decode("decode", "cuda", seed=Dk + Dv, N=3, H=2, steps=4, dtype=dtype)
    nrm = lambda x: (x[..., :Dk].float() / torch.linalg.vector_norm(x[..., :Dk].float(), dim=-1, keepdim=True)).to(x.dtype)
    q = [nrm(x) for x in inp["q"]]
    k = [nrm(x) for x in inp["k"]]
    v = [x[..., :Dv].contiguous() for x in inp["v"]]
    la = [x[..., :Dk].contiguous() for x in inp["log_alpha"]]
    state = inp["state"][:, :, :Dk, :Dv].contiguous()
    st = host64(state)
    tau = TAU[torch.bfloat16 if dtype == "bf16" else torch.float32]
    for t in range(4):
        o = kda.decode_step(q[t], k[t], v[t], la[t], inp["beta"][t], state)
        torch.cuda.synchronize()
        o_ref, st = oracle.decode_step(q[t], k[t], v[t], la[t], inp["beta"][t], st)
        assert assert_parity(o, o_ref, tau, f"decode Dk={Dk} Dv={Dv} o step {t}") < 1e-5
    assert assert_parity(state, st, tau, f"decode Dk={Dk} Dv={Dv} state") < 1e-5
