"""Gated DeltaNet (scalar gate per token and head) on the GPU, through the C-ABI,
against the fp64 GDN oracle, at the KDA parity bar."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_55_amd import kda, workloads
from kda_testlib import TAU, assert_parity, host64, log, oracle_threads

pytestmark = pytest.mark.gpu


def _shrink(inp, D):
    """Keeps the first D channels (re-normalising q, k) for smaller head dims."""
    out = dict(inp)
    for name in ("q", "k"):
        x = inp[name][..., :D].float()
        out[name] = (x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)).to(inp[name].dtype)
    out["v"] = inp["v"][..., :D].contiguous()
    if inp["init_state"] is not None:
        out["init_state"] = inp["init_state"][:, :, :D, :D].contiguous()
    return out


def _gpu(inp, chunk=None):
    q = inp["q"]
    B, T, H, _ = q.shape
    Dv = inp["v"].shape[-1]
    o = torch.full((B, T, H, Dv), float("nan"), device="cuda")
    fs = torch.full((inp["N"], H, q.shape[-1], Dv), float("nan"), device="cuda")
    o, fs = kda.gdn_chunk_fwd(q, inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["init_state"],
                              inp["cu_seqlens"], chunk or inp["chunk"], out=o, final_state=fs)
    torch.cuda.synchronize()
    return o, fs


def _check(inp, o, fs, tau, heads=None, T=None, label=""):
    hs = (lambda x: x) if heads is None else (lambda x: x[:, :, heads])
    tc = (lambda x: x) if T is None else (lambda x: x[:, :T])
    s0 = inp["init_state"]
    if s0 is not None and heads is not None:
        s0 = s0[:, heads]
    o_ref, s_ref = oracle.gdn_forward(*(tc(hs(inp[n])) for n in ("q", "k", "v", "log_alpha", "beta")),
                                      s0, inp["cu_seqlens"], n_threads=oracle_threads())
    assert_parity(tc(hs(o)), o_ref, tau, f"{label} o")
    if T is None:
        assert_parity(fs if heads is None else fs[:, heads], s_ref, tau, f"{label} final state")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 64, 128])
@pytest.mark.parametrize("C", [16, 64])
def test_gdn_ragged_small(dtype, D, C):
    """T = 157 (no multiple of any chunk size), 3 heads, random initial state."""
    log(f"gdn ragged dtype={dtype} D={D} C={C}")
    inp = workloads.make_prefill("prefill", "cuda", seed=100 + D + C, T=157, H=3, dtype=dtype,
                                 gate="scalar")
    if D != 128:
        inp = _shrink(inp, D)
    o, fs = _gpu(inp, chunk=C)
    _check(inp, o, fs, TAU[torch.bfloat16 if dtype == "bf16" else torch.float32],
           label=f"gdn {dtype} D={D} C={C}")


@pytest.mark.parametrize("shift", [0.0, 3.0])
def test_gdn_prefill_workload_full(shift):
    """T = 4096, H = 32, d = 128, bf16, random initial state, scalar gates."""
    log(f"gdn prefill workload shift={shift}")
    inp = workloads.make_prefill("prefill", "cuda", seed=1, shift=shift, gate="scalar")
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.bfloat16], label=f"gdn prefill shift={shift}")


def test_gdn_varlen_with_resets():
    lens = [1, 64, 65, 130, 7, 0, 200, 33]
    inp = workloads.make_prefill("varlen", "cuda", seed=15, H=3, lengths=lens, gate="scalar")
    g = torch.Generator(device="cuda").manual_seed(19)
    inp["init_state"] = 0.02 * torch.randn((len(lens), 3, 128, 128), device="cuda", generator=g)
    inp["log_alpha"][0, 100, 1] = float("-inf")  # one head reset inside a chunk
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.bfloat16], label="gdn varlen")


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "bf16"), (32, "f32")])
def test_gdn_agrees_with_kda_on_the_broadcast_gate(D, dtype):
    """The scalar gate broadcast over key channels through kda_chunk_fwd: the same
    function, computed by the channel-wise path (the d = 128 bf16 scalar-gate
    path forms its Gram tiles differently, so the two agree to rounding; the
    general kernel reads the same values either way, so there they are equal)."""
    inp = workloads.make_prefill("varlen", "cuda", seed=16, H=4, lengths=[300, 1, 129],
                                 gate="scalar", dtype=dtype)
    if D != 128:
        inp = _shrink(inp, D)
    o, fs = _gpu(inp)
    la_b = inp["log_alpha"][..., None].expand(*inp["log_alpha"].shape, D).contiguous()
    ok, fk = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], la_b, inp["beta"], None, inp["cu_seqlens"], 64)
    torch.cuda.synchronize()
    if D == 128 and dtype == "bf16":
        assert_parity(o, host64(ok), 3e-3, "gdn vs kda broadcast o")
        assert_parity(fs, host64(fk), 3e-3, "gdn vs kda broadcast final state")
    else:
        assert torch.equal(o, ok) and torch.equal(fs, fk)


@pytest.mark.timeout(600)
def test_gdn_long_workload_sampled():
    """T = 1,048,576, H = 32 with scalar gates: o of 6 heads over the first 16384
    tokens and, for one head, every output and the final state."""
    log("gdn long workload T=1M H=32")
    inp = workloads.make_prefill("long", "cuda", 0)
    inp["log_alpha"] = workloads.scalar_log_alpha((1, inp["T"], 32), 3.0, "cuda", seed=1)
    o, fs = kda.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], None, None, 64)
    torch.cuda.synchronize()
    assert torch.isfinite(fs).all()
    _check(inp, o, fs, TAU[torch.bfloat16], heads=[1, 8, 15, 17, 24, 30], T=16384,
           label="gdn long (6 heads, 16k tokens)")
    _check(inp, o, fs, TAU[torch.bfloat16], heads=[12], label="gdn long head 12 full")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 128])
def test_gdn_decode_steps(dtype, D):
    log(f"gdn decode dtype={dtype} D={D}")
    inp = workloads.make_decode("decode", "cuda", seed=D + 7, N=3, H=2, steps=6, dtype=dtype, D=D,
                                gate="scalar")
    inp["log_alpha"][3][1, 0] = float("-inf")  # a reset of one (n, h) at step 3
    state = inp["state"].clone()
    st = host64(inp["state"])
    tau = TAU[torch.bfloat16 if dtype == "bf16" else torch.float32]
    for t in range(6):
        o = kda.gdn_decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_alpha"][t],
                                inp["beta"][t], state)
        torch.cuda.synchronize()
        o_ref, st = oracle.gdn_decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_alpha"][t],
                                           inp["beta"][t], st)
        assert assert_parity(o, o_ref, tau, f"gdn decode o step {t}") < 1e-5
    assert assert_parity(state, st, tau, "gdn decode state") < 1e-5


def test_gdn_decode_workload_sampled_units():
    """256 sequences x 32 heads, 64 steps: 32 sampled (n, h) units recomputed by the oracle."""
    log("gdn decode workload")
    inp = workloads.make_decode("decode", "cuda", seed=0, gate="scalar")
    w = inp["workload"]
    rng = np.random.default_rng(1)
    units = [(int(rng.integers(w.N)), int(rng.integers(w.H))) for _ in range(32)]
    ns = torch.tensor([u[0] for u in units], device="cuda")
    hs = torch.tensor([u[1] for u in units], device="cuda")
    st = host64(inp["state"][ns, hs])[:, None]
    state = inp["state"].clone()
    sl = lambda x: x[ns, hs][:, None]
    for t in range(w.steps):
        o = kda.gdn_decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_alpha"][t],
                                inp["beta"][t], state)
        o_ref, st = oracle.gdn_decode_step(sl(inp["q"][t]), sl(inp["k"][t]), sl(inp["v"][t]),
                                           sl(inp["log_alpha"][t]), sl(inp["beta"][t]), st)
        if t % 16 == 15:
            torch.cuda.synchronize()
            assert_parity(sl(o), o_ref, TAU[torch.bfloat16], f"gdn decode workload o step {t}")
    torch.cuda.synchronize()
    assert_parity(sl(state), st, TAU[torch.bfloat16], "gdn decode workload states")


def test_gdn_abi_rejects_misaligned_and_null():
    inp = workloads.make_decode("decode", "cuda", seed=3, N=2, H=2, steps=1, gate="scalar")
    state = inp["state"].clone()
    with pytest.raises(kda.KdaError):
        kda.gdn_decode_step(inp["q"][0], inp["k"][0], inp["v"][0], None, inp["beta"][0], state)
    # a scalar gate only needs 4-byte alignment: an odd-element slice is accepted
    la = torch.zeros(2 * 2 + 1, device="cuda")[1:].view(2, 2)
    kda.gdn_decode_step(inp["q"][0], inp["k"][0], inp["v"][0], la, inp["beta"][0], state)
    torch.cuda.synchronize()


def test_gdn_empty_inputs():
    """T = 0 keeps the initial state; N = 0 decode is a no-op."""
    inp = workloads.make_prefill("prefill", "cuda", seed=17, T=0, H=2, gate="scalar")
    o, fs = _gpu(inp)
    assert o.numel() == 0 and torch.equal(fs, inp["init_state"])
    z = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((0, 2, 128, 128), device="cuda")
    out = kda.gdn_decode_step(z, z, z, torch.empty((0, 2), device="cuda"), torch.empty((0, 2), device="cuda"), st)
    torch.cuda.synchronize()
    assert out.numel() == 0
