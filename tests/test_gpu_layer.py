"""The KDA layer (fused prologue + recurrence + epilogue) on the GPU, through the
C-ABI, against the fp64 layer oracle, at the operator's bf16 parity bar.

The prefill applies 1/|q| and 1/|k| in fp32 at every use of the bf16 inputs;
rounding the normalised vectors back to bf16 instead would by itself cost
about 8e-2 of the output's RMS under this max-error metric (seen with the
oracle on the CPU), so the kernels never do."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_55_amd import kda, workloads
from kda_testlib import TAU, assert_parity, host64, log, oracle_threads

pytestmark = pytest.mark.gpu

L2_EPS, NORM_EPS = 1e-6, 1e-5
NAMES = ("q", "k", "v", "x_alpha", "x_beta", "out_gate")


def _gpu(inp):
    B, T, H, D = inp["q"].shape
    o = torch.full((B, T, H, D), float("nan"), device="cuda")
    fs = torch.full((inp["N"], H, D, D), float("nan"), device="cuda")
    o, fs = kda.layer_chunk_fwd(*(inp[n] for n in NAMES), inp["norm_weight"], L2_EPS, NORM_EPS,
                                inp["init_state"], inp["cu_seqlens"], out=o, final_state=fs)
    torch.cuda.synchronize()
    return o, fs


def _check(inp, o, fs, heads=None, T=None, label=""):
    hs = (lambda x: x) if heads is None else (lambda x: x[:, :, heads])
    tc = (lambda x: x) if T is None else (lambda x: x[:, :T])
    s0 = inp["init_state"]
    if s0 is not None and heads is not None:
        s0 = s0[:, heads]
    out_ref, s_ref = oracle.layer_forward(*(tc(hs(inp[n])) for n in NAMES), inp["norm_weight"], L2_EPS,
                                          NORM_EPS, s0, inp["cu_seqlens"], n_threads=oracle_threads())
    assert_parity(tc(hs(o)), out_ref, TAU[torch.bfloat16], f"{label} out")
    if T is None:
        assert_parity(fs if heads is None else fs[:, heads], s_ref, TAU[torch.bfloat16], f"{label} final state")


@pytest.mark.parametrize("T", [1, 63, 157])
def test_layer_ragged_small(T):
    log(f"layer ragged T={T}")
    inp = workloads.make_layer_prefill("prefill", "cuda", seed=200 + T, T=T, H=3)
    o, fs = _gpu(inp)
    _check(inp, o, fs, label=f"layer T={T}")


def test_layer_prefill_workload_full():
    """T = 4096, H = 32, d = 128 raw projections, random initial state: every output."""
    log("layer prefill workload")
    inp = workloads.make_layer_prefill("prefill", "cuda", seed=2)
    o, fs = _gpu(inp)
    _check(inp, o, fs, label="layer prefill 4096x32")


def test_layer_varlen_with_resets():
    lens = [1, 64, 65, 130, 7, 0, 200, 33]
    inp = workloads.make_layer_prefill("varlen", "cuda", seed=21, H=3, lengths=lens)
    g = torch.Generator(device="cuda").manual_seed(23)
    inp["init_state"] = 0.02 * torch.randn((len(lens), 3, 128, 128), device="cuda", generator=g)
    inp["x_alpha"][0, 90, 2] = float("inf")   # one head reset inside a chunk
    o, fs = _gpu(inp)
    _check(inp, o, fs, label="layer varlen")


def test_layer_many_units_short_sequences():
    """The state pass exchanges each row's sum of squares between the eight
    workgroups of a (sequence, head) unit: 96 sequences x 5 heads = 480 units,
    3,840 workgroups (many more than are resident at once), lengths 1..200."""
    log("layer varlen 96 x 5 heads")
    rng = np.random.default_rng(31)
    lens = [int(x) for x in rng.integers(1, 201, size=96)]
    inp = workloads.make_layer_prefill("varlen", "cuda", seed=31, H=5, lengths=lens)
    o, fs = _gpu(inp)
    _check(inp, o, fs, label="layer varlen 96x5")


def test_layer_workspace_contents_and_reuse():
    """The exchange words carry a per-call tag: a workspace full of leftover
    bytes, or one last used by another call, gives the same output bit for bit
    (and the oracle's)."""
    log("layer workspace reuse")
    inp = workloads.make_layer_prefill("prefill", "cuda", seed=32, T=300, H=5)
    other = workloads.make_layer_prefill("prefill", "cuda", seed=33, T=300, H=5)
    B, T, H, D = inp["q"].shape
    ws = torch.full((kda.layer_workspace_size(B, T, H),), 0xFF, dtype=torch.uint8, device="cuda")

    def run(x):
        o = torch.full((B, T, H, D), float("nan"), device="cuda")
        fs = torch.full((x["N"], H, D, D), float("nan"), device="cuda")
        kda.layer_chunk_fwd(*(x[n] for n in NAMES), x["norm_weight"], L2_EPS, NORM_EPS, x["init_state"],
                            None, out=o, final_state=fs, workspace=ws)
        torch.cuda.synchronize()
        return o, fs

    o1, fs1 = run(inp)
    run(other)
    o2, fs2 = run(inp)
    assert torch.equal(o1, o2) and torch.equal(fs1, fs2)
    _check(inp, o1, fs1, label="layer, workspace of 0xff bytes")


def test_layer_prologue_matches_unfused_operator():
    """The fused prologue against the plain operator's fp32 path fed the prologue
    computed by torch in fp32 (normalised q and k, -softplus, sigmoid); both
    outputs go through the epilogue oracle."""
    inp = workloads.make_layer_prefill("prefill", "cuda", seed=24, T=300, H=2)
    o, fs = _gpu(inp)
    nrm = lambda x: x / torch.sqrt((x * x).sum(-1, keepdim=True) + L2_EPS)
    qn, kn = nrm(inp["q"].float()), nrm(inp["k"].float())
    la = -torch.nn.functional.softplus(inp["x_alpha"].float())
    beta = torch.sigmoid(inp["x_beta"].float())
    o2, fs2 = kda.chunk_fwd(qn, kn, inp["v"].float(), la, beta, inp["init_state"], None, 32)
    torch.cuda.synchronize()
    ref = oracle.layer.rmsnorm_gate(host64(o2), host64(inp["out_gate"]), host64(inp["norm_weight"]), NORM_EPS)
    assert_parity(o, ref, TAU[torch.bfloat16], "fused vs unfused prologue out")
    assert_parity(fs, host64(fs2), TAU[torch.bfloat16], "fused vs unfused prologue final state")


@pytest.mark.timeout(600)
def test_layer_long_workload_sampled():
    """T = 1,048,576, H = 32 raw projections: out of 6 heads over the first 16384
    tokens and, for one head, every output and its final state."""
    log("layer long workload T=1M H=32")
    inp = workloads.make_layer_prefill("long", "cuda", 0)
    o, fs = kda.layer_chunk_fwd(*(inp[n] for n in NAMES), inp["norm_weight"], L2_EPS, NORM_EPS)
    torch.cuda.synchronize()
    assert torch.isfinite(fs).all()
    _check(inp, o, fs, heads=[2, 7, 13, 19, 23, 29], T=16384, label="layer long (6 heads, 16k)")
    _check(inp, o, fs, heads=[21], label="layer long head 21 full")


@pytest.mark.parametrize("D", [16, 64, 128])
def test_layer_decode_steps(D):
    log(f"layer decode D={D}")
    inp = workloads.make_layer_decode("decode", "cuda", seed=300 + D, N=3, H=2, steps=6, D=D)
    inp["x_alpha"][2][0, 1] = float("inf")  # a reset of one (n, h) at step 2
    state = inp["state"].clone()
    st = host64(inp["state"])
    for t in range(6):
        args = [inp[n][t] for n in NAMES]
        o = kda.layer_decode_step(*args, inp["norm_weight"], state, L2_EPS, NORM_EPS)
        torch.cuda.synchronize()
        o_ref, st = oracle.layer_decode_step(*args, inp["norm_weight"], L2_EPS, NORM_EPS, st)
        # fp32 throughout (q, k normalised in fp32)
        assert assert_parity(o, o_ref, TAU[torch.bfloat16], f"layer decode out step {t}") < 1e-4
    assert assert_parity(state, st, TAU[torch.bfloat16], "layer decode state") < 1e-4


def test_layer_decode_workload_sampled_units():
    log("layer decode workload")
    inp = workloads.make_layer_decode("decode", "cuda", seed=0)
    N, H, steps = inp["N"], inp["H"], inp["steps"]
    rng = np.random.default_rng(2)
    units = [(int(rng.integers(N)), int(rng.integers(H))) for _ in range(32)]
    ns = torch.tensor([u[0] for u in units], device="cuda")
    hs = torch.tensor([u[1] for u in units], device="cuda")
    sl = lambda x: x[ns, hs][:, None]
    st = host64(sl(inp["state"]))
    state = inp["state"].clone()
    for t in range(steps):
        args = [inp[n][t] for n in NAMES]
        o = kda.layer_decode_step(*args, inp["norm_weight"], state, L2_EPS, NORM_EPS)
        o_ref, st = oracle.layer_decode_step(*(sl(a) for a in args), inp["norm_weight"], L2_EPS, NORM_EPS, st)
        if t % 16 == 15:
            torch.cuda.synchronize()
            assert_parity(sl(o), o_ref, TAU[torch.bfloat16], f"layer decode workload out step {t}")
    torch.cuda.synchronize()
    assert_parity(sl(state), st, TAU[torch.bfloat16], "layer decode workload states")


def test_layer_empty_and_zero_length_sequences():
    """T = 0 keeps the initial state; zero-length sequences inside a varlen
    batch keep theirs; N = 0 decode is a no-op."""
    inp = workloads.make_layer_prefill("prefill", "cuda", seed=26, T=0, H=2)
    o, fs = _gpu(inp)
    assert o.numel() == 0 and torch.equal(fs, inp["init_state"])
    inp = workloads.make_layer_prefill("varlen", "cuda", seed=27, H=2, lengths=[0, 70, 0, 5, 0])
    g = torch.Generator(device="cuda").manual_seed(28)
    inp["init_state"] = 0.02 * torch.randn((5, 2, 128, 128), device="cuda", generator=g)
    o, fs = _gpu(inp)
    for n in (0, 2, 4):
        assert torch.equal(fs[n], inp["init_state"][n])
    _check(inp, o, fs, label="layer varlen with empty sequences")
    z = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((0, 2, 128, 128), device="cuda")
    out = kda.layer_decode_step(z, z, z, z, torch.empty((0, 2), dtype=torch.bfloat16, device="cuda"), z,
                                inp["norm_weight"], st)
    torch.cuda.synchronize()
    assert out.numel() == 0
