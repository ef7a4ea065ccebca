"""Chunked prefill on the GPU (through the C-ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_55_amd import kda, workloads
from kda_testlib import TAU, StreamingParity, assert_parity, host64, log, oracle_threads, rel_err

pytestmark = pytest.mark.gpu


def _gpu(inp, chunk=None, poison=True, init_state="inp"):
    q = inp["q"]
    B, T, H, Dk = q.shape
    Dv = inp["v"].shape[-1]
    N = inp["N"]
    o = torch.full((B, T, H, Dv), float("nan"), device="cuda") if poison else None
    fs = torch.full((N, H, Dk, Dv), float("nan"), device="cuda") if poison else None
    s0 = inp["init_state"] if init_state == "inp" else init_state
    o, fs = kda.chunk_fwd(q, inp["k"], inp["v"], inp["log_alpha"], inp["beta"], s0,
                          inp["cu_seqlens"], chunk or inp["chunk"], out=o, final_state=fs)
    torch.cuda.synchronize()
    return o, fs


def _oracle(inp, heads=None, T=None):
    sl = (lambda x: x) if heads is None else (lambda x: x[:, :, heads])
    tcut = (lambda x: x) if T is None else (lambda x: x[:, :T])
    s0 = inp["init_state"]
    if s0 is not None and heads is not None:
        s0 = s0[:, heads]
    return oracle.forward(tcut(sl(inp["q"])), tcut(sl(inp["k"])), tcut(sl(inp["v"])),
                          tcut(sl(inp["log_alpha"])), tcut(sl(inp["beta"])), s0,
                          inp["cu_seqlens"], n_threads=oracle_threads())


def _check(inp, o, fs, tau, heads=None, label=""):
    o_ref, s_ref = _oracle(inp, heads)
    og = o if heads is None else o[:, :, heads]
    fg = fs if heads is None else fs[:, heads]
    e1 = assert_parity(og, o_ref, tau, f"{label} o")
    e2 = assert_parity(fg, s_ref, tau, f"{label} final state")
    return e1, e2


def test_tiny_fp32_workload():
    """fp32 inputs, T=64, H=1, d=16, 16-token chunks: the 1e-4 bar."""
    inp = workloads.make_prefill("tiny", "cuda", 0)
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.float32], label="tiny")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("C", [16, 32, 64])
def test_ragged_small(dtype, D, C):
    """T not a multiple of any chunk size, several heads, random initial state."""
    log(f"ragged dtype={dtype} D={D} C={C}")
    inp = workloads.make_prefill("prefill", "cuda", seed=D + C, T=157, H=3, dtype=dtype)
    if D != 128:
        inp = _shrink(inp, D)
    o, fs = _gpu(inp, chunk=C)
    tau = TAU[torch.bfloat16 if dtype == "bf16" else torch.float32]
    _check(inp, o, fs, tau, label=f"{dtype} D={D} C={C}")


def _shrink(inp, D):
    """Keeps the first D channels (re-normalising q, k) for smaller head dims."""
    out = dict(inp)
    for name in ("q", "k"):
        x = inp[name][..., :D].float()
        out[name] = (x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)).to(inp[name].dtype)
    out["v"] = inp["v"][..., :D].contiguous()
    out["log_alpha"] = inp["log_alpha"][..., :D].contiguous()
    if inp["init_state"] is not None:
        out["init_state"] = inp["init_state"][:, :, :D, :D].contiguous()
    return out


@pytest.mark.parametrize("shift", [0.0, 2.0, 3.0])
def test_gate_ranges_bf16(shift):
    inp = workloads.make_prefill("prefill", "cuda", seed=11, T=700, H=4, shift=shift)
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.bfloat16], label=f"shift={shift}")


def test_prefill_workload_full():
    """T=4096, H=32, d=128, bf16, random initial state: every output checked."""
    log("prefill workload T=4096 H=32")
    inp = workloads.make_prefill("prefill", "cuda", 0)
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.bfloat16], label="prefill 4096x32")


def test_varlen_small_with_resets():
    lens = [1, 64, 65, 130, 7, 0, 200, 33]
    inp = workloads.make_prefill("varlen", "cuda", seed=5, H=3, lengths=lens)
    g = torch.Generator(device="cuda").manual_seed(9)
    inp["init_state"] = 0.02 * torch.randn((len(lens), 3, 128, 128), device="cuda", generator=g)
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.bfloat16], label="varlen small")


@pytest.mark.parametrize("Dk,Dv", [(128, 16), (32, 32), (64, 64)])
def test_varlen_many_units_narrow_values(Dk, Dv):
    """The state passes decode (sequence, head, slab) from a one-dimensional
    block index with Dv / 16 slabs per unit: 37 sequences x 3 heads = 111 units
    (not a multiple of eight) at 1, 2 and 4 slabs, lengths 0..300, random
    initial state, bf16."""
    log(f"varlen 37x3 Dk={Dk} Dv={Dv}")
    rng = np.random.default_rng(Dk + Dv)
    lens = [int(x) for x in rng.integers(0, 301, size=37)]
    inp = _shrink2(workloads.make_prefill("varlen", "cuda", seed=50 + Dv, H=3, lengths=lens), Dk, Dv)
    g = torch.Generator(device="cuda").manual_seed(51)
    inp["init_state"] = 0.02 * torch.randn((len(lens), 3, Dk, Dv), device="cuda", generator=g)
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.bfloat16], label=f"varlen 37x3 Dk={Dk} Dv={Dv}")


def _whole_tensor_check(inp, o, fs, label, group=16):
    """Every head, token and final state against the oracle, a group of heads
    at a time (host copies of the inputs in their own dtypes; the oracle widens
    each token in C), with max|err| / RMS taken over the whole tensors."""
    import time
    H = inp["H"]
    t0 = time.time()
    host = {n: inp[n].cpu() for n in ("q", "k", "v", "log_alpha", "beta")}
    cu = inp["cu_seqlens"]
    so, ss = StreamingParity(f"{label} o (all heads, all tokens)"), StreamingParity(f"{label} final state (all)")
    t_oracle = 0.0
    for h0 in range(0, H, group):
        h1 = min(H, h0 + group)
        s0 = None if inp["init_state"] is None else inp["init_state"][:, h0:h1]
        ta = time.time()
        o_ref, s_ref = oracle.forward_native(host["q"], host["k"], host["v"], host["log_alpha"], host["beta"],
                                             s0, cu, heads=(h0, h1), n_threads=oracle_threads())
        t_oracle += time.time() - ta
        og = o[:, :, h0:h1].cpu()
        for j in range(h1 - h0):
            so.add(og[:, :, j], o_ref[:, :, j])
        ss.add(fs[:, h0:h1], s_ref)
        del o_ref, og
        log(f"  heads {h0}..{h1 - 1} checked ({time.time() - t0:.0f} s)")
    log(f"  oracle {t_oracle:.1f} s on {oracle_threads()} threads; whole check {time.time() - t0:.1f} s")
    tau = TAU[torch.bfloat16]
    return so.check(tau), ss.check(tau)


@pytest.mark.timeout(600)
def test_varlen_workload_whole():
    """16 packed sequences (~131k tokens), 5% resets, H=32: every output and
    every final state of every head."""
    inp = workloads.make_prefill("varlen", "cuda", 0)
    log(f"varlen workload T={inp['T']}")
    o, fs = _gpu(inp)
    _whole_tensor_check(inp, o, fs, "varlen 16 seqs")


@pytest.mark.timeout(1200)
def test_long_workload_whole():
    """T=1,048,576, H=32 in the launch the benchmark times: every one of the
    33.5 M outputs (x 128) and all 32 final states against the oracle, with the
    outputs NaN-poisoned beforehand so that an unwritten value fails."""
    inp = workloads.make_prefill("long", "cuda", 0)
    log("long workload T=1M H=32")
    o, fs = _gpu(inp)
    _whole_tensor_check(inp, o, fs, "long 1M")


def test_chunk_size_invariance():
    inp = workloads.make_prefill("prefill", "cuda", seed=3, T=333, H=2)
    res = [_gpu(inp, chunk=C) for C in (16, 32, 64)]
    for C, (o, fs) in zip((32, 64), res[1:]):
        assert rel_err(o, host64(res[0][0])) < 5e-3, C
        assert rel_err(fs, host64(res[0][1])) < 5e-3, C


def test_split_resume_and_final_state_alias():
    inp = workloads.make_prefill("prefill", "cuda", seed=4, T=400, H=2)
    o, fs = _gpu(inp)
    T1 = 150
    a = {k: (v[:, :T1].contiguous() if k in ("q", "k", "v", "log_alpha", "beta") else v)
         for k, v in inp.items()}
    b = {k: (v[:, T1:].contiguous() if k in ("q", "k", "v", "log_alpha", "beta") else v)
         for k, v in inp.items()}
    oa, fa = _gpu(a)
    # continue in place: final_state aliases init_state
    ob, fb = kda.chunk_fwd(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], fa, None, 64,
                           final_state=fa)
    torch.cuda.synchronize()
    o2 = torch.cat([oa, ob], dim=1)
    assert rel_err(o2, host64(o)) < 5e-3
    assert rel_err(fb, host64(fs)) < 5e-3
    assert fb.data_ptr() == fa.data_ptr()


def test_prefill_equals_decode_steps():
    inp = workloads.make_prefill("prefill", "cuda", seed=6, T=96, H=2)
    o, fs = _gpu(inp)
    st = inp["init_state"].clone()
    outs = []
    for t in range(96):
        outs.append(kda.decode_step(inp["q"][:, t].contiguous(), inp["k"][:, t].contiguous(),
                                    inp["v"][:, t].contiguous(), inp["log_alpha"][:, t].contiguous(),
                                    inp["beta"][:, t].contiguous(), st))
    torch.cuda.synchronize()
    od = torch.stack(outs, dim=1)
    assert rel_err(o, host64(od)) < 5e-3
    assert rel_err(fs, host64(st)) < 5e-3


def test_varlen_equals_separate_calls():
    lens = [70, 1, 129, 64]
    inp = workloads.make_prefill("varlen", "cuda", seed=7, H=2, lengths=lens)
    o, fs = _gpu(inp)
    cu = inp["cu_seqlens"].cpu().tolist()
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        sub = {k: (v[:, a:b].contiguous() if k in ("q", "k", "v", "log_alpha", "beta") else v)
               for k, v in inp.items()}
        sub["cu_seqlens"] = None
        sub["N"] = 1
        on, fn = _gpu(sub)
        assert torch.equal(on, o[:, a:b]), n
        assert torch.equal(fn[0], fs[n]), n


def test_deterministic_and_all_outputs_written():
    inp = workloads.make_prefill("varlen", "cuda", seed=8, H=2, lengths=[100, 37, 0, 64])
    o1, f1 = _gpu(inp)
    o2, f2 = _gpu(inp)
    assert torch.isfinite(o1).all() and torch.isfinite(f1).all()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_extreme_decay_and_partial_neg_inf():
    """Gates far outside the workloads' range (exact per-element path for
    diagonal tiles) and -inf on scattered channels (clamped to -88)."""
    inp = workloads.make_prefill("prefill", "cuda", seed=12, T=200, H=2)
    g = torch.Generator(device="cuda").manual_seed(3)
    inp["log_alpha"] = inp["log_alpha"] * 12.0
    mask = torch.rand(inp["log_alpha"].shape, device="cuda", generator=g) < 0.03
    inp["log_alpha"][mask] = float("-inf")
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.bfloat16], label="extreme decay")


def test_zero_length_and_empty():
    # T = 0: final state equals the initial state, o is empty
    inp = workloads.make_prefill("prefill", "cuda", seed=13, T=0, H=2)
    o, fs = _gpu(inp)
    assert o.numel() == 0
    assert torch.equal(fs, inp["init_state"])


def test_empty_varlen_without_workspace():
    """T = 0 with cu_seqlens (three empty sequences) and a NULL workspace, through
    the C ABI: each final state is its initial state, nothing else is written."""
    import ctypes
    lib = kda.load()
    H, D, N = 2, 128, 3
    q = torch.zeros((1, 0, H, D), dtype=torch.bfloat16, device="cuda")
    la = torch.zeros((1, 0, H, D), device="cuda")
    be = torch.zeros((1, 0, H), device="cuda")
    o = torch.zeros((1, 0, H, D), device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(21)
    s0 = torch.randn((N, H, D, D), device="cuda", generator=g)
    fs = torch.full((N, H, D, D), float("nan"), device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    for fn in (lib.kda_chunk_fwd, lib.gdn_chunk_fwd):
        fs.fill_(float("nan"))
        gate = la if fn is lib.kda_chunk_fwd else be
        rc = fn(p(q), p(q), p(q), p(gate), p(be), p(s0), p(cu), 1, 0, H, D, D, N, kda.KDA_BF16, 64,
                p(o), p(fs), None, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, lib.kda_last_error()
        torch.cuda.synchronize()
        assert torch.equal(fs, s0)
    fs.fill_(float("nan"))
    rc = lib.kda_dplr_chunk_fwd(p(q), p(q), p(q), p(q), p(q), p(la), p(s0), p(cu), 1, 0, H, D, N, kda.KDA_BF16,
                                64, p(o), p(fs), None, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.kda_last_error()
    torch.cuda.synchronize()
    assert torch.equal(fs, s0)


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (32, "f32")])
def test_dense_batch_with_resets(D, dtype):
    """B = 3 independent sequences in one dense call (partial last chunk, random
    initial states, full-token resets) against the oracle's dense batch."""
    log(f"dense batch D={D} {dtype}")
    parts = [workloads.make_prefill("prefill", "cuda", seed=40 + b, T=200, H=3, dtype=dtype) for b in range(3)]
    inp = {k: torch.cat([p_[k] for p_ in parts], dim=0) for k in ("q", "k", "v", "log_alpha", "beta")}
    if D != 128:
        for k in ("q", "k"):
            x = inp[k][..., :D].float()
            inp[k] = (x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)).to(inp[k].dtype)
        inp["v"] = inp["v"][..., :D].contiguous()
        inp["log_alpha"] = inp["log_alpha"][..., :D].contiguous()
    g = torch.Generator(device="cuda").manual_seed(17)
    inp["log_alpha"][1, 37] = float("-inf")     # a reset inside a chunk of sequence 1
    inp["log_alpha"][2, 64] = float("-inf")     # a reset on a chunk boundary of sequence 2
    inp["init_state"] = 0.02 * torch.randn((3, 3, D, D), device="cuda", generator=g)
    inp.update(cu_seqlens=None, chunk=64, N=3)
    o, fs = _gpu(inp)
    tau = TAU[torch.bfloat16 if dtype == "bf16" else torch.float32]
    _check(inp, o, fs, tau, label=f"dense batch D={D} {dtype}")


def _shrink2(inp, Dk, Dv):
    """Keeps the first Dk key channels (re-normalising q, k) and Dv value columns."""
    out = dict(inp)
    for name in ("q", "k"):
        x = inp[name][..., :Dk].float()
        out[name] = (x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)).to(inp[name].dtype)
    out["v"] = inp["v"][..., :Dv].contiguous()
    out["log_alpha"] = inp["log_alpha"][..., :Dk].contiguous()
    if inp["init_state"] is not None:
        out["init_state"] = inp["init_state"][:, :, :Dk, :Dv].contiguous()
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Dk,Dv", [(16, 32), (32, 16), (64, 128), (128, 64), (16, 128), (128, 16)])
def test_unequal_key_and_value_dims(dtype, Dk, Dv):
    """d_k != d_v: T = 157 (ragged), 3 heads, random initial state, 64-token chunks."""
    log(f"prefill Dk={Dk} Dv={Dv} {dtype}")
    inp = _shrink2(workloads.make_prefill("prefill", "cuda", seed=Dk + 3 * Dv, T=157, H=3, dtype=dtype), Dk, Dv)
    o, fs = _gpu(inp, chunk=64)
    _check(inp, o, fs, TAU[torch.bfloat16 if dtype == "bf16" else torch.float32], label=f"Dk={Dk} Dv={Dv} {dtype}")


def test_slow_decay_gate_variant():
    """The harder precision case: log_alpha = logsigmoid(N(0,1) + 2) per channel
    (mean alpha ~ 0.85, long memory) on the 4096-token workload, every output."""
    log("prefill 4096x32 slow decay")
    inp = workloads.make_prefill("prefill", "cuda", seed=31)
    g = torch.Generator(device="cuda").manual_seed(32)
    x = torch.randn(inp["log_alpha"].shape, device="cuda", generator=g)
    inp["log_alpha"] = torch.nn.functional.logsigmoid(x + 2.0)
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.bfloat16], label="slow decay 4096x32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_degenerate_token_values(dtype):
    """Tokens with beta = 0 (no write), alpha = 1 on every channel (no decay),
    k = 0 (nothing erased or written), q = 0 (zero readout), v = 0, and a reset
    on a chunk's first token, mixed into a ragged 3-head sequence."""
    log(f"degenerate values {dtype}")
    inp = workloads.make_prefill("prefill", "cuda", seed=41, T=300, H=3, dtype=dtype)
    if dtype == "f32":
        inp = _shrink(inp, 64)
    inp["beta"][0, 10:20] = 0.0
    inp["log_alpha"][0, 30:45] = 0.0
    inp["k"][0, 50:53] = 0
    inp["q"][0, 60:70, 1] = 0
    inp["v"][0, 80:90, 2] = 0
    inp["log_alpha"][0, 128] = float("-inf")
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.bfloat16 if dtype == "bf16" else torch.float32], label=f"degenerate {dtype}")
    assert torch.all(o[0, 60:70, 1] == 0)


@pytest.mark.parametrize("e", [-10, -8, 7, 10, 14])
def test_value_scale_within_the_fp16_operand_range(e):
    """v (and the initial state) scaled by 2^e, exact in bf16: o and the final
    state scale by 2^e and stay within the bound while the state and U fit
    fp16's range (v ~ N(0,1) times 2^-10 .. 2^14; 2^7 is the "v x 100" case)."""
    inp = workloads.make_prefill("prefill", "cuda", seed=81, T=777, H=2, shift=-2.0)
    inp["v"] = (inp["v"].float() * 2.0 ** e).to(torch.bfloat16)
    inp["init_state"] = inp["init_state"] * 2.0 ** e
    o, fs = _gpu(inp)
    _check(inp, o, fs, TAU[torch.bfloat16], label=f"v x 2^{e}")


def test_value_scale_past_the_fp16_operand_range():
    """At v ~ N(0,1) x 2^16 (|v| up to ~3e5), U exceeds fp16's largest finite
    value and the bf16 path's output is not finite: the limit the header
    states.  The fp32-input path (fp32 matrix cores throughout) is finite and
    within its bound on the same inputs."""
    inp = workloads.make_prefill("prefill", "cuda", seed=82, T=300, H=2, shift=-2.0, init="zeros")
    inp["v"] = (inp["v"].float() * 2.0 ** 16).to(torch.bfloat16)
    o, fs = _gpu(inp)
    assert not bool(torch.isfinite(o).all())
    f32 = {**inp, **{n: inp[n].float() for n in ("q", "k", "v")}}
    o32, fs32 = _gpu(f32, chunk=64)
    _check(f32, o32, fs32, TAU[torch.float32], label="fp32 path, v x 2^16")
