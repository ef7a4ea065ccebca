"""Benchmark of the KDA hot path on one MI355X.

One step = one chunked prefill (kda_chunk_fwd) over the 1M-token workload
(B=1, T=1,048,576, H=32, d_k=d_v=128, 64-token chunks, bf16 q/k/v, fp32 gates)
followed by the 64 consecutive decode steps (kda_decode_step) of the decode
workload (256 sequences x 32 heads, 128x128 fp32 states).  Inputs are seeded
synthetic tensors already resident in HBM; outputs and workspaces are
preallocated.  `value` is prefill tokens/s; the decode step's HBM GB/s is
reported next to it.  Times come from HIP events on the stream the kernels run
on: W warm-up passes (default 3), then K timed ones (default 10), each prefill
preceded by a 512 MiB write that flushes L2 and the MALL; reported times are
medians (means beside them).  The fp64 CPU oracle is timed on a bounded sample of the same prefill
workload on the host cores (cpu_baseline).

After the timed KDA steps, the Gated DeltaNet (scalar-gate) variant is timed
on the same tensors with one log gate per (token, head) -- gdn_chunk_fwd over
the 1M-token workload and 64 gdn_decode_step calls -- and reported in the
"gdn" object of the same JSON line; then the KDA layer (fused prologue and
epilogue, kda_layer_chunk_fwd / kda_layer_decode_step) in the "layer" object;
then the general diagonal-plus-low-rank recurrence (kda_dplr_chunk_fwd over the
same 1M-token q, k, v and gates, and 64 kda_dplr_decode_step calls on the decode
workload) in the "dplr" object; then the backward
(kda_chunk_bwd) over all 1,048,576 tokens of the same prefill inputs in the
"backward" object.

python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

Profiling helpers (the commands that made the summaries under profiles/):
  python bench.py --only prefill|decode|copy|backward|dplr ...   one part only, for rocprofv3
      (copy: a plain device-to-device copy of COPY_BYTES, the counter calibration)
  python bench.py --summarize-trace DIR            markdown table of rocprofv3
      --kernel-trace --stats output (DIR/run_kernel_stats.csv)
  python bench.py --summarize-counters FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR [MFMA_DIR]
          [--backward-counters BWD_FETCH_DIR BWD_WRITE_DIR]
      writes profiles/traffic.json from the rocprofv3 --pmc runs (the backward's: every
      dispatch of one --only backward call summed)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12        # MI355X HBM3E bytes/s
COPY_BYTES = 1 << 31     # size of the calibration copy (read once, written once)
FLUSH_BYTES = 1 << 29    # cache flush written before each timed prefill (> the 256 MB MALL)
BF16_PEAK = 2.5e15       # MI355X dense bf16/fp16 matrix flop/s


def prefill_alg_bytes(T, H, Dk, Dv, N, in_bytes=2, init=False, gate_per_head=None):
    """Algorithmic HBM bytes of one prefill: q, k, v read, log_alpha and beta
    read, o written, final state written (and the initial state read).
    gate_per_head: fp32 gates per (token, head) -- Dk for KDA, 1 for GDN."""
    g = Dk if gate_per_head is None else gate_per_head
    per_tok_head = in_bytes * (2 * Dk + Dv) + 4 * g + 4 + 4 * Dv
    state = N * H * Dk * Dv * 4
    return T * H * per_tok_head + state * (2 if init else 1)


def prefill_alg_flops(T, H, Dk, Dv, C):
    """6 d_k d_v + C (3 d_k + 2 d_v) + C^2 / 3 per token and head (the three
    state contractions, the intra-chunk products counted on their triangles,
    and the triangular inverse)."""
    return T * H * (6 * Dk * Dv + C * (3 * Dk + 2 * Dv) + C * C / 3)


def layer_alg_bytes(T, H, Dk, Dv, N, decode=False):
    """The KDA layer's algorithmic bytes: bf16 q, k, v, x_alpha, x_beta and output
    gate read, fp32 output written, the state written (decode: read and written);
    the RMSNorm weight is negligible."""
    per = 2 * (2 * Dk + Dv) + 2 * Dk + 2 + 2 * Dv + 4 * Dv
    state = N * H * Dk * Dv * 4
    return T * H * per + state * (2 if decode else 1)


def backward_alg_bytes(T, H, Dk, Dv, in_bytes=2):
    """kda_chunk_bwd, per token and head: q, k, v (in_bytes each element),
    log_alpha, beta and d_o read; dq, dk, dv, dlog_alpha, dbeta written (fp32)."""
    read = in_bytes * (2 * Dk + Dv) + 4 * Dk + 4 + 4 * Dv
    write = 4 * (3 * Dk + Dv) + 4
    return T * H * (read + write)


def dplr_alg_bytes(T, H, D, N, in_bytes=2):
    """kda_dplr_chunk_fwd: q, k, v, a, b read (in_bytes each element), log_alpha
    read (fp32, per channel), o written (fp32), final state written."""
    return T * H * (5 * in_bytes * D + 4 * D + 4 * D) + N * H * D * D * 4


def dplr_decode_alg_bytes(N, H, D, in_bytes=2):
    """State read and written once, plus the token's q, k, v, a, b, log_alpha and o."""
    return N * H * (8 * D * D + 5 * in_bytes * D + 4 * D + 4 * D)


def decode_alg_bytes(N, H, Dk, Dv, in_bytes=2, gate_per_head=None):
    """State read and written once, plus the token's q, k, v, log_alpha, beta, o
    (gate_per_head: Dk for KDA, 1 for GDN)."""
    g = Dk if gate_per_head is None else gate_per_head
    return N * H * (8 * Dk * Dv + in_bytes * (2 * Dk + Dv) + 4 * g + 4 + 4 * Dv)


# what the line's copied counter fields are: figures of the committed summary,
# not measured in the run that prints them (null when the summary was taken on
# other kernel sources)
COUNTER_SOURCE = ("profiles/traffic.json: rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, copy-calibrated; "
                  "MfmaUtil) of an earlier run on these exact kernel sources (source digest checked)")


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_55_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per launch (fetch + write, copy-calibrated) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel sources;
    else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    ent = rec.get("launches", {}).get(key)
    return None if ent is None else ent.get("hbm_bytes")


# Kernels of each C-ABI launch on the 1M-token prefill / 256x32-state decode
# workloads (rocprofv3 names, shortened).  The state pass is one kernel for
# the KDA and GDN prefills (its traffic does not depend on the gate); the
# layer's is its own kernel with the RMSNorm and output gate fused.
KDA_INTRA = "kda::intra_wide_kernel<0>"
GDN_INTRA = "kda::intra_wide_kernel<1>"
STATE = "kda::state_kernel<64, 128, 128, true, false>"
KDA_DECODE = "kda::decode_step_kernel<128, 128, true, 0>"
GDN_DECODE = "kda::decode_step_kernel<128, 128, true, 1>"
LAYER_INTRA = "kda::intra_wide_kernel<2>"
LAYER_STATE = "kda::layer_state_kernel"
LAYER_DECODE = "kda::decode_step_kernel<128, 128, true, 2>"
DPLR_INTRA = "kda::dplr_intra_kernel<64, 128, true>"
DPLR_STATE = "kda::dplr_state_kernel<64, 128, 128, true>"
DPLR_DECODE = "kda::decode_step_kernel<128, 128, true, 3>"
LAUNCH_KERNELS = {
    "kda_chunk_fwd": (KDA_INTRA, STATE),
    "kda_decode_step": (KDA_DECODE,),
    "gdn_chunk_fwd": (GDN_INTRA, STATE),
    "gdn_decode_step": (GDN_DECODE,),
    "kda_layer_chunk_fwd": (LAYER_INTRA, LAYER_STATE),
    "kda_layer_decode_step": (LAYER_DECODE,),
    "kda_dplr_chunk_fwd": (DPLR_INTRA, DPLR_STATE),
    "kda_dplr_decode_step": (DPLR_DECODE,),
}


def _short(name):
    """Kernel name without return type, anonymous namespace and parameter list."""
    return name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def _kernel_rows(csv_path):
    import csv
    with open(csv_path) as f:
        return list(csv.DictReader(f))


def summarize_trace(d):
    """Markdown table of the library's kernels from rocprofv3 --stats output."""
    rows = _kernel_rows(os.path.join(d, "run_kernel_stats.csv"))
    print("| kernel | calls | total us | avg us | min us | max us |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        name = r["Name"]
        if "kda::" not in name:
            continue
        short = _short(name)
        print(f"| `{short}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
              f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")


def _last_dispatch_counters(d, counter):
    """{kernel name: value of `counter` (summed over instances) in its last dispatch}."""
    import glob
    (path,) = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    per = {}
    for r in _kernel_rows(path):
        if r["Counter_Name"] != counter:
            continue
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    last = {}
    for (disp, name), v in sorted(per.items()):
        last[name] = v
    return last


def _call_counters(d, counter):
    """`counter` summed over every dispatch of the library's kernels in a run
    that makes one C-ABI call (the backward: many dispatches per call)."""
    import glob
    (path,) = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    tot, n = 0.0, set()
    for r in _kernel_rows(path):
        if r["Counter_Name"] == counter and "kda::" in r["Kernel_Name"]:
            tot += float(r["Counter_Value"])
            n.add(int(r["Dispatch_Id"]))
    return tot, len(n)


def _counter_commands(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, mfma_dir, bwd_dirs=None):
    """The rocprofv3 runs (each counter in its own run; <repo> is the repository root and
    each run's output is the directory given here) and this summary's command line."""
    prof = "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} --output-format csv -d <repo>/{d} -o run -- " \
           "python3 <repo>/bench.py {a}"
    bench_args = "--steps 1 --warmup 0 --no-cpu-baseline --no-backward --no-configs"
    cmds = [prof.format(c="FETCH_SIZE", d=fetch_dir, a=bench_args),
            prof.format(c="WRITE_SIZE", d=write_dir, a=bench_args),
            prof.format(c="FETCH_SIZE", d=copy_fetch_dir, a="--only copy --steps 2"),
            prof.format(c="WRITE_SIZE", d=copy_write_dir, a="--only copy --steps 2")]
    if mfma_dir:
        cmds.append(prof.format(c="MfmaUtil", d=mfma_dir, a=bench_args))
    if bwd_dirs:
        cmds.append(prof.format(c="FETCH_SIZE", d=bwd_dirs[0], a="--only backward --steps 1 --warmup 0"))
        cmds.append(prof.format(c="WRITE_SIZE", d=bwd_dirs[1], a="--only backward --steps 1 --warmup 0"))
    dirs = [fetch_dir, write_dir, copy_fetch_dir, copy_write_dir] + ([mfma_dir] if mfma_dir else [])
    cmd = "python bench.py --summarize-counters " + " ".join(dirs)
    if bwd_dirs:
        cmd += " --backward-counters " + " ".join(bwd_dirs)
    cmds.append(cmd)
    return cmds


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, mfma_dir=None, bwd_dirs=None):
    fetch = _last_dispatch_counters(fetch_dir, "FETCH_SIZE")
    write = _last_dispatch_counters(write_dir, "WRITE_SIZE")
    cf = _last_dispatch_counters(copy_fetch_dir, "FETCH_SIZE")
    cw = _last_dispatch_counters(copy_write_dir, "WRITE_SIZE")
    copy_name = max(cf, key=cf.get)  # the calibration copy is the largest dispatch
    fetch_scale = COPY_BYTES / (cf[copy_name] * 1024.0)
    write_scale = COPY_BYTES / (cw[copy_name] * 1024.0)
    kernels = {}
    for name in sorted(set(fetch) | set(write)):
        if "kda::" not in name:
            continue
        short = _short(name)
        fb = fetch.get(name, 0.0) * 1024.0 * fetch_scale
        wb = write.get(name, 0.0) * 1024.0 * write_scale
        kernels[short] = {"fetch_kib_raw": fetch.get(name), "write_kib_raw": write.get(name),
                          "fetch_bytes": fb, "write_bytes": wb, "hbm_bytes": fb + wb}
    if mfma_dir:  # rocprofv3's MfmaUtil: matrix-core busy cycles / (GPU active cycles x SIMDs), percent
        util = _last_dispatch_counters(mfma_dir, "MfmaUtil")
        for name, v in util.items():
            if _short(name) in kernels:
                kernels[_short(name)]["mfma_busy_pct"] = v
    launches = {}
    for launch, names in LAUNCH_KERNELS.items():
        if all(n in kernels for n in names):
            launches[launch] = {"kernels": list(names),
                                "hbm_bytes": sum(kernels[n]["hbm_bytes"] for n in names)}
    if bwd_dirs:  # one kda_chunk_bwd call over the 1M-token workload: every dispatch summed
        bf, nf = _call_counters(bwd_dirs[0], "FETCH_SIZE")
        bw, nw = _call_counters(bwd_dirs[1], "WRITE_SIZE")
        launches["kda_chunk_bwd"] = {"kernels": "every dispatch of one call", "dispatches": nf,
                                     "fetch_bytes": bf * 1024.0 * fetch_scale,
                                     "write_bytes": bw * 1024.0 * write_scale,
                                     "hbm_bytes": bf * 1024.0 * fetch_scale + bw * 1024.0 * write_scale}
    rec = {"source_digest": source_digest(),
           "commands": _counter_commands(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, mfma_dir, bwd_dirs),
           "note": "per-launch bytes of the last dispatch of each kernel; each counter scaled by what it reads "
                   "for a plain device copy of copy_bytes (read once, written once)",
           "calibration": {"copy_bytes": COPY_BYTES, "copy_kernel": _short(copy_name),
                           "fetch_kib": cf[copy_name], "write_kib": cw[copy_name],
                           "fetch_scale": fetch_scale, "write_scale": write_scale},
           "kernels": kernels, "launches": launches}
    out = os.path.join(ROOT, "profiles", "traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def measured_mfma_busy(launch):
    """{kernel: rocprofv3 MfmaUtil percent} for the kernels of one C-ABI launch,
    from the committed counter summary when it matches the current kernel
    sources, else {}."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return {}
    names = rec.get("launches", {}).get(launch, {}).get("kernels", [])
    kern = rec.get("kernels", {})
    return {k: kern[k]["mfma_busy_pct"] for k in names if "mfma_busy_pct" in kern.get(k, {})}


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def backward_leg(torch, kda, pin, dev, C):
    """kda_chunk_bwd over all tokens of the long prefill inputs, with
    d_o ~ N(0, 1) and preallocated gradients and workspace (one segment's
    packages and states, and a checkpoint per segment: about 4.3 GB at 1M
    tokens).  Returns (call, T_B)."""
    T, H, Dk, Dv = pin["T"], pin["H"], pin["q"].shape[-1], pin["v"].shape[-1]
    T_B = T
    bq, bk, bv, bla, bbeta = (pin[n][:, :T_B] for n in ("q", "k", "v", "log_alpha", "beta"))
    bgen = torch.Generator(device=dev)
    bgen.manual_seed(4)
    b_do = torch.randn((1, T_B, H, Dv), generator=bgen, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    b_grads = (torch.empty((1, T_B, H, Dk), **f32), torch.empty((1, T_B, H, Dk), **f32),
               torch.empty((1, T_B, H, Dv), **f32), torch.empty((1, T_B, H, Dk), **f32),
               torch.empty((1, T_B, H), **f32), None)
    b_ws = torch.empty(kda.bwd_workspace_size(1, T_B, H, Dk, 0, torch.bfloat16, C), dtype=torch.uint8,
                       device=dev)

    def backward():
        kda.chunk_bwd(bq, bk, bv, bla, bbeta, b_do, None, None, None, C, grads=b_grads, workspace=b_ws)

    return backward, T_B


def dplr_leg(torch, kda, workloads, pin, dev, C):
    """kda_dplr_chunk_fwd over the long prefill inputs with low-rank vectors from
    workloads.dplr_vectors (made in 128k-token slices to bound the temporaries),
    preallocated output and workspace.  Returns (call, (a, b))."""
    T, H, D = pin["T"], pin["H"], pin["q"].shape[-1]
    a = torch.empty_like(pin["k"])
    b = torch.empty_like(pin["k"])
    step = 1 << 17
    for i, t0 in enumerate(range(0, T, step)):
        part = {n: pin[n][:, t0:t0 + step] for n in ("k", "beta", "log_alpha")}
        a[:, t0:t0 + step], b[:, t0:t0 + step] = workloads.dplr_vectors(part, seed=10 + i)
        del part
    o = torch.empty((1, T, H, D), dtype=torch.float32, device=dev)
    fs = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.dplr_workspace_size(1, T, H, D, 0, torch.bfloat16, C), dtype=torch.uint8, device=dev)

    def dplr():
        kda.dplr_chunk_fwd(pin["q"], pin["k"], pin["v"], a, b, pin["log_alpha"], None, None, C,
                           out=o, final_state=fs, workspace=ws)

    return dplr, (a, b)


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def _parity(got, ref):
    """max|got - ref| / RMS(ref) over the whole tensor (got: torch, ref: fp64 numpy)."""
    import numpy as np
    g = got.detach().to("cpu").double().numpy()
    return float(np.max(np.abs(g - ref)) / np.sqrt(np.mean(ref * ref)))


def config_legs(torch, kda, workloads, oracle, dev, steps, flush, threads):
    """The other workloads, each timed and checked against the oracle in full:
    the tiny fp32 case (a launch-latency figure), the 4096-token prefill, the
    packed varlen prefill and the decode workload; the oracle is timed on the
    same inputs on all host threads and on one.  Returns {name: record}."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    out = {}

    def prefill_record(name, inp, reps, flush_each, tau):
        q = inp["q"]
        B, T, H, Dk = q.shape
        Dv = inp["v"].shape[-1]
        N, C = inp["N"], inp["chunk"]
        bf = q.dtype == torch.bfloat16
        cu = inp["cu_seqlens"]
        o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
        fs = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, kda.workspace_size(B, T, H, Dk, Dv, 0 if cu is None else N, q.dtype, C)),
                         dtype=torch.uint8, device=dev)
        call = lambda: kda.chunk_fwd(q, inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["init_state"],
                                     cu, C, out=o, final_state=fs, workspace=ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            if flush_each:
                flush.zero_()
            e0, e1 = ev(), ev()
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        t = _median(ts)
        Ttot = B * T
        by = prefill_alg_bytes(Ttot, H, Dk, Dv, N, in_bytes=2 if bf else 4, init=inp["init_state"] is not None)
        fl = prefill_alg_flops(Ttot, H, Dk, Dv, C)
        # the oracle on the same inputs: all host threads, then one thread on head 0
        t0 = time.perf_counter()
        o_ref, s_ref = oracle.forward_native(q, inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                             inp["init_state"], cu, n_threads=threads)
        t_all = time.perf_counter() - t0
        s0 = None if inp["init_state"] is None else inp["init_state"][:, :1]
        t0 = time.perf_counter()
        oracle.forward_native(q, inp["k"], inp["v"], inp["log_alpha"], inp["beta"], s0, cu, heads=(0, 1),
                              n_threads=1)
        t_one = time.perf_counter() - t0
        rec = {"T": Ttot, "H": H, "d_k": Dk, "d_v": Dv, "chunk": C, "dtype": "bf16" if bf else "f32",
               "ms_median": t * 1e3, "ms_mean": sum(ts) / len(ts) * 1e3, "tokens_per_s": Ttot / t,
               "alg_bytes": by, "alg_flops": fl, "hbm_frac_algorithmic": by / t / HBM_PEAK,
               "mfma_frac_algorithmic": fl / t / BF16_PEAK,
               "parity": {"o": _parity(o, o_ref), "final_state": _parity(fs, s_ref), "tau": tau,
                          "scope": "every output and final state against the fp64 oracle"},
               "cpu_baseline": {"value": Ttot / t_all, "unit": "tokens/s", "cores": min(threads, N * H),
                                "kind": "oracle", "sample": f"the whole workload ({t_all:.2f} s wall)",
                                "value_1_thread": Ttot / t_one / H,
                                "sample_1_thread": f"head 0, every token, one thread ({t_one:.2f} s wall), "
                                                   f"scaled to H={H} tokens/s"}}
        return rec, call

    # tiny fp32 workload: T=64, H=1, d=16, 16-token chunks -- launch-bound
    tiny = workloads.make_prefill("tiny", dev, 0)
    rec, call = prefill_record("tiny", tiny, 200, False, 1e-4)
    n_calls = 1000
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_calls):
        call()
    torch.cuda.synchronize()
    rec["us_per_call_back_to_back"] = (time.perf_counter() - t0) / n_calls * 1e6
    rec["us_per_call_median"] = rec.pop("ms_median") * 1e3
    rec["us_per_call_mean"] = rec.pop("ms_mean") * 1e3
    rec["workload"] = "KDA tiny: B=1 T=64 H=1 d=16 chunk=16 fp32, zero initial state (HIP events around each call)"
    out["tiny"] = rec
    _step("tiny workload done")

    # the 4096-token prefill, 240 MB: fits in the 256 MB MALL, so each timed call
    # follows the cache flush
    pre = workloads.make_prefill("prefill", dev, 0)
    rec, _ = prefill_record("prefill", pre, steps, True, 2e-2)
    rec["workload"] = ("KDA prefill: B=1 T=4096 H=32 d=128 chunk=64 bf16, log_alpha=-softplus(N(0,1)+2), "
                       "initial state N(0,0.02^2); L2 and MALL flushed before each timed call")
    out["prefill"] = rec
    del pre
    _step("4096-token workload done")

    # the packed varlen prefill: 16 sequences, ragged lengths, 5% resets
    var = workloads.make_prefill("varlen", dev, 0)
    rec, _ = prefill_record("varlen", var, steps, True, 2e-2)
    rec["workload"] = ("KDA varlen: 16 packed sequences, lengths U[1,16384] (none a multiple of 64), H=32 d=128 "
                       "chunk=64 bf16, log_alpha=-softplus(N(0,1)), 5% full-token resets, zero initial states")
    rec["n_seqs"] = var["N"]
    out["varlen"] = rec
    del var
    _step("varlen workload done")

    # the decode workload in full: 64 steps on 256 x 32 states, against the
    # oracle (threaded over the states)
    din = workloads.make_decode("decode", dev, 0)
    dw = din["workload"]
    st = din["state"].clone()
    outs = [torch.empty((dw.N, dw.H, dw.Dv), dtype=torch.float32, device=dev) for _ in range(dw.steps)]
    for t in range(dw.steps):
        kda.decode_step(din["q"][t], din["k"][t], din["v"][t], din["log_alpha"][t], din["beta"][t], st, out=outs[t])
    torch.cuda.synchronize()
    import numpy as np
    st_ref = din["state"].detach().to("cpu").double().numpy()
    err_o, ss_o, n_o = 0.0, 0.0, 0
    t0 = time.perf_counter()
    for t in range(dw.steps):
        o_ref, st_ref = oracle.decode_step_native(din["q"][t], din["k"][t], din["v"][t], din["log_alpha"][t],
                                                  din["beta"][t], st_ref, n_threads=threads)
        g = outs[t].detach().to("cpu").double().numpy()
        err_o = max(err_o, float(np.max(np.abs(g - o_ref))))
        ss_o += float(np.sum(o_ref * o_ref))
        n_o += o_ref.size
    t_all = time.perf_counter() - t0
    sub = slice(0, 16)  # one thread: 16 sequences x 32 heads, 64 steps
    st1 = din["state"][sub].detach().to("cpu").double().numpy()
    t0 = time.perf_counter()
    for t in range(dw.steps):
        _, st1 = oracle.decode_step_native(din["q"][t][sub], din["k"][t][sub], din["v"][t][sub],
                                           din["log_alpha"][t][sub], din["beta"][t][sub], st1, n_threads=1)
    t_one = time.perf_counter() - t0
    out["decode"] = {
        "workload": "KDA decode: 256 seqs x 32 heads, 128x128 fp32 states N(0,0.02^2), 64 steps, bf16 tokens",
        "parity": {"o": err_o / np.sqrt(ss_o / n_o), "final_state": _parity(st, st_ref), "tau": 2e-2,
                   "scope": "every output of the 64 steps and every final state against the fp64 oracle"},
        "cpu_baseline": {"value": dw.N * dw.steps / t_all, "unit": "tokens/s (one token per sequence and step)",
                         "cores": threads, "kind": "oracle",
                         "sample": f"the whole workload, 8192 states x 64 steps ({t_all:.2f} s wall)",
                         "value_1_thread": 16 * dw.steps / t_one,
                         "sample_1_thread": f"16 sequences x 32 heads x 64 steps on one thread ({t_one:.2f} s wall)"},
    }
    del din, outs, st
    _step("decode workload done")
    return out


def context_legs(torch, kda, pin, o, fs, ws, C, steps, flush):
    """Prefill tokens/s at T = 65,536, 262,144 and 1,048,576 (prefixes of the
    long workload, flushed before each call), and one decode step of the 32
    heads continuing from each prefill's final state: the per-token cost of a
    linear-time recurrence with a fixed-size state does not grow with T."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    H = pin["H"]
    rec = {"prefill": [], "decode_step_after_prefill": []}
    Ts = [t for t in (1 << 16, 1 << 18, 1 << 20) if t <= pin["T"]]
    od = torch.empty((1, H, o.shape[-1]), dtype=torch.float32, device=dev_of(o))
    for T in Ts:
        args = [pin[n][:, :T] for n in ("q", "k", "v", "log_alpha", "beta")]
        oo = o[:, :T]
        call = lambda: kda.chunk_fwd(*args, None, None, C, out=oo, final_state=fs, workspace=ws)
        call()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(3, steps // 2)):
            flush.zero_()
            e0, e1 = ev(), ev()
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        t = _median(ts)
        rec["prefill"].append({"T": T, "ms_median": t * 1e3, "tokens_per_s": T / t})
        # decode steps continuing this sequence (token T from the inputs' next row)
        nt = T % pin["T"]
        tok = [pin[n][0, nt:nt + 1].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")]
        st = fs.clone()
        for _ in range(3):
            kda.decode_step(*tok, st, out=od)
        ds = []
        for _ in range(20):
            e0, e1 = ev(), ev()
            e0.record(stream)
            kda.decode_step(*tok, st, out=od)
            e1.record(stream)
            torch.cuda.synchronize()
            ds.append(e0.elapsed_time(e1) * 1e3)
        rec["decode_step_after_prefill"].append({"context_T": T, "us_per_step_median": _median(ds)})
    rec["note"] = ("decode steps here are one sequence x 32 heads (2 MiB of state): launch-bound, "
                   "the figure shows no dependence on the context length")
    return rec


_T0 = time.perf_counter()


def _step(msg):
    """One progress line on stderr as each leg of the run ends."""
    print(f"[bench {time.perf_counter() - _T0:7.1f} s] {msg}", file=sys.stderr, flush=True)


def dev_of(t):
    return t.device


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward leg (the forward profiles use this: the backward's own "
                         "forward pass runs the same kernels at another size)")
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--chunk", type=int, default=None, help="prefill chunk size (default: the workload's)")
    ap.add_argument("--no-dplr", action="store_true", help="skip the general DPLR prefill leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload legs (tiny, 4096-token, varlen, decode) and the T sweep")
    ap.add_argument("--only", choices=["prefill", "decode", "copy", "backward", "dplr"], default=None,
                    help="run one part only (for profilers); prints no JSON line")
    ap.add_argument("--workload", choices=["long", "prefill", "varlen", "tiny"], default="long",
                    help="with --only prefill: the prefill workload to run (default: the 1M-token one)")
    ap.add_argument("--summarize-trace", metavar="DIR", default=None)
    ap.add_argument("--backward-counters", nargs=2, metavar="DIR", default=None,
                    help="with --summarize-counters: FETCH_DIR WRITE_DIR of one backward call")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR", default=None,
                    help="FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR [MFMA_UTIL_DIR]")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, bwd_dirs=args.backward_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the KDA operator here runs on a single "
              f"MI355X (got --gpus {args.gpus}); heads and sequences would shard across "
              f"GPUs with no communication, which this benchmark does not launch.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_55_amd import kda, workloads

    dev = "cuda:0"
    torch.cuda.set_device(0)
    lib = kda.load()

    if args.only == "copy":
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        return

    if args.only == "prefill" and args.workload != "long":
        # one of the smaller prefill workloads alone (a kernel trace per workload)
        pw = workloads.make_prefill(args.workload, dev, 0)
        wl = pw["workload"]
        ow = torch.empty(tuple(pw["q"].shape[:3]) + (wl.Dv,), dtype=torch.float32, device=dev)
        fw = torch.empty((pw["N"], wl.H, wl.Dk, wl.Dv), dtype=torch.float32, device=dev)
        for _ in range(args.warmup + args.steps):
            kda.chunk_fwd(pw["q"], pw["k"], pw["v"], pw["log_alpha"], pw["beta"], pw["init_state"],
                          pw["cu_seqlens"], wl.chunk, out=ow, final_state=fw)
        torch.cuda.synchronize()
        return

    # ---- inputs (seeded, synthetic, resident in HBM) ----------------------------
    pin = workloads.make_prefill("long", dev, 0)
    w = pin["workload"]
    T, H, Dk, Dv, C, N = pin["T"], w.H, w.Dk, w.Dv, (args.chunk or w.chunk), pin["N"]
    o = torch.empty((1, T, H, Dv), dtype=torch.float32, device=dev)
    fs = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    ws_bytes = kda.workspace_size(1, T, H, Dk, Dv, 0, torch.bfloat16, C)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    din = workloads.make_decode("decode", dev, 0)
    dw = din["workload"]
    dsteps = args.decode_steps or dw.steps
    state0 = din["state"]
    state = state0.clone()
    od = torch.empty((dw.N, dw.H, dw.Dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def prefill():
        kda.chunk_fwd(pin["q"], pin["k"], pin["v"], pin["log_alpha"], pin["beta"], None, None, C,
                      out=o, final_state=fs, workspace=ws)

    def decode(t):
        kda.decode_step(din["q"][t], din["k"][t], din["v"][t], din["log_alpha"][t],
                        din["beta"][t], state, out=od)

    if args.only == "dplr":
        del ws
        dplr, _ = dplr_leg(torch, kda, workloads, pin, dev, C)
        for _ in range(args.warmup + args.steps):
            dplr()
        torch.cuda.synchronize()
        return
    if args.only == "backward":
        backward, _ = backward_leg(torch, kda, pin, dev, C)
        for _ in range(args.warmup + args.steps):
            backward()
        torch.cuda.synchronize()
        return
    if args.only:
        for _ in range(args.warmup + args.steps):
            if args.only == "prefill":
                prefill()
            else:
                for t in range(dsteps):
                    decode(t)
        torch.cuda.synchronize()
        return

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def warm(prefill_fn, decode_fn):
        for _ in range(args.warmup):
            prefill_fn()
            for t in range(dsteps):
                decode_fn(t)
        torch.cuda.synchronize()

    # written before each timed prefill so that no input starts in L2 or the
    # 256 MB MALL (outside the timed region)
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def timed(prefill_fn, decode_fn):
        """K timed passes: per-call prefill ms and per-step decode ms (HIP events)."""
        pre, dec = [], []
        for _ in range(args.steps):
            flush.zero_()
            e0, e1 = ev(), ev()
            e0.record(stream)
            prefill_fn()
            e1.record(stream)
            de = [ev() for _ in range(dsteps + 1)]
            de[0].record(stream)
            for t in range(dsteps):
                decode_fn(t)
                de[t + 1].record(stream)
            torch.cuda.synchronize()
            pre.append(e0.elapsed_time(e1))
            dec.extend(de[t].elapsed_time(de[t + 1]) for t in range(dsteps))
        return pre, dec

    warm(prefill, decode)
    t_start = time.perf_counter()
    pre_ms, dec_ms = timed(prefill, decode)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    _step("1M-token prefill and decode timed")

    # the oracle on a sample of the same 1M-token workload: its time is the CPU
    # baseline, its outputs check the prefill just timed (o still holds them)
    long_cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        heads = (0, 16)
        T_s = 262144
        hostq = {n: pin[n][:, :T_s].detach().to("cpu") for n in ("q", "k", "v", "log_alpha", "beta")}
        t0 = time.perf_counter()
        o_ref, _ = oracle.forward_native(hostq["q"], hostq["k"], hostq["v"], hostq["log_alpha"], hostq["beta"],
                                         heads=heads, n_threads=threads)
        dt = time.perf_counter() - t0
        par = _parity(o[:, :T_s, heads[0]:heads[1]], o_ref)
        del o_ref
        T_1 = 65536
        t0 = time.perf_counter()
        oracle.forward_native(hostq["q"][:, :T_1], hostq["k"][:, :T_1], hostq["v"][:, :T_1],
                              hostq["log_alpha"][:, :T_1], hostq["beta"][:, :T_1], heads=(0, 1), n_threads=1)
        dt1 = time.perf_counter() - t0
        del hostq
        # the metric's unit is tokens/s at H=32: token-heads/s divided by 32
        long_cpu = {
            "value": T_s * (heads[1] - heads[0]) / dt / H,
            "unit": "tokens/s",
            "cores": min(threads, heads[1] - heads[0]),
            "kind": "oracle",
            "sample": f"fp64 token loop on heads 0-15 x first {T_s} tokens of the long "
                      f"prefill workload ({dt:.1f} s wall), scaled to H=32 tokens/s",
            "value_1_thread": T_1 / dt1 / H,
            "sample_1_thread": f"head 0 x first {T_1} tokens on one thread ({dt1:.1f} s wall), "
                               f"scaled to H=32 tokens/s",
            "host_cpu": host_cpu_model(),
            "host_threads": os.cpu_count(),
        }
        long_parity = {"o": par, "tau": 2e-2,
                       "scope": f"o of heads 0-15 over the first {T_s} tokens (the oracle sample above) of the "
                                f"timed call; every output is checked in the GPU tests"}

        _step("oracle sample of the 1M-token prefill done")

    ctx = None if args.no_configs else context_legs(torch, kda, pin, o, fs, ws, C, args.steps, flush)

    _step("context sweep done")
    # ---- Gated DeltaNet on the same tensors: one log gate per (token, head) ----
    gdn_la = workloads.scalar_log_alpha((1, T, H), w.shift, dev, seed=1)
    gdn_dla = workloads.scalar_log_alpha((dsteps, dw.N, dw.H), dw.shift, dev, seed=2)
    gstate = state0.clone()

    def gdn_prefill():
        kda.gdn_chunk_fwd(pin["q"], pin["k"], pin["v"], gdn_la, pin["beta"], None, None, C,
                          out=o, final_state=fs, workspace=ws)

    def gdn_decode(t):
        kda.gdn_decode_step(din["q"][t], din["k"][t], din["v"][t], gdn_dla[t],
                            din["beta"][t], gstate, out=od)

    warm(gdn_prefill, gdn_decode)
    g_pre_ms, g_dec_ms = timed(gdn_prefill, gdn_decode)
    del gdn_la, gdn_dla

    _step("Gated DeltaNet timed")
    # ---- the KDA layer: raw bf16 projections in, prologue and epilogue fused ----
    lg = torch.Generator(device=dev)
    lg.manual_seed(3)
    bfn = lambda shape, shift=0.0: (torch.randn(shape, generator=lg, device=dev) + shift).to(torch.bfloat16)
    l_xa = bfn((1, T, H, Dk), w.shift)
    l_xb = bfn((1, T, H))
    l_g = bfn((1, T, H, Dv))
    l_w = 0.5 + torch.rand((Dv,), generator=lg, device=dev)
    ld_xa = bfn((dsteps, dw.N, dw.H, dw.Dk), dw.shift)
    ld_xb = bfn((dsteps, dw.N, dw.H))
    ld_g = bfn((dsteps, dw.N, dw.H, dw.Dv))
    lstate = state0.clone()

    # the layer's workspace: the prefill's plus its row-norm exchange
    l_ws = torch.empty(kda.layer_workspace_size(1, T, H), dtype=torch.uint8, device=dev)

    def layer_prefill():
        kda.layer_chunk_fwd(pin["q"], pin["k"], pin["v"], l_xa, l_xb, l_g, l_w, 1e-6, 1e-5,
                            out=o, final_state=fs, workspace=l_ws)

    def layer_decode(t):
        kda.layer_decode_step(din["q"][t], din["k"][t], din["v"][t], ld_xa[t], ld_xb[t], ld_g[t], l_w,
                              lstate, 1e-6, 1e-5, out=od)

    warm(layer_prefill, layer_decode)
    l_pre_ms, l_dec_ms = timed(layer_prefill, layer_decode)
    del l_xa, l_xb, l_g, ld_xa, ld_xb, ld_g, l_ws

    _step("KDA layer timed")
    # ---- the general DPLR recurrence on the same q, k, v and gates (kda_dplr_chunk_fwd)
    d_ms = []
    if not args.no_dplr:
        dplr, d_bufs = dplr_leg(torch, kda, workloads, pin, dev, C)
        for _ in range(args.warmup):
            dplr()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            flush.zero_()
            e0, e1 = ev(), ev()
            e0.record(stream)
            dplr()
            e1.record(stream)
            torch.cuda.synchronize()
            d_ms.append(e0.elapsed_time(e1))
        del dplr
        # DPLR decode steps on the decode workload's states and tokens
        dg = torch.Generator(device=dev)
        dg.manual_seed(5)
        da, db_ = [], []
        for t in range(dsteps):
            kt = din["k"][t]
            da.append((-din["beta"][t][..., None] * kt.float()).to(kt.dtype))
            dub = kt.float() + 0.5 * torch.randn(kt.shape, generator=dg, device=dev)
            db_.append((torch.exp(din["log_alpha"][t]) * dub / torch.linalg.vector_norm(dub, dim=-1, keepdim=True))
                       .to(kt.dtype))
        del dub
        dstate = state0.clone()

        def dplr_decode(t):
            kda.dplr_decode_step(din["q"][t], din["k"][t], din["v"][t], da[t], db_[t], din["log_alpha"][t],
                                 dstate, out=od)

        for _ in range(args.warmup):
            for t in range(dsteps):
                dplr_decode(t)
        torch.cuda.synchronize()
        dd_ms = []
        for _ in range(args.steps):
            de = [ev() for _ in range(dsteps + 1)]
            de[0].record(stream)
            for t in range(dsteps):
                dplr_decode(t)
                de[t + 1].record(stream)
            torch.cuda.synchronize()
            dd_ms.extend(de[t].elapsed_time(de[t + 1]) for t in range(dsteps))
        del da, db_, dstate

    _step("DPLR timed")
    # ---- the backward (kda_chunk_bwd) over the same inputs (the forward's
    # workspace is no longer needed)
    del ws
    b_ms = []
    if not args.no_backward:
        backward, T_B = backward_leg(torch, kda, pin, dev, C)
        for _ in range(args.warmup):
            backward()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            flush.zero_()
            e0, e1 = ev(), ev()
            e0.record(stream)
            backward()
            e1.record(stream)
            torch.cuda.synchronize()
            b_ms.append(e0.elapsed_time(e1))
        del backward

    _step("backward timed")
    pre_ms.sort()
    dec_sorted = sorted(dec_ms)
    # medians of the timed calls and steps (means reported beside them)
    t_pre = pre_ms[len(pre_ms) // 2] / 1e3
    t_dec = dec_sorted[len(dec_sorted) // 2] / 1e3
    tok_s = T / t_pre
    pb = prefill_alg_bytes(T, H, Dk, Dv, N)
    pf = prefill_alg_flops(T, H, Dk, Dv, C)
    db = decode_alg_bytes(dw.N, dw.H, dw.Dk, dw.Dv)
    dec_gbs = db / t_dec / 1e9

    g_pre_ms.sort()
    g_dec_sorted = sorted(g_dec_ms)
    g_t_pre = g_pre_ms[len(g_pre_ms) // 2] / 1e3
    g_t_dec = g_dec_sorted[len(g_dec_sorted) // 2] / 1e3
    g_pb = prefill_alg_bytes(T, H, Dk, Dv, N, gate_per_head=1)
    g_db = decode_alg_bytes(dw.N, dw.H, dw.Dk, dw.Dv, gate_per_head=1)

    l_pre_ms.sort()
    l_dec_sorted = sorted(l_dec_ms)
    l_t_pre = l_pre_ms[len(l_pre_ms) // 2] / 1e3
    l_t_dec = l_dec_sorted[len(l_dec_sorted) // 2] / 1e3
    l_pb = layer_alg_bytes(T, H, Dk, Dv, N)
    l_db = layer_alg_bytes(dw.N, dw.H, dw.Dk, dw.Dv, dw.N, decode=True)  # one token per sequence

    result = {
        "metric": "KDA prefill tokens/s (H=32,d=128, T=1M) + decode step HBM GB/s, 1 MI355X",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "KDA long prefill B=1 T=1048576 H=32 d_k=d_v=128 chunk=64 bf16 q/k/v, "
                        "fp32 gates/state, log_alpha=-softplus(N(0,1)+3); then KDA decode "
                        "256 seqs x 32 heads x 128x128 fp32 state, 64 steps",
            "T": T, "H": H, "d_k": Dk, "d_v": Dv, "chunk": C,
            "decode_states": dw.N * dw.H, "decode_steps": dsteps,
        },
        "prefill": {
            "ms_mean": sum(pre_ms) / len(pre_ms), "ms_median": t_pre * 1e3,
            "tokens_per_s": tok_s,
            "hbm_frac_algorithmic": pb / t_pre / HBM_PEAK,
            "mfma_frac_algorithmic": pf / t_pre / BF16_PEAK,
            "mfma_busy_pct_counter": measured_mfma_busy("kda_chunk_fwd") or None,
            "mfma_busy_pct_counter_source": COUNTER_SOURCE,
            "alg_bytes": pb, "alg_flops": pf,
        },
        "decode": {
            "us_per_step_mean": sum(dec_ms) / len(dec_ms) * 1e3,
            "us_per_step_median": t_dec * 1e6,
            "GB_per_s": dec_gbs,
            "hbm_frac": db / t_dec / HBM_PEAK,
            "alg_bytes_per_step": db,
        },
        "roofline": {
            "kernel": "kda_chunk_fwd (intra_wide_kernel<0> + state_kernel<64,128,128,bf16>)",
            "bound": "hbm",
            "achieved": pb / t_pre / 1e9,
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": pb / t_pre / HBM_PEAK,
            "traffic": measured_traffic("kda_chunk_fwd"),
            "traffic_source": COUNTER_SOURCE,
        },
        "decode_roofline": {
            "kernel": "decode_step_kernel<128,128,bf16,0>",
            "bound": "hbm",
            "achieved": dec_gbs,
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": db / t_dec / HBM_PEAK,
            "traffic": measured_traffic("kda_decode_step"),
        },
    }

    result["gdn"] = {
        "workload": "Gated DeltaNet (one log gate per token and head, -softplus(N(0,1)+3)) on the "
                    "same q/k/v/beta tensors: gdn_chunk_fwd over the 1M-token prefill, then 64 "
                    "gdn_decode_step calls on 256 seqs x 32 heads",
        "prefill": {
            "ms_mean": sum(g_pre_ms) / len(g_pre_ms), "ms_median": g_t_pre * 1e3,
            "tokens_per_s": T / g_t_pre,
            "hbm_frac_algorithmic": g_pb / g_t_pre / HBM_PEAK,
            "mfma_frac_algorithmic": pf / g_t_pre / BF16_PEAK,
            "alg_bytes": g_pb, "alg_flops": pf,
            "roofline": {"kernel": "gdn_chunk_fwd (intra_wide_kernel<1> + state_kernel)",
                         "bound": "hbm", "achieved": g_pb / g_t_pre / 1e9,
                         "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": g_pb / g_t_pre / HBM_PEAK,
                         "traffic": measured_traffic("gdn_chunk_fwd")},
        },
        "decode": {
            "us_per_step_mean": sum(g_dec_ms) / len(g_dec_ms) * 1e3,
            "us_per_step_median": g_t_dec * 1e6,
            "GB_per_s": g_db / g_t_dec / 1e9,
            "hbm_frac": g_db / g_t_dec / HBM_PEAK,
            "alg_bytes_per_step": g_db,
            "traffic": measured_traffic("gdn_decode_step"),
        },
    }

    result["layer"] = {
        "workload": "KDA layer (kda_layer_chunk_fwd / kda_layer_decode_step): bf16 q, k, v as "
                    "above taken as raw projections, x_alpha ~ N(0,1)+3, x_beta, output gate ~ "
                    "N(0,1) bf16, RMSNorm weight U[0.5,1.5]; prologue (L2Norm, -softplus, sigmoid) "
                    "and epilogue (RMSNorm x weight x sigmoid gate) fused",
        "prefill": {
            "ms_mean": sum(l_pre_ms) / len(l_pre_ms), "ms_median": l_t_pre * 1e3,
            "tokens_per_s": T / l_t_pre,
            "hbm_frac_algorithmic": l_pb / l_t_pre / HBM_PEAK,
            "alg_bytes": l_pb,
            "roofline": {"kernel": "kda_layer_chunk_fwd (intra_wide_kernel<2> + layer_state_kernel)",
                         "bound": "hbm", "achieved": l_pb / l_t_pre / 1e9,
                         "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": l_pb / l_t_pre / HBM_PEAK,
                         "traffic": measured_traffic("kda_layer_chunk_fwd")},
        },
        "decode": {
            "us_per_step_mean": sum(l_dec_ms) / len(l_dec_ms) * 1e3,
            "us_per_step_median": l_t_dec * 1e6,
            "GB_per_s": l_db / l_t_dec / 1e9,
            "hbm_frac": l_db / l_t_dec / HBM_PEAK,
            "alg_bytes_per_step": l_db,
            "traffic": measured_traffic("kda_layer_decode_step"),
        },
    }

    if d_ms:
        d_ms.sort()
        d_t = d_ms[len(d_ms) // 2] / 1e3
        d_bytes = dplr_alg_bytes(T, H, Dk, N)
        result["dplr"] = {
            "workload": "kda_dplr_chunk_fwd, S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T, over the "
                        "same 1M-token q, k, v and log_alpha (H=32, d=128, chunk 64, bf16), a = -beta * k, "
                        "b = alpha * unit(k + 0.5 N(0,1)) in bf16",
            "ms_mean": sum(d_ms) / len(d_ms), "ms_median": d_t * 1e3,
            "tokens_per_s": T / d_t,
            "time_vs_kda_prefill": d_t / t_pre,
            "alg_bytes": d_bytes,
            "hbm_frac_algorithmic": d_bytes / d_t / HBM_PEAK,
            "roofline": {"kernel": "kda_dplr_chunk_fwd (dplr_intra_kernel + dplr_state_kernel)",
                         "bound": "hbm", "achieved": d_bytes / d_t / 1e9, "peak": HBM_PEAK / 1e9,
                         "unit": "GB/s", "frac": d_bytes / d_t / HBM_PEAK,
                         "traffic": measured_traffic("kda_dplr_chunk_fwd")},
        }
        dd_ms.sort()
        dd_t = dd_ms[len(dd_ms) // 2] / 1e3
        dd_bytes = dplr_decode_alg_bytes(dw.N, dw.H, dw.Dk)
        result["dplr"]["decode"] = {
            "workload": "kda_dplr_decode_step on the decode workload's 256 x 32 fp32 states and tokens, 64 "
                        "consecutive steps, a = -beta * k, b = alpha * unit(k + 0.5 N(0,1)) (bf16)",
            "us_per_step_mean": sum(dd_ms) / len(dd_ms) * 1e3, "us_per_step_median": dd_t * 1e6,
            "GB_per_s": dd_bytes / dd_t / 1e9, "hbm_frac": dd_bytes / dd_t / HBM_PEAK,
            "alg_bytes_per_step": dd_bytes,
            "traffic": measured_traffic("kda_dplr_decode_step"),
        }
        if not args.no_cpu_baseline:
            import oracle
            threads = max(1, min(16, os.cpu_count() or 1))
            heads, T_s = list(range(16)), 131072
            sl = lambda x: x[:, :T_s, heads].detach().to("cpu").double().numpy()
            args_d = [sl(pin[n]) for n in ("q", "k", "v")] + [sl(x) for x in d_bufs] + [sl(pin["log_alpha"])]
            t0 = time.perf_counter()
            oracle.dplr_forward(*args_d, n_threads=threads)
            dtd = time.perf_counter() - t0
            result["dplr"]["cpu_baseline"] = {
                "value": T_s * len(heads) / dtd / H, "unit": "tokens/s", "cores": min(threads, len(heads)),
                "kind": "oracle",
                "sample": f"fp64 DPLR token loop on heads 0-15 x first {T_s} tokens of the same inputs "
                          f"({dtd:.1f} s wall), scaled to H=32 tokens/s"}
        del d_bufs

    if b_ms:
        b_ms.sort()
        b_t = b_ms[len(b_ms) // 2] / 1e3
        b_bytes = backward_alg_bytes(T_B, H, Dk, Dv)
        result["backward"] = {
            "workload": f"kda_chunk_bwd over the {T_B} tokens of the long prefill workload (H=32, "
                        f"d=128, chunk 64, bf16 q/k/v, fp32 gates), d_o ~ N(0,1) fp32, no initial or "
                        f"final state: gradients of q, k, v, log_alpha and beta (fp32)",
            "T": T_B,
            "ms_mean": sum(b_ms) / len(b_ms), "ms_median": b_t * 1e3,
            "tokens_per_s": T_B / b_t,
            "alg_bytes": b_bytes,
            "hbm_frac_algorithmic": b_bytes / b_t / HBM_PEAK,
            "roofline": {"kernel": "kda_chunk_bwd (segment checkpoints, then per segment: packages and "
                                   "saved states recomputed, bwd_state_kernel, intra_bwd_kernel)",
                         "bound": "hbm", "achieved": b_bytes / b_t / 1e9, "peak": HBM_PEAK / 1e9,
                         "unit": "GB/s", "frac": b_bytes / b_t / HBM_PEAK,
                         "traffic": measured_traffic("kda_chunk_bwd")},
        }

    if b_ms and not args.no_cpu_baseline:
        import numpy as np
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        heads, T_s = list(range(16)), 16384
        sl = lambda x: x[:, :T_s, heads].detach().to("cpu").double().numpy()
        args_b = [sl(pin[k]) for k in ("q", "k", "v", "log_alpha", "beta")]
        d_o_s = np.random.default_rng(4).standard_normal(args_b[2].shape)
        t0 = time.perf_counter()
        oracle.backward(*args_b, d_o=d_o_s, n_threads=threads)
        dtb = time.perf_counter() - t0
        result["backward"]["cpu_baseline"] = {
            "value": T_s * len(heads) / dtb / H, "unit": "tokens/s", "cores": min(threads, len(heads)),
            "kind": "oracle",
            "sample": f"fp64 reverse-mode token loop on heads 0-15 x first {T_s} tokens of the long prefill "
                      f"workload ({dtb:.1f} s wall), scaled to H=32 tokens/s"}

    if long_cpu is not None:
        result["cpu_baseline"] = long_cpu
        result["prefill"]["parity"] = long_parity
    if ctx is not None:
        result["context_sweep"] = ctx
    if not args.no_configs:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        result["configs"] = config_legs(torch, kda, workloads, oracle, dev, args.steps, flush, threads)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
