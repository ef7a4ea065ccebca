"""Regenerates the operand-precision table of the prefill kernels' design.

Not a test (run it by hand: ``python tests/precision_table.py [--quick]``).
Each row emulates, with ``chunk_model.chunk_forward``'s ``rnd`` hooks, the
operand precision of every matrix product of the chunked prefill and reports
max|o - o_oracle| / RMS(o_oracle) and the same for the final state, against
the fp64 token-loop oracle on the same bf16 inputs.  Workloads are scaled-down
versions of the bf16 workloads (same gates, head dim 128, 64-token chunks):
  prefill  log_alpha = -softplus(N(0,1) + 2), random initial state
  slow     log_alpha = logsigmoid(N(0,1) + 2) (mean alpha ~ 0.85: long memory)
  long     log_alpha = -softplus(N(0,1) + 3), a longer sequence
  varlen   log_alpha = -softplus(N(0,1)), 5% full-token resets, ragged lengths
"""
from __future__ import annotations

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
from chunk_model import chunk_forward, product, to_bf16  # noqa: E402


def workload(name, T, H, seed=0):
    rng = np.random.default_rng(seed)
    d = 128
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = to_bf16(unit(rng.standard_normal((1, T, H, d))))
    k = to_bf16(unit(rng.standard_normal((1, T, H, d))))
    v = to_bf16(rng.standard_normal((1, T, H, d)))
    x = rng.standard_normal((1, T, H, d))
    be = (1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, H))))).astype(np.float32).astype(np.float64)
    s0, cu = None, None
    if name == "prefill":
        la = -np.log1p(np.exp(x + 2.0))
        s0 = 0.02 * rng.standard_normal((1, H, d, d))
    elif name == "slow":
        la = -np.log1p(np.exp(-(x + 2.0)))
        s0 = 0.02 * rng.standard_normal((1, H, d, d))
    elif name == "long":
        la = -np.log1p(np.exp(x + 3.0))
    else:
        la = -np.log1p(np.exp(x))
        la[:, rng.random(T) < 0.05] = -np.inf
        cuts = np.sort(rng.choice(np.arange(1, T), 5, replace=False))
        cu = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    la = la.astype(np.float32).astype(np.float64)
    return q, k, v, la, be, s0, cu


# the bf16 path of the kernels: Gram tiles on the diagonal bf16 hi/lo (three
# products), below it plain fp16; WY and fold products bf16 hi/lo; [W; Q'] S
# fp16; Kt fp16 against U fp16 hi/lo
KERNEL = {"APd": product("bf16x3"), "APo": product("f16"), "WU": product("bf16x3"), "QW": product("bf16x3"),
          "WS": product("f16"), "QS": product("f16"), "KU": product("f16x2R")}

ROWS = [
    ("all bf16", {g: product("bf16") for g in ("AP", "WU", "QW", "WS", "QS", "KU")}),
    ("kernel", KERNEL),
    ("kernel with every Gram tile bf16 hi/lo", dict(KERNEL, APo=product("bf16x3"))),
    ("kernel, Gram tiles below the diagonal plain bf16", dict(KERNEL, APo=product("bf16"))),
    ("kernel, WY plain fp16", dict(KERNEL, WU=product("f16"))),
    ("kernel, fold products plain fp16", dict(KERNEL, QW=product("f16"))),
    ("kernel, Kt U plain fp16", dict(KERNEL, KU=product("f16"))),
    ("kernel, Kt U fp16 hi/lo both", dict(KERNEL, KU=product("f16x3"))),
    ("all fp32", {g: product("f32") for g in ("AP", "WU", "QW", "WS", "QS", "KU")}),
]


def rel(a, b):
    return float(np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b)))


def main(quick=False):
    sizes = {"prefill": (2048, 2), "slow": (2048, 2), "long": (8192, 1), "varlen": (4096, 2)}
    if quick:
        sizes = {k: (T // 4, 1) for k, (T, H) in sizes.items()}
    data = {n: workload(n, *sizes[n]) for n in sizes}
    refs = {n: oracle.forward(q, k, v, la, be, s0, cu) for n, (q, k, v, la, be, s0, cu) in data.items()}
    print("| operands | " + " | ".join(f"{n} o / S" for n in data) + " |")
    print("|---|" + "---|" * len(data))
    for label, rnd in ROWS:
        cells = []
        for n, (q, k, v, la, be, s0, cu) in data.items():
            o, s = chunk_forward(q, k, v, la, be, s0, cu, 64, rnd=rnd, fold=True)
            cells.append(f"{rel(o, refs[n][0]):.1e} / {rel(s, refs[n][1]):.1e}")
        print(f"| {label} | " + " | ".join(cells) + " |", flush=True)


if __name__ == "__main__":
    main("--quick" in sys.argv)
