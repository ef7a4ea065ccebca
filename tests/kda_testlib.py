"""Helpers shared by the GPU parity tests: tolerance checks against the oracle
and host copies of device tensors.  The tolerances are the operator's parity
bar: max|gpu - oracle| <= tau * RMS(oracle) over the whole tensor, with
tau = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs, for o and for states."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

TAU = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def log(msg: str):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def host64(x):
    return x.detach().to("cpu").double().numpy()


def rel_err(got, ref) -> float:
    """max|got - ref| / RMS(ref) (got: torch or numpy, ref: numpy fp64)."""
    g = host64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if not np.all(np.isfinite(g)):
        return float("inf")
    rms = float(np.sqrt(np.mean(r * r)))
    err = float(np.max(np.abs(g - r))) if g.size else 0.0
    if rms == 0.0:
        return 0.0 if err == 0.0 else float("inf")
    return err / rms


def assert_parity(got, ref, tau, what):
    e = rel_err(got, ref)
    log(f"  {what}: max|err|/RMS = {e:.3e} (bound {tau:g})")
    assert e <= tau, f"{what}: max|err|/RMS = {e:.3e} exceeds {tau:g}"
    return e


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


class StreamingParity:
    """max|got - ref| / RMS(ref) over a whole tensor that is compared piece by
    piece (a head or a step at a time), so neither side is ever held whole in
    fp64: a running max|err| and sum of ref^2 over every element."""

    def __init__(self, what: str):
        self.what = what
        self.err = 0.0
        self.ss = 0.0
        self.n = 0
        self.finite = True

    def add(self, got, ref):
        g = host64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
        r = np.asarray(ref, np.float64)
        assert g.shape == r.shape, (g.shape, r.shape)
        if g.size == 0:
            return
        if not np.all(np.isfinite(g)):
            self.finite = False
        self.err = max(self.err, float(np.max(np.abs(g - r))))
        self.ss += float(np.sum(r * r))
        self.n += r.size

    def check(self, tau) -> float:
        rms = float(np.sqrt(self.ss / max(self.n, 1)))
        e = float("inf") if not self.finite else (self.err / rms if rms > 0 else (0.0 if self.err == 0 else float("inf")))
        log(f"  {self.what}: max|err|/RMS = {e:.3e} over {self.n} values (bound {tau:g})")
        assert e <= tau, f"{self.what}: max|err|/RMS = {e:.3e} exceeds {tau:g}"
        return e
