"""The benchmark's algorithmic-work formulas against the per-token counts they
are built from (host only; no GPU)."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(spec)
spec.loader.exec_module(bench)

T, H, D = 1 << 20, 32, 128


def test_prefill_bytes_and_flops():
    # bf16 q, k, v (2 B each element), fp32 log_alpha per channel, fp32 beta, fp32 o
    per = 2 * (2 * D + D) + 4 * D + 4 + 4 * D
    assert per == 1796
    assert bench.prefill_alg_bytes(T, H, D, D, 1) == T * H * per + H * D * D * 4
    assert abs(bench.prefill_alg_bytes(T, H, D, D, 1) / 1e9 - 60.27) < 0.01
    # one gate per token and head for GDN
    assert bench.prefill_alg_bytes(T, H, D, D, 1, gate_per_head=1) == T * H * (per - 4 * D + 4) + H * D * D * 4
    flops = bench.prefill_alg_flops(T, H, D, D, 64)
    assert flops == T * H * (6 * D * D + 64 * 5 * D + 64 * 64 / 3)


def test_decode_bytes():
    # the state read and written once per head, plus the token's tensors
    per = 8 * D * D + 2 * 3 * D + 4 * D + 4 + 4 * D
    assert bench.decode_alg_bytes(256, 32, D, D) == 256 * 32 * per
    assert abs(bench.decode_alg_bytes(256, 32, D, D) / 1e9 - 1.0885) < 1e-4
    assert bench.dplr_decode_alg_bytes(256, 32, D) == 256 * 32 * (8 * D * D + 5 * 2 * D + 8 * D)


def test_dplr_and_backward_bytes():
    assert bench.dplr_alg_bytes(T, H, D, 1) == T * H * (5 * 2 * D + 8 * D) + H * D * D * 4
    Tb = 1 << 18
    read = 2 * 3 * D + 4 * D + 4 + 4 * D
    write = 4 * 4 * D + 4
    assert bench.backward_alg_bytes(Tb, H, D, D) == Tb * H * (read + write)
    assert abs(bench.backward_alg_bytes(Tb, H, D, D) / 1e9 - 32.3) < 0.1
