"""The benchmark's roofline arithmetic, on the CPU: the per-token-head byte and flop counts and the
bounds reported beside each prefill time, checked against values worked out by hand from the
definitions (algorithmic bytes: q, k, v, log-decay, beta read once in bf16 and o written once in
fp32; flops: the three dk x dv products per token, the triangular tile halves and the decay)."""
import math
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_bytes_and_flops_per_token_head():
    # 2 * (3 * 128 + 128 + 1) + 4 * 128 = 1,026 + 512
    assert bench.prefill_bytes_per_token_head(128, 128) == 1538
    # 6 * 128 * 128 + 16 * (3 * 128 + 2 * 128) + 2 * 128 * 128 / 16 = 98,304 + 10,240 + 2,048
    assert bench.prefill_flops_per_token_head(128, 128) == 110592
    # decode: the fp32 state read and written, one token's inputs, o
    assert bench.decode_bytes_per_head(128, 128) == 2 * 128 * 128 * 4 + 1026 + 512
    assert bench.window_bytes_per_head(128, 128, 4) == 2 * 128 * 128 * 4 + 4 * 1538


def test_bounds_of_the_varlen_workload():
    th = 1048576 * 96
    flops = th * bench.prefill_flops_per_token_head(128, 128)
    alg = th * bench.prefill_bytes_per_token_head(128, 128) + 27 * 96 * 128 * 128 * 4
    seqlens = [40000] * 26 + [1048576 - 26 * 40000]
    b = bench.bound_fields(flops, alg, 56.0, seqlens, 96)
    assert b["t_hbm_ms"] == pytest.approx(alg / 8e12 * 1e3)
    assert b["t_mfma_ms"] == pytest.approx(flops / 2.5e15 * 1e3)
    assert b["active_bound"] == "hbm"  # AI ~ 72 flop/B, below the ~312 flop/B ridge
    ai = flops / alg
    assert 70 < ai < 73
    assert b["attainable_tflops"] == pytest.approx(ai * 8.0)
    # below the ridge the attainable fraction is the HBM fraction
    assert b["attainable_frac"] == pytest.approx(alg / (56.0e-3) / 8e12)
    assert b["time_over_bound"] == pytest.approx(56.0 / b["t_hbm_ms"])
    assert b["longest_chain_steps"] == 2500  # the 40,000-token sequences (the last holds 8,576)
    steps = (26 * math.ceil(40000 / 16) + math.ceil((1048576 - 26 * 40000) / 16)) * 96 / 256
    assert b["chain_steps_per_cu"] == pytest.approx(steps)
    assert b["ns_per_chain_step_per_cu"] == pytest.approx(56.0e6 / steps)


def test_bounds_above_the_ridge_and_with_empty_sequences():
    # an intensity above the ridge binds on the matrix cores
    b = bench.bound_fields(1e15, 1e12, 1.0, [64], 1)
    assert b["active_bound"] == "mfma" and b["attainable_tflops"] == bench.MFMA_BF16_PEAK_TFLOPS
    # empty sequences keep every field finite
    b = bench.bound_fields(1e9, 1e9, 1.0, [0, 0], 1)
    assert all(math.isfinite(v) for v in b.values() if isinstance(v, float))
