"""GPU parity of the single-pass prefill (bf16 inputs, dk = dv = 128: the chunk-local work and the
recurrence in one kernel) against the fp64 oracle, for every workgroup shape it has, and against
the two-kernel path (kda_chunk_local + kda_inter_chunk) on the same inputs; the K3 layer through
kda_prefill on every head.  Outputs start as NaN so unwritten rows cannot pass."""
import numpy as np
import pytest
import torch

import gated_delta_rule_51_amd as kda
import workloads
from parity import TOL, assert_close, oracle_prefill, rel_err, say

pytestmark = pytest.mark.gpu

RAGGED = [17, 0, 1, 33, 100, 16, 15, 48, 49]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


def _nan(shape, dev):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=dev)


def _fused(dev, x, nseq, H, init=None, shape=(0, 0)):
    N = x["q"].shape[0]
    o, fin = _nan((N, H, 128), dev), _nan((nseq, H, 128, 128), dev)
    kda.kda_prefill_single_pass(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], init,
                                consumers=shape[0], slices=shape[1], o=o, final_state=fin)
    return o, fin


def _two_kernel(dev, x, nseq, H, init=None):
    N = x["q"].shape[0]
    ws = kda.alloc_workspace(N, nseq, H, 128, 128, torch.bfloat16, dev)
    kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
    return kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws, init)


@pytest.mark.parametrize("H,shape", [(2, (2, 1)), (8, (4, 1)), (32, (4, 2)), (32, (0, 0))],
                         ids=["2x1", "4x1", "4x2", "chosen"])
def test_fused_shapes_ragged_against_oracle(dev, H, shape):
    """Empty, one-token, exact-chunk and ragged sequences with an initial state, through every
    workgroup shape of the single-pass kernel (2 consumers of one 16-column slice, 4 of one,
    4 of two) and the shape it chooses itself."""
    seqlens = RAGGED
    w = workloads.custom(seqlens, H, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=H)
    init = workloads.random_state(len(seqlens), H, 128, 128, device=dev, seed=H)
    say(f"  case: single pass H={H} chains={H * len(seqlens)} shape={shape}")
    o, fin = _fused(dev, x, len(seqlens), H, init, shape)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(x, init)
    assert_close(o, o_ref, TOL[torch.bfloat16], "o")
    assert_close(fin, f_ref, TOL[torch.bfloat16], "final_state")
    o2, f2 = _two_kernel(dev, x, len(seqlens), H, init)
    torch.cuda.synchronize()
    # the two paths differ only in rounding order (the inverse, the operand splits)
    assert rel_err(o, o2) <= 2e-3 and rel_err(fin, f2) <= 2e-3


def test_fused_gate_and_beta_extremes(dev):
    """g at the -5 floor and at 0, beta exactly 0 and 1, through the single-pass kernel."""
    seqlens, H = [64, 37, 130], 4
    w = workloads.custom(seqlens, H, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=9)
    g, b = x["log_alpha"], x["beta"]
    g[0::3] = -5.0
    g[1::5] = 0.0
    b[0::4] = 0.0
    b[1::4] = 1.0
    o, fin = _fused(dev, x, len(seqlens), H)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(x)
    assert_close(o, o_ref, TOL[torch.bfloat16], "o")
    assert_close(fin, f_ref, TOL[torch.bfloat16], "final_state")


def test_fused_strong_decay(dev):
    """Log-decay uniform on [-5, 0): 16-token cumulative decays down to -80, the range the
    bounded-decay argument allows (e^{-G} up to e^80 in the key operands)."""
    seqlens, H = [200, 77], 4
    w = workloads.custom(seqlens, H, 128, 128, torch.bfloat16, gate="uniform")
    x = workloads.prefill_inputs(w, device=dev, seed=5)
    o, fin = _fused(dev, x, len(seqlens), H)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(x)
    assert_close(o, o_ref, TOL[torch.bfloat16], "o")
    assert_close(fin, f_ref, TOL[torch.bfloat16], "final_state")


def test_fused_final_state_may_alias_initial_state(dev):
    seqlens, H = [50, 20], 2
    w = workloads.custom(seqlens, H, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=4)
    init = workloads.random_state(2, H, 128, 128, device=dev, seed=4)
    o_ref, f_ref = oracle_prefill(x, init)
    st = init.clone()
    kda.kda_prefill_single_pass(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], st,
                                final_state=st)
    torch.cuda.synchronize()
    assert_close(st, f_ref, TOL[torch.bfloat16], "final_state (in place)")


def test_fused_is_deterministic(dev):
    w = workloads.custom([300, 1000, 7], 16, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=8)
    a = _fused(dev, x, 3, 16)
    b = _fused(dev, x, 3, 16)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_workload3_k3_layer_every_head(dev):
    """B=1, H=96, T=65,536 through kda_prefill (the path it chooses for this shape), every head
    against the oracle (in groups of 16 heads to bound host memory)."""
    w = workloads.workload(3)
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    say(f"  case: K3 layer, all {w.H} heads")
    o = _nan((w.total_tokens, w.H, 128), dev)
    fin = _nan((1, w.H, 128, 128), dev)
    kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], o=o, final_state=fin)
    torch.cuda.synchronize()
    err_o = err_f = 0.0
    ss_o = ss_f = 0.0
    for h0 in range(0, w.H, 16):
        hs = list(range(h0, h0 + 16))
        o_ref, f_ref = oracle_prefill(x, heads=hs)
        go = o[:, hs].double().cpu().numpy()
        gf = fin[:, hs].double().cpu().numpy()
        assert np.all(np.isfinite(go)) and np.all(np.isfinite(gf))
        err_o = max(err_o, float(np.max(np.abs(go - o_ref))))
        err_f = max(err_f, float(np.max(np.abs(gf - f_ref))))
        ss_o += float(np.sum(o_ref * o_ref))
        ss_f += float(np.sum(f_ref * f_ref))
    eo = err_o / (ss_o / o.numel()) ** 0.5
    ef = err_f / (ss_f / fin.numel()) ** 0.5
    say(f"    o: max|err|/rms = {eo:.3e}; final_state: {ef:.3e} (tol 1e-2)")
    assert eo <= TOL[torch.bfloat16] and ef <= TOL[torch.bfloat16]
    del x, o, fin
    torch.cuda.empty_cache()
