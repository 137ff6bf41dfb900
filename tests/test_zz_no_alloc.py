"""kda_prefill_noalloc (the prefill for callers that cannot allocate: its workspace is the
library's static per-device scratch) against kda_prefill on the same inputs, through the C ABI:
two calls in a row, the second on a smaller input, so the second call runs on scratch the first
one left behind.  (bf16 with dk = dv = 128 runs in one kernel that needs no workspace; the other
shapes use the scratch.)  Both go through the same kernels, so the results must match bit for bit (which
is inside the oracle bar the prefill itself is tested to)."""
import pytest
import torch

import gated_delta_rule_51_amd as kda
import workloads
from parity import TOL, assert_close, oracle_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


def _run_both(dev, seqlens, H, d, dtype, seed, init):
    w = workloads.custom(seqlens, H, d, d, dtype)
    x = workloads.prefill_inputs(w, device=dev, seed=seed)
    s0 = workloads.random_state(len(seqlens), H, d, d, device=dev, seed=seed) if init else None
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], s0)
    nan = lambda shape: torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    o1, f1 = nan((w.total_tokens, H, d)), nan((len(seqlens), H, d, d))
    kda.kda_prefill_noalloc(*args, o=o1, final_state=f1)
    o2, f2 = kda.kda_prefill(*args)
    torch.cuda.synchronize()
    print(f"  case: seqlens={seqlens} H={H} d={d} {dtype} init={init}", flush=True)
    assert torch.equal(o1, o2), "o differs from kda_prefill"
    assert torch.equal(f1, f2), "final state differs from kda_prefill"
    return x, s0, o1, f1


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 16)])
def test_noalloc_matches_prefill_twice(dev, dtype, d):
    # first call: 3 sequences, ragged; second: smaller, on the scratch the first one left
    x, s0, o, f = _run_both(dev, [1000, 37, 517], 8, d, dtype, seed=1, init=True)
    o_ref, f_ref = oracle_prefill(x, s0)
    assert_close(o, o_ref, TOL[dtype], "o (first call) vs oracle")
    assert_close(f, f_ref, TOL[dtype], "final_state (first call) vs oracle")
    _run_both(dev, [70, 5], 3, d, dtype, seed=2, init=False)


def test_noalloc_rejects_problems_above_the_scratch(dev):
    # (floor(N/16) + nseq) * H slot-heads of 2 KiB: 65,536 fit in 128 MiB (a shape that runs the
    # two phases; bf16 with dk = dv = 128 runs in one kernel and needs no workspace)
    H, d = 64, 64
    ok_tokens = 16 * (65536 // H - 1)
    too_many = ok_tokens + 32
    w = workloads.custom([too_many], H, d, d, torch.bfloat16)
    assert kda.kda_prefill_workspace_bytes(too_many, 1, H, d, d) > (128 << 20)
    assert kda.kda_prefill_workspace_bytes(ok_tokens, 1, H, d, d) <= (128 << 20)
    x = workloads.prefill_inputs(w, device=dev, seed=3)
    o = torch.full((too_many, H, d), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(kda.KDAError) as ei:
        kda.kda_prefill_noalloc(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], o=o)
    assert ei.value.code == 7
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)
