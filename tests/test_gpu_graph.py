"""HIP graph replay of the benchmark's step (kda_chunk_local, kda_inter_chunk, then one
kda_decode_step from the final states), through the C ABI: the three launches captured once
with torch's graph capture and replayed several times, with eager launches of the same step
on other inputs and host synchronisations between the replays.  Every replay must reproduce
the eager outputs bit for bit (the kernels are deterministic and the library records only
kernel launches)."""
import pytest
import torch

import gated_delta_rule_51_amd as kda
import workloads
from parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


def test_step_graph_replays_match_eager(dev):
    seqlens, H, d = [300, 77, 512], 4, 128
    w = workloads.custom(seqlens, H, d, d, torch.bfloat16, "neg_softplus")
    dw = workloads.custom([1] * len(seqlens), H, d, d, torch.bfloat16, "neg_softplus")
    xs = [workloads.prefill_inputs(w, device=dev, seed=s) for s in (11, 12)]
    ds = [workloads.decode_step_inputs(dw, 0, device=dev, seed=s) for s in (11, 12)]
    N, nseq = w.total_tokens, len(seqlens)
    ws = kda.alloc_workspace(N, nseq, H, d, d, torch.bfloat16, dev)
    o = torch.empty((N, H, d), dtype=torch.float32, device=dev)
    fin = torch.empty((nseq, H, d, d), dtype=torch.float32, device=dev)
    od = torch.empty((nseq, H, d), dtype=torch.float32, device=dev)

    def step(i):
        x, dd = xs[i], ds[i]
        kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
        kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws, None,
                            o=o, final_state=fin)
        kda.kda_decode_step(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], fin, o=od)

    say(f"  case: graph of the step, seqlens={seqlens} H={H} d={d} bf16, 3 replays")
    ref = []
    for i in (0, 1):
        step(i)
        torch.cuda.synchronize()
        ref.append((o.clone(), fin.clone(), od.clone()))
    step(0)  # warm the capture's first use of the buffers
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(0)
    for rep in range(3):
        step(1)  # eager work on the other inputs between replays
        torch.cuda.synchronize()
        assert torch.equal(o, ref[1][0]) and torch.equal(fin, ref[1][1]) and torch.equal(od, ref[1][2])
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((o, fin, od), ref[0], ("o", "final_state", "decode o")):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
