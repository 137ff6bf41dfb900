"""GPU parity of the context-parallel prefill (kda_prefill_cp, through the C ABI): every
sequence split into R chunk-aligned segments run as independent chains, the incoming states
recovered by a scan over the segments' affine maps.  Against the fp64 oracle at the prefill's
bar (1e-2 RMS for bf16 inputs, 1e-5 for fp32), and against the plain two-kernel prefill on the
same inputs; kda_prefill's own choice of it for few long chains; segments whose transition the
device-side bound declares negligible (the M pass skipped) next to segments where it is not."""
import pytest
import torch

import gated_delta_rule_51_amd as kda
import workloads
from parity import TOL, assert_close, oracle_prefill, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


def _two_kernel(x, S0=None):
    """The plain prefill (chunk-local then inter-chunk, no context parallelism)."""
    N, H, dk = x["q"].shape
    dv = x["v"].shape[2]
    nseq = x["cu_seqlens"].numel() - 1
    ws = kda.alloc_workspace(N, nseq, H, dk, dv, x["q"].dtype, x["q"].device)
    kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
    return kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws, S0)


def _cp_case(dev, seqlens, H, dk, dv, dtype, R, seed=0, init=True, heads=None):
    w = workloads.custom(seqlens, H, dk, dv, dtype, "neg_softplus")
    x = workloads.prefill_inputs(w, device=dev, seed=seed)
    S0 = workloads.random_state(len(seqlens), H, dk, dv, device=dev, seed=seed) if init else None
    say(f"  case: cp R={R} seqlens={list(seqlens)[:6]} H={H} dk={dk} dv={dv} {dtype} init={init}")
    # outputs start as NaN, so a row or state the kernels never write cannot pass
    o = torch.full((w.total_tokens, H, dv), float("nan"), dtype=torch.float32, device=dev)
    fin = torch.full((len(seqlens), H, dk, dv), float("nan"), dtype=torch.float32, device=dev)
    kda.kda_prefill_cp(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], S0, segments=R,
                       o=o, final_state=fin)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(x, S0, heads=heads)
    if heads is not None:
        o, fin = o[:, heads], fin[:, heads]
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(fin, f_ref, TOL[dtype], "final_state")
    return x, S0, o, fin


# Segments shorter than a chunk, sequences shorter than R chunks (empty segments), an empty
# sequence, ragged tails; R = 1 (the plain recurrence run three times) up to 7.
@pytest.mark.parametrize("dtype,dk,dv,R", [(torch.float32, 16, 16, 3), (torch.float32, 32, 64, 1),
                                           (torch.float32, 64, 16, 7), (torch.bfloat16, 128, 128, 4),
                                           (torch.bfloat16, 32, 128, 2), (torch.bfloat16, 128, 64, 5)])
def test_cp_matches_oracle(dev, dtype, dk, dv, R):
    _cp_case(dev, [200, 17, 0, 33, 1, 96], 2, dk, dv, dtype, R, seed=dk + dv + R)


def test_cp_without_initial_state(dev):
    _cp_case(dev, [129, 64], 3, 128, 128, torch.bfloat16, 4, seed=9, init=False)


def test_cp_agrees_with_prefill(dev):
    """The same inputs through kda_prefill and kda_prefill_cp (R = 4): the two differ only by
    the order of fp32 rounding in the state, far inside the bf16 bar."""
    w = workloads.custom([500, 260, 31], 4, 128, 128, torch.bfloat16, "neg_softplus")
    x = workloads.prefill_inputs(w, device=dev, seed=5)
    S0 = workloads.random_state(3, 4, 128, 128, device=dev, seed=5)
    o1, f1 = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], S0)
    o2, f2 = kda.kda_prefill_cp(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], S0, segments=4)
    torch.cuda.synchronize()
    assert_close(o2, o1.double().cpu().numpy(), 1e-3, "o (cp vs prefill)")
    assert_close(f2, f1.double().cpu().numpy(), 1e-3, "final_state (cp vs prefill)")


def test_cp_batched_workload_sampled_heads(dev):
    """The batched workload's shape (B=4 x 2048 tokens, H=8, d=128, bf16) with R = 4 segments
    per sequence (128 chains instead of 32), the oracle on 2 sampled heads."""
    w = workloads.workload(2)
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    say("  case: cp R=4, B=4 T=2048 H=8 d=128, heads [2, 5]")
    o, fin = kda.kda_prefill_cp(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], segments=4)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(x, None, heads=[2, 5])
    assert_close(o[:, [2, 5]], o_ref, TOL[torch.bfloat16], "o")
    assert_close(fin[:, [2, 5]], f_ref, TOL[torch.bfloat16], "final_state")



def test_cp_few_heads_long_sequence(dev):
    """Where context parallelism pays: one 65,536-token sequence with 12 heads (the K3 layer's
    share of one device when its 96 heads are split eight ways), R = 10 segments as timed by
    the benchmark.  The oracle on 2 sampled heads, and every head against the plain prefill.
    With the workload's decay and erase rates a 6,554-token segment forgets its incoming
    state entirely (its map M is about 1e-10 in norm), so here the log-decay is scaled by 1e-4
    and beta by 1e-2: each segment's map then keeps about half of the incoming state (norm
    ratio 0.46 in a CPU estimate) and the scan's products count."""
    w = workloads.custom([65536], 12, 128, 128, torch.bfloat16, "neg_softplus")
    x = workloads.prefill_inputs(w, device=dev, seed=3)
    x["log_alpha"] = (x["log_alpha"].float() * 1e-4).to(torch.bfloat16)
    x["beta"] = (x["beta"].float() * 1e-2).to(torch.bfloat16)
    say("  case: cp R=10, T=65536 H=12 d=128, log-decay x 1e-4, beta x 1e-2, heads [3, 10] + all vs plain")
    o, fin = kda.kda_prefill_cp(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], segments=10)
    o1, f1 = _two_kernel(x)
    torch.cuda.synchronize()
    assert_close(o, o1.double().cpu().numpy(), 1e-3, "o (cp vs prefill)")
    assert_close(fin, f1.double().cpu().numpy(), 1e-3, "final_state (cp vs prefill)")
    o_ref, f_ref = oracle_prefill(x, None, heads=[3, 10], nthreads=2)
    assert_close(o[:, [3, 10]], o_ref, TOL[torch.bfloat16], "o")
    assert_close(fin[:, [3, 10]], f_ref, TOL[torch.bfloat16], "final_state")

def test_cp_long_sequence_workload_rates(dev):
    """One 65,536-token sequence with 12 heads at R = 10 with the workload's own decay and write
    rates (where a segment's map is far below fp32 resolution, so the scan must not disturb the
    exact states; every segment's M pass is skipped there): outputs start as NaN, every head
    against the plain prefill, the oracle on heads 0-7 (one per residue mod 8)."""
    w = workloads.custom([65536], 12, 128, 128, torch.bfloat16, "neg_softplus")
    x = workloads.prefill_inputs(w, device=dev, seed=4)
    o = torch.full((65536, 12, 128), float("nan"), dtype=torch.float32, device=dev)
    fin = torch.full((1, 12, 128, 128), float("nan"), dtype=torch.float32, device=dev)
    say("  case: cp R=10, T=65536 H=12 d=128, workload rates")
    kda.kda_prefill_cp(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], segments=10, o=o,
                       final_state=fin)
    o1, f1 = _two_kernel(x)
    torch.cuda.synchronize()
    assert_close(o, o1.double().cpu().numpy(), 1e-3, "o (cp vs prefill)")
    assert_close(fin, f1.double().cpu().numpy(), 1e-3, "final_state (cp vs prefill)")
    hs = list(range(8))
    o_ref, f_ref = oracle_prefill(x, None, heads=hs)
    assert_close(o[:, hs], o_ref, TOL[torch.bfloat16], "o")
    assert_close(fin[:, hs], f_ref, TOL[torch.bfloat16], "final_state")


def test_cp_negligible_and_kept_transitions_in_one_sequence(dev):
    """One 65,536-token sequence, 4 heads, R = 8: the first half at the workload's rates (the
    bound declares those segments' transitions negligible and their M pass is skipped), the
    second half with the log-decay scaled by 1e-4 and beta by 1e-2 (transitions kept, the scan's
    products count), so one scan mixes both kinds; plus a second sequence of 20,000 tokens.
    Against the oracle on 2 heads and the plain prefill on every head."""
    seqlens, H = [65536, 20000], 4
    w = workloads.custom(seqlens, H, 128, 128, torch.bfloat16, "neg_softplus")
    x = workloads.prefill_inputs(w, device=dev, seed=6)
    g, b = x["log_alpha"].float(), x["beta"].float()
    g[32768:65536] *= 1e-4
    b[32768:65536] *= 1e-2
    x["log_alpha"], x["beta"] = g.to(torch.bfloat16), b.to(torch.bfloat16)
    S0 = workloads.random_state(2, H, 128, 128, device=dev, seed=6)
    o = torch.full((sum(seqlens), H, 128), float("nan"), dtype=torch.float32, device=dev)
    fin = torch.full((2, H, 128, 128), float("nan"), dtype=torch.float32, device=dev)
    say("  case: cp R=8, seqlens [65536, 20000] H=4, half the first sequence at workload rates, half scaled")
    kda.kda_prefill_cp(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], S0, segments=8, o=o,
                       final_state=fin)
    o1, f1 = _two_kernel(x, S0)
    torch.cuda.synchronize()
    assert_close(o, o1.double().cpu().numpy(), 1e-3, "o (cp vs plain)")
    assert_close(fin, f1.double().cpu().numpy(), 1e-3, "final_state (cp vs plain)")
    o_ref, f_ref = oracle_prefill(x, S0, heads=[1, 2], nthreads=2)
    assert_close(o[:, [1, 2]], o_ref, TOL[torch.bfloat16], "o")
    assert_close(fin[:, [1, 2]], f_ref, TOL[torch.bfloat16], "final_state")


def test_prefill_chooses_cp_for_few_long_chains(dev):
    """kda_prefill on one 65,536-token sequence with 12 heads (12 chains, 65,536 tokens each)
    runs context parallelism with R = 10 -- bit for bit kda_prefill_cp(segments=10) -- and on 65
    heads (more chains than it takes) the plain two-kernel prefill, bit for bit."""
    w = workloads.custom([65536], 12, 128, 128, torch.bfloat16, "neg_softplus")
    x = workloads.prefill_inputs(w, device=dev, seed=7)
    assert kda.kda_prefill_workspace_bytes(65536, 1, 12, 128, 128) == \
        kda.load_library().kda_prefill_cp_workspace_bytes(65536, 1, 12, 128, 128, 1, 10)
    o1, f1 = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"])
    o2, f2 = kda.kda_prefill_cp(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], segments=10)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    del x, o1, f1, o2, f2
    w = workloads.custom([16384], 65, 128, 128, torch.bfloat16, "neg_softplus")
    x = workloads.prefill_inputs(w, device=dev, seed=8)
    o1, f1 = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"])
    o2, f2 = _two_kernel(x)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_cp_no_tokens(dev):
    """N = 0: every segment is empty, so the final states are the initial ones exactly."""
    H, dk, dv = 2, 32, 64
    e = torch.empty((0, H, dk), dtype=torch.bfloat16, device=dev)
    ev = torch.empty((0, H, dv), dtype=torch.bfloat16, device=dev)
    eb = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(4, dtype=torch.int32, device=dev)
    S0 = torch.randn((3, H, dk, dv), device=dev)
    o, fin = kda.kda_prefill_cp(e, e, ev, e, eb, cu, S0, segments=3)
    torch.cuda.synchronize()
    assert o.shape == (0, H, dv)
    assert torch.equal(fin, S0)
