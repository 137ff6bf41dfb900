"""GPU parity of the prefill backward pass (kda_prefill_backward, through the C ABI) against
the fp64 oracle's reverse mode.  The backward computes in fp32 for both input dtypes."""
import numpy as np
import pytest
import torch

import gated_delta_rule_51_amd as kda
import oracle
import workloads
from parity import assert_close, say

pytestmark = pytest.mark.gpu

# fp32 arithmetic throughout (inputs of either dtype are exact in it): the fp32 bar, except for
# the log-decay gradient, a sum of per-token increments larger than the result (they partly
# cancel), so its error relative to its own RMS is the largest (measured up to 1.4e-5): 5e-5.
TOLS = {"dq": 1e-5, "dk": 1e-5, "dv": 1e-5, "dlog_alpha": 5e-5, "dbeta": 1e-5, "dinit": 1e-5}
NAMES = tuple(TOLS)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


def _case(dev, seqlens, H, dk, dv, dtype, seed, init=True, dfinal=True, gate="neg_softplus"):
    w = workloads.custom(seqlens, H, dk, dv, dtype, gate)
    x = workloads.prefill_inputs(w, device=dev, seed=seed)
    N, nseq = w.total_tokens, len(seqlens)
    gen = torch.Generator(device=dev).manual_seed(1000 + seed)
    d_o = torch.randn((N, H, dv), generator=gen, device=dev)
    S0 = workloads.random_state(nseq, H, dk, dv, device=dev, seed=seed) if init else None
    dF = torch.randn((nseq, H, dk, dv), generator=gen, device=dev) if dfinal else None
    return x, d_o, S0, dF


def _check(dev, x, d_o, S0, dF, heads=None, tols=TOLS):
    got = kda.kda_prefill_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], d_o, x["cu_seqlens"], S0, dF)
    torch.cuda.synchronize()
    sel = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    cpu = {n: sel(x[n]).cpu() for n in ("q", "k", "v", "log_alpha", "beta")}
    ref = oracle.backward(cpu["q"], cpu["k"], cpu["v"], cpu["log_alpha"], cpu["beta"], sel(d_o).cpu(),
                          cu_seqlens=x["cu_seqlens"].cpu(), init_state=None if S0 is None else sel(S0).cpu(),
                          dfinal=None if dF is None else sel(dF).cpu())
    for n in NAMES:
        assert_close(sel(got[n]), ref[n], tols[n], n)
    return got


@pytest.mark.parametrize("dtype,dk,dv", [(torch.float32, 16, 16), (torch.float32, 32, 64),
                                         (torch.bfloat16, 128, 128), (torch.bfloat16, 64, 16)])
def test_backward_matches_oracle(dev, dtype, dk, dv):
    """Ragged and empty sequences, a one-token sequence, initial state and final-state gradient."""
    seqlens = [40, 0, 17, 16, 1]
    x, d_o, S0, dF = _case(dev, seqlens, 2, dk, dv, dtype, seed=dk + dv)
    say(f"  case: backward seqlens={seqlens} H=2 dk={dk} dv={dv} {dtype}")
    _check(dev, x, d_o, S0, dF)


# The sweeps put NS 16-column slices of dv in one workgroup, NS the smallest of 1, 2, 4, 8 for
# which the (sequence, head, slice-group) grid stays within 256 workgroups, with 3, 2, 4, 4
# producer waves; these shapes take each NS, and dk = 16 with two producers leaves one of
# them without a channel block.
@pytest.mark.parametrize("seqlens,H,dk,dv,dtype,ns", [
    ([70, 23], 24, 128, 128, torch.bfloat16, 2),   # 2 x 24 x 8 = 384 slices
    ([50], 96, 128, 128, torch.bfloat16, 4),       # 768 slices (the K3 layer's grouping)
    ([37, 20], 96, 64, 128, torch.float32, 8),     # 1,536 slices
    ([45], 64, 16, 128, torch.bfloat16, 2),        # dk = 16: one channel block, two producers
])
def test_backward_slice_groupings(dev, seqlens, H, dk, dv, dtype, ns):
    x, d_o, S0, dF = _case(dev, seqlens, H, dk, dv, dtype, seed=H + dk)
    say(f"  case: backward seqlens={seqlens} H={H} dk={dk} dv={dv} {dtype} (NS = {ns})")
    _check(dev, x, d_o, S0, dF)


def test_backward_without_initial_state_or_final_gradient(dev):
    x, d_o, _, _ = _case(dev, [33, 5], 3, 128, 64, torch.bfloat16, seed=3, init=False, dfinal=False)
    say("  case: backward without init / d_final")
    _check(dev, x, d_o, None, None)


def test_backward_strong_decay(dev):
    """log-decay uniform on [-5, 0): the chunk factors e^{+-G} span the full e^{80} range."""
    x, d_o, S0, dF = _case(dev, [64, 29], 2, 64, 64, torch.float32, seed=4, gate="uniform")
    say("  case: backward, strong decay")
    _check(dev, x, d_o, S0, dF)


def test_backward_no_tokens(dev):
    """N = 0: the initial state's gradient is the final state's."""
    H, dk, dv = 2, 32, 32
    e = torch.empty((0, H, dk), dtype=torch.bfloat16, device=dev)
    ev = torch.empty((0, H, dv), dtype=torch.bfloat16, device=dev)
    eb = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(3, dtype=torch.int32, device=dev)
    dF = torch.randn((2, H, dk, dv), device=dev)
    got = kda.kda_prefill_backward(e, e, ev, e, eb, torch.empty((0, H, dv), device=dev), cu, None, dF)
    torch.cuda.synchronize()
    assert torch.equal(got["dinit"], dF)


def test_backward_batched_workload_sampled_heads(dev):
    """The batched workload's shape (B=4 x 2048 tokens, H=8, d=128, bf16): the whole backward
    on the GPU, the oracle on 2 sampled heads of every sequence."""
    w = workloads.workload(2)
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    gen = torch.Generator(device=dev).manual_seed(7)
    d_o = torch.randn((w.total_tokens, w.H, w.dv), generator=gen, device=dev)
    dF = torch.randn((w.nseq, w.H, w.dk, w.dv), generator=gen, device=dev)
    say("  case: backward B=4 T=2048 H=8 d=128, heads [1, 6]")
    _check(dev, x, d_o, None, dF, heads=[1, 6])


# A 65,536-token sequence runs the fp32 recurrences through 4,096 chunk steps each way, and
# the largest deviation over 16.8 M values of a gradient grows past the short cases' 1e-5
# (measured 1.3e-5 for dv, 1.4e-5 for dlog_alpha): 5e-5 for every gradient here, still far
# below the 1e-2 bar stated for bf16 inputs.
TOLS_LONG = {n: 5e-5 for n in NAMES}


def test_backward_k3_layer_sampled_heads(dev):
    """The K3 layer's shape (B=1, 65,536 tokens, H=96, d=128, bf16): the whole backward on the
    GPU in the launch configuration the benchmark times (four slice waves per workgroup) and
    with the log-decay carry over 4,096 chunks; the oracle on 2 sampled heads."""
    w = workloads.workload(3)
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    gen = torch.Generator(device=dev).manual_seed(11)
    d_o = torch.randn((w.total_tokens, w.H, w.dv), generator=gen, device=dev)
    dF = torch.randn((w.nseq, w.H, w.dk, w.dv), generator=gen, device=dev)
    say("  case: backward B=1 T=65536 H=96 d=128, heads [5, 77]")
    _check(dev, x, d_o, None, dF, heads=[5, 77], tols=TOLS_LONG)


def test_backward_is_deterministic(dev):
    """No atomics anywhere: two calls on the same inputs agree bit for bit."""
    x, d_o, S0, dF = _case(dev, [300, 45, 1], 24, 128, 128, torch.bfloat16, seed=21)
    runs = [kda.kda_prefill_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], d_o, x["cu_seqlens"], S0,
                                     dF) for _ in range(2)]
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(runs[0][n], runs[1][n]), f"{n} differs between two identical calls"


def _slabbed(x, d_o, S0, dF, slab):
    return kda.kda_prefill_backward_slabbed(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], d_o, S0, dF,
                                           slab_tokens=slab)


@pytest.mark.parametrize("T,slab,dtype,dk,dv", [(1000, 256, torch.bfloat16, 128, 128), (700, 96, torch.float32, 32, 64),
                                                (50, 64, torch.bfloat16, 64, 32), (512, 256, torch.bfloat16, 128, 64)])
def test_backward_slabbed_matches_oracle(dev, T, slab, dtype, dk, dv):
    """One sequence cut into slabs (a ragged last slab, a single slab, slabs ending exactly at
    the sequence's end), with an initial state and a final-state gradient: every gradient
    against the oracle's reverse mode, and against the unsliced backward."""
    x, d_o, S0, dF = _case(dev, [T], 3, dk, dv, dtype, seed=T + slab)
    say(f"  case: slabbed backward T={T} slab={slab} H=3 dk={dk} dv={dv} {dtype}")
    got = _slabbed(x, d_o, S0, dF, slab)
    whole = kda.kda_prefill_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], d_o, x["cu_seqlens"], S0, dF)
    torch.cuda.synchronize()
    cpu = {n: x[n].cpu() for n in ("q", "k", "v", "log_alpha", "beta")}
    ref = oracle.backward(cpu["q"], cpu["k"], cpu["v"], cpu["log_alpha"], cpu["beta"], d_o.cpu(),
                          cu_seqlens=x["cu_seqlens"].cpu(), init_state=S0.cpu(), dfinal=dF.cpu())
    for n in NAMES:
        assert_close(got[n], ref[n], TOLS[n], n)
        assert_close(got[n], whole[n].double().cpu().numpy(), 2e-6, n + " (slabbed vs whole)")


def test_backward_slabbed_k3_layer_against_whole(dev):
    """The K3 layer's shape (65,536 tokens, 96 heads) in slabs of 16,384 tokens: a quarter of
    the unsliced backward's workspace (15 GB instead of 60 GB); every gradient of every head
    against the unsliced backward (the same fp32 arithmetic, cut at the slab boundaries)."""
    w = workloads.workload(3)
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    gen = torch.Generator(device=dev).manual_seed(11)
    d_o = torch.randn((w.total_tokens, w.H, w.dv), generator=gen, device=dev)
    dF = torch.randn((1, w.H, w.dk, w.dv), generator=gen, device=dev)
    nb_slab = kda.kda_prefill_backward_slabbed_workspace_bytes(w.total_tokens, w.H, 128, 128, 16384)
    nb_whole = int(kda.load_library().kda_prefill_backward_workspace_bytes(w.total_tokens, 1, w.H, 128, 128, 1))
    say(f"  case: slabbed backward K3 layer, workspace {nb_slab / 2**30:.1f} GiB vs {nb_whole / 2**30:.1f} GiB")
    assert nb_slab < nb_whole / 3.5
    got = _slabbed(x, d_o, None, dF, 16384)
    torch.cuda.synchronize()
    whole = kda.kda_prefill_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], d_o, x["cu_seqlens"], None,
                                     dF)
    torch.cuda.synchronize()
    for n in NAMES:
        assert_close(got[n], whole[n].double().cpu().numpy(), 5e-6, n + " (slabbed vs whole)")
    del x, d_o, dF, got, whole
    torch.cuda.empty_cache()


def test_backward_slabbed_262k_tokens(dev):
    """262,144 tokens x 96 heads (four times the K3 layer; the unsliced backward would need
    238 GB of workspace): slabs of 16,384 tokens, the oracle's reverse mode on one head (fp32
    chains of 16,384 chunk steps each way: the long-sequence bar)."""
    N, H = 262144, 96
    w = workloads.custom([N], H, 128, 128, torch.bfloat16, "neg_softplus")
    x = workloads.prefill_inputs(w, device=dev, seed=2)
    gen = torch.Generator(device=dev).manual_seed(13)
    d_o = torch.randn((N, H, 128), generator=gen, device=dev)
    say(f"  case: slabbed backward T={N} H={H}, workspace "
        f"{kda.kda_prefill_backward_slabbed_workspace_bytes(N, H, 128, 128, 16384) / 2**30:.1f} GiB, oracle on head 40")
    got = _slabbed(x, d_o, None, None, 16384)
    torch.cuda.synchronize()
    hs = [40]
    cpu = {n: x[n][:, hs].cpu() for n in ("q", "k", "v", "log_alpha", "beta")}
    ref = oracle.backward(cpu["q"], cpu["k"], cpu["v"], cpu["log_alpha"], cpu["beta"], d_o[:, hs].cpu(),
                          cu_seqlens=x["cu_seqlens"].cpu())
    for n in NAMES:
        assert_close(got[n][:, hs], ref[n], TOLS_LONG[n], n)
    del x, d_o, got
    torch.cuda.empty_cache()
