"""Guard regions and launch-order independence on the GPU.

Guard regions: every output, in/out and workspace buffer the calls below write is the interior
of a larger allocation whose 4 KiB before and after hold a sentinel bit pattern; after the call
the sentinels must be unchanged, bit for bit (a write past either end of a buffer -- a wrong
row stride, a ragged tail, a grid larger than the work -- fails here even where the values
inside the buffer are right).  Shapes with ragged tails and heads that do not fill the last
workgroup, for each kernel family: the single-pass and the two-kernel prefill, decode steps,
decode windows in both forms, the layer window's one-chunk form (its workspace and convolution
cache included), the fused layer prefill and the backward's workspace.

Launch-order independence: the same sequences packed in another order map their (sequence,
head) chains to other workgroups (the longest-first order ranks them anew) and to other
dispatch positions; every sequence's outputs and final state must be identical bit for bit.
A race through LDS or a dependence on which workgroup runs a chain would show as a difference."""
import pytest
import torch

import gated_delta_rule_51_amd as kda
import workloads
from parity import say

pytestmark = pytest.mark.gpu

GUARD_BYTES = 4096
SENTINEL = {torch.float32: 0x7FC0DEAD, torch.bfloat16: 0x7FA1, torch.uint8: 0xA5, torch.int32: 0x5EED5EED}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


class Guarded:
    """A tensor of `shape` inside a flat allocation with GUARD_BYTES of sentinel on each side."""

    def __init__(self, shape, dtype, dev, fill=None):
        esz = torch.empty((), dtype=dtype).element_size()
        raw_dtype = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[esz]
        self.g = GUARD_BYTES // esz
        self.n = 1
        for s in shape:
            self.n *= s
        self.flat = torch.empty(self.n + 2 * self.g, dtype=dtype, device=dev)
        v = SENTINEL[dtype]
        self.bits = v - (1 << (8 * esz)) if esz > 1 and v >= 1 << (8 * esz - 1) else v  # as the signed view
        self.raw = self.flat.view(raw_dtype)
        self.raw.fill_(self.bits)
        self.t = self.flat[self.g:self.g + self.n].view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self, what):
        torch.cuda.synchronize()
        bad_h = int((self.raw[:self.g] != self.bits).sum())
        bad_t = int((self.raw[self.g + self.n:] != self.bits).sum())
        assert bad_h == 0 and bad_t == 0, f"{what}: {bad_h} guard elements before and {bad_t} after were written"


def _prefill_guarded(dev, seqlens, H, dk, dv, dtype, seed, init=True):
    w = workloads.custom(seqlens, H, dk, dv, dtype)
    x = workloads.prefill_inputs(w, device=dev, seed=seed)
    N, nseq = sum(seqlens), len(seqlens)
    st = workloads.random_state(nseq, H, dk, dv, device=dev, seed=seed) if init else None
    o = Guarded((N, H, dv), torch.float32, dev)
    f = Guarded((nseq, H, dk, dv), torch.float32, dev)
    nbytes = kda.kda_prefill_workspace_bytes(N, nseq, H, dk, dv, dtype)
    ws = Guarded((max(nbytes, 4) // 4,), torch.float32, dev) if nbytes > 0 else None
    say(f"  case: guarded prefill seqlens={seqlens} H={H} dk={dk} dv={dv} {dtype} workspace={nbytes}")
    kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], st, o=o.t, final_state=f.t,
                    workspace=None if ws is None else ws.t)
    o.check("o")
    f.check("final_state")
    if ws is not None:
        ws.check("workspace")
    assert torch.isfinite(o.t).all() and torch.isfinite(f.t).all()


def test_guards_two_kernel_prefill(dev):
    """Few chains: chunk-local + inter-chunk with a workspace; ragged tails, several head sizes."""
    _prefill_guarded(dev, [37, 1, 130], 3, 128, 128, torch.bfloat16, 1)
    _prefill_guarded(dev, [33, 17], 5, 64, 32, torch.bfloat16, 2)
    _prefill_guarded(dev, [19, 40], 2, 16, 64, torch.float32, 3, init=False)


def test_guards_single_pass_prefill(dev):
    """At least 256 chains (the single-pass kernel, no workspace): 3 x 90 chains, ragged tails."""
    _prefill_guarded(dev, [45, 16, 77], 90, 128, 128, torch.bfloat16, 4)


def test_guards_decode_step_and_windows(dev):
    B, H, T = 5, 7, 8  # 35 heads: the last workgroups of the persistent grids are partly empty
    w = workloads.custom([1] * B, H, 128, 128, torch.bfloat16)
    init = workloads.random_state(B, H, 128, 128, device=dev, seed=5)
    d = workloads.decode_step_inputs(w, 0, device=dev, seed=5)
    st = Guarded((B, H, 128, 128), torch.float32, dev, fill=init)
    o = Guarded((B, H, 128), torch.float32, dev)
    say(f"  case: guarded decode step B={B} H={H}")
    kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], st.t, o=o.t)
    st.check("decode state")
    o.check("decode o")
    x = workloads.decode_window_inputs(w, T, 0, device=dev, seed=6)
    acc = torch.tensor([0, 3, 8, 5, 1], dtype=torch.int32, device=dev)
    for form in (1, 2):
        st = Guarded((B, H, 128, 128), torch.float32, dev, fill=init)
        o = Guarded((B, T, H, 128), torch.float32, dev)
        say(f"  case: guarded decode window B={B} T={T} H={H} form={form}")
        kda.kda_decode_window(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], st.t, acc, o=o.t, form=form)
        st.check(f"window state (form {form})")
        o.check(f"window o (form {form})")


def test_guards_layer_window_one_chunk(dev):
    """The layer window's one-chunk form: o, y, the committed state and convolution cache, and
    the workspace the prologue pass writes."""
    B, T, H, dk, dv = 3, 4, 5, 128, 128
    C = 2 * dk + dv
    prev = {"qkv": workloads.layer_inputs(B * T, H, C, torch.bfloat16, nseq=B, device=dev, seed=7)["x"]
            .view(B, T, H, C).contiguous(),
            "gate": workloads.layer_inputs(B * T, H, dk, torch.bfloat16, device=dev, seed=8)["z"].view(B, T, H, dk)
            .contiguous(),
            "beta": workloads.decode_window_inputs(workloads.custom([1] * B, H, dk, dv), T, 0, device=dev,
                                                   seed=9)["beta"]}
    li = workloads.layer_inputs(B * T, H, C, torch.bfloat16, nseq=B, device=dev, seed=10)
    lz = workloads.layer_inputs(B * T, H, dk, torch.bfloat16, device=dev, seed=11)
    lu = workloads.layer_inputs(B * T, H, dv, torch.bfloat16, device=dev, seed=12)
    beta = workloads.decode_window_inputs(workloads.custom([1] * B, H, dk, dv), T, 1, device=dev, seed=9)["beta"]
    init = workloads.random_state(B, H, dk, dv, device=dev, seed=13)
    st = Guarded((B, H, dk, dv), torch.float32, dev, fill=init)
    cache = Guarded((B, H, C, 3), torch.float32, dev, fill=li["conv_cache"][:B])
    o = Guarded((B, T, H, dv), torch.float32, dev)
    y = Guarded((B, T, H, dv), torch.bfloat16, dev)
    need = kda.kda_decode_layer_window_workspace_bytes(B, T, T, H, dk, dv, torch.bfloat16)
    assert need > 0
    ws = Guarded((need,), torch.uint8, dev)
    acc = torch.tensor([2, 0, 4], dtype=torch.int32, device=dev)
    say(f"  case: guarded layer window B={B} T={T} H={H}, one chunk")
    kda.kda_decode_layer_window_replay(prev, acc, li["x"].view(B, T, H, C).contiguous(),
                                       lz["z"].view(B, T, H, dk).contiguous(), beta, li["conv_w"], cache.t, st.t,
                                       dk=dk, gate_A_log=lz["A_log"], out_gate=lu["u"].view(B, T, H, dv).contiguous(),
                                       norm_w=lu["norm_w"], o=o.t, y=y.t, form=2, workspace=ws.t)
    for g, name in ((st, "state"), (cache, "convolution cache"), (o, "o"), (y, "y"), (ws, "workspace")):
        g.check(name)


def test_guards_layer_prefill_and_backward_workspace(dev):
    seqlens = [50, 3, 29]
    N, nseq, H, d = sum(seqlens), len(seqlens), 3, 128
    w = workloads.custom(seqlens, H, d, d, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=14)
    li = workloads.layer_inputs(N, H, 3 * d, torch.bfloat16, nseq=nseq, device=dev, seed=15)
    lz = workloads.layer_inputs(N, H, d, torch.bfloat16, device=dev, seed=16)
    lu = workloads.layer_inputs(N, H, d, torch.bfloat16, device=dev, seed=17)
    q, k, v = (li["x"][:, :, i * d:(i + 1) * d].contiguous() for i in range(3))
    o = Guarded((N, H, d), torch.float32, dev)
    f = Guarded((nseq, H, d, d), torch.float32, dev)
    y = Guarded((N, H, d), torch.bfloat16, dev)
    cout = Guarded((nseq, H, 3 * d, 3), torch.float32, dev)
    nbytes = kda.kda_prefill_layer_workspace_bytes(N, nseq, H, d, d, torch.bfloat16)
    ws = Guarded((max(nbytes, 4) // 4,), torch.float32, dev)
    say(f"  case: guarded layer prefill seqlens={seqlens} H={H}")
    kda.kda_prefill_layer(q, k, v, li["conv_w"], lz["z"], lz["A_log"], x["beta"], x["cu_seqlens"],
                          conv_cache=li["conv_cache"], conv_cache_out=cout.t, out_gate=lu["u"], norm_w=lu["norm_w"],
                          o=o.t, final_state=f.t, y=y.t, workspace=ws.t)
    for g, name in ((o, "o"), (f, "final_state"), (y, "y"), (cout, "convolution cache out"), (ws, "workspace")):
        g.check("layer prefill " + name)
    d_o = torch.randn((N, H, d), dtype=torch.float32, device=dev)
    nb = int(kda.load_library().kda_prefill_backward_workspace_bytes(N, nseq, H, d, d, kda.KDA_BF16))
    assert nb > 0
    wsb = Guarded((nb // 4,), torch.float32, dev)
    say("  case: guarded backward workspace")
    g = kda.kda_prefill_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], d_o, x["cu_seqlens"],
                                 workspace=wsb.t)
    wsb.check("backward workspace")
    assert all(torch.isfinite(t).all() for t in g.values() if t is not None)


def _repack(x, seqlens, order):
    """The same sequences packed in `order`."""
    cu = workloads.cu_seqlens_of(seqlens)
    out = {}
    for n in ("q", "k", "v", "log_alpha", "beta"):
        out[n] = torch.cat([x[n][cu[s]:cu[s + 1]] for s in order]).contiguous()
    new_lens = [seqlens[s] for s in order]
    out["cu_seqlens"] = torch.tensor(workloads.cu_seqlens_of(new_lens), dtype=torch.int32, device=x["q"].device)
    return out, new_lens


@pytest.mark.parametrize("H", [4, 40])
def test_prefill_is_independent_of_launch_order(dev, H):
    """Seven sequences in two packing orders: with 4 heads (28 chains: the two-kernel path, the
    inter-chunk kernel's longest-first order) and 40 heads (280 chains: the single pass), every
    sequence's o and final state bit for bit the same."""
    seqlens = [300, 17, 64, 129, 5, 211, 48]
    w = workloads.custom(seqlens, H, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=18)
    init = workloads.random_state(len(seqlens), H, 128, 128, device=dev, seed=18)
    o1, f1 = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], init)
    order = [5, 2, 0, 6, 1, 4, 3]
    y, lens = _repack(x, seqlens, order)
    o2, f2 = kda.kda_prefill(y["q"], y["k"], y["v"], y["log_alpha"], y["beta"], y["cu_seqlens"],
                             init[order].contiguous())
    torch.cuda.synchronize()
    cu1, cu2 = workloads.cu_seqlens_of(seqlens), workloads.cu_seqlens_of(lens)
    say(f"  case: launch order, {len(seqlens)} sequences x {H} heads")
    for j, s in enumerate(order):
        assert torch.equal(o1[cu1[s]:cu1[s + 1]], o2[cu2[j]:cu2[j + 1]]), f"sequence {s}: o depends on the order"
        assert torch.equal(f1[s], f2[j]), f"sequence {s}: final state depends on the order"


def test_decode_window_is_independent_of_batch_order(dev):
    """The decode window (one-chunk form) over a batch in two orders: per sequence identical."""
    B, H, T = 9, 5, 8
    w = workloads.custom([1] * B, H, 128, 128, torch.bfloat16)
    x = workloads.decode_window_inputs(w, T, 0, device=dev, seed=19)
    init = workloads.random_state(B, H, 128, 128, device=dev, seed=19)
    acc = workloads.window_accept(B, T, device=dev, seed=19)
    s1 = init.clone()
    o1 = kda.kda_decode_window(*(x[n] for n in ("q", "k", "v", "log_alpha", "beta")), s1, acc)
    perm = torch.tensor([4, 8, 0, 2, 7, 1, 6, 3, 5], device=dev)
    s2 = init[perm].contiguous()
    o2 = kda.kda_decode_window(*(x[n][perm].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")), s2,
                               acc[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o1[perm], o2) and torch.equal(s1[perm], s2)


def test_check_cu_seqlens(dev):
    """The opt-in device check of cu_seqlens: -1 for valid offsets (empty sequences included),
    else the first index that breaks the contract."""
    def check(cu, N):
        return int(kda.kda_check_cu_seqlens(torch.tensor(cu, dtype=torch.int32, device=dev), N).item())
    assert check([0, 5, 5, 12], 12) == -1
    assert check([0, 0], 0) == -1
    assert check([1, 5, 12], 12) == 0          # does not start at 0
    assert check([0, 7, 5, 12], 12) == 2       # decreasing
    assert check([0, 5, 11], 12) == 2          # does not end at N
    assert check([0, 5, 13, 12], 12) == 2      # beyond N
    assert check([0, -1, 3], 3) == 1           # negative
    big = list(range(0, 3 * 5000 + 1, 3))      # 5,000 sequences: several strides of the workgroup
    assert check(big, 15000) == -1
    big[4321] = big[4320] - 1
    assert check(big, 15000) == 4321
