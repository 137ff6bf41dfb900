"""GPU parity of speculative decoding as a serving loop runs it (kda_decode_window_replay): each
call replays the previous window's accepted prefix (counts known only after that window ran),
commits the state after it, and runs the new window without committing it.  Against the fp64
oracle's decode steps window by window, and against the same schedule through kda_decode_window
with the accepted counts given at launch (the committed states bit for bit).  Outputs start as
NaN.  From 6 tokens per call (T + Tp) the replay runs as one chunk on the matrix cores."""
import numpy as np
import pytest
import torch

import gated_delta_rule_51_amd as kda
import oracle
import workloads
from oracle import layer
from parity import TOL, assert_close, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_alpha", "beta")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


def _np(t):
    return t.detach().cpu().double().numpy()


def _serving_loop(dev, B, T, H, dk, dv, dtype, windows, seed, accepts=None):
    """Windows of T tokens for B sequences; accepted counts per window drawn uniform on [0, T]
    (or given).  Returns the windows' inputs, the accepted counts, the GPU outputs per window
    and the committed state after a final replay."""
    w = workloads.custom([1] * B, H, dk, dv, dtype)
    xs = [workloads.decode_window_inputs(w, T, i, device=dev, seed=seed) for i in range(windows)]
    if accepts is None:
        accepts = [workloads.window_accept(B, T, device=dev, seed=seed + i) for i in range(windows)]
    init = workloads.random_state(B, H, dk, dv, device=dev, seed=seed)
    state = init.clone()
    outs = []
    for i, x in enumerate(xs):
        prev = None if i == 0 else {"q": xs[i - 1]["q"], "k": xs[i - 1]["k"], "v": xs[i - 1]["v"],
                                    "gate": xs[i - 1]["log_alpha"], "beta": xs[i - 1]["beta"]}
        o = torch.full((B, T, H, dv), float("nan"), dtype=torch.float32, device=dev)
        o, _ = kda.kda_decode_window_replay(prev, None if i == 0 else accepts[i - 1], x["q"], x["k"], x["v"],
                                            x["log_alpha"], x["beta"], state, o=o)
        outs.append(o)
    # commit the last window's accepted prefix (a one-token window whose output is not used)
    last = xs[-1]
    one = workloads.decode_window_inputs(w, 1, windows * T, device=dev, seed=seed)
    kda.kda_decode_window_replay({"q": last["q"], "k": last["k"], "v": last["v"], "gate": last["log_alpha"],
                                  "beta": last["beta"]}, accepts[-1], one["q"], one["k"], one["v"],
                                 one["log_alpha"], one["beta"], state)
    torch.cuda.synchronize()
    return xs, accepts, init, outs, state


def _oracle_loop(xs, accepts, init):
    """The oracle: per window, T steps from the committed state give the outputs; the committed
    state then advances by the window's first accepted tokens."""
    committed = _np(init).copy()
    outs = []
    for x, acc in zip(xs, accepts):
        acc = [int(a) for a in acc.cpu()]
        B, T = x["q"].shape[:2]
        st = committed.copy()
        o_w = []
        for t in range(T):
            step = [_np(x[n][:, t]) for n in NAMES]
            o_t, st = oracle.decode(*step, st, inplace=True)
            o_w.append(o_t)
            for b in range(B):
                if acc[b] == t + 1:
                    committed[b] = st[b]
        outs.append(np.stack(o_w, axis=1))
    return outs, committed


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 16, 64),
                                         (torch.bfloat16, 64, 32)])
def test_replay_serving_loop_matches_oracle(dev, dtype, dk, dv):
    """Six sequences, five windows of 4 tokens, accepted counts uniform on [0, 4] (nothing and
    everything accepted both occur): every window's outputs and the committed state after the
    last replay against the oracle; sequences that never accept keep their state bit for bit."""
    B, T, H = 6, 4, 3
    accepts = [torch.tensor(a, dtype=torch.int32, device=dev) for a in
               ([0, 4, 2, 1, 3, 0], [4, 0, 2, 3, 1, 0], [2, 2, 0, 4, 4, 0], [1, 3, 4, 0, 2, 0], [3, 1, 1, 2, 0, 0])]
    say(f"  case: replay loop B={B} T={T} H={H} dk={dk} dv={dv} {dtype}, 5 windows")
    xs, accepts, init, outs, state = _serving_loop(dev, B, T, H, dk, dv, dtype, 5, seed=dk + dv, accepts=accepts)
    o_ref, s_ref = _oracle_loop(xs, accepts, init)
    for i, (o, r) in enumerate(zip(outs, o_ref)):
        assert_close(o, r, TOL[dtype], f"window {i} o")
    assert_close(state, s_ref, TOL[dtype], "committed state")
    assert torch.equal(state[5], init[5]), "a sequence that accepted nothing changed its state"


@pytest.mark.parametrize("T,form", [(2, 1), (5, 2)])
def test_replay_equals_windows_with_known_acceptance(dev, T, form):
    """The same schedule through kda_decode_window, which needs the accepted counts at launch:
    window i with accept = acc_i commits what the replay call of window i + 1 commits, bit for
    bit, and window i + 1 from that state (accept = 0) gives the replay call's outputs.  With
    T + Tp = 4 tokens per call both run token by token and the outputs agree bit for bit; with
    10 the replay runs as one chunk (the window through form 2 as well), whose outputs come
    from a chunk that starts before the replayed tokens, so they agree to the bar."""
    B, H, W = 8, 4, 4
    xs, accepts, init, outs, state = _serving_loop(dev, B, T, H, 128, 128, torch.bfloat16, W, seed=7)
    ref = init.clone()
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    for i, x in enumerate(xs):
        o_ref = kda.kda_decode_window(*(x[n] for n in NAMES), ref.clone(), zero, form=form)
        torch.cuda.synchronize()
        if form == 1:
            assert torch.equal(outs[i], o_ref), f"window {i}: outputs differ from kda_decode_window"
        else:
            assert_close(outs[i], _np(o_ref), TOL[torch.bfloat16], f"window {i} o against the window form")
        kda.kda_decode_window(*(x[n] for n in NAMES), ref, accepts[i], output_o=False, form=form)
    torch.cuda.synchronize()
    assert torch.equal(state, ref), "committed state differs from kda_decode_window with known counts"


def test_replay_fused_gate_and_epilogue(dev):
    """Decay logits with the per-head gate and the output epilogue fused in, through replays of
    accepted prefixes: outputs and the committed state against the oracles (gate, recurrence,
    epilogue) window by window."""
    B, T, H, W, d = 4, 3, 2, 3, 128
    w = workloads.custom([1] * B, H, d, d, torch.bfloat16)
    xs = [workloads.decode_window_inputs(w, T, i, device=dev, seed=13) for i in range(W)]
    lz = [workloads.layer_inputs(B * T, H, d, torch.bfloat16, device=dev, seed=30 + i) for i in range(W)]
    A_log = lz[0]["A_log"]
    z = [l["z"].view(B, T, H, d).contiguous() for l in lz]
    u = [l["u"].view(B, T, H, d).contiguous() for l in lz]
    norm_w = lz[0]["norm_w"]
    accepts = [torch.tensor(a, dtype=torch.int32, device=dev) for a in ([3, 0, 1, 2], [1, 2, 3, 0], [0, 3, 2, 1])]
    init = workloads.random_state(B, H, d, d, device=dev, seed=13)
    state = init.clone()
    committed = _np(init).copy()
    for i, x in enumerate(xs):
        prev = None if i == 0 else {"q": xs[i - 1]["q"], "k": xs[i - 1]["k"], "v": xs[i - 1]["v"], "gate": z[i - 1],
                                    "beta": xs[i - 1]["beta"]}
        o, y = kda.kda_decode_window_replay(prev, None if i == 0 else accepts[i - 1], x["q"], x["k"], x["v"], z[i],
                                            x["beta"], state, gate_A_log=A_log, out_gate=u[i], norm_w=norm_w)
        torch.cuda.synchronize()
        if i > 0:  # the state committed by this call: the previous window's accepted prefix
            assert_close(state, committed, TOL[torch.bfloat16], f"state committed in call {i}")
        st = committed.copy()
        o_w = []
        acc = [int(a) for a in accepts[i].cpu()]
        nxt = committed.copy()
        for t in range(T):
            g = layer.gate(_np(z[i][:, t]), _np(A_log))
            o_t, st = oracle.decode(_np(x["q"][:, t]), _np(x["k"][:, t]), _np(x["v"][:, t]), g, _np(x["beta"][:, t]),
                                    st, inplace=True)
            o_w.append(o_t)
            for b in range(B):
                if acc[b] == t + 1:
                    nxt[b] = st[b]
        o_ref = np.stack(o_w, axis=1)
        assert_close(o, o_ref, TOL[torch.bfloat16], f"window {i} o")
        y_ref = layer.out_norm_gate(o_ref, _np(u[i]), _np(norm_w), 1e-6)
        yv = _np(y)
        rms = float(np.sqrt(np.mean(y_ref * y_ref)))
        assert np.all(np.abs(yv - y_ref) <= TOL[torch.bfloat16] * rms + 2.0 ** -8 * np.abs(y_ref)), f"window {i} y"
        committed = nxt


def test_replay_workload_shape(dev):
    """The decode workload's shape (B=256 x H=96, bf16): three windows of 4 with seeded accepted
    counts, the committed state and the last window's outputs on 48 sampled heads."""
    B, T, H, W = 256, 4, 96, 3
    xs, accepts, init, outs, state = _serving_loop(dev, B, T, H, 128, 128, torch.bfloat16, W, seed=0)
    idx = [(b, h) for b in range(0, B, 43) for h in range(0, H, 13)][:48]
    bs = sorted({b for b, _ in idx})
    sub = lambda t: t[bs].contiguous()
    xs_s = [{n: sub(x[n]) for n in NAMES} for x in xs]
    acc_s = [sub(a) for a in accepts]
    o_ref, s_ref = _oracle_loop(xs_s, acc_s, sub(init))
    assert_close(sub(outs[-1]), o_ref[-1], TOL[torch.bfloat16], "last window o (sampled sequences)")
    assert_close(sub(state), s_ref, TOL[torch.bfloat16], "committed state (sampled sequences)")
