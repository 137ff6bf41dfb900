"""GPU parity of decode windows evaluated as one chunk on the matrix cores (kda_decode_window_form
with form 2, and the automatic choice from 6 tokens on for bf16 with dk = dv = 128): against the
fp64 oracle's decode steps (outputs of every token; state after each sequence's accepted count),
the committed state bit for bit independent of the drafts after the accepted prefix, the replay of
a serving loop through the same form, and the decode workload's shape.  Outputs start as NaN."""
import numpy as np
import pytest
import torch

import gated_delta_rule_51_amd as kda
import oracle
import workloads
from parity import TOL, assert_close, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_alpha", "beta")
BF = torch.bfloat16


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


def _np(t):
    return t.detach().cpu().double().numpy()


def _oracle_window(x, init, accepts):
    """T oracle decode steps from ``init``; the state kept per sequence is the one after its first
    accepts[b] tokens.  Returns (o [B, T, H, dv], state [B, H, dk, dv]) in float64."""
    T = x["q"].shape[1]
    st = _np(init)
    snaps, outs = [st], []
    for t in range(T):
        ot, st = oracle.decode(*(_np(x[n][:, t]) for n in NAMES), st)
        outs.append(ot)
        snaps.append(st)
    return np.stack(outs, axis=1), np.stack([snaps[a][b] for b, a in enumerate(accepts)])


def _case(dev, B, T, H, accept, seed, form=2, gate="neg_softplus", edit=None, output_o=True):
    w = workloads.custom([1] * B, H, 128, 128, BF, gate)
    x = workloads.decode_window_inputs(w, T, 0, device=dev, seed=seed)
    if edit is not None:
        edit(x)
    init = workloads.random_state(B, H, 128, 128, device=dev, seed=seed)
    state = init.clone()
    acc = None if accept is None else torch.tensor(accept, dtype=torch.int32, device=dev)
    say(f"  case: chunk-form window B={B} T={T} H={H} accept={accept} form={form} gate={gate}")
    o = torch.full((B, T, H, 128), float("nan"), dtype=torch.float32, device=dev) if output_o else None
    o = kda.kda_decode_window(*(x[n] for n in NAMES), state, acc, o=o, output_o=output_o, form=form)
    torch.cuda.synchronize()
    accepts = [T] * B if accept is None else [min(max(a, 0), T) for a in accept]
    o_ref, st_ref = _oracle_window(x, init, accepts)
    if output_o:
        assert_close(o, o_ref, TOL[BF], "window o")
    assert_close(state, st_ref, TOL[BF], "window state")
    for b, a in enumerate(accepts):
        if a == 0:
            assert torch.equal(state[b], init[b]), f"sequence {b} accepted nothing but its state changed"
    return x, init, state, o


@pytest.mark.parametrize("T", [1, 3, 8, 11, 16])
def test_chunk_window_matches_oracle(dev, T):
    """Seven sequences, accepted counts 0, 1, T/2, T - 1, T and two out of range."""
    acc = [0, 1, T // 2, T - 1, T, T + 5, -2]
    _case(dev, len(acc), T, 3, acc, seed=100 + T)


def test_chunk_window_without_accept_or_outputs(dev):
    _case(dev, 3, 8, 2, None, seed=5)
    _case(dev, 4, 12, 2, [3, 0, 12, 7], seed=6, output_o=False)


def test_chunk_window_strong_decay(dev):
    """Log-decay uniform on [-5, 0), and at the bound -5 for every channel and token of a
    16-token window (a cumulative decay of -80, the chunk form's widest range)."""
    _case(dev, 6, 16, 2, [0, 5, 8, 13, 15, 16], seed=31, gate="uniform")

    def floor(x):
        x["log_alpha"].fill_(-5.0)
    _case(dev, 6, 16, 2, [0, 1, 2, 9, 15, 16], seed=32, edit=floor)


def test_chunk_window_is_the_automatic_choice_from_six_tokens(dev):
    """kda_decode_window picks the chunk form for T >= 6 (bf16, 128 x 128): bit for bit the
    explicit form 2; below 6 tokens it keeps the token-by-token form (form 1)."""
    w = workloads.custom([1] * 5, 4, 128, 128, BF)
    init = workloads.random_state(5, 4, 128, 128, device=dev, seed=2)
    acc = torch.tensor([0, 3, 8, 5, 2], dtype=torch.int32, device=dev)
    for T, form in ((8, 2), (12, 2), (6, 2), (5, 1), (4, 1)):
        x = workloads.decode_window_inputs(w, T, 0, device=dev, seed=T)
        s1, s2 = init.clone(), init.clone()
        o1 = kda.kda_decode_window(*(x[n] for n in NAMES), s1, acc)
        o2 = kda.kda_decode_window(*(x[n] for n in NAMES), s2, acc, form=form)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2), f"T={T}: automatic choice is not form {form}"


def test_chunk_window_commit_depends_only_on_accepted_prefix(dev):
    """The committed state after a tokens of a T-token window equals, bit for bit, the chunk
    form's state for a window of those a tokens alone (all accepted), and the drafts after the
    prefix can be anything: a window whose drafts past a are replaced commits the same state."""
    B, H, T = 4, 3, 12
    w = workloads.custom([1] * B, H, 128, 128, BF)
    x = workloads.decode_window_inputs(w, T, 0, device=dev, seed=9)
    init = workloads.random_state(B, H, 128, 128, device=dev, seed=9)
    for a in (1, 5, 11):
        acc = torch.full((B,), a, dtype=torch.int32, device=dev)
        s_full, s_pre, s_alt = init.clone(), init.clone(), init.clone()
        kda.kda_decode_window(*(x[n] for n in NAMES), s_full, acc, form=2)
        kda.kda_decode_window(*(x[n][:, :a].contiguous() for n in NAMES), s_pre, None, form=2)
        y = {n: x[n].clone() for n in NAMES}
        for n in NAMES:
            y[n][:, a:] = torch.flip(x[n][:, a:], dims=[0])  # other sequences' drafts
        kda.kda_decode_window(*(y[n] for n in NAMES), s_alt, acc, form=2)
        torch.cuda.synchronize()
        assert torch.equal(s_full, s_pre), f"a={a}: committed state differs from the prefix window's"
        assert torch.equal(s_full, s_alt), f"a={a}: committed state depends on the drafts after the prefix"


def test_chunk_and_token_forms_agree(dev):
    """Form 1 (token by token, near-exact fp32) and form 2 on the same windows: within the bar."""
    B, H, T = 6, 4, 10
    w = workloads.custom([1] * B, H, 128, 128, BF)
    x = workloads.decode_window_inputs(w, T, 0, device=dev, seed=12)
    init = workloads.random_state(B, H, 128, 128, device=dev, seed=12)
    acc = workloads.window_accept(B, T, device=dev, seed=12)
    s1, s2 = init.clone(), init.clone()
    o1 = kda.kda_decode_window(*(x[n] for n in NAMES), s1, acc, form=1)
    o2 = kda.kda_decode_window(*(x[n] for n in NAMES), s2, acc, form=2)
    torch.cuda.synchronize()
    assert_close(o2, _np(o1), TOL[BF], "chunk vs token form o")
    assert_close(s2, _np(s1), TOL[BF], "chunk vs token form state")


def test_chunk_window_many_heads_per_workgroup(dev):
    """1,200 heads: more than the persistent grid holds, so workgroups loop over heads with
    each sequence's own accepted count; every head checked."""
    B, H, T = 300, 4, 8
    _case(dev, B, T, H, workloads.window_accept(B, T, seed=3).tolist(), seed=3)


def test_chunk_window_replay_serving_loop(dev):
    """Windows of 8 with the previous window's accepted prefix replayed in front (at most 16
    tokens per call, so the automatic choice is the chunk form): every window's outputs and the
    committed state after a final replay against the oracle's steps window by window."""
    B, T, H, W = 6, 8, 3, 4
    w = workloads.custom([1] * B, H, 128, 128, BF)
    xs = [workloads.decode_window_inputs(w, T, i, device=dev, seed=40) for i in range(W)]
    accepts = [torch.tensor(a, dtype=torch.int32, device=dev) for a in
               ([0, 8, 3, 1, 5, 7], [8, 0, 2, 6, 4, 0], [1, 1, 8, 0, 3, 2], [5, 2, 0, 8, 8, 1])]
    init = workloads.random_state(B, H, 128, 128, device=dev, seed=40)
    state = init.clone()
    say(f"  case: chunk-form replay loop B={B} T={T} H={H}, {W} windows")
    outs = []
    for i, x in enumerate(xs):
        prev = None if i == 0 else {"q": xs[i - 1]["q"], "k": xs[i - 1]["k"], "v": xs[i - 1]["v"],
                                    "gate": xs[i - 1]["log_alpha"], "beta": xs[i - 1]["beta"]}
        o = torch.full((B, T, H, 128), float("nan"), dtype=torch.float32, device=dev)
        o, _ = kda.kda_decode_window_replay(prev, None if i == 0 else accepts[i - 1], x["q"], x["k"], x["v"],
                                            x["log_alpha"], x["beta"], state, o=o)
        outs.append(o)
    last = xs[-1]
    one = workloads.decode_window_inputs(w, 1, W * T, device=dev, seed=40)
    kda.kda_decode_window_replay({"q": last["q"], "k": last["k"], "v": last["v"], "gate": last["log_alpha"],
                                  "beta": last["beta"]}, accepts[-1], one["q"], one["k"], one["v"],
                                 one["log_alpha"], one["beta"], state)
    torch.cuda.synchronize()
    committed = _np(init)
    for i, (x, acc) in enumerate(zip(xs, accepts)):
        acc = [int(a) for a in acc.cpu()]
        st = committed.copy()
        o_w, nxt = [], committed.copy()
        for t in range(T):
            o_t, st = oracle.decode(*(_np(x[n][:, t]) for n in NAMES), st)
            o_w.append(o_t)
            for b in range(B):
                if acc[b] == t + 1:
                    nxt[b] = st[b]
        assert_close(outs[i], np.stack(o_w, axis=1), TOL[BF], f"window {i} o")
        committed = nxt
    assert_close(state, committed, TOL[BF], "committed state")


def test_chunk_window_workload_shape(dev):
    """The decode workload's shape (B=256 x H=96), two windows of 8 with seeded accepted counts
    through kda_decode_window (the chunk form); the oracle on 48 sampled heads."""
    w = workloads.workload(4)
    B, H, T = w.nseq, w.H, 8
    state = workloads.decode_initial_state(B, H, w.dk, w.dv, device=dev)
    rng = np.random.default_rng(7)
    bi = torch.tensor(rng.integers(0, B, 48), device=dev)
    hi = torch.tensor(rng.integers(0, H, 48), device=dev)
    ref_state = state[bi, hi].cpu().double().numpy()
    say(f"  case: chunk-form window B={B} H={H} T={T}, 2 windows")
    for win in range(2):
        x = workloads.decode_window_inputs(w, T, win, device=dev)
        acc = workloads.window_accept(B, T, device=dev, seed=win)
        o = torch.full((B, T, H, w.dv), float("nan"), dtype=torch.float32, device=dev)
        o = kda.kda_decode_window(*(x[n] for n in NAMES), state, acc, o=o)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all(), "an output row was not written"
        sub = {n: x[n][bi, :, hi].unsqueeze(2).contiguous() for n in NAMES}
        o_ref, st = _oracle_window(sub, torch.from_numpy(ref_state).unsqueeze(1), acc[bi].tolist())
        ref_state = st[:, 0]
        assert_close(o[bi, :, hi], o_ref[:, :, 0], TOL[BF], f"window {win} o")
        assert_close(state[bi, hi], ref_state, TOL[BF], f"window {win} state")
    del state
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [6, 8, 16])
def test_chunk_window_gate_from_logits(dev, T):
    """kda_decode_window_fused with decay logits and the per-head gate from 6 tokens on runs as
    one chunk (the gate in fp32, split hi + lo for the chunk's decay sums), with the epilogue:
    outputs, y and the state after each accepted count against the oracles (gate, decode steps,
    epilogue)."""
    from oracle import layer
    B, H = 5, 3
    w = workloads.custom([1] * B, H, 128, 128, BF)
    x = workloads.decode_window_inputs(w, T, 0, device=dev, seed=70 + T)
    lk = workloads.layer_inputs(B * T, H, 128, BF, device=dev, seed=71 + T)
    lv = workloads.layer_inputs(B * T, H, 128, BF, device=dev, seed=72 + T)
    z = lk["z"].view(B, T, H, 128).contiguous()
    u = lv["u"].view(B, T, H, 128).contiguous()
    init = workloads.random_state(B, H, 128, 128, device=dev, seed=T)
    state = init.clone()
    accepts = [0, 1, T // 2, T - 1, T]
    acc = torch.tensor(accepts, dtype=torch.int32, device=dev)
    say(f"  case: chunk-form window with the gate from logits B={B} T={T} H={H}")
    o = torch.full((B, T, H, 128), float("nan"), dtype=torch.float32, device=dev)
    o, y = kda.kda_decode_window_fused(x["q"], x["k"], x["v"], z, x["beta"], state, acc, gate_A_log=lk["A_log"],
                                       out_gate=u, norm_w=lv["norm_w"], o=o)
    torch.cuda.synchronize()
    g = layer.gate(_np(lk["z"]), _np(lk["A_log"])).reshape(B, T, H, 128)
    y_dict = dict(x)
    y_dict["log_alpha"] = torch.from_numpy(g)
    o_ref, st_ref = _oracle_window(y_dict, init, accepts)
    assert_close(o, o_ref, TOL[BF], "o")
    assert_close(state, st_ref, TOL[BF], "state")
    assert torch.equal(state[0], init[0]), "sequence 0 accepted nothing but its state changed"
    y_ref = layer.out_norm_gate(o_ref, _np(u), _np(lv["norm_w"]), 1e-6)
    rms = float(np.sqrt(np.mean(y_ref * y_ref)))
    assert np.all(np.abs(_np(y) - y_ref) <= TOL[BF] * rms + 2.0 ** -8 * np.abs(y_ref)), "y"
