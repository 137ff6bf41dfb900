"""GPU parity of the layer core's speculative-decoding call (kda_decode_layer_window_replay): each
call replays the previous window's accepted prefix through ShortConv + Swish (+ L2 for q, k), the
gate and the recurrence, commits the state and the convolution cache after it, and runs the new
window without committing it.  Against the stage oracles (oracle/layer.py: ShortConv, gate,
epilogue) and the fp64 recurrence oracle window by window; the committed cache exactly (it holds
inputs); and against successive kda_decode_layer_step calls.  Outputs start as NaN."""
import numpy as np
import pytest
import torch

import gated_delta_rule_51_amd as kda
import oracle
import workloads
from oracle import layer
from parity import TOL, assert_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


def _np(t):
    return t.detach().cpu().double().numpy()


def _inputs(dev, B, T, H, dk, dv, dtype, W, seed, fused):
    """W windows of raw q | k | v rows, decay logits (or log-decay) and beta; the layer's weights."""
    C = 2 * dk + dv
    wins = []
    for i in range(W):
        lx = workloads.layer_inputs(B * T, H, C, dtype, nseq=B, device=dev, seed=seed + 10 * i)
        lz = workloads.layer_inputs(B * T, H, dk, dtype, device=dev, seed=seed + 10 * i + 1)
        x = workloads.decode_window_inputs(workloads.custom([1] * B, H, dk, dv, dtype), T, i, device=dev, seed=seed)
        wins.append({"qkv": lx["x"].view(B, T, H, C).contiguous(),
                     "gate": (lz["z"] if fused else x["log_alpha"].view(B * T, H, dk)).view(B, T, H, dk).contiguous(),
                     "beta": x["beta"]})
    base = workloads.layer_inputs(B, H, C, dtype, nseq=B, device=dev, seed=seed + 5)
    lw = workloads.layer_inputs(B, H, dk, dtype, device=dev, seed=seed + 6)
    lu = [workloads.layer_inputs(B * T, H, dv, dtype, device=dev, seed=seed + 10 * i + 2) for i in range(W)]
    extra = {"conv_w": base["conv_w"], "cache": base["conv_cache"], "A_log": lw["A_log"] if fused else None,
             "u": [l["u"].view(B, T, H, dv).contiguous() for l in lu] if fused else None,
             "norm_w": workloads.layer_inputs(1, H, dv, dtype, device=dev, seed=seed + 7)["norm_w"] if fused else None}
    return wins, extra


def _oracle_window(x, committed, cache, conv_w, A_log, dk, acc):
    """One window from the committed state and cache, per sequence: outputs of every token, and the
    state and cache after its first acc[b] tokens."""
    qkv, gate, beta = _np(x["qkv"]), _np(x["gate"]), _np(x["beta"])
    B, T, H, C = qkv.shape
    w = _np(conv_w)
    o = np.zeros((B, T, H, C - 2 * dk))
    st_out, c_out = committed.copy(), cache.copy()
    for b in range(B):
        parts = {}
        for name, lo, hi, l2 in (("q", 0, dk, True), ("k", dk, 2 * dk, True), ("v", 2 * dk, C, False)):
            parts[name] = layer.short_conv(qkv[b, :, :, lo:hi], w[:, lo:hi], None, cache[b:b + 1, :, lo:hi],
                                           l2norm=l2, eps=1e-6)[0]
        g = layer.gate(gate[b], _np(A_log)) if A_log is not None else gate[b]
        st = committed[b:b + 1].copy()
        for t in range(T):
            o_t, st = oracle.decode(parts["q"][t][None], parts["k"][t][None], parts["v"][t][None], g[t][None],
                                    beta[b, t][None], st)
            o[b, t] = o_t[0]
            if acc[b] == t + 1:
                st_out[b] = st[0]
        c_out[b] = layer.short_conv(qkv[b, :acc[b]], w, None, cache[b:b + 1])[1][0] if acc[b] > 0 else cache[b]
    return o, st_out, c_out


@pytest.mark.parametrize("dtype,dk,dv,fused", [(torch.bfloat16, 128, 128, True), (torch.float32, 16, 64, False),
                                               (torch.bfloat16, 64, 32, True), (torch.bfloat16, 128, 128, False)])
def test_layer_window_serving_loop_matches_oracles(dev, dtype, dk, dv, fused):
    """Five sequences, four windows of 4 tokens, accepted counts 0..4 (nothing and everything
    accepted both occur), with and without the gate from logits and the epilogue: outputs (and y)
    of every window, and the state and cache committed by a final replay."""
    B, T, H, W = 5, 4, 3, 4
    wins, ex = _inputs(dev, B, T, H, dk, dv, dtype, W, seed=dk + dv, fused=fused)
    accepts = [torch.tensor(a, dtype=torch.int32, device=dev) for a in
               ([0, 4, 2, 1, 3], [4, 0, 3, 2, 1], [1, 2, 0, 4, 4], [3, 1, 4, 0, 2])]
    state0 = workloads.random_state(B, H, dk, dv, device=dev, seed=dk)
    state, cache = state0.clone(), ex["cache"].clone()
    say(f"  case: layer window loop B={B} T={T} H={H} dk={dk} dv={dv} {dtype} fused={fused}")
    outs = []
    for i, x in enumerate(wins):
        prev = None if i == 0 else wins[i - 1]
        o = torch.full((B, T, H, dv), float("nan"), dtype=torch.float32, device=dev)
        o, y = kda.kda_decode_layer_window_replay(prev, None if i == 0 else accepts[i - 1], x["qkv"], x["gate"],
                                                  x["beta"], ex["conv_w"], cache, state, dk=dk, gate_A_log=ex["A_log"],
                                                  out_gate=ex["u"][i] if fused else None, norm_w=ex["norm_w"], o=o)
        outs.append((o, y))
    one, _ = _inputs(dev, B, 1, H, dk, dv, dtype, 1, seed=99, fused=fused)
    kda.kda_decode_layer_window_replay(wins[-1], accepts[-1], one[0]["qkv"], one[0]["gate"], one[0]["beta"],
                                       ex["conv_w"], cache, state, dk=dk, gate_A_log=ex["A_log"])
    torch.cuda.synchronize()
    committed, c_ref = _np(state0), _np(ex["cache"])
    for i, x in enumerate(wins):
        acc = [int(a) for a in accepts[i].cpu()]
        o_ref, committed, c_ref = _oracle_window(x, committed, c_ref, ex["conv_w"], ex["A_log"], dk, acc)
        assert_close(outs[i][0], o_ref, TOL[dtype], f"window {i} o")
        if fused:
            y_ref = layer.out_norm_gate(o_ref, _np(ex["u"][i]), _np(ex["norm_w"]), 1e-6)
            yv = _np(outs[i][1])
            rms = float(np.sqrt(np.mean(y_ref * y_ref)))
            assert np.all(np.abs(yv - y_ref) <= TOL[dtype] * rms + 2.0 ** -8 * np.abs(y_ref)), f"window {i} y"
    assert_close(state, committed, TOL[dtype], "committed state")
    assert np.array_equal(_np(cache), c_ref), "committed convolution cache"


def test_layer_window_equals_layer_steps(dev):
    """A window from the committed state and cache gives, token by token, the outputs of
    kda_decode_layer_step calls from copies of them (the same per-token arithmetic, 1e-5), and a
    replay of all T tokens commits their state and cache."""
    B, T, H, dk, dv = 4, 5, 2, 128, 128
    wins, ex = _inputs(dev, B, T, H, dk, dv, torch.bfloat16, 1, seed=3, fused=True)
    x = wins[0]
    state0 = workloads.random_state(B, H, dk, dv, device=dev, seed=3)
    s_w, c_w = state0.clone(), ex["cache"].clone()
    o_w, _ = kda.kda_decode_layer_window_replay(None, None, x["qkv"], x["gate"], x["beta"], ex["conv_w"], c_w, s_w,
                                                dk=dk, gate_A_log=ex["A_log"])
    s_s, c_s = state0.clone(), ex["cache"].clone()
    o_s = []
    for t in range(T):
        o_t, _ = kda.kda_decode_layer_step(x["qkv"][:, t].contiguous(), ex["conv_w"], c_s, x["gate"][:, t].contiguous(),
                                           x["beta"][:, t].contiguous(), s_s, dk=dk, gate_A_log=ex["A_log"])
        o_s.append(o_t)
    torch.cuda.synchronize()
    assert torch.equal(s_w, state0) and torch.equal(c_w, ex["cache"]), "the window committed something"
    assert_close(o_w, _np(torch.stack(o_s, dim=1)), 1e-5, "window vs layer steps o")
    full = torch.full((B,), T, dtype=torch.int32, device=dev)
    one, _ = _inputs(dev, B, 1, H, dk, dv, torch.bfloat16, 1, seed=8, fused=True)
    kda.kda_decode_layer_window_replay(x, full, one[0]["qkv"], one[0]["gate"], one[0]["beta"], ex["conv_w"], c_w,
                                       s_w, dk=dk, gate_A_log=ex["A_log"])
    torch.cuda.synchronize()
    assert_close(s_w, _np(s_s), 1e-5, "state committed by the replay vs layer steps")
    assert torch.equal(c_w, c_s), "cache committed by the replay vs layer steps"
