"""GPU parity of the layer core's speculative-decoding call (kda_decode_layer_window_replay): each
call replays the previous window's accepted prefix through ShortConv + Swish (+ L2 for q, k), the
gate and the recurrence, commits the state and the convolution cache after it, and runs the new
window without committing it.  Against the stage oracles (oracle/layer.py: ShortConv, gate,
epilogue) and the fp64 recurrence oracle window by window; the committed cache exactly (it holds
inputs); and against successive kda_decode_layer_step calls.  Both evaluation forms: token by
token (q, k, v and the decay stay fp32: against the oracle stages in fp64), and (bf16, dk = dv =
128, 6 to 16 tokens with the replay) the prologue pass + one chunk on the matrix cores, whose
prologue rounds its outputs to bf16 as the layer prefill does (against the oracle stages with
their outputs rounded to bf16).  Outputs start as NaN."""
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


def _bf16(a):
    """fp64 array rounded to bf16 (nearest even), back in fp64."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).double().numpy()


def _chunk_form(dtype, dk, dv, T, Tp, form):
    """Whether kda_decode_layer_window_replay evaluates a call as one chunk."""
    return form != 1 and dtype == torch.bfloat16 and dk == dv == 128 and 6 <= T + Tp <= 16


def _oracle_window(x, committed, cache, conv_w, A_log, dk, acc, rounded=False):
    """One window from the committed state and cache, per sequence: outputs of every token, and the
    state and cache after its first acc[b] tokens.  rounded: the prologue's outputs (convolved and
    normalised q, k, v; the log-decay) rounded to bf16 before the recurrence."""
    rnd = _bf16 if rounded else (lambda a: a)
    qkv, gate, beta = _np(x["qkv"]), _np(x["gate"]), _np(x["beta"])
    B, T, H, C = qkv.shape
    w = _np(conv_w)
    o = np.zeros((B, T, H, C - 2 * dk))
    st_out, c_out = committed.copy(), cache.copy()
    for b in range(B):
        parts = {}
        for name, lo, hi, l2 in (("q", 0, dk, True), ("k", dk, 2 * dk, True), ("v", 2 * dk, C, False)):
            parts[name] = rnd(layer.short_conv(qkv[b, :, :, lo:hi], w[:, lo:hi], None, cache[b:b + 1, :, lo:hi],
                                               l2norm=l2, eps=1e-6)[0])
        g = rnd(layer.gate(gate[b], _np(A_log))) if A_log is not None else gate[b]
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
    of every window, and the state and cache committed by a final replay.  (bf16 128 x 128: the
    first window and the final replay of one token run token by token, the replaying windows as
    one chunk.)"""
    _serving_loop(dev, dtype, dk, dv, fused, B=5, T=4, H=3,
                  accepts=([0, 4, 2, 1, 3], [4, 0, 3, 2, 1], [1, 2, 0, 4, 4], [3, 1, 4, 0, 2]))


@pytest.mark.parametrize("form", [1, 2])
def test_layer_window_forms_with_eight_token_windows(dev, form):
    """Windows of 8 tokens with up to 8 replayed (16 rows: the largest one-chunk case), accepted
    counts 0..8, gate from logits and epilogue, in each form explicitly."""
    _serving_loop(dev, torch.bfloat16, 128, 128, True, B=6, T=8, H=2,
                  accepts=([0, 8, 3, 1, 5, 7], [8, 0, 2, 6, 4, 0], [1, 1, 8, 0, 3, 2]), form=form)


def _serving_loop(dev, dtype, dk, dv, fused, B, T, H, accepts, form=None):
    W = len(accepts)
    wins, ex = _inputs(dev, B, T, H, dk, dv, dtype, W, seed=dk + dv, fused=fused)
    accepts = [torch.tensor(a, dtype=torch.int32, device=dev) for a in accepts]
    state0 = workloads.random_state(B, H, dk, dv, device=dev, seed=dk)
    state, cache = state0.clone(), ex["cache"].clone()
    say(f"  case: layer window loop B={B} T={T} H={H} dk={dk} dv={dv} {dtype} fused={fused} form={form}")
    outs = []
    for i, x in enumerate(wins):
        prev = None if i == 0 else wins[i - 1]
        o = torch.full((B, T, H, dv), float("nan"), dtype=torch.float32, device=dev)
        f = form if (form != 2 or i > 0 or T >= 6) else None  # (a first window below 6 tokens has no chunk form)
        o, y = kda.kda_decode_layer_window_replay(prev, None if i == 0 else accepts[i - 1], x["qkv"], x["gate"],
                                                  x["beta"], ex["conv_w"], cache, state, dk=dk, gate_A_log=ex["A_log"],
                                                  out_gate=ex["u"][i] if fused else None, norm_w=ex["norm_w"], o=o,
                                                  form=f)
        outs.append((o, y))
    one, _ = _inputs(dev, B, 1, H, dk, dv, dtype, 1, seed=99, fused=fused)
    kda.kda_decode_layer_window_replay(wins[-1], accepts[-1], one[0]["qkv"], one[0]["gate"], one[0]["beta"],
                                       ex["conv_w"], cache, state, dk=dk, gate_A_log=ex["A_log"],
                                       form=form if (form != 2 or 1 + T >= 6) else None)
    torch.cuda.synchronize()
    # call i runs window i (from the state committed by call i) and commits window i - 1's prefix;
    # the last call commits the last window's
    chunk = [_chunk_form(dtype, dk, dv, T, 0 if i == 0 else T, form) for i in range(W)]
    chunk.append(_chunk_form(dtype, dk, dv, 1, T, form))
    committed, c_ref = _np(state0), _np(ex["cache"])
    for i, x in enumerate(wins):
        acc = [int(a) for a in accepts[i].cpu()]
        o_ref = _oracle_window(x, committed, c_ref, ex["conv_w"], ex["A_log"], dk, acc, chunk[i])[0]
        _, committed, c_ref = _oracle_window(x, committed, c_ref, ex["conv_w"], ex["A_log"], dk, acc, chunk[i + 1])
        assert_close(outs[i][0], o_ref, TOL[dtype], f"window {i} o ({'one chunk' if chunk[i] else 'token by token'})")
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
                                       s_w, dk=dk, gate_A_log=ex["A_log"], form=1)
    torch.cuda.synchronize()
    assert_close(s_w, _np(s_s), 1e-5, "state committed by the replay vs layer steps")
    assert torch.equal(c_w, c_s), "cache committed by the replay vs layer steps"


def test_layer_window_chunk_form_is_the_automatic_choice(dev):
    """From 6 tokens (window plus replay) on, bf16 with dk = dv = 128, the call without a form
    is bit for bit the one-chunk form (workspace allocated by the binding, or the caller's);
    each form meets its oracle on o, y and the committed state, and both commit the same cache
    exactly."""
    B, T, H, dk, dv = 4, 4, 3, 128, 128
    wins, ex = _inputs(dev, B, T, H, dk, dv, torch.bfloat16, 2, seed=21, fused=True)
    acc = torch.tensor([0, 4, 2, 3], dtype=torch.int32, device=dev)
    state0 = workloads.random_state(B, H, dk, dv, device=dev, seed=21)
    res = {}
    need = kda.kda_decode_layer_window_workspace_bytes(B, T, T, H, dk, dv, torch.bfloat16)
    assert need == 1024 * B * H * 2 * T
    for name, form, ws in (("auto", None, None), ("given", None, torch.empty(need, dtype=torch.uint8, device=dev)),
                           ("chunk", 2, None), ("token", 1, None)):
        st, cc = state0.clone(), ex["cache"].clone()
        o = torch.full((B, T, H, dv), float("nan"), dtype=torch.float32, device=dev)
        o, y = kda.kda_decode_layer_window_replay(wins[0], acc, wins[1]["qkv"], wins[1]["gate"], wins[1]["beta"],
                                                  ex["conv_w"], cc, st, dk=dk, gate_A_log=ex["A_log"],
                                                  out_gate=ex["u"][1], norm_w=ex["norm_w"], o=o, form=form,
                                                  workspace=ws)
        torch.cuda.synchronize()
        res[name] = (o, y, st, cc)
    for name in ("auto", "given"):
        assert all(torch.equal(a, b) for a, b in zip(res[name], res["chunk"])), f"{name} is not the chunk form"
    oc, yc, sc, cc = res["chunk"]
    ot, yt, stt, ct = res["token"]
    assert torch.equal(cc, ct), "the forms committed different caches"
    acc_l = [int(a) for a in acc.cpu()]
    committed = _oracle_window(wins[0], _np(state0), _np(ex["cache"]), ex["conv_w"], ex["A_log"], dk, acc_l, True)[1]
    o_ref = _oracle_window(wins[1], committed, _np(cc), ex["conv_w"], ex["A_log"], dk, [0] * B, True)[0]
    assert_close(oc, o_ref, TOL[torch.bfloat16], "one-chunk form o")
    assert_close(sc, committed, TOL[torch.bfloat16], "one-chunk form committed state")
    committed = _oracle_window(wins[0], _np(state0), _np(ex["cache"]), ex["conv_w"], ex["A_log"], dk, acc_l)[1]
    o_ref_t = _oracle_window(wins[1], committed, _np(ct), ex["conv_w"], ex["A_log"], dk, [0] * B)[0]
    assert_close(ot, o_ref_t, 1e-4, "token form o")
    assert_close(stt, committed, 1e-4, "token form committed state")
    for yv, orf, name in ((yc, o_ref, "one chunk"), (yt, o_ref_t, "token by token")):
        yr = layer.out_norm_gate(orf, _np(ex["u"][1]), _np(ex["norm_w"]), 1e-6)
        rms = float(np.sqrt(np.mean(yr * yr)))
        assert np.all(np.abs(_np(yv) - yr) <= TOL[torch.bfloat16] * rms + 2.0 ** -8 * np.abs(yr)), f"{name} y"
    with pytest.raises(ValueError):
        kda.kda_decode_layer_window_replay(None, None, wins[1]["qkv"], wins[1]["gate"], wins[1]["beta"], ex["conv_w"],
                                           ex["cache"].clone(), state0.clone(), dk=dk, form=2)  # 4 tokens: no chunk form


def test_layer_window_workload_shape_sampled_heads(dev):
    """The decode workload's shape (B=256 x H=96) in the launch configuration the benchmark times:
    windows of 4 with the previous window's accepted prefix replayed (T + Tp = 8: one chunk, the
    prologue pass over 24,576 heads), gate from logits; two calls.  On 48 sampled (sequence,
    head) pairs: the prologue's bf16 rows in the workspace within one bf16 rounding of the fp64
    stage oracles; the recurrence oracle fed those rows (the recurrence's own inputs -- an
    oracle that rounds by itself lands a few heavy-tailed values on the other side of a bf16
    boundary) against o and the committed state; the committed cache exactly."""
    w = workloads.workload(4)
    B, H, T, dk, dv = w.nseq, w.H, 4, 128, 128
    C = 2 * dk + dv
    wins = []
    for i in range(3):
        lx = workloads.layer_inputs(B * T, H, C, torch.bfloat16, nseq=B, device=dev, seed=60 + i)
        lz = workloads.layer_inputs(B * T, H, dk, torch.bfloat16, device=dev, seed=70 + i)
        xw = workloads.decode_window_inputs(w, T, i, device=dev)
        wins.append({"qkv": lx["x"].view(B, T, H, C), "gate": lz["z"].view(B, T, H, dk), "beta": xw["beta"]})
    conv_w, A_log = lx["conv_w"], lz["A_log"]
    cache = workloads.layer_inputs(B, H, C, torch.bfloat16, nseq=B, device=dev, seed=80)["conv_cache"]
    state = workloads.decode_initial_state(B, H, dk, dv, device=dev)
    accs = [workloads.window_accept(B, T, device=dev, seed=s, lo=0) for s in (1, 2)]
    rng = np.random.default_rng(11)
    bi, hi = rng.integers(0, B, 48), rng.integers(0, H, 48)
    bt, ht = torch.tensor(bi, device=dev), torch.tensor(hi, device=dev)
    ref_state = state[bt, ht].double().cpu().numpy()
    ref_cache = cache[bt, ht].double().cpu().numpy()
    need = kda.kda_decode_layer_window_workspace_bytes(B, T, T, H, dk, dv, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    cw, A = _np(conv_w), _np(A_log)
    say(f"  case: layer window B={B} H={H} T={T} with replay, 48 sampled heads")
    for i in (1, 2):
        o = torch.full((B, T, H, dv), float("nan"), dtype=torch.float32, device=dev)
        o, _ = kda.kda_decode_layer_window_replay(wins[i - 1], accs[i - 1], wins[i]["qkv"], wins[i]["gate"],
                                                  wins[i]["beta"], conv_w, cache, state, dk=dk, gate_A_log=A_log,
                                                  o=o, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all(), "an output row was not written"
        wb = ws.view(torch.bfloat16)
        cur = wb[:4 * B * T * H * 128].view(4, B, T, H, 128)[:, bt, :, ht].double().cpu().numpy()  # [48, 4, T, 128]
        pre = wb[4 * B * T * H * 128:].view(4, B, T, H, 128)[:, bt, :, ht].double().cpu().numpy()
        o_got = o[bt, :, ht].double().cpu().numpy()
        acc = accs[i - 1].cpu().numpy()
        o_ref = np.zeros_like(o_got)
        worst = 0.0
        for n in range(48):
            b, h = int(bi[n]), int(hi[n])
            rp = int(acc[b])
            rows = np.concatenate([_np(wins[i - 1]["qkv"][b, :rp, h]), _np(wins[i]["qkv"][b, :, h])])  # [rp + T, C]
            z = np.concatenate([_np(wins[i - 1]["gate"][b, :rp, h]), _np(wins[i]["gate"][b, :, h])])
            beta = np.concatenate([_np(wins[i - 1]["beta"][b, :rp, h]), _np(wins[i]["beta"][b, :, h])])
            # the prologue's rows against the stage oracles, within one bf16 rounding
            got = np.concatenate([pre[n][:, :rp], cur[n]], axis=1)  # [4 (q, k, v, g), rp + T, 128]
            stage = []
            for lo, l2 in ((0, True), (dk, True), (2 * dk, False)):
                stage.append(layer.short_conv(rows[:, None, lo:lo + 128], cw[h:h + 1, lo:lo + 128], None,
                                              ref_cache[n][None, None, lo:lo + 128], l2norm=l2, eps=1e-6)[0][:, 0])
            stage.append(layer.gate(z[:, None], A[h:h + 1])[:, 0])
            for j in range(4):
                ref = stage[j]
                tol = 2.0 ** -8 * np.abs(ref) + 1e-6 * np.sqrt(np.mean(ref * ref))
                assert np.all(np.abs(got[j] - ref) <= tol), f"call {i}, pair {n}: prologue output {'qkvg'[j]}"
            # the recurrence on those rows; the state commits after the prefix
            st = ref_state[n][None, None]
            committed = st
            for t in range(rp + T):
                ot, st = oracle.decode(got[0, t][None, None], got[1, t][None, None], got[2, t][None, None],
                                       got[3, t][None, None], beta[t][None, None], st)
                if t + 1 == rp:
                    committed = st
                if t >= rp:
                    o_ref[n, t - rp] = ot[0, 0]
            ref_state[n] = committed[0, 0]
            ref_cache[n] = layer.short_conv(rows[:rp, None], cw[h:h + 1], None, ref_cache[n][None, None])[1][0, 0] \
                if rp > 0 else ref_cache[n]
        assert_close(o_got, o_ref, TOL[torch.bfloat16], f"call {i} o (sampled heads)")
    assert_close(state[bt, ht], ref_state, TOL[torch.bfloat16], "committed state (sampled heads)")
    assert np.array_equal(cache[bt, ht].double().cpu().numpy(), ref_cache), "committed convolution cache"
    del state, cache, ws
    torch.cuda.empty_cache()
