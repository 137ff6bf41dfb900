"""GPU parity of the layer's passes around the recurrence (decay gate, ShortConv prologue,
RMSNorm + output-gate epilogue) against the fp64 layer oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import gated_delta_rule_51_amd as kda
import oracle
import workloads
from oracle import layer
from parity import TOL, assert_close, oracle_prefill, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


def _np(t):
    return t.detach().cpu().double().numpy()


def assert_rounded(x, ref, dtype, what):
    """fp32 results: the recurrence's bar (max|err| <= 1e-5 RMS(ref)).  Results written in
    bf16 are the fp32 value rounded to nearest: per element within half a unit in the last
    place (at most 2^-8 |ref|) plus the fp32 evaluation error."""
    if dtype == torch.float32:
        return assert_close(x, ref, TOL[torch.float32], what)
    xv, ref = _np(x), np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(xv - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * rms
    say(f"    {what}: max(err / bound) = {float(np.max(err / bound)) if ref.size else 0.0:.3f}")
    assert np.all(np.isfinite(xv)), f"{what}: non-finite"
    assert np.all(err <= bound), f"{what}: bf16 result off by more than half an ulp"


def _bf16_round(x):
    return torch.from_numpy(np.asarray(x)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("dtype,dk", [(torch.float32, 16), (torch.float32, 128), (torch.bfloat16, 128),
                                      (torch.bfloat16, 32)])
def test_gate_matches_oracle(dev, dtype, dk):
    x = workloads.layer_inputs(37, 3, dk, dtype, device=dev, seed=dk)
    say(f"  case: gate N=37 H=3 dk={dk} {dtype}")
    g = kda.kda_gate(x["z"], x["A_log"])
    torch.cuda.synchronize()
    ref = layer.gate(_np(x["z"]), _np(x["A_log"]))
    err = np.abs(_np(g) - ref)
    # fp32: the fp32 bar relative to the gate's range |g_min| = 5; bf16: the result is rounded
    # to the input dtype, so at most one unit in the last place (2^-7 relative) off
    tol = 1e-5 * 5 if dtype == torch.float32 else 2.0 ** -7 * np.abs(ref) + 1e-7
    assert np.all(err <= tol), f"gate error {err.max():.3e}"
    assert np.all(_np(g) >= -5.0) and np.all(_np(g) <= 0.0)
    z2 = x["z"].clone()
    kda.kda_gate(z2, x["A_log"], out=z2)  # in place
    torch.cuda.synchronize()
    assert torch.equal(z2, g)


def test_gate_feeds_prefill(dev):
    """Decay logits -> kda_gate -> kda_prefill against the oracle recurrence run on the
    oracle's gate (rounded to bf16, the dtype the recurrence takes)."""
    w = workloads.custom([40, 9], 2, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=8)
    li = workloads.layer_inputs(49, 2, 128, torch.bfloat16, device=dev, seed=8)
    g = kda.kda_gate(li["z"], li["A_log"])
    o, fin = kda.kda_prefill(x["q"], x["k"], x["v"], g, x["beta"], x["cu_seqlens"])
    torch.cuda.synchronize()
    g_ref = _bf16_round(layer.gate(_np(li["z"]), _np(li["A_log"])))
    x2 = dict(x)
    x2["log_alpha"] = torch.from_numpy(g_ref).to(torch.bfloat16).to(dev)
    o_ref, f_ref = oracle_prefill(x2)
    assert_close(o, o_ref, TOL[torch.bfloat16], "o")
    assert_close(fin, f_ref, TOL[torch.bfloat16], "final_state")


@pytest.mark.parametrize("dtype,d", [(torch.float32, 16), (torch.float32, 128), (torch.bfloat16, 128),
                                     (torch.bfloat16, 64)])
@pytest.mark.parametrize("l2norm", [False, True])
@pytest.mark.parametrize("with_cache", [False, True])
def test_short_conv_matches_oracle(dev, dtype, d, l2norm, with_cache):
    """Packed sequences of 5, 0, 1, 2, 17 and 33 tokens (empty, shorter than the filter,
    several lanes of rows), with and without an incoming cache."""
    seqlens = [5, 0, 1, 2, 17, 33]
    cu = torch.tensor(workloads.cu_seqlens_of(seqlens), dtype=torch.int32, device=dev)
    N, H = sum(seqlens), 3
    li = workloads.layer_inputs(N, H, d, dtype, nseq=len(seqlens), device=dev, seed=d + 7)
    cache = li["conv_cache"] if with_cache else None
    say(f"  case: short_conv seqlens={seqlens} H={H} d={d} {dtype} l2norm={l2norm} cache={with_cache}")
    y, c_out = kda.kda_short_conv(li["x"], li["conv_w"], cu, cache, l2norm=l2norm, eps=1e-6)
    torch.cuda.synchronize()
    y_ref, c_ref = layer.short_conv(_np(li["x"]), _np(li["conv_w"]), _np(cu),
                                    None if cache is None else _np(cache), l2norm=l2norm, eps=1e-6)
    assert_rounded(y, y_ref, dtype, "y")
    assert np.array_equal(_np(c_out), c_ref), "cache_out is a copy of inputs and must be exact"
    if with_cache:  # the cache updated in place
        c2 = cache.clone()
        kda.kda_short_conv(li["x"], li["conv_w"], cu, c2, l2norm=l2norm, eps=1e-6, cache_out=c2)
        torch.cuda.synchronize()
        assert torch.equal(c2, c_out)


def test_short_conv_resumes_across_calls(dev):
    """A sequence in two calls, the second starting from the first call's cache, equals
    one call (bitwise: every output reads the same inputs)."""
    li = workloads.layer_inputs(40, 2, 128, torch.bfloat16, device=dev, seed=3)
    y_all, c_all = kda.kda_short_conv(li["x"], li["conv_w"], l2norm=True)
    y1, c1 = kda.kda_short_conv(li["x"][:13].contiguous(), li["conv_w"], l2norm=True)
    y2, c2 = kda.kda_short_conv(li["x"][13:].contiguous(), li["conv_w"], None, c1, l2norm=True)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2]), y_all)
    assert torch.equal(c2, c_all)


@pytest.mark.parametrize("dtype,dv", [(torch.float32, 16), (torch.float32, 128), (torch.bfloat16, 128),
                                      (torch.bfloat16, 32)])
def test_out_norm_gate_matches_oracle(dev, dtype, dv):
    li = workloads.layer_inputs(41, 3, dv, dtype, device=dev, seed=dv + 1)
    say(f"  case: out_norm_gate N=41 H=3 dv={dv} {dtype}")
    y = kda.kda_out_norm_gate(li["o"], li["u"], li["norm_w"], 1e-6)
    torch.cuda.synchronize()
    ref = layer.out_norm_gate(_np(li["o"]), _np(li["u"]), _np(li["norm_w"]), 1e-6)
    assert_rounded(y, ref, dtype, "y")
    z = kda.kda_out_norm_gate(torch.zeros_like(li["o"]), li["u"], li["norm_w"], 1e-6)
    torch.cuda.synchronize()
    assert torch.count_nonzero(z) == 0


def test_layer_passes_k3_shape_sampled_rows(dev):
    """The K3 layer shape (65,536 tokens x 96 heads, d = 128, bf16): every pass over the
    whole tensor, the oracle on 256 sampled (token, head) rows (the conv on the 4 tokens
    each sampled output reads)."""
    N, H, d = 65536, 96, 128
    li = workloads.layer_inputs(N, H, d, torch.bfloat16, device=dev, seed=11)
    say(f"  case: layer passes N={N} H={H} d={d} bf16")
    g = kda.kda_gate(li["z"], li["A_log"])
    y, _ = kda.kda_short_conv(li["x"], li["conv_w"], l2norm=True)
    e = kda.kda_out_norm_gate(li["o"], li["u"], li["norm_w"], 1e-6)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    ts = rng.integers(0, N, 256)
    hs = rng.integers(0, H, 256)
    ti, hi = torch.tensor(ts, device=dev), torch.tensor(hs, device=dev)
    A = _np(li["A_log"])
    g_ref = np.stack([layer.gate(_np(li["z"][t:t + 1, h:h + 1]), A[h:h + 1])[0, 0] for t, h in zip(ts, hs)])
    err = np.abs(_np(g[ti, hi]) - g_ref)
    assert np.all(err <= 2.0 ** -7 * np.abs(g_ref) + 1e-7), f"gate error {err.max():.3e}"
    y_ref = []
    for t, h in zip(ts, hs):
        lo = max(0, t - 3)
        yy, _ = layer.short_conv(_np(li["x"][lo:t + 1, h:h + 1]), _np(li["conv_w"][h:h + 1]), l2norm=True,
                                 eps=1e-6)
        y_ref.append(yy[-1, 0])
    assert_rounded(y[ti, hi], np.stack(y_ref), torch.bfloat16, "conv rows")
    e_ref = layer.out_norm_gate(_np(li["o"][ti, hi]), _np(li["u"][ti, hi]), _np(li["norm_w"]), 1e-6)
    assert_rounded(e[ti, hi], e_ref, torch.bfloat16, "epilogue rows")
    del li, g, y, e
    torch.cuda.empty_cache()


# ----------------------------------------------------------------- fused decode

def _assert_y(y, ref, dtype, what):
    """The epilogue's output carries the recurrence's error (the 1e-2 / 1e-5 RMS bar) and,
    in bf16, its rounding (half an ulp, at most 2^-8 |ref|)."""
    yv, ref = _np(y), np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = TOL[dtype] * rms + (2.0 ** -8 * np.abs(ref) if dtype == torch.bfloat16 else 0.0)
    say(f"    {what}: max(err / bound) = {float(np.max(np.abs(yv - ref) / bound)):.3f}")
    assert np.all(np.isfinite(yv)) and np.all(np.abs(yv - ref) <= bound), f"{what} off"


def _decode_case(dev, dtype, dk, dv, B=3, H=4, seed=0):
    w = workloads.custom([1] * B, H, dk, dv, dtype)
    x = workloads.decode_step_inputs(w, 0, device=dev, seed=seed)
    lk = workloads.layer_inputs(B, H, dk, dtype, device=dev, seed=seed)
    lv = workloads.layer_inputs(B, H, dv, dtype, device=dev, seed=seed + 100)
    state = workloads.random_state(B, H, dk, dv, device=dev, seed=seed)
    return x, lk, lv, state


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 16, 64),
                                         (torch.bfloat16, 64, 32), (torch.float32, 128, 128)])
def test_decode_step_fused_matches_oracle(dev, dtype, dk, dv):
    """Gate from logits and the RMSNorm + Sigmoid epilogue inside the decode kernel, against
    the oracle gate, the oracle recurrence and the oracle epilogue in sequence."""
    x, lk, lv, state0 = _decode_case(dev, dtype, dk, dv, seed=dk + dv)
    say(f"  case: fused decode B=3 H=4 dk={dk} dv={dv} {dtype}")
    st = state0.clone()
    o, y = kda.kda_decode_step_fused(x["q"], x["k"], x["v"], lk["z"], x["beta"], st, gate_A_log=lk["A_log"],
                                     out_gate=lv["u"], norm_w=lv["norm_w"], norm_eps=1e-6)
    torch.cuda.synchronize()
    g = layer.gate(_np(lk["z"]), _np(lk["A_log"]))
    o_ref, s_ref = oracle.decode(_np(x["q"]), _np(x["k"]), _np(x["v"]), g, _np(x["beta"]), _np(state0))
    y_ref = layer.out_norm_gate(o_ref, _np(lv["u"]), _np(lv["norm_w"]), 1e-6)
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(st, s_ref, TOL[dtype], "state")
    _assert_y(y, y_ref, dtype, "y")
    # each fusion alone, and y without o
    st = state0.clone()
    o2, y2 = kda.kda_decode_step_fused(x["q"], x["k"], x["v"], lk["z"], x["beta"], st, gate_A_log=lk["A_log"])
    st3 = state0.clone()
    o3, y3 = kda.kda_decode_step_fused(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], st3,
                                       out_gate=lv["u"], norm_w=lv["norm_w"], output_o=False)
    torch.cuda.synchronize()
    assert y2 is None and o3 is None
    assert torch.equal(o2, o)
    o3_ref, _ = oracle.decode(_np(x["q"]), _np(x["k"]), _np(x["v"]), _np(x["log_alpha"]), _np(x["beta"]),
                              _np(state0))
    _assert_y(y3, layer.out_norm_gate(o3_ref, _np(lv["u"]), _np(lv["norm_w"]), 1e-6), dtype, "y (epilogue only)")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_window_fused_matches_oracle(dev, dtype):
    B, T, H, dk, dv = 3, 5, 2, 128, 128
    w = workloads.custom([1] * B, H, dk, dv, dtype)
    x = workloads.decode_window_inputs(w, T, 0, device=dev, seed=41)
    lk = workloads.layer_inputs(B * T, H, dk, dtype, device=dev, seed=41)
    lv = workloads.layer_inputs(B * T, H, dv, dtype, device=dev, seed=42)
    z = lk["z"].view(B, T, H, dk)
    u = lv["u"].view(B, T, H, dv)
    state0 = workloads.random_state(B, H, dk, dv, device=dev, seed=41)
    st = state0.clone()
    acc = torch.tensor([0, 3, 5], dtype=torch.int32, device=dev)
    say(f"  case: fused window B={B} T={T} H={H} {dtype}")
    o, y = kda.kda_decode_window_fused(x["q"], x["k"], x["v"], z, x["beta"], st, acc, gate_A_log=lk["A_log"],
                                       out_gate=u, norm_w=lv["norm_w"], norm_eps=1e-6)
    torch.cuda.synchronize()
    g = layer.gate(_np(lk["z"]), _np(lk["A_log"])).reshape(B, T, H, dk)
    s = _np(state0)
    snaps, outs = [s], []
    for t in range(T):
        ot, s = oracle.decode(_np(x["q"][:, t]), _np(x["k"][:, t]), _np(x["v"][:, t]), g[:, t],
                              _np(x["beta"][:, t]), s)
        outs.append(ot)
        snaps.append(s)
    o_ref = np.stack(outs, axis=1)
    s_ref = np.stack([snaps[a][b] for b, a in enumerate([0, 3, 5])])
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(st, s_ref, TOL[dtype], "state")
    assert torch.equal(st[0], state0[0])
    _assert_y(y, layer.out_norm_gate(o_ref, _np(u), _np(lv["norm_w"]), 1e-6), dtype, "y")


def test_layer_passes_with_no_tokens(dev):
    """N = 0: nothing to compute; the ShortConv cache of empty sequences passes through."""
    H, d = 2, 64
    z = torch.empty((0, H, d), dtype=torch.bfloat16, device=dev)
    A = torch.zeros((H,), dtype=torch.float32, device=dev)
    assert kda.kda_gate(z, A).shape == (0, H, d)
    cu = torch.zeros(3, dtype=torch.int32, device=dev)
    li = workloads.layer_inputs(1, H, d, torch.bfloat16, nseq=2, device=dev, seed=5)
    y, c = kda.kda_short_conv(z, li["conv_w"], cu, li["conv_cache"], l2norm=True)
    e = kda.kda_out_norm_gate(torch.empty((0, H, d), dtype=torch.float32, device=dev), z, li["norm_w"])
    torch.cuda.synchronize()
    assert y.shape == (0, H, d) and e.shape == (0, H, d)
    assert torch.equal(c, li["conv_cache"])


def test_fused_window_of_one_token_equals_fused_step(dev):
    """A one-token fused window and the fused decode step (same kernels' arithmetic per token)."""
    x, lk, lv, state0 = _decode_case(dev, torch.bfloat16, 128, 128, B=4, H=3, seed=9)
    s1, s2 = state0.clone(), state0.clone()
    o1, y1 = kda.kda_decode_step_fused(x["q"], x["k"], x["v"], lk["z"], x["beta"], s1, gate_A_log=lk["A_log"],
                                       out_gate=lv["u"], norm_w=lv["norm_w"])
    w = {n: t.unsqueeze(1).contiguous() for n, t in x.items()}
    o2, y2 = kda.kda_decode_window_fused(w["q"], w["k"], w["v"], lk["z"].unsqueeze(1).contiguous(), w["beta"], s2,
                                         gate_A_log=lk["A_log"], out_gate=lv["u"].unsqueeze(1).contiguous(),
                                         norm_w=lv["norm_w"])
    torch.cuda.synchronize()
    assert_close(o2[:, 0], _np(o1), 1e-6, "o")
    assert_close(s2, _np(s1), 1e-6, "state")
    _assert_y(y2[:, 0], _np(y1), torch.bfloat16, "y")


def test_short_conv_decode_mode(dev):
    """Without cu_seqlens every token is its own sequence (a decode step): B tokens, each
    convolved with its sequence's cache, and the cache shifted by one, in place."""
    B, H, d = 6, 3, 128
    li = workloads.layer_inputs(B, H, d, torch.bfloat16, nseq=B, device=dev, seed=13)
    cache = li["conv_cache"].clone()
    y, c = kda.kda_short_conv(li["x"], li["conv_w"], "decode", cache, l2norm=True, cache_out=cache)
    torch.cuda.synchronize()
    cu = np.arange(B + 1)
    y_ref, c_ref = layer.short_conv(_np(li["x"]), _np(li["conv_w"]), cu, _np(li["conv_cache"]), l2norm=True,
                                    eps=1e-6)
    assert_rounded(y, y_ref, torch.bfloat16, "y")
    assert np.array_equal(_np(cache), c_ref)


def test_layer_pipeline_end_to_end(dev):
    """ShortConv (q, k with L2, v) -> gate -> prefill -> epilogue through the library, against
    the same pipeline in the oracles, fed with the library's own bf16 roundings of each
    intermediate (the recurrence takes its inputs in bf16)."""
    seqlens = [37, 20]
    N, H, dk, dv = sum(seqlens), 2, 128, 128
    cu = torch.tensor(workloads.cu_seqlens_of(seqlens), dtype=torch.int32, device=dev)
    lq = workloads.layer_inputs(N, H, dk, torch.bfloat16, nseq=2, device=dev, seed=21)
    lk = workloads.layer_inputs(N, H, dk, torch.bfloat16, nseq=2, device=dev, seed=22)
    lv = workloads.layer_inputs(N, H, dv, torch.bfloat16, nseq=2, device=dev, seed=23)
    beta = torch.sigmoid(torch.randn((N, H), generator=torch.Generator(device=dev).manual_seed(5),
                                     device=dev)).to(torch.bfloat16)
    q, _ = kda.kda_short_conv(lq["x"], lq["conv_w"], cu, l2norm=True)
    k, _ = kda.kda_short_conv(lk["x"], lk["conv_w"], cu, l2norm=True)
    v, _ = kda.kda_short_conv(lv["x"], lv["conv_w"], cu)
    g = kda.kda_gate(lk["z"], lk["A_log"])
    o, fin = kda.kda_prefill(q, k, v, g, beta, cu)
    y = kda.kda_out_norm_gate(o, lv["u"], lv["norm_w"], 1e-6)
    torch.cuda.synchronize()
    # each stage against its oracle on the library's inputs to that stage
    for name, got, ref in (
            ("q", q, layer.short_conv(_np(lq["x"]), _np(lq["conv_w"]), _np(cu), l2norm=True)[0]),
            ("k", k, layer.short_conv(_np(lk["x"]), _np(lk["conv_w"]), _np(cu), l2norm=True)[0]),
            ("v", v, layer.short_conv(_np(lv["x"]), _np(lv["conv_w"]), _np(cu))[0])):
        assert_rounded(got, ref, torch.bfloat16, name)
    x = {"q": q, "k": k, "v": v, "log_alpha": g, "beta": beta, "cu_seqlens": cu}
    o_ref, f_ref = oracle_prefill(x)
    assert_close(o, o_ref, TOL[torch.bfloat16], "o")
    assert_close(fin, f_ref, TOL[torch.bfloat16], "final_state")
    _assert_y(y, layer.out_norm_gate(o_ref, _np(lv["u"]), _np(lv["norm_w"]), 1e-6), torch.bfloat16, "y")


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 16, 64),
                                         (torch.bfloat16, 64, 32)])
def test_decode_layer_step_matches_oracle(dev, dtype, dk, dv):
    """ShortConv (+ L2 for q, k) from the cache, gate, recurrence and epilogue in one launch,
    against the oracles in sequence; the cache after the step is exact (it holds inputs)."""
    B, H = 3, 4
    C = 2 * dk + dv
    lx = workloads.layer_inputs(B, H, C, dtype, nseq=B, device=dev, seed=dk + 3 * dv)
    lk = workloads.layer_inputs(B, H, dk, dtype, device=dev, seed=dk + 1)
    lv = workloads.layer_inputs(B, H, dv, dtype, device=dev, seed=dv + 2)
    beta = workloads.decode_step_inputs(workloads.custom([1] * B, H, dk, dv, dtype), 0, device=dev, seed=4)["beta"]
    state0 = workloads.random_state(B, H, dk, dv, device=dev, seed=dk)
    st, cache = state0.clone(), lx["conv_cache"].clone()
    say(f"  case: decode layer step B={B} H={H} dk={dk} dv={dv} {dtype}")
    o, y = kda.kda_decode_layer_step(lx["x"], lx["conv_w"], cache, lk["z"], beta, st, dk=dk, l2_eps=1e-6,
                                     gate_A_log=lk["A_log"], out_gate=lv["u"], norm_w=lv["norm_w"], norm_eps=1e-6)
    torch.cuda.synchronize()
    cu = np.arange(B + 1)
    x, w, c0 = _np(lx["x"]), _np(lx["conv_w"]), _np(lx["conv_cache"])
    parts = {}
    for name, lo, hi, l2 in (("q", 0, dk, True), ("k", dk, 2 * dk, True), ("v", 2 * dk, C, False)):
        parts[name] = layer.short_conv(x[..., lo:hi], w[:, lo:hi], cu, c0[:, :, lo:hi], l2norm=l2, eps=1e-6)
    g = layer.gate(_np(lk["z"]), _np(lk["A_log"]))
    o_ref, s_ref = oracle.decode(parts["q"][0], parts["k"][0], parts["v"][0], g, _np(beta), _np(state0))
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(st, s_ref, TOL[dtype], "state")
    _assert_y(y, layer.out_norm_gate(o_ref, _np(lv["u"]), _np(lv["norm_w"]), 1e-6), dtype, "y")
    c_ref = np.concatenate([parts[n][1] for n in ("q", "k", "v")], axis=2)
    assert np.array_equal(_np(cache), c_ref), "conv cache after the step"
