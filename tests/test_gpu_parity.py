"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Bar: max|x - ref| <= tol * RMS(ref) per output tensor, tol = 1e-2 for bf16 inputs with
fp32 state, 1e-5 for fp32 inputs.  Inputs are seeded and synthetic (workloads module),
generated on the GPU and copied to the host for the oracle.  Full-size workloads are
run in full on the GPU and checked on a sample of heads the oracle recomputes exactly.
"""
import numpy as np
import pytest
import torch

import chunk_model
import gated_delta_rule_51_amd as kda
import oracle
import workloads
from parity import TOL, assert_close, oracle_prefill, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    return torch.device("cuda:0")


def _prefill_case(dev, seqlens, H, dk, dv, dtype, seed=0, gate="neg_softplus", init=False,
                  heads=None, edit=None):
    w = workloads.custom(seqlens, H, dk, dv, dtype, gate)
    x = workloads.prefill_inputs(w, device=dev, seed=seed)
    if edit is not None:
        edit(x)
    init_state = workloads.random_state(len(seqlens), H, dk, dv, device=dev, seed=seed) if init else None
    say(f"  case: seqlens={list(seqlens)[:8]}{'...' if len(seqlens) > 8 else ''} N={w.total_tokens} "
        f"H={H} dk={dk} dv={dv} {dtype} init={init}")
    # outputs start as NaN, so a row or state the kernels never write cannot pass
    o = torch.full((w.total_tokens, H, dv), float("nan"), dtype=torch.float32, device=dev)
    fin = torch.full((len(seqlens), H, dk, dv), float("nan"), dtype=torch.float32, device=dev)
    kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], init_state,
                    o=o, final_state=fin)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(x, init_state, heads=heads)
    if heads is not None:
        o, fin = o[:, heads], fin[:, heads]
    tol = TOL[dtype]
    assert_close(o, o_ref, tol, "o")
    assert_close(fin, f_ref, tol, "final_state")
    return x, o, fin


# ----------------------------------------------------------------- chunk-local phase

def decode_workspace(ws, H, dtype):
    """The workspace holds, per (chunk slot, head), T' then A_qk as 16x16 MFMA A-operand
    fragments: lane 16g + m holds row m, columns 4g..4g+3 ({hi[4], lo[4]} bf16 for bf16
    inputs, 4 fp32 for fp32 inputs).  Returns [slots, H, 2, 16, 16] float64."""
    if dtype == torch.float32:
        fr = ws.cpu().double().numpy().reshape(-1, H, 2, 4, 16, 4)           # [.., g, m, j]
    else:
        b = ws.cpu().view(torch.bfloat16).double().numpy().reshape(-1, H, 2, 4, 16, 8)
        fr = b[..., :4] + b[..., 4:]
    # M[m][4g + j] = fr[g][m][j]
    return np.ascontiguousarray(fr.transpose(0, 1, 2, 4, 3, 5)).reshape(fr.shape[0], H, 2, 16, 16)


@pytest.mark.parametrize("dtype,dk", [(torch.float32, 16), (torch.float32, 128),
                                      (torch.bfloat16, 64), (torch.bfloat16, 128)])
def test_chunk_local_matches_chunked_model(dev, dtype, dk):
    """Kernel 1's T' = (I + A_kk)^-1 diag(beta) and A_qk for every chunk against the fp64
    chunked-form model on the same (rounded) inputs."""
    seqlens, H = [40, 16, 7], 2
    w = workloads.custom(seqlens, H, dk, 16, dtype)
    x = workloads.prefill_inputs(w, device=dev, seed=3)
    say(f"  case: chunk_local dk={dk} {dtype}")
    nseq = len(seqlens)
    ws = kda.alloc_workspace(w.total_tokens, nseq, H, dk, 16, dtype, dev)
    ws.fill_(float("nan"))
    kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
    torch.cuda.synchronize()
    wsn = decode_workspace(ws, H, dtype)
    cpu = {n: x[n].cpu().double().numpy() for n in ("q", "k", "v", "log_alpha", "beta")}
    _, _, kept = chunk_model.prefill(cpu["q"], cpu["k"], cpu["v"], cpu["log_alpha"], cpu["beta"],
                                     cu_seqlens=workloads.cu_seqlens_of(seqlens), keep=True)
    cu = workloads.cu_seqlens_of(seqlens)
    tol_t = 1e-5 if dtype == torch.float32 else 2e-2
    tol_a = 1e-5 if dtype == torch.float32 else 1e-3
    for (s, h, j), loc in kept.items():
        slot = cu[s] // 16 + s + j
        n = loc["Tp"].shape[0]
        Tp = np.zeros((16, 16))
        Tp[:n, :n] = loc["Tp"]
        Aq = np.zeros((16, 16))
        Aq[:n, :n] = loc["Aqk"]
        gT, gA = wsn[slot, h, 0], wsn[slot, h, 1]
        eT = np.max(np.abs(gT - Tp)) / np.max(np.abs(Tp))
        eA = np.max(np.abs(gA - Aq)) / np.max(np.abs(Aq))
        assert eT <= tol_t and eA <= tol_a, f"chunk (s={s},h={h},j={j}): T' err {eT:.2e}, A_qk err {eA:.2e}"


# ----------------------------------------------------------------- the five workloads

def test_workload1_tiny_fp32_prefill(dev):
    w = workloads.workload(1)
    _prefill_case(dev, w.seqlens, w.H, w.dk, w.dv, w.dtype, gate=w.gate)


def test_workload1_tiny_fp32_decode(dev):
    """The tiny workload stepped token by token through the decode kernel."""
    w = workloads.workload(1)
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    T = w.total_tokens
    state = torch.zeros((1, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    outs = []
    for t in range(T):
        outs.append(kda.kda_decode_step(*(x[n][t:t + 1].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")),
                                        state).clone())
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(x)
    assert_close(torch.cat(outs), o_ref, TOL[torch.float32], "decode o (64 steps)")
    assert_close(state, f_ref, TOL[torch.float32], "decode state")


def test_workload2_batched_prefill(dev):
    w = workloads.workload(2)
    _prefill_case(dev, w.seqlens, w.H, w.dk, w.dv, w.dtype)


def test_workload3_k3_layer_sampled_heads(dev):
    """B=1, H=96, T=65,536: full run on the GPU, oracle on 4 heads."""
    w = workloads.workload(3)
    heads = [0, 31, 64, 95]
    _prefill_case(dev, w.seqlens, w.H, w.dk, w.dv, w.dtype, heads=heads)
    torch.cuda.empty_cache()


def test_workload4_decode_every_head(dev):
    """B=256 x H=96, 128 steps from a unit-Frobenius random state; the oracle carries all 24,576
    heads' fp64 states through the same 128 steps, and every output and final state is checked."""
    w = workloads.workload(4)
    B, H = w.nseq, w.H
    state = workloads.decode_initial_state(B, H, w.dk, w.dv, device=dev)
    ref_state = state.cpu().double().numpy()  # [B, H, dk, dv], advanced in place by the oracle
    err = ss = 0.0
    say(f"  case: decode B={B} H={H} steps={w.decode_steps}, every head")
    o = torch.full((B, H, w.dv), float("nan"), dtype=torch.float32, device=dev)
    for step in range(w.decode_steps):
        x = workloads.decode_step_inputs(w, step, device=dev)
        kda.kda_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], state, o=o)
        got = o.cpu().double().numpy()
        orf, ref_state = oracle.decode(*(x[n].cpu() for n in ("q", "k", "v", "log_alpha", "beta")), ref_state,
                                       inplace=True)
        assert np.all(np.isfinite(got)), f"step {step}: non-finite output"
        err = max(err, float(np.max(np.abs(got - orf))))
        ss += float(np.sum(orf * orf))
        o.fill_(float("nan"))
    torch.cuda.synchronize()
    e = err / (ss / (w.decode_steps * o.numel())) ** 0.5
    say(f"    decode o (128 steps, every head): max|err|/rms = {e:.3e}")
    assert e <= TOL[torch.bfloat16]
    assert_close(state, ref_state, TOL[torch.bfloat16], "decode state after 128 steps (every head)")
    del state
    torch.cuda.empty_cache()


# ----------------------------------------------------------------- decode windows

def _oracle_window(x, init, accepts):
    """T oracle decode steps from ``init``; the state kept per sequence is the one after its
    first accepts[b] tokens.  Returns (o [B, T, H, dv], state [B, H, dk, dv]) in float64."""
    T = x["q"].shape[1]
    st = init.detach().cpu().double().numpy()
    snaps, outs = [st], []
    for t in range(T):
        ot, st = oracle.decode(*(x[n][:, t].cpu() for n in ("q", "k", "v", "log_alpha", "beta")), st)
        outs.append(ot)
        snaps.append(st)
    return np.stack(outs, axis=1), np.stack([snaps[a][b] for b, a in enumerate(accepts)])


def _window_case(dev, B, T, H, dk, dv, dtype, accept, seed=0, output_o=True, gate="neg_softplus", edit=None):
    w = workloads.custom([1] * B, H, dk, dv, dtype, gate)
    x = workloads.decode_window_inputs(w, T, 0, device=dev, seed=seed)
    if edit is not None:
        edit(x)
    init = workloads.random_state(B, H, dk, dv, device=dev, seed=seed)
    state = init.clone()
    acc = None if accept is None else torch.tensor(accept, dtype=torch.int32, device=dev)
    say(f"  case: window B={B} T={T} H={H} dk={dk} dv={dv} {dtype} accept={accept} o={output_o}")
    o = torch.full((B, T, H, dv), float("nan"), dtype=torch.float32, device=dev) if output_o else None
    o = kda.kda_decode_window(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], state, acc,
                              output_o=output_o, o=o)
    torch.cuda.synchronize()
    accepts = [T] * B if accept is None else [min(max(a, 0), T) for a in accept]
    o_ref, st_ref = _oracle_window(x, init, accepts)
    if output_o:
        assert_close(o, o_ref, TOL[dtype], "window o")
    else:
        assert o is None
    assert_close(state, st_ref, TOL[dtype], "window state")
    for b, a in enumerate(accepts):
        if a == 0:
            assert torch.equal(state[b], init[b]), f"sequence {b} accepted nothing but its state changed"
    return x, init, state, o


@pytest.mark.parametrize("dtype,dk,dv", [(torch.float32, 16, 16), (torch.float32, 128, 128),
                                         (torch.bfloat16, 128, 128), (torch.bfloat16, 64, 32),
                                         (torch.bfloat16, 32, 128), (torch.float32, 16, 64)])
def test_decode_window_matches_oracle(dev, dtype, dk, dv):
    """Five sequences, windows of 5 drafts, accepted counts 0, 2, 5 and two out of range."""
    _window_case(dev, 5, 5, 3, dk, dv, dtype, [0, 2, 5, 9, -3], seed=dk + dv)


def test_decode_window_without_accept_or_outputs(dev):
    _window_case(dev, 2, 3, 2, 128, 128, torch.bfloat16, None, seed=3)
    _window_case(dev, 3, 4, 2, 128, 64, torch.bfloat16, [1, 4, 3], seed=4, output_o=False)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_window_long_strong_decay(dev, dtype):
    """Windows of 20 tokens with log-decay uniform on [-5, 0) and, in a second case, at the
    bound -5 for every channel and token; accepted counts 0 to 20."""
    acc = [0, 7, 8, 9, 16, 17, 20]
    _window_case(dev, 7, 20, 2, 128, 128, dtype, acc, seed=21, gate="uniform")

    def floor(x):
        x["log_alpha"].fill_(-5.0)
    _window_case(dev, 7, 20, 2, 64, 128, dtype, acc, seed=22, edit=floor)


def test_decode_window_equals_decode_steps(dev):
    """A fully accepted window in the token-by-token form and the same tokens through
    kda_decode_step one by one; a window of one token and a single step."""
    w = workloads.custom([1] * 4, 3, 128, 128, torch.bfloat16)
    x = workloads.decode_window_inputs(w, 6, 0, device=dev, seed=11)
    init = workloads.random_state(4, 3, 128, 128, device=dev, seed=11)
    sw, ss = init.clone(), init.clone()
    ow = kda.kda_decode_window(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], sw, form=1)
    os_ = torch.stack([kda.kda_decode_step(*(x[n][:, t].contiguous()
                                             for n in ("q", "k", "v", "log_alpha", "beta")), ss)
                       for t in range(6)], dim=1)
    torch.cuda.synchronize()
    assert_close(ow, os_, 1e-6, "window vs steps o")
    assert_close(sw, ss, 1e-6, "window vs steps state")
    s1, s2 = init.clone(), init.clone()
    o1 = kda.kda_decode_window(*(x[n][:, :1].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")), s1)
    o2 = kda.kda_decode_step(*(x[n][:, 0].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")), s2)
    torch.cuda.synchronize()
    assert_close(o1[:, 0], o2, 1e-6, "one-token window vs step o")
    assert_close(s1, s2, 1e-6, "one-token window vs step state")


def test_decode_window_many_heads_per_workgroup(dev):
    """1,100 heads of 128x128: more than the persistent grid holds, so workgroups carry the
    state of a second head in the other register set; every head checked."""
    _window_case(dev, 550, 3, 2, 128, 128, torch.float32,
                 workloads.window_accept(550, 3, seed=5).tolist(), seed=5)


def test_decode_window_workload_sampled_heads(dev):
    """The decode workload's shape (B=256 x H=96), windows of 4 drafts, two windows in a row
    with seeded accepted counts; oracle on 48 sampled heads."""
    w = workloads.workload(4)
    B, H, T = w.nseq, w.H, 4
    state = workloads.decode_initial_state(B, H, w.dk, w.dv, device=dev)
    rng = np.random.default_rng(1)
    bi = torch.tensor(rng.integers(0, B, 48), device=dev)
    hi = torch.tensor(rng.integers(0, H, 48), device=dev)
    ref_state = state[bi, hi].cpu().double().numpy()        # [48, dk, dv], as 48 sequences of 1 head
    say(f"  case: decode window B={B} H={H} T={T}, 2 windows")
    for win in range(2):
        x = workloads.decode_window_inputs(w, T, win, device=dev)
        acc = workloads.window_accept(B, T, device=dev, seed=win)
        o = kda.kda_decode_window(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], state, acc)
        torch.cuda.synchronize()
        sub = {n: x[n][bi, :, hi].unsqueeze(2).contiguous() for n in ("q", "k", "v", "log_alpha", "beta")}
        accepts = acc[bi].tolist()
        o_ref, st = _oracle_window(sub, torch.from_numpy(ref_state).unsqueeze(1), accepts)
        ref_state = st[:, 0]
        assert_close(o[bi, :, hi], o_ref[:, :, 0], TOL[torch.bfloat16], f"window {win} o")
        assert_close(state[bi, hi], ref_state, TOL[torch.bfloat16], f"window {win} state")
    del state
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_workload5_varlen_1m_sampled_heads(dev):
    """1,048,576 packed tokens in 27 log-uniform sequences, H=96, through kda_prefill (the
    single-pass kernel for this shape): outputs start as NaN; the oracle on 8 heads, one per
    residue mod 8 (the XCD each chain runs on), every sequence, in groups of 4 heads."""
    w = workloads.workload(5)
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    heads = [0, 13, 26, 39, 52, 65, 78, 91]
    assert sorted(h % 8 for h in heads) == list(range(8))
    o = torch.full((w.total_tokens, w.H, w.dv), float("nan"), dtype=torch.float32, device=dev)
    fin = torch.full((w.nseq, w.H, w.dk, w.dv), float("nan"), dtype=torch.float32, device=dev)
    say(f"  case: varlen 1M, {w.nseq} sequences, heads {heads}")
    kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], o=o, final_state=fin)
    torch.cuda.synchronize()
    err = {"o": 0.0, "f": 0.0}
    ss = {"o": 0.0, "f": 0.0}
    for g0 in range(0, len(heads), 4):
        hs = heads[g0:g0 + 4]
        o_ref, f_ref = oracle_prefill(x, heads=hs)
        for key, got, ref in (("o", o[:, hs], o_ref), ("f", fin[:, hs], f_ref)):
            g = got.double().cpu().numpy()
            assert np.all(np.isfinite(g)), f"{key}: non-finite (unwritten) values on heads {hs}"
            err[key] = max(err[key], float(np.max(np.abs(g - ref))))
            ss[key] += float(np.sum(ref * ref))
        del o_ref, f_ref
    eo = err["o"] / (ss["o"] / (w.total_tokens * len(heads) * w.dv)) ** 0.5
    ef = err["f"] / (ss["f"] / (w.nseq * len(heads) * w.dk * w.dv)) ** 0.5
    say(f"    o: max|err|/rms = {eo:.3e}; final_state: {ef:.3e} (tol 1e-2)")
    assert eo <= TOL[torch.bfloat16] and ef <= TOL[torch.bfloat16]
    del x, o, fin
    torch.cuda.empty_cache()


# ----------------------------------------------------------------- edge cases

@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128), (128, 128)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ragged_lengths_and_shapes(dev, dk, dv, dtype):
    """Empty, single-token, exact-chunk and ragged sequences, with an initial state."""
    _prefill_case(dev, [17, 0, 1, 33, 100, 16, 15], 3, dk, dv, dtype, seed=dk + dv, init=True)


@pytest.mark.parametrize("shape", [(2, 4), (4, 4)])
def test_ragged_lengths_warp_specialised_shapes(dev, shape):
    """The warp-specialised inter-chunk shapes on empty, single-chunk, two-chunk and
    ragged sequences with an initial state (every remainder of the three-chunk unrolled
    loop)."""
    seqlens, H = [17, 0, 1, 33, 100, 16, 15, 48, 49], 2
    w = workloads.custom(seqlens, H, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=21)
    init = workloads.random_state(len(seqlens), H, 128, 128, device=dev, seed=21)
    ws = kda.alloc_workspace(w.total_tokens, len(seqlens), H, 128, 128, torch.bfloat16, dev)
    kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
    o = torch.full((w.total_tokens, H, 128), float("nan"), dtype=torch.float32, device=dev)
    fin = torch.full((len(seqlens), H, 128, 128), float("nan"), dtype=torch.float32, device=dev)
    say(f"  case: warp-specialised shape {shape}")
    kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws, init, o=o, final_state=fin,
                        consumers=shape[0], producers=shape[1])
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(x, init)
    assert_close(o, o_ref, TOL[torch.bfloat16], "o")
    assert_close(fin, f_ref, TOL[torch.bfloat16], "final_state")


def test_zero_tokens(dev):
    """N = 0: every final state equals its initial state."""
    H, d = 2, 64
    z = torch.empty((0, H, d), dtype=torch.bfloat16, device=dev)
    zb = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(3, dtype=torch.int32, device=dev)
    init = workloads.random_state(2, H, d, d, device=dev)
    o, fin = kda.kda_prefill(z, z, z, z, zb, cu, init)
    torch.cuda.synchronize()
    assert o.shape == (0, H, d) and torch.equal(fin, init)


def test_gate_and_beta_extremes(dev):
    """g at the -5 floor and at 0, beta exactly 0 and 1."""
    def edit(x):
        g, b = x["log_alpha"], x["beta"]
        g[0::3] = -5.0
        g[1::5] = 0.0
        b[0::4] = 0.0
        b[1::4] = 1.0
    _prefill_case(dev, [64, 37], 4, 128, 128, torch.bfloat16, seed=9, init=True, edit=edit)
    _prefill_case(dev, [64, 37], 2, 32, 32, torch.float32, seed=9, gate="uniform", init=True, edit=edit)


def test_final_state_may_alias_initial_state(dev):
    w = workloads.custom([50, 20], 2, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=4)
    init = workloads.random_state(2, 2, 128, 128, device=dev, seed=4)
    o1, f1 = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], init.clone())
    buf = init.clone()
    o2, f2 = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], buf,
                             final_state=buf)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, buf)


# ----------------------------------------------------------------- cross-path invariants

def test_decode_steps_match_prefill(dev):
    """T decode steps and one prefill of T tokens agree (both also against the oracle)."""
    w = workloads.custom([45], 3, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=5)
    init = workloads.random_state(1, 3, 128, 128, device=dev, seed=5)
    o_p, f_p = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], init)
    state = init.clone()
    outs = [kda.kda_decode_step(*(x[n][t:t + 1].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")),
                                state) for t in range(45)]
    torch.cuda.synchronize()
    o_d = torch.cat(outs)
    o_ref, f_ref = oracle_prefill(x, init)
    assert_close(o_d, o_ref, TOL[torch.bfloat16], "decode o")
    assert_close(state, f_ref, TOL[torch.bfloat16], "decode state")
    assert_close(o_d, o_p.double().cpu().numpy(), TOL[torch.bfloat16], "decode vs prefill o")


def test_split_prefill_resumes_exactly(dev):
    """prefill(0:t1) then prefill(t1:T, init = final_1) against prefill(0:T) and the oracle."""
    w = workloads.custom([300], 2, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=6)
    o, f = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"])
    parts = []
    state = None
    for a, b in ((0, 123), (123, 300)):
        sl = [x[n][a:b].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")]
        op, state = kda.kda_prefill(*sl, None, state)
        parts.append(op)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(x)
    assert_close(torch.cat(parts), o_ref, TOL[torch.bfloat16], "split o")
    assert_close(state, f_ref, TOL[torch.bfloat16], "split final state")
    assert rel_err(torch.cat(parts), o.double().cpu().numpy()) <= TOL[torch.bfloat16]


def test_varlen_packing_equals_separate_calls(dev):
    seqlens = [70, 5, 33]
    w = workloads.custom(seqlens, 2, 64, 64, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=7)
    o, f = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"])
    cu = workloads.cu_seqlens_of(seqlens)
    for s in range(len(seqlens)):
        sl = [x[n][cu[s]:cu[s + 1]].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")]
        os_, fs = kda.kda_prefill(*sl)
        torch.cuda.synchronize()
        # chunk boundaries are aligned to each sequence's start in both calls: identical arithmetic
        assert torch.equal(os_, o[cu[s]:cu[s + 1]]) and torch.equal(fs[0], f[s])


def test_bitwise_deterministic(dev):
    w = workloads.custom([200, 77], 4, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=8)
    r1 = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"])
    r2 = kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"])
    st = workloads.random_state(4, 8, 128, 128, device=dev)
    st1, st2 = st.clone(), st.clone()
    d = workloads.decode_step_inputs(workloads.custom([1] * 4, 8, 128, 128), 0, device=dev)
    o1 = kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], st1)
    o2 = kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], st2)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])
    assert torch.equal(o1, o2) and torch.equal(st1, st2)


def test_graph_replays_match_eager(dev):
    """The three-call step (chunk-local, inter-chunk, decode of one more token from the
    final states) captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager result bitwise.  The library
    enqueues kernels only (no memsets, no allocation), so it can be captured."""
    w = workloads.custom([256, 256], 2, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=31)
    d = workloads.decode_step_inputs(workloads.custom([1, 1], 2, 128, 128), 0, device=dev, seed=32)
    ws = kda.alloc_workspace(w.total_tokens, w.nseq, w.H, w.dk, w.dv, torch.bfloat16, dev)
    o = torch.empty((w.total_tokens, w.H, w.dv), dtype=torch.float32, device=dev)
    fin = torch.empty((w.nseq, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    od = torch.empty((w.nseq, w.H, w.dv), dtype=torch.float32, device=dev)

    def step():
        kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
        kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws, None,
                            o=o, final_state=fin)
        kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], fin, o=od)

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), fin.clone(), od.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        o.zero_(), fin.zero_(), od.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {r}")
        assert torch.equal(o, ref[0]) and torch.equal(fin, ref[1]) and torch.equal(od, ref[2])
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(od, ref[2])


def test_workgroup_shape_variants_agree(dev):
    """Every workgroup shape of the warp-specialised inter-chunk kernel and of the single-pass
    prefill meets the bar, is bitwise reproducible on its own, and agrees with the other shapes
    (the per-channel decay sums and the inverse are grouped differently per kernel, so shapes
    agree to the tolerance, not bitwise)."""
    w = workloads.custom([130, 64], 3, 128, 128, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=10)
    o_ref, f_ref = oracle_prefill(x)
    ws = kda.alloc_workspace(w.total_tokens, 2, 3, 128, 128, torch.bfloat16, dev)
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"])

    def two_kernel(shape):
        kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
        return kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws,
                                   consumers=shape[0], producers=shape[1])

    def single_pass(shape):
        return kda.kda_prefill_single_pass(*args, consumers=shape[0], slices=shape[1])

    runs = [(f"inter-chunk {s}", two_kernel, s) for s in ((4, 4), (2, 4))]
    runs += [(f"single pass {s}", single_pass, s) for s in ((2, 1), (4, 1), (4, 2))]
    outs = []
    for name, fn, shape in runs:
        say(name)
        outs.append(fn(shape))
        again = fn(shape)
        torch.cuda.synchronize()
        assert torch.equal(outs[-1][0], again[0]) and torch.equal(outs[-1][1], again[1])
        assert_close(outs[-1][0], o_ref, TOL[torch.bfloat16], f"o ({name})")
        assert_close(outs[-1][1], f_ref, TOL[torch.bfloat16], f"final_state ({name})")
    for o, f in outs[1:]:
        assert rel_err(o, outs[0][0].double().cpu().numpy()) <= TOL[torch.bfloat16]
        assert rel_err(f, outs[0][1].double().cpu().numpy()) <= TOL[torch.bfloat16]
