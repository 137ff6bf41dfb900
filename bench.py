"""Benchmark of the MI355X KDA library (one GPU).

One step = one pass of the whole hot path over one batch: the chunk-local kernel, the
inter-chunk kernel (prefill of the batch) and one decode step per sequence continuing
from the prefill's final states.  The headline batch is B=4, H=8, T=2048, dk=dv=128,
bf16 inputs, fp32 state.  Three input sets are rotated so the ~105 MB working set
cannot stay resident in the 256 MB Infinity Cache.  --graph also times the step replayed
from HIP graphs (its three launches captured once per input set), reported beside the
eager time.

The JSON line also carries, measured in the same run:
  * "k3_layer": prefill of B=1, H=96, T=65,536 (the K3 layer shape),
  * "decode":   128 recurrent steps over B=256 x H=96 heads (1.6 GB of fp32 state),
  * "decode_window_4" / "_8": the same 128 steps as windows of 4 or 8 draft tokens
    (speculative verification: one state read and write per window),
  * "layer": the passes around the recurrence (decay gate, ShortConv prologue, RMSNorm +
    output-gate epilogue) on the K3 layer shape, and the fused decode step against the
    same operations as separate launches,
  * "backward": the prefill backward on the batched workload and the K3 layer,
  * "context_parallel": the prefill with every sequence split into R segments (intra-device
    context parallelism) against the plain prefill, on the batched workload, the K3 layer and
    the K3 layer's 65,536-token sequence with 12 heads (its share of one device when the 96
    heads are split eight ways),
  * "varlen_1m": prefill of 1,048,576 packed tokens in log-uniform sequences,
each with tokens/s (or GB/s), TFLOP/s and the fraction of the roofline that bounds it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only main|k3|decode|layer|backward|cp|varlen|none]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
CHUNK = 16


def prefill_flops_per_token_head(dk: int, dv: int) -> float:
    """Algorithmic flops per token-head of the chunked prefill: the three dk x dv products per
    token (K+ S, Q+ S, K~^T Delta), the triangular halves of the 16x16 tiles (A_kk, A_qk,
    T' (V - K+S), A_qk Delta), and the state decay."""
    return 6 * dk * dv + CHUNK * (3 * dk + 2 * dv) + 2 * dk * dv / CHUNK


def prefill_bytes_per_token_head(dk: int, dv: int, in_bytes: int = 2) -> float:
    """Algorithmic HBM bytes per token-head: q, k, log_alpha, v, beta read once, o (fp32) written once."""
    return in_bytes * (3 * dk + dv + 1) + 4 * dv


def inter_chunk_bytes_per_token_head(dk: int, dv: int, in_bytes: int = 2) -> float:
    """The inter-chunk kernel's own algorithmic traffic: q, k, log_alpha, v read, o written, and the
    chunk-local matrices T' and A_qk (2 x 16 x 16 fp32 per 16 tokens) read."""
    return in_bytes * (3 * dk + dv) + 4 * dv + 2 * 16 * 16 * 4 / CHUNK


def decode_bytes_per_head(dk: int, dv: int, in_bytes: int = 2) -> float:
    """Decode step: fp32 state read + written, q, k, log_alpha, v, beta read, o written."""
    return 2 * dk * dv * 4 + in_bytes * (3 * dk + dv + 1) + 4 * dv


def window_bytes_per_head(dk: int, dv: int, T: int, in_bytes: int = 2) -> float:
    """Decode window of T tokens: fp32 state read + written once, T tokens of inputs read and
    outputs written."""
    return 2 * dk * dv * 4 + T * (in_bytes * (3 * dk + dv + 1) + 4 * dv)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


KERNEL_SOURCES = ("gated_delta_rule_51_amd/csrc/inter_chunk.hip", "gated_delta_rule_51_amd/csrc/inter_chunk_ws.hip",
                  "gated_delta_rule_51_amd/csrc/kda_device.hpp", "gated_delta_rule_51_amd/csrc/kda_launch.hpp")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "inter_chunk_batched_prefill_traffic.txt")


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """(HBM bytes per inter-chunk launch, HIP kernel name) from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or (None, None) when it is missing or was taken on
    different kernel sources."""
    try:
        fields = {}
        with open(TRAFFIC_SUMMARY) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    fields[key.strip()] = val.strip()
        if fields.get("kernel_source_sha256_16") != kernel_source_hash():
            return None, None
        return float(fields["traffic_bytes_per_launch"]), fields.get("kernel")
    except (OSError, KeyError, ValueError):
        return None, None


def copy_calibration(torch, dev, gib: float = 1.0, reps: int = 3) -> None:
    """A plain device copy of known size (read + write gib GiB each), so hardware byte
    counters collected over this run can be scaled to true bytes."""
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


class Timer:
    """HIP events on torch's current stream (the stream every KDA call is enqueued on)."""

    def __init__(self, torch, n: int):
        self.torch = torch
        self.start = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self.end = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self.i = 0

    def __enter__(self):
        self.start[self.i].record()
        return self

    def __exit__(self, *exc):
        self.end[self.i].record()
        self.i += 1

    def mean_ms(self) -> float:
        return sum(s.elapsed_time(e) for s, e in zip(self.start[:self.i], self.end[:self.i])) / max(self.i, 1)


def cpu_baseline(workload, seed: int = 0) -> dict:
    """The fp64 oracle (as it stands) on the host cores: the whole headline batch
    (prefill of every sequence and head, then one decode token per sequence)."""
    import numpy as np
    import torch

    import oracle
    import workloads

    x = workloads.prefill_inputs(workload, device="cpu", seed=seed)
    d = workloads.decode_step_inputs(workloads.custom([1] * workload.nseq, workload.H, workload.dk, workload.dv),
                                     0, device="cpu", seed=seed)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    names = ("q", "k", "v", "log_alpha", "beta")
    args = [x[n].double().numpy() for n in names]
    dargs = [d[n].double().numpy() for n in names]
    threads = min(cores, workload.nseq * workload.H)  # the oracle runs one thread per (sequence, head) at most
    # the whole batch, repeated until about 10 s of host time have been measured
    reps, dt = 0, 0.0
    while dt < 10.0 or reps < 1:
        t0 = time.perf_counter()
        _, fin = oracle.prefill(*args, cu_seqlens=x["cu_seqlens"].numpy(), nthreads=threads)
        oracle.decode(*dargs, fin, nthreads=threads)
        dt += time.perf_counter() - t0
        reps += 1
    tokens = (workload.total_tokens + workload.nseq) * reps
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": dt, "repetitions": reps,
            "sample": f"whole batch, {reps} times: prefill of {workload.nseq}x{workload.seqlens[0]} tokens x "
                      f"{workload.H} heads (dk=dv={workload.dk}) + 1 decode token per sequence, fp64, "
                      f"{threads} threads"}


def bench_main(args, torch, kda, workloads, dev):
    w = workloads.workload(2)
    N, H, dk, dv, nseq = w.total_tokens, w.H, w.dk, w.dv, w.nseq
    sets = [workloads.prefill_inputs(w, device=dev, seed=s) for s in range(3)]
    dw = workloads.custom([1] * nseq, H, dk, dv)
    dsets = [workloads.decode_step_inputs(dw, 0, device=dev, seed=s) for s in range(3)]
    ws = kda.alloc_workspace(N, nseq, H, dk, dv, torch.bfloat16, dev)
    o = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    fin = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=dev)
    od = torch.empty((nseq, H, dv), dtype=torch.float32, device=dev)
    n_ev = args.warmup + args.steps
    t_cl, t_ic, t_dec = Timer(torch, n_ev), Timer(torch, n_ev), Timer(torch, n_ev)

    def step(i, timed):
        x, d = sets[i % 3], dsets[i % 3]
        if timed:
            with t_cl:
                kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
            with t_ic:
                kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws, None,
                                    o=o, final_state=fin)
            with t_dec:
                kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], fin, o=od)
        else:
            kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
            kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws, None,
                                o=o, final_state=fin)
            kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], fin, o=od)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    # wall-clock of exactly K untimed-by-event steps (no per-kernel events inside)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, False)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    graph_ms = None
    if args.graph:
        # the same steps replayed from HIP graphs (one per input set: the three launches of a
        # step captured once); on this stack a replay costs more than the launch gaps it removes
        graphs = []
        for i in range(3):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i, False)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % 3].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % 3].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        del graphs
    # per-kernel durations: the same K steps again with HIP events around each launch
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    ms_cl, ms_ic, ms_dec = t_cl.mean_ms(), t_ic.mean_ms(), t_dec.mean_ms()
    tokens = N + nseq
    th = N * H
    flops = th * prefill_flops_per_token_head(dk, dv)
    return {
        "w": w, "wall_ms": wall_ms, "graph_ms": graph_ms, "tokens": tokens, "ms_chunk_local": ms_cl, "ms_inter_chunk": ms_ic,
        "ms_decode": ms_dec, "prefill_tflops": flops / ((ms_cl + ms_ic) * 1e-3) / 1e12,
        "ic_bytes": th * inter_chunk_bytes_per_token_head(dk, dv) + nseq * H * dk * dv * 4,
        "cl_bytes": th * (2 * (2 * dk + dk + 1)) + (N // 16 + nseq) * H * 2048,
    }


def bench_prefill_workload(index, torch, kda, workloads, dev, reps: int):
    w = workloads.workload(index)
    N, H, dk, dv, nseq = w.total_tokens, w.H, w.dk, w.dv, w.nseq
    log(f"[bench] generating workload {w.name}: {w.notes}")
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    ws = kda.alloc_workspace(N, nseq, H, dk, dv, torch.bfloat16, dev)
    o = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    fin = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=dev)
    t_cl, t_ic = Timer(torch, reps + 1), Timer(torch, reps + 1)

    def run():
        with t_cl:
            kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
        with t_ic:
            kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws, None,
                                o=o, final_state=fin)

    run()
    torch.cuda.synchronize()
    t_cl.i = t_ic.i = 0
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    ms_cl, ms_ic = t_cl.mean_ms(), t_ic.mean_ms()
    ms = ms_cl + ms_ic
    th = N * H
    flops = th * prefill_flops_per_token_head(dk, dv)
    alg_bytes = th * prefill_bytes_per_token_head(dk, dv) + nseq * H * dk * dv * 4
    res = {
        "workload": w.name, "tokens": N, "heads": H, "sequences": nseq, "ms": round(ms, 4),
        "ms_chunk_local": round(ms_cl, 4), "ms_inter_chunk": round(ms_ic, 4),
        "tokens_per_s": N / (ms * 1e-3), "tflops": flops / (ms * 1e-3) / 1e12,
        "mfma_peak_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "hbm_gbs_algorithmic": alg_bytes / (ms * 1e-3) / 1e9,
        "hbm_roofline_frac": alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "t_hbm_ms": alg_bytes / (HBM_PEAK_GBS * 1e9) * 1e3,
    }
    if index == 5:
        res["seqlens"] = list(w.seqlens)
    del x, ws, o, fin
    torch.cuda.empty_cache()
    return res


def bench_decode(torch, kda, workloads, dev, steps):
    w = workloads.workload(4)
    B, H, dk, dv = w.nseq, w.H, w.dk, w.dv
    state = workloads.decode_initial_state(B, H, dk, dv, device=dev)
    o = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    # one untimed warm-up step on a scratch copy of the state
    scratch = state.clone()
    kda.kda_decode_step(steps[0]["q"], steps[0]["k"], steps[0]["v"], steps[0]["log_alpha"], steps[0]["beta"],
                        scratch, o=o)
    del scratch
    torch.cuda.synchronize()
    t = Timer(torch, w.decode_steps)
    for x in steps:
        with t:
            kda.kda_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], state, o=o)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    per_step = B * H * decode_bytes_per_head(dk, dv)
    gbs = per_step / (ms * 1e-3) / 1e9
    res = {"workload": w.name, "heads": B * H, "steps": w.decode_steps, "ms_per_step": round(ms, 5),
           "bytes_per_step": per_step, "gbs": gbs, "hbm_peak_frac": gbs / HBM_PEAK_GBS,
           "tokens_per_s": B / (ms * 1e-3)}
    del state, o
    torch.cuda.empty_cache()
    return res


def bench_decode_window(torch, kda, workloads, dev, steps, T: int):
    """The decode workload's steps regrouped into windows of T drafts (speculative verification):
    one kda_decode_window call per window, accepted counts uniform on [1, T] per sequence."""
    w = workloads.workload(4)
    B, H, dk, dv = w.nseq, w.H, w.dk, w.dv
    state = workloads.decode_initial_state(B, H, dk, dv, device=dev)
    names = ("q", "k", "v", "log_alpha", "beta")
    nwin = len(steps) // T
    wins = [{n: torch.stack([steps[i * T + t][n] for t in range(T)], dim=1).contiguous() for n in names}
            for i in range(nwin)]
    accs = [workloads.window_accept(B, T, device=dev, seed=i, lo=1) for i in range(nwin)]
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    scratch = state.clone()
    kda.kda_decode_window(*(wins[0][n] for n in names), scratch, accs[0], o=o)
    del scratch
    torch.cuda.synchronize()
    t = Timer(torch, nwin)
    for x, a in zip(wins, accs):
        with t:
            kda.kda_decode_window(*(x[n] for n in names), state, a, o=o)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    per_win = B * H * window_bytes_per_head(dk, dv, T)
    gbs = per_win / (ms * 1e-3) / 1e9
    accepted = float(torch.stack(accs).double().mean()) * B
    res = {"workload": f"{w.name}_window", "T": T, "heads": B * H, "windows": nwin,
           "ms_per_window": round(ms, 5), "bytes_per_window": per_win, "gbs": gbs,
           "hbm_peak_frac": gbs / HBM_PEAK_GBS, "draft_tokens_per_s": B * T / (ms * 1e-3),
           "accepted_tokens_per_s": accepted / (ms * 1e-3)}
    del state, wins, o
    torch.cuda.empty_cache()
    return res


def _event_ms(torch, fn, reps: int) -> float:
    """Mean milliseconds per call of fn() over reps back-to-back calls on torch's current stream
    (every library call is enqueued there), after one untimed call."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_layer(torch, kda, workloads, dev):
    """The layer's passes around the recurrence.  Prefill side, on the K3 layer shape (65,536
    tokens x 96 heads, d = 128, bf16): the decay gate, the ShortConv prologue of q (with L2
    norm) and the epilogue, each one HBM pass (GB/s of algorithmic bytes against 8 TB/s).
    Decode side, on the decode workload (B=256 x H=96) and at B=4: one fused launch (gate +
    step + epilogue) against the same three operations as separate launches, and the whole
    layer core per token (ShortConv of q, k, v + gate + step + epilogue) in one launch against
    six."""
    N, H, d = 65536, 96, 128
    li = workloads.layer_inputs(N, H, d, torch.bfloat16, device=dev, seed=0)
    g = torch.empty_like(li["z"])
    y = torch.empty_like(li["x"])
    e = torch.empty_like(li["u"])
    cache = torch.empty((1, H, d, 3), dtype=torch.float32, device=dev)
    elems = N * H * d
    res = {"shape": {"tokens": N, "heads": H, "d": d, "dtype": "bf16"}}
    for name, fn, nbytes in (
            ("gate", lambda: kda.kda_gate(li["z"], li["A_log"], out=g), 4 * elems),
            ("short_conv_l2", lambda: kda.kda_short_conv(li["x"], li["conv_w"], l2norm=True, cache_out=cache, y=y),
             4 * elems),
            ("out_norm_gate", lambda: kda.kda_out_norm_gate(li["o"], li["u"], li["norm_w"], 1e-6, y=e),
             8 * elems)):
        ms = _event_ms(torch, fn, 10)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 5), "bytes": nbytes, "gbs": gbs, "hbm_peak_frac": gbs / HBM_PEAK_GBS}
    del li, g, y, e
    torch.cuda.empty_cache()

    # the whole prefill layer core on the same shape: ShortConv of q, k (with L2) and v, the
    # gate, chunk-local + inter-chunk, the epilogue (eight launches)
    w3 = workloads.workload(3)
    x3 = workloads.prefill_inputs(w3, device=dev, seed=0)
    lq = workloads.layer_inputs(N, H, d, torch.bfloat16, device=dev, seed=7)
    cu = x3["cu_seqlens"]
    ws = kda.alloc_workspace(N, 1, H, d, d, torch.bfloat16, dev)
    bufs = {n: torch.empty_like(x3["q"]) for n in ("q", "k", "v", "g")}
    o3 = torch.empty((N, H, d), dtype=torch.float32, device=dev)
    fin3 = torch.empty((1, H, d, d), dtype=torch.float32, device=dev)
    y3 = torch.empty_like(x3["q"])
    cache3 = torch.empty((1, H, d, 3), dtype=torch.float32, device=dev)

    def layer_prefill():
        kda.kda_short_conv(x3["q"], lq["conv_w"], cu, l2norm=True, cache_out=cache3, y=bufs["q"])
        kda.kda_short_conv(x3["k"], lq["conv_w"], cu, l2norm=True, cache_out=cache3, y=bufs["k"])
        kda.kda_short_conv(x3["v"], lq["conv_w"], cu, cache_out=cache3, y=bufs["v"])
        kda.kda_gate(lq["z"], lq["A_log"], out=bufs["g"])
        kda.kda_prefill(bufs["q"], bufs["k"], bufs["v"], bufs["g"], x3["beta"], cu, o=o3, final_state=fin3,
                        workspace=ws)
        kda.kda_out_norm_gate(o3, lq["u"], lq["norm_w"], 1e-6, y=y3)

    ms = _event_ms(torch, layer_prefill, 5)
    res["prefill_layer_k3"] = {"tokens": N, "heads": H, "ms": round(ms, 5), "tokens_per_s": N / (ms * 1e-3),
                               "launches": 8}
    del x3, lq, ws, bufs, o3, fin3, y3, cache3
    torch.cuda.empty_cache()

    w4 = workloads.workload(4)
    step0 = workloads.decode_step_inputs(w4, 0, device=dev)
    for B in (w4.nseq, 4):
        Hd, dk, dv = w4.H, w4.dk, w4.dv
        x = {n: t[:B].contiguous() for n, t in step0.items()}
        lk = workloads.layer_inputs(B, Hd, dk, torch.bfloat16, device=dev, seed=1)
        lv = workloads.layer_inputs(B, Hd, dv, torch.bfloat16, device=dev, seed=2)
        state = workloads.decode_initial_state(B, Hd, dk, dv, device=dev)
        o = torch.empty((B, Hd, dv), dtype=torch.float32, device=dev)
        yv = torch.empty((B, Hd, dv), dtype=torch.bfloat16, device=dev)
        gz = torch.empty_like(lk["z"])

        def fused():
            kda.kda_decode_step_fused(x["q"], x["k"], x["v"], lk["z"], x["beta"], state, gate_A_log=lk["A_log"],
                                      out_gate=lv["u"], norm_w=lv["norm_w"], output_o=False, y=yv)

        def separate():
            kda.kda_gate(lk["z"], lk["A_log"], out=gz)
            kda.kda_decode_step(x["q"], x["k"], x["v"], gz, x["beta"], state, o=o)
            kda.kda_out_norm_gate(o, lv["u"], lv["norm_w"], 1e-6, y=yv)

        reps = 50 if B > 16 else 500
        ms_f, ms_s = _event_ms(torch, fused, reps), _event_ms(torch, separate, reps)
        res[f"decode_b{B}"] = {"batch": B, "heads": Hd, "ms_fused": round(ms_f, 5), "ms_separate": round(ms_s, 5),
                               "speedup": ms_s / ms_f}

        # the whole layer core per token: ShortConv of q, k, v from their caches, gate, step,
        # epilogue -- one launch against six
        C = 2 * dk + dv
        lx = workloads.layer_inputs(B, Hd, C, torch.bfloat16, nseq=B, device=dev, seed=5)
        qkv, cw, cache = lx["x"], lx["conv_w"], lx["conv_cache"]
        parts = [(0, dk, True), (dk, 2 * dk, True), (2 * dk, C, False)]
        xs = [qkv[..., lo:hi].contiguous() for lo, hi, _ in parts]
        ws = [cw[:, lo:hi].contiguous() for lo, hi, _ in parts]
        cs = [cache[:, :, lo:hi].contiguous() for lo, hi, _ in parts]
        ys = [torch.empty_like(xx) for xx in xs]

        def layer_fused():
            kda.kda_decode_layer_step(qkv, cw, cache, lk["z"], x["beta"], state, dk=dk, gate_A_log=lk["A_log"],
                                      out_gate=lv["u"], norm_w=lv["norm_w"], output_o=False, y=yv)

        def layer_separate():
            for (lo, hi, l2), xx, ww, cc, yy in zip(parts, xs, ws, cs, ys):
                kda.kda_short_conv(xx, ww, "decode", cc, l2norm=l2, cache_out=cc, y=yy)
            kda.kda_gate(lk["z"], lk["A_log"], out=gz)
            kda.kda_decode_step(ys[0], ys[1], ys[2], gz, x["beta"], state, o=o)
            kda.kda_out_norm_gate(o, lv["u"], lv["norm_w"], 1e-6, y=yv)

        ms_f, ms_s = _event_ms(torch, layer_fused, reps), _event_ms(torch, layer_separate, reps)
        res[f"decode_layer_b{B}"] = {"batch": B, "heads": Hd, "ms_fused": round(ms_f, 5),
                                     "ms_separate": round(ms_s, 5), "speedup": ms_s / ms_f}
        del x, lk, lv, state, o, yv, gz, lx, xs, ws, cs, ys

    # windows of 4 drafts at B=256: the fused call (gate in the window kernel, epilogue as a
    # second launch over o) against gate + window + epilogue as three launches
    B, T, Hd, dk, dv = w4.nseq, 4, w4.H, w4.dk, w4.dv
    xw = workloads.decode_window_inputs(w4, T, 0, device=dev)
    lk = workloads.layer_inputs(B * T, Hd, dk, torch.bfloat16, device=dev, seed=3)
    lv = workloads.layer_inputs(B * T, Hd, dv, torch.bfloat16, device=dev, seed=4)
    z, u = lk["z"].view(B, T, Hd, dk), lv["u"].view(B, T, Hd, dv)
    acc = workloads.window_accept(B, T, device=dev, seed=0, lo=1)
    state = workloads.decode_initial_state(B, Hd, dk, dv, device=dev)
    o = torch.empty((B, T, Hd, dv), dtype=torch.float32, device=dev)
    yv = torch.empty((B, T, Hd, dv), dtype=torch.bfloat16, device=dev)
    gz = torch.empty_like(z)

    def wfused():
        kda.kda_decode_window_fused(xw["q"], xw["k"], xw["v"], z, xw["beta"], state, acc, gate_A_log=lk["A_log"],
                                    out_gate=u, norm_w=lv["norm_w"], o=o, output_o=False, y=yv)

    def wseparate():
        kda.kda_gate(lk["z"], lk["A_log"], out=gz.view(B * T, Hd, dk))
        kda.kda_decode_window(xw["q"], xw["k"], xw["v"], gz, xw["beta"], state, acc, o=o)
        kda.kda_out_norm_gate(o.view(B * T, Hd, dv), lv["u"], lv["norm_w"], 1e-6, y=yv.view(B * T, Hd, dv))

    ms_f, ms_s = _event_ms(torch, wfused, 20), _event_ms(torch, wseparate, 20)
    res["decode_window4_b256"] = {"batch": B, "T": T, "heads": Hd, "ms_fused": round(ms_f, 5),
                                  "ms_separate": round(ms_s, 5), "speedup": ms_s / ms_f}
    del xw, lk, lv, state, o, yv, gz
    torch.cuda.empty_cache()
    return res


def bench_backward(index, torch, kda, workloads, dev, reps: int):
    """The prefill backward (kda_prefill_backward) on a prefill workload, with the forward time of
    the same call for reference.  Per token-head the backward moves, at least, its inputs (q, k,
    log_alpha, v, beta and dO) and gradients (fp32), and the per-chunk state and adjoint
    checkpoints: written once and read once, 4 x dk x dv x 4 B per 16 tokens."""
    w = workloads.workload(index)
    log(f"[bench] generating workload {w.name} for the backward")
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    N, H, dk, dv = w.total_tokens, w.H, w.dk, w.dv
    gen = torch.Generator(device=dev).manual_seed(1)
    d_o = torch.randn((N, H, dv), generator=gen, device=dev)
    d_f = torch.randn((w.nseq, H, dk, dv), generator=gen, device=dev)
    nbytes = int(kda.load_library().kda_prefill_backward_workspace_bytes(N, w.nseq, H, dk, dv, 1))
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)

    def bwd():
        kda.kda_prefill_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], d_o, x["cu_seqlens"], None, d_f,
                                 workspace=ws)

    def fwd():
        kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"])

    ms_b = _event_ms(torch, bwd, reps)
    ms_f = _event_ms(torch, fwd, reps)
    per_th = 2 * (3 * dk + dv + 1) + 4 * dv + 4 * (3 * dk + dv + 1) + 4 * 4 * dk * dv / CHUNK
    gbs = N * H * per_th / (ms_b * 1e-3) / 1e9
    res = {"workload": w.name, "tokens": N, "heads": H, "ms_backward": round(ms_b, 4), "ms_forward": round(ms_f, 4),
           "backward_over_forward": ms_b / ms_f, "tokens_per_s": N / (ms_b * 1e-3),
           "algorithmic_bytes": N * H * per_th, "gbs": gbs, "hbm_peak_frac": gbs / HBM_PEAK_GBS,
           "workspace_bytes": nbytes}
    del x, d_o, d_f, ws
    torch.cuda.empty_cache()
    return res


def bench_cp(wl, torch, kda, workloads, dev, segments, reps: int):
    """Intra-device context parallelism (kda_prefill_cp): every sequence in R segments run as
    independent chains (three recurrence passes and a scan), against kda_prefill on the same
    inputs.  wl is a workload index or a Workload."""
    w = workloads.workload(wl) if isinstance(wl, int) else wl
    log(f"[bench] generating workload {w.name} for context parallelism")
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    N = w.total_tokens
    lib = kda.load_library()
    ws = kda.alloc_workspace(N, w.nseq, w.H, w.dk, w.dv, x["q"].dtype, dev)

    def plain():
        kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], workspace=ws)
    res = {"workload": w.name, "ms_prefill": round(_event_ms(torch, plain, reps), 4)}
    del ws
    for R in segments:
        nb = int(lib.kda_prefill_cp_workspace_bytes(N, w.nseq, w.H, w.dk, w.dv, 1, R))
        wcp = torch.empty(nb // 4, dtype=torch.float32, device=dev)

        def cp():
            kda.kda_prefill_cp(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], segments=R,
                               workspace=wcp)
        ms = _event_ms(torch, cp, reps)
        res[f"ms_cp_{R}"] = round(ms, 4)
        res[f"cp_{R}_over_prefill"] = round(ms / res["ms_prefill"], 3)
        del wcp
    del x
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="all",
                    choices=["all", "main", "k3", "decode", "layer", "backward", "cp", "varlen", "none"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the headline step as HIP graph replays (reported beside the eager time)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU; --gpus must be 1 (heads and sequences shard "
              "across GPUs with no exchange -- see the design notes)", file=sys.stderr)
        return 2

    import torch

    import gated_delta_rule_51_amd as kda
    import workloads

    if not os.path.exists(kda.LIBRARY):
        import __graft_entry__

        __graft_entry__.build()
    kda.load_library()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(torch, dev)
    out = {"metric": "KDA prefill tokens/s + TFLOP/s (% MFMA peak); decode state GB/s (% HBM peak)",
           "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic"}

    if args.only in ("all", "main"):
        log("[bench] headline step: batched prefill B=4 H=8 T=2048 + 1 decode token per sequence")
        m = bench_main(args, torch, kda, workloads, dev)
        w = m["w"]
        out["value"] = m["tokens"] / (m["wall_ms"] * 1e-3)
        out["ms_per_step"] = round(m["wall_ms"], 5)
        if m["graph_ms"] is not None:
            out["ms_per_step_graph_replay"] = round(m["graph_ms"], 5)
        out["config"] = {"workload": "batched_prefill_then_decode", "batch": w.nseq, "heads": w.H,
                         "seq_len": w.seqlens[0], "dk": w.dk, "dv": w.dv, "chunk": CHUNK,
                         "inputs": "bf16", "state": "fp32", "output": "fp32",
                         "step": "kda_chunk_local + kda_inter_chunk over the batch, then kda_decode_step "
                                 "(1 token per sequence) from the final states",
                         "input_sets_rotated": 3}
        kernels = {"chunk_local": m["ms_chunk_local"], "inter_chunk": m["ms_inter_chunk"],
                   "decode": m["ms_decode"]}
        out["kernel_ms"] = {k: round(v, 5) for k, v in kernels.items()}
        out["prefill_tflops"] = m["prefill_tflops"]
        out["prefill_mfma_peak_frac"] = m["prefill_tflops"] / MFMA_BF16_PEAK_TFLOPS
        dom = max(("chunk_local", "inter_chunk"), key=lambda k: kernels[k])
        b = m["ic_bytes"] if dom == "inter_chunk" else m["cl_bytes"]
        ach = b / (kernels[dom] * 1e-3) / 1e9
        traffic, hip_kernel = measured_traffic() if dom == "inter_chunk" else (None, None)
        out["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": traffic,
                           "algorithmic_bytes_per_launch": b}
        if hip_kernel:
            out["roofline"]["hip_kernel"] = hip_kernel
        if not args.no_cpu_baseline:
            log("[bench] cpu baseline: fp64 oracle on the same batch")
            out["cpu_baseline"] = cpu_baseline(w)
    if args.only in ("all", "k3"):
        log("[bench] K3 layer prefill B=1 H=96 T=65536")
        out["k3_layer"] = bench_prefill_workload(3, torch, kda, workloads, dev, reps=5)
    if args.only in ("all", "decode"):
        log("[bench] recurrent decode B=256 H=96, 128 steps")
        w4 = workloads.workload(4)
        steps = [workloads.decode_step_inputs(w4, s, device=dev) for s in range(w4.decode_steps)]
        out["decode"] = bench_decode(torch, kda, workloads, dev, steps)
        for T in (4, 8):
            log(f"[bench] decode windows of {T} drafts (speculative verification), B=256 H=96")
            out[f"decode_window_{T}"] = bench_decode_window(torch, kda, workloads, dev, steps, T)
        del steps
        torch.cuda.empty_cache()
    if args.only in ("all", "backward"):
        log("[bench] prefill backward: batched workload and the K3 layer")
        out["backward"] = {"batched": bench_backward(2, torch, kda, workloads, dev, reps=5),
                           "k3_layer": bench_backward(3, torch, kda, workloads, dev, reps=2)}
    if args.only in ("all", "cp"):
        log("[bench] intra-device context parallelism: batched workload and the K3 layer")
        out["context_parallel"] = {"batched": bench_cp(2, torch, kda, workloads, dev, (2, 4, 8), reps=10),
                                   "k3_layer": bench_cp(3, torch, kda, workloads, dev, (2, 4), reps=2),
                                   "k3_sequence_12_heads": bench_cp(
                                       workloads.custom([65536], 12, 128, 128, name="k3_sequence_12_heads"),
                                       torch, kda, workloads, dev, (4, 8, 10, 16), reps=3)}
    if args.only in ("all", "layer"):
        log("[bench] layer passes (gate, ShortConv, epilogue) and the fused decode step")
        out["layer"] = bench_layer(torch, kda, workloads, dev)
    if args.only in ("all", "varlen"):
        log("[bench] varlen 1M-token prefill")
        out["varlen_1m"] = bench_prefill_workload(5, torch, kda, workloads, dev, reps=3)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
