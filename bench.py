"""Benchmark of the MI355X KDA library (one GPU).

One step = one pass of the whole hot path over one batch: the prefill of the 1,048,576-token
varlen workload (27 packed sequences of log-uniform length in [512, 262,144], H=96, dk=dv=128,
bf16 inputs, fp32 state and output) and one decode step per sequence continuing from the
prefill's final states.  The inputs (155 GB) are resident in HBM before timing starts and far
exceed the 256 MB Infinity Cache.  The headline line carries:
  * value / ms_per_step: tokens (prefill tokens + one decode token per sequence) per second over
    K steps bracketed by device synchronisation, plus median and minimum step times from HIP
    events;
  * roofline: the dominant kernel's algorithmic bytes (q, k, v, log_alpha, beta read once, o
    written once, final states written) over its average launch time from HIP events on the
    stream it runs on, against 8 TB/s, with HBM traffic from committed rocprofv3 counters;
  * parity: the outputs of the last timed step (o, the decode output and the state after the
    decode step) against the fp64 oracle on 8 heads (one per residue mod 8) of every sequence;
  * cpu_baseline: the oracle's time on those 8 heads, extrapolated to all 96, with the CPU model,
    the threads it used and a single-thread rate.

Sub-objects of the same line, each measured in the same run:
  * "batched": prefill of B=4, H=8, T=2048 + one decode token (three input sets rotated),
  * "k3_layer": prefill of B=1, H=96, T=65,536 (the K3 layer shape),
  * "decode":   128 recurrent steps over B=256 x H=96 heads (1.6 GB of fp32 state),
  * "decode_window_4" / "_8": the same 128 steps as windows of 4 or 8 draft tokens
    (speculative verification: one state read and write per window),
  * "layer": the passes around the recurrence (decay gate, ShortConv prologue, RMSNorm +
    output-gate epilogue) on the K3 layer shape, and the fused decode step against the
    same operations as separate launches,
  * "backward": the prefill backward on the batched workload and the K3 layer,
  * "context_parallel": the prefill with every sequence split into R segments (intra-device
    context parallelism) against the plain prefill.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--only main|batched|k3|decode|layer|backward|cp|none]
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


def decode_bytes_per_head(dk: int, dv: int, in_bytes: int = 2) -> float:
    """Decode step: fp32 state read + written, q, k, log_alpha, v, beta read, o written."""
    return 2 * dk * dv * 4 + in_bytes * (3 * dk + dv + 1) + 4 * dv


def window_bytes_per_head(dk: int, dv: int, T: int, in_bytes: int = 2) -> float:
    """Decode window of T tokens: fp32 state read + written once, T tokens of inputs read and
    outputs written."""
    return 2 * dk * dv * 4 + T * (in_bytes * (3 * dk + dv + 1) + 4 * dv)


N_CU = 256  # MI355X compute units


def bound_fields(flops: float, alg_bytes: float, ms: float, seqlens, H: int) -> dict:
    """The prefill's ceilings beside its time: HBM time and matrix-core time of the algorithmic
    bytes and flops (the active bound is the larger), the attainable rate min(MFMA peak,
    arithmetic intensity x HBM peak) and the fraction of it reached, and the serial-chain view:
    chunk steps of the longest (sequence, head) chain and of an even share of all chains per
    compute unit, with the time per step of each."""
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
    att = min(MFMA_BF16_PEAK_TFLOPS, flops / alg_bytes * HBM_PEAK_GBS / 1e3)
    longest = max(1, -(-max(seqlens) // CHUNK))
    per_cu = max(1.0, sum(-(-n // CHUNK) for n in seqlens) * H / N_CU)
    return {"t_hbm_ms": t_hbm, "t_mfma_ms": t_mfma, "active_bound": "hbm" if t_hbm >= t_mfma else "mfma",
            "time_over_bound": ms / max(t_hbm, t_mfma), "attainable_tflops": att,
            "attainable_frac": flops / (ms * 1e-3) / 1e12 / att,
            "longest_chain_steps": longest, "ns_per_longest_chain_step": ms * 1e6 / longest,
            "chain_steps_per_cu": per_cu, "ns_per_chain_step_per_cu": ms * 1e6 / per_cu}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def host_info() -> dict:
    """CPU model and the logical cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return {"cpu_model": model, "cores_available": cores}


KERNEL_SOURCES = ("gated_delta_rule_51_amd/csrc/prefill_fused.hip", "gated_delta_rule_51_amd/csrc/kda_device.hpp")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "prefill_varlen_1m_traffic.txt")


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        path = os.path.join(ROOT, rel)
        if os.path.exists(path):
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(path: str = TRAFFIC_SUMMARY):
    """(HBM bytes per launch, HIP kernel name) from a committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or (None, None) when it is missing or was taken on different kernel
    sources."""
    try:
        fields = {}
        with open(path) as f:
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


# heads the oracle recomputes on the headline workload: one per residue mod 8 (the XCD a
# (sequence, head) chain runs on is its index mod 8, and with 96 heads that is the head mod 8)
PARITY_HEADS = (0, 13, 26, 39, 52, 65, 78, 91)


def oracle_check(x, o, od, state, d, heads, tol: float, group: int = 4) -> dict:
    """Run the fp64 oracle on ``heads`` of every sequence of the prefill inputs ``x`` (device
    tensors), then one decode step with the decode inputs ``d``; compare with the GPU's prefill
    output ``o``, decode output ``od`` and state after the decode step ``state``.  Heads go
    through the oracle ``group`` at a time (host memory: ~5.4 GB of fp64 per head at 1M tokens).
    Returns the errors (max|err| / RMS(ref), pooled over the heads) and the oracle's wall time."""
    import numpy as np

    import oracle

    info = host_info()
    threads = info["cores_available"]
    names = ("q", "k", "v", "log_alpha", "beta")
    cu = x["cu_seqlens"].cpu().numpy()
    err = {"o": [0.0, 0.0], "decode_o": [0.0, 0.0], "state": [0.0, 0.0]}  # [sum sq ref, max abs err]
    seconds = 0.0
    for g0 in range(0, len(heads), group):
        hs = list(heads[g0:g0 + group])
        cpu = {n: x[n][:, hs].contiguous().cpu() for n in names}
        t0 = time.perf_counter()
        o_ref, f_ref = oracle.prefill(*(cpu[n] for n in names), cu_seqlens=cu, nthreads=threads)
        seconds += time.perf_counter() - t0
        del cpu
        od_ref, s_ref = oracle.decode(*(d[n][:, hs].contiguous().cpu() for n in names), f_ref, nthreads=threads)
        for key, got, ref in (("o", o[:, hs], o_ref), ("decode_o", od[:, hs], od_ref), ("state", state[:, hs], s_ref)):
            g = got.contiguous().cpu().double().numpy()
            if not np.all(np.isfinite(g)):
                err[key][1] = float("inf")
            err[key][0] += float(np.sum(ref * ref))
            err[key][1] = max(err[key][1], float(np.max(np.abs(g - ref))) if ref.size else 0.0)
        del o_ref, f_ref, od_ref, s_ref
    counts = {"o": o[:, list(heads)].numel(), "decode_o": od[:, list(heads)].numel(),
              "state": state[:, list(heads)].numel()}
    out = {"heads": list(heads), "tol_max_err_over_rms": tol}
    for key, (ss, mx) in err.items():
        rms = (ss / max(counts[key], 1)) ** 0.5
        out[f"{key}_max_err_over_rms"] = mx / rms if rms > 0 else mx
    out["pass"] = all(out[f"{k}_max_err_over_rms"] <= tol for k in err)
    return {"parity": out, "oracle_seconds": seconds, "threads": threads, "cpu_model": info["cpu_model"]}


def oracle_single_thread_rate(x, seqlen: int = 8192) -> float:
    """Token-heads per second of the oracle on one thread: the first ``seqlen`` tokens of the
    longest sequence, head 0."""
    import numpy as np

    import oracle

    cu = x["cu_seqlens"].cpu().numpy()
    lens = np.diff(cu)
    s = int(np.argmax(lens))
    n = int(min(seqlen, lens[s]))
    a, b = int(cu[s]), int(cu[s]) + n
    cpu = [x[nm][a:b, :1].contiguous().cpu() for nm in ("q", "k", "v", "log_alpha", "beta")]
    t0 = time.perf_counter()
    oracle.prefill(*cpu, nthreads=1)
    return n / (time.perf_counter() - t0)


def bench_headline(args, torch, kda, workloads, dev, cpu_baseline: bool = True) -> dict:
    """The headline step on the varlen 1M workload: kda_prefill over 1,048,576 packed tokens
    (27 sequences, H=96, dk=dv=128, bf16), then kda_decode_step of one more token per sequence
    from the final states.  Returns the fields of the JSON line."""
    import statistics

    w = workloads.workload(5)
    N, H, dk, dv, nseq = w.total_tokens, w.H, w.dk, w.dv, w.nseq
    log(f"[bench] generating workload {w.name}: {w.notes}")
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    dw = workloads.custom([1] * nseq, H, dk, dv)
    dsets = [workloads.decode_step_inputs(dw, 0, device=dev, seed=s) for s in range(3)]
    ws_bytes = kda.kda_prefill_workspace_bytes(N, nseq, H, dk, dv, torch.bfloat16)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=dev) if ws_bytes else None
    single_pass = ws_bytes == 0
    o = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    fin = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=dev)
    od = torch.empty((nseq, H, dv), dtype=torch.float32, device=dev)
    args_x = (x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"])

    def prefill():
        kda.kda_prefill(*args_x, o=o, final_state=fin, workspace=ws)

    def step(i):
        d = dsets[i % 3]
        prefill()
        kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], fin, o=od)

    log(f"[bench] headline: {args.warmup} warm-up + {args.steps} timed steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    step_ms = [a.elapsed_time(b) for a, b in ev]
    last = (args.steps - 1) % 3  # decode inputs of the last timed step

    # parity of the last timed step's outputs, and the oracle's time on the same heads
    check = None
    if cpu_baseline:
        log(f"[bench] oracle on heads {PARITY_HEADS} of every sequence (parity of the timed outputs)")
        check = oracle_check(x, o, od, fin, dsets[last], PARITY_HEADS, tol=1e-2)
        log(f"[bench] parity: {check['parity']}")

    # per-kernel durations: HIP events on the stream every call is enqueued on (torch's
    # current stream) around the prefill (one kernel on this shape) and the decode step
    reps = max(3, min(args.steps, 10))
    t_pf, t_dec = Timer(torch, reps), Timer(torch, reps)
    for i in range(reps):
        d = dsets[i % 3]
        with t_pf:
            prefill()
        with t_dec:
            kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], fin, o=od)
    torch.cuda.synchronize()
    kernels = {"prefill": t_pf.mean_ms(), "decode": t_dec.mean_ms()}
    # the two-kernel path (chunk-local pass, then the recurrence) on the same inputs, for reference
    two = None
    if single_pass and not args.no_two_kernel:
        wsp = kda.alloc_workspace(N, nseq, H, dk, dv, torch.bfloat16, dev)
        t_cl, t_ic = Timer(torch, 3), Timer(torch, 3)
        for _ in range(3):
            with t_cl:
                kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], wsp)
            with t_ic:
                kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], wsp, None,
                                    o=o, final_state=fin)
        torch.cuda.synchronize()
        two = {"chunk_local_ms": round(t_cl.mean_ms(), 4), "inter_chunk_ms": round(t_ic.mean_ms(), 4),
               "total_ms": round(t_cl.mean_ms() + t_ic.mean_ms(), 4)}
        del wsp
    th = N * H
    prefill_ms = kernels["prefill"]
    flops = th * prefill_flops_per_token_head(dk, dv)
    alg_bytes = th * prefill_bytes_per_token_head(dk, dv) + nseq * H * dk * dv * 4
    ach = alg_bytes / (prefill_ms * 1e-3) / 1e9
    traffic, hip_kernel = measured_traffic()
    res = {
        "value": (N + nseq) / (wall_ms * 1e-3), "ms_per_step": round(wall_ms, 4),
        "ms_per_step_median": round(statistics.median(step_ms), 4), "ms_per_step_min": round(min(step_ms), 4),
        "config": {"workload": w.name, "tokens": N, "sequences": nseq, "seqlens": list(w.seqlens), "heads": H,
                   "dk": dk, "dv": dv, "chunk": CHUNK, "inputs": "bf16", "state": "fp32", "output": "fp32",
                   "step": "kda_prefill over the packed batch, then kda_decode_step (1 token per sequence) "
                           "from the final states"},
        "kernel_ms": {k: round(v, 4) for k, v in kernels.items()},
        "prefill": {"ms": round(prefill_ms, 4), "single_pass": single_pass, "tokens_per_s": N / (prefill_ms * 1e-3),
                    "tflops": flops / (prefill_ms * 1e-3) / 1e12,
                    "mfma_peak_frac": flops / (prefill_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                    "hbm_gbs_algorithmic": ach, "hbm_roofline_frac": ach / HBM_PEAK_GBS,
                    **bound_fields(flops, alg_bytes, prefill_ms, w.seqlens, H)},
        "roofline": {"kernel": "prefill" if single_pass else "prefill (chunk_local + inter_chunk)",
                     "hip_kernel": hip_kernel or ("prefill_fused_kernel<128,128,4,2>" if single_pass else None),
                     "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes_per_launch": alg_bytes,
                     "bytes_formula": "N*H*(2*(3*dk+dv+1) + 4*dv) + nseq*H*dk*dv*4"},
    }
    if two is not None:
        res["prefill"]["two_kernel_path"] = two
    if check is not None:
        res["parity"] = check["parity"]
        frac = len(PARITY_HEADS) / H
        t_full = check["oracle_seconds"] / frac
        st_rate = oracle_single_thread_rate(x)
        res["cpu_baseline"] = {
            "value": (N + nseq) / t_full, "unit": "tokens/s", "cores": check["threads"], "kind": "oracle",
            "cpu_model": check["cpu_model"], "seconds_measured": round(check["oracle_seconds"], 3),
            "extrapolated": True,
            "sample": f"fp64 oracle prefill of all {nseq} sequences on heads {list(PARITY_HEADS)} "
                      f"({len(PARITY_HEADS)} of {H}), {check['threads']} threads; time scaled by {H}/"
                      f"{len(PARITY_HEADS)} to the whole workload (the decode token is not timed)",
            "single_thread_token_heads_per_s": st_rate,
            "single_thread_tokens_per_s": st_rate / H}
    del x, ws, o, fin, od, dsets
    torch.cuda.empty_cache()
    return res


def bench_batched(args, torch, kda, workloads, dev):
    """B=4, H=8, T=2048 (three input sets rotated, ~105 MB each, so no set stays in the 256 MB
    Infinity Cache): kda_prefill then one decode token per sequence from the final states."""
    w = workloads.workload(2)
    N, H, dk, dv, nseq = w.total_tokens, w.H, w.dk, w.dv, w.nseq
    sets = [workloads.prefill_inputs(w, device=dev, seed=s) for s in range(3)]
    dw = workloads.custom([1] * nseq, H, dk, dv)
    dsets = [workloads.decode_step_inputs(dw, 0, device=dev, seed=s) for s in range(3)]
    o = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    fin = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=dev)
    od = torch.empty((nseq, H, dv), dtype=torch.float32, device=dev)
    n_ev = args.steps
    t_pf, t_dec = Timer(torch, n_ev), Timer(torch, n_ev)

    def step(i, timed):
        x, d = sets[i % 3], dsets[i % 3]
        if timed:
            with t_pf:
                kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], o=o,
                                final_state=fin)
            with t_dec:
                kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], fin, o=od)
        else:
            kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], o=o,
                            final_state=fin)
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
        # the same steps replayed from HIP graphs (one per input set: the launches of a step
        # captured once)
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
    ms_pf, ms_dec = t_pf.mean_ms(), t_dec.mean_ms()
    tokens = N + nseq
    th = N * H
    flops = th * prefill_flops_per_token_head(dk, dv)
    return {"w": w, "wall_ms": wall_ms, "graph_ms": graph_ms, "tokens": tokens, "ms_prefill": ms_pf,
            "ms_decode": ms_dec, "prefill_tflops": flops / (ms_pf * 1e-3) / 1e12}


def bench_prefill_workload(index, torch, kda, workloads, dev, reps: int):
    """kda_prefill on a prefill workload (one kernel for bf16 with dk = dv = 128), and the two-kernel
    path (kda_chunk_local + kda_inter_chunk) on the same inputs for reference."""
    w = workloads.workload(index)
    N, H, dk, dv, nseq = w.total_tokens, w.H, w.dk, w.dv, w.nseq
    log(f"[bench] generating workload {w.name}: {w.notes}")
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    o = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    fin = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=dev)
    args_x = (x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"])
    # three rounds of reps calls after the warm-up (the first calls after the inputs are generated
    # run slower); the median round is reported, the fastest beside it
    rounds = sorted(_event_ms(torch, lambda: kda.kda_prefill(*args_x, o=o, final_state=fin), reps)
                    for _ in range(3))
    ms, ms_min = rounds[1], rounds[0]
    ws = kda.alloc_workspace(N, nseq, H, dk, dv, torch.bfloat16, dev)
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
    th = N * H
    flops = th * prefill_flops_per_token_head(dk, dv)
    alg_bytes = th * prefill_bytes_per_token_head(dk, dv) + nseq * H * dk * dv * 4
    res = {
        "workload": w.name, "tokens": N, "heads": H, "sequences": nseq, "ms": round(ms, 4),
        "ms_min": round(ms_min, 4),
        "two_kernel_path": {"ms_chunk_local": round(ms_cl, 4), "ms_inter_chunk": round(ms_ic, 4),
                            "ms": round(ms_cl + ms_ic, 4)},
        "tokens_per_s": N / (ms * 1e-3), "tflops": flops / (ms * 1e-3) / 1e12,
        "mfma_peak_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "hbm_gbs_algorithmic": alg_bytes / (ms * 1e-3) / 1e9,
        "hbm_roofline_frac": alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        **bound_fields(flops, alg_bytes, ms, w.seqlens, H),
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
    # context beside the published peak: torch's device-to-device copy of the state (the same
    # bytes read and written once)
    dst = torch.empty_like(state)
    ms_copy = _event_ms(torch, lambda: dst.copy_(state), 10)
    res["torch_copy_gbs"] = 2 * state.numel() * 4 / (ms_copy * 1e-3) / 1e9
    del state, o, dst
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
           "form": "one chunk (matrix cores)" if T >= 6 else "token by token",
           "ms_per_window": round(ms, 5), "bytes_per_window": per_win, "gbs": gbs,
           "hbm_peak_frac": gbs / HBM_PEAK_GBS, "draft_tokens_per_s": B * T / (ms * 1e-3),
           "accepted_tokens_per_s": accepted / (ms * 1e-3)}
    if T >= 6:  # the token-by-token form on the same windows, for comparison
        state2 = workloads.decode_initial_state(B, H, dk, dv, device=dev)
        t1 = Timer(torch, nwin)
        for x, a in zip(wins, accs):
            with t1:
                kda.kda_decode_window(*(x[n] for n in names), state2, a, o=o, form=1)
        torch.cuda.synchronize()
        res["ms_per_window_token_form"] = round(t1.mean_ms(), 5)
        del state2
    del state, wins, o
    torch.cuda.empty_cache()
    return res


def bench_decode_window_replay(torch, kda, workloads, dev, steps, T: int):
    """The same windows as a serving loop runs them: each kda_decode_window_replay call replays
    the previous window's accepted prefix (counts drawn uniform on [1, T], known only after that
    window ran), commits the state after it, and runs the new window without committing it."""
    w = workloads.workload(4)
    B, H, dk, dv = w.nseq, w.H, w.dk, w.dv
    state = workloads.decode_initial_state(B, H, dk, dv, device=dev)
    names = ("q", "k", "v", "log_alpha", "beta")
    nwin = len(steps) // T
    wins = [{n: torch.stack([steps[i * T + t][n] for t in range(T)], dim=1).contiguous() for n in names}
            for i in range(nwin)]
    accs = [workloads.window_accept(B, T, device=dev, seed=i, lo=1) for i in range(nwin)]
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)

    def prev_of(i):
        x = wins[i - 1]
        return {"q": x["q"], "k": x["k"], "v": x["v"], "gate": x["log_alpha"], "beta": x["beta"]}
    scratch = state.clone()
    kda.kda_decode_window_replay(prev_of(1), accs[0], *(wins[1][n] for n in names), scratch, o=o)
    del scratch
    torch.cuda.synchronize()
    t = Timer(torch, nwin - 1)
    for i in range(1, nwin):  # window 0 only supplies the first replay
        x = wins[i]
        with t:
            kda.kda_decode_window_replay(prev_of(i), accs[i - 1], *(x[n] for n in names), state, o=o)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    replayed = float(torch.stack(accs[:-1]).double().mean())
    # state read + written once, T new and (on average) `replayed` replayed tokens of inputs, T outputs
    per_call = B * H * (window_bytes_per_head(dk, dv, T) + replayed * (2 * (3 * dk + dv + 1)))
    gbs = per_call / (ms * 1e-3) / 1e9
    res = {"workload": f"{w.name}_window_replay", "T": T, "heads": B * H, "calls": nwin - 1,
           "ms_per_call": round(ms, 5), "replayed_tokens_mean": replayed, "gbs": gbs,
           "hbm_peak_frac": gbs / HBM_PEAK_GBS, "accepted_tokens_per_s": replayed * B / (ms * 1e-3),
           "draft_tokens_per_s": B * T / (ms * 1e-3)}
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
    del bufs, ws
    torch.cuda.empty_cache()

    # the same layer core with the prologue fused into the recurrence's loads: ShortConv + Swish
    # (+ L2) of the raw q, k, v and the gate inside chunk-local and inter-chunk, then the cache
    # copy and the epilogue (four launches)
    wsl = torch.empty(kda.kda_prefill_layer_workspace_bytes(N, 1, H) // 4 + 4, dtype=torch.float32, device=dev)
    conv_w3 = torch.cat([lq["conv_w"]] * 3, dim=1).contiguous()
    cache3c = torch.zeros((1, H, 3 * d, 3), dtype=torch.float32, device=dev)

    def layer_prefill_fused():
        kda.kda_prefill_layer(x3["q"], x3["k"], x3["v"], conv_w3, lq["z"], lq["A_log"], x3["beta"], cu,
                              conv_cache_out=cache3c, out_gate=lq["u"], norm_w=lq["norm_w"], o=o3,
                              final_state=fin3, y=y3, workspace=wsl)

    ms_f = _event_ms(torch, layer_prefill_fused, 5)
    res["prefill_layer_k3_fused"] = {"tokens": N, "heads": H, "ms": round(ms_f, 5),
                                     "tokens_per_s": N / (ms_f * 1e-3), "launches": 4,
                                     "speedup_vs_separate": ms / ms_f}
    del x3, lq, o3, fin3, y3, cache3, wsl, conv_w3, cache3c
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

    # windows of 8 with the gate from logits and the epilogue: one chunk on the matrix cores (the
    # gate in fp32 inside the chunk kernel), against the gate pass + the window + the epilogue pass
    T8 = 8
    w8 = workloads.workload(4)
    x8 = workloads.decode_window_inputs(w8, T8, 0, device=dev)
    k8 = workloads.layer_inputs(B * T8, Hd, dk, torch.bfloat16, device=dev, seed=5)
    v8 = workloads.layer_inputs(B * T8, Hd, dv, torch.bfloat16, device=dev, seed=6)
    z8, u8 = k8["z"].view(B, T8, Hd, dk), v8["u"].view(B, T8, Hd, dv)
    acc8 = workloads.window_accept(B, T8, device=dev, seed=0, lo=1)
    o8 = torch.empty((B, T8, Hd, dv), dtype=torch.float32, device=dev)
    y8 = torch.empty((B, T8, Hd, dv), dtype=torch.bfloat16, device=dev)
    g8 = torch.empty_like(z8)

    def w8fused():
        kda.kda_decode_window_fused(x8["q"], x8["k"], x8["v"], z8, x8["beta"], state, acc8, gate_A_log=k8["A_log"],
                                    out_gate=u8, norm_w=v8["norm_w"], o=o8, output_o=False, y=y8)

    def w8separate():
        kda.kda_gate(k8["z"], k8["A_log"], out=g8.view(B * T8, Hd, dk))
        kda.kda_decode_window(x8["q"], x8["k"], x8["v"], g8, x8["beta"], state, acc8, o=o8)
        kda.kda_out_norm_gate(o8.view(B * T8, Hd, dv), v8["u"], v8["norm_w"], 1e-6, y=y8.view(B * T8, Hd, dv))

    ms_f8, ms_s8 = _event_ms(torch, w8fused, 20), _event_ms(torch, w8separate, 20)
    res["decode_window8_b256"] = {"batch": B, "T": T8, "heads": Hd, "ms_fused": round(ms_f8, 5),
                                  "ms_separate": round(ms_s8, 5), "speedup": ms_s8 / ms_f8}
    del x8, k8, v8, z8, u8, acc8, o8, y8, g8

    # the layer core's speculative-decoding call at B=256, T=4: the previous window's accepted
    # prefix replayed and the new window run through ShortConv (+ L2), gate and recurrence, the
    # state and convolution cache committed after the prefix, then the epilogue pass; the one-chunk
    # form (prologue pass + chunk kernel, chosen for T + Tp = 8) and the token-by-token kernel
    C = 2 * dk + dv
    lwins = []
    for i in range(3):
        lx = workloads.layer_inputs(B * T, Hd, C, torch.bfloat16, nseq=B, device=dev, seed=20 + i)
        lz = workloads.layer_inputs(B * T, Hd, dk, torch.bfloat16, device=dev, seed=30 + i)
        lwins.append({"qkv": lx["x"].view(B, T, Hd, C), "gate": lz["z"].view(B, T, Hd, dk), "beta": xw["beta"]})
    conv_w = lx["conv_w"]
    cache = workloads.layer_inputs(B, Hd, C, torch.bfloat16, nseq=B, device=dev, seed=40)["conv_cache"]
    calls = [0]

    need = kda.kda_decode_layer_window_workspace_bytes(B, T, T, Hd, dk, dv, torch.bfloat16)
    lws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def lwin(form):
        i = calls[0] = calls[0] + 1
        kda.kda_decode_layer_window_replay(lwins[(i - 1) % 3], acc, lwins[i % 3]["qkv"], lwins[i % 3]["gate"],
                                           lwins[i % 3]["beta"], conv_w, cache, state, dk=dk,
                                           gate_A_log=lk["A_log"], out_gate=u, norm_w=lv["norm_w"], o=o, y=yv,
                                           form=form, workspace=lws if form != 1 else None)

    ms_l = _event_ms(torch, lambda: lwin(None), 20)
    ms_t = _event_ms(torch, lambda: lwin(1), 20)
    replayed = float(acc.double().mean())
    # algorithmic HBM bytes: the state and the convolution cache (fp32, 3 inputs per channel) read
    # and written once per head; per replayed token its raw q | k | v row, gate logits and beta;
    # per window token those, o (fp32), u and y
    bpt_r = 2 * (C + dk + 1)
    bpt_w = bpt_r + 4 * dv + 2 * dv + 2 * dv
    nbytes = B * Hd * (2 * dk * dv * 4 + 2 * C * 3 * 4 + replayed * bpt_r + T * bpt_w)
    res["decode_layer_window_replay4_b256"] = {"batch": B, "T": T, "heads": Hd, "form": "one chunk" if need else
                                               "token by token", "ms_per_call": round(ms_l, 5),
                                               "ms_token_by_token": round(ms_t, 5),
                                               "replayed_tokens_mean": replayed,
                                               "token_steps_per_s": B * (T + replayed) / (ms_l * 1e-3),
                                               "hbm_gbs_algorithmic": nbytes / (ms_l * 1e-3) / 1e9,
                                               "hbm_roofline_frac": nbytes / (ms_l * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del xw, lk, lv, state, o, yv, gz, lwins, cache, lws
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
    del ws
    torch.cuda.empty_cache()
    if w.nseq == 1 and N > 16384:
        # one long sequence: the slabbed backward, one slab's workspace at a time
        slab = 16384
        nb2 = kda.kda_prefill_backward_slabbed_workspace_bytes(N, H, dk, dv, slab, x["q"].dtype)
        ws2 = torch.empty(nb2 // 4 + 4, dtype=torch.float32, device=dev)

        def bwd_slabbed():
            kda.kda_prefill_backward_slabbed(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], d_o, None, d_f,
                                             slab_tokens=slab, workspace=ws2)
        ms_s = _event_ms(torch, bwd_slabbed, reps)
        res["slabbed"] = {"slab_tokens": slab, "ms_backward": round(ms_s, 4), "over_unsliced": ms_s / ms_b,
                          "workspace_bytes": nb2}
        del ws2
    del x, d_o, d_f
    torch.cuda.empty_cache()
    return res


def bench_cp(wl, torch, kda, workloads, dev, segments, reps: int):
    """Intra-device context parallelism (kda_prefill_cp): every sequence in R segments run as
    independent chains (up to three recurrence passes and a scan), against the plain two-kernel
    prefill on the same inputs, and kda_prefill with its own choice between them.  wl is a
    workload index or a Workload."""
    w = workloads.workload(wl) if isinstance(wl, int) else wl
    log(f"[bench] generating workload {w.name} for context parallelism")
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    N = w.total_tokens
    lib = kda.load_library()
    ws = kda.alloc_workspace(N, w.nseq, w.H, w.dk, w.dv, x["q"].dtype, dev)

    def plain():
        kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
        kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws)
    res = {"workload": w.name, "ms_prefill": round(_event_ms(torch, plain, reps), 4)}
    del ws
    nb = kda.kda_prefill_workspace_bytes(N, w.nseq, w.H, w.dk, w.dv, x["q"].dtype)
    wp = torch.empty(max(nb, 16) // 4, dtype=torch.float32, device=dev)

    def auto():
        kda.kda_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"], workspace=wp)
    res["ms_kda_prefill"] = round(_event_ms(torch, auto, reps), 4)
    res["kda_prefill_uses_cp"] = nb != kda.kda_chunk_workspace_bytes(N, w.nseq, w.H, w.dk, w.dv, x["q"].dtype) \
        and nb > 0
    del wp
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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default="all",
                    choices=["all", "main", "batched", "k3", "decode", "layer", "backward", "cp", "none"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-two-kernel", action="store_true",
                    help="skip timing the two-kernel prefill path beside the single-pass kernel")
    ap.add_argument("--graph", action="store_true",
                    help="also time the batched step as HIP graph replays (reported beside the eager time)")
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
        log("[bench] headline step: varlen 1M prefill (27 sequences, H=96) + 1 decode token per sequence")
        out.update(bench_headline(args, torch, kda, workloads, dev, cpu_baseline=not args.no_cpu_baseline))
    if args.only in ("all", "batched"):
        log("[bench] batched prefill B=4 H=8 T=2048 + 1 decode token per sequence")
        m = bench_batched(args, torch, kda, workloads, dev)
        w = m["w"]
        kernels = {"prefill": m["ms_prefill"], "decode": m["ms_decode"]}
        th = w.total_tokens * w.H
        alg = th * prefill_bytes_per_token_head(w.dk, w.dv) + w.nseq * w.H * w.dk * w.dv * 4
        out["batched"] = {
            "workload": w.name, "batch": w.nseq, "heads": w.H, "seq_len": w.seqlens[0], "input_sets_rotated": 3,
            "ms_per_step": round(m["wall_ms"], 5), "tokens_per_s": m["tokens"] / (m["wall_ms"] * 1e-3),
            "kernel_ms": {k: round(v, 5) for k, v in kernels.items()},
            "prefill_tflops": m["prefill_tflops"],
            "prefill_hbm_frac": alg / (m["ms_prefill"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "prefill_bounds": bound_fields(th * prefill_flops_per_token_head(w.dk, w.dv), alg, m["ms_prefill"],
                                           w.seqlens, w.H)}
        if m["graph_ms"] is not None:
            out["batched"]["ms_per_step_graph_replay"] = round(m["graph_ms"], 5)
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
            out[f"decode_window_replay_{T}"] = bench_decode_window_replay(torch, kda, workloads, dev, steps, T)
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
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
