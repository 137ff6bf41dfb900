"""Helpers for the GPU parity tests: error metric, oracle runs on GPU-generated inputs."""
import sys

import numpy as np
import torch

import oracle

# max|x - ref| <= TOL * RMS(ref), per output tensor (o, final state), pooled over all
# sequences and heads of a case.  bf16 inputs with fp32 state: 1e-2; fp32 inputs: 1e-5.
TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-5}
NAMES = ("q", "k", "v", "log_alpha", "beta")


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def rel_err(x, ref) -> float:
    x = x.detach().double().cpu().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float64)
    ref = ref.detach().double().cpu().numpy() if isinstance(ref, torch.Tensor) else np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(x - ref)))
    if rms == 0.0:
        return err
    return err / rms


def assert_close(x, ref, tol, what):
    e = rel_err(x, ref)
    say(f"    {what}: max|err|/rms = {e:.3e} (tol {tol:.0e})")
    assert np.all(np.isfinite(x.detach().double().cpu().numpy() if isinstance(x, torch.Tensor) else x)), \
        f"{what}: non-finite"
    assert e <= tol, f"{what}: max|err|/RMS(ref) = {e:.3e} > {tol:.1e}"
    return e


def oracle_prefill(x, init_state=None, heads=None, nthreads=0):
    """Oracle on the inputs dict ``x`` (device tensors), optionally on a subset of heads."""
    sel = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    cpu = {n: sel(x[n]).contiguous().cpu() for n in NAMES}
    init = None
    if init_state is not None:
        init = (init_state if heads is None else init_state[:, heads]).contiguous().cpu()
    return oracle.prefill(cpu["q"], cpu["k"], cpu["v"], cpu["log_alpha"], cpu["beta"],
                          cu_seqlens=x["cu_seqlens"].cpu(), init_state=init, nthreads=nthreads)
