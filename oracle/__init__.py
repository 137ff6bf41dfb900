"""fp64 CPU oracle for the KDA recurrence -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and shares
no code with it (the C source ``kda_oracle.c`` is compiled on its own by gcc).

It evaluates, per (sequence, head), the plain token-by-token definition from the
Kimi K3 report digest (discuss.pytorch.kr, section "Kimi Delta Attention"):

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t,      alpha_t = exp(g_t)

in IEEE double.  The arithmetic lives in ``kda_oracle.c``; this module only
widens inputs to float64, checks shapes and calls the C entry points.

Pins (what fixes this oracle other than itself) are the ``-m "not gpu"`` tests
in ``tests/test_oracle_pins.py`` and ``tests/test_oracle_mutants.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kda_oracle.c")
LIBRARY = os.path.join(_HERE, "libkda_oracle.so")

_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    cmd = ["gcc", "-O3", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
           *extra_flags, source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (CPU); the oracle never touches a device
        x = x.detach().to("cpu")
        import torch  # local import: torch is only needed for this conversion

        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(_f64p)


class Oracle:
    """ctypes handle on one compiled copy of the oracle."""

    def __init__(self, library: str = LIBRARY):
        if not os.path.exists(library):
            if library != LIBRARY:
                raise FileNotFoundError(library)
            build()
        self.library = library
        lib = ctypes.CDLL(library)
        lib.kda_oracle_prefill_f64.restype = ctypes.c_int
        lib.kda_oracle_prefill_f64.argtypes = [
            _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _i64p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _f64p, _f64p, ctypes.c_int]
        lib.kda_oracle_backward_f64.restype = ctypes.c_int
        lib.kda_oracle_backward_f64.argtypes = [
            _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _i64p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p]
        lib.kda_oracle_decode_f64.restype = ctypes.c_int
        lib.kda_oracle_decode_f64.argtypes = [
            _f64p, _f64p, _f64p, _f64p, _f64p, _f64p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _f64p, ctypes.c_int]
        self._lib = lib

    def prefill(self, q, k, v, log_alpha, beta, cu_seqlens=None, init_state=None,
                nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Run the recurrence over packed sequences.

        q, k, log_alpha: [N, H, dk]; v: [N, H, dv]; beta: [N, H];
        cu_seqlens: [nseq + 1] (None = one sequence of N tokens);
        init_state: [nseq, H, dk, dv] or None (zeros).
        Returns (o [N, H, dv], final_state [nseq, H, dk, dv]) in float64.
        """
        q, k, v, g, b = (_as_f64(t) for t in (q, k, v, log_alpha, beta))
        N, H, dk = q.shape
        dv = v.shape[2]
        if k.shape != (N, H, dk) or g.shape != (N, H, dk) or v.shape[:2] != (N, H) or b.shape != (N, H):
            raise ValueError("oracle.prefill: inconsistent input shapes")
        if cu_seqlens is None:
            cu = np.array([0, N], dtype=np.int64)
        else:
            if hasattr(cu_seqlens, "detach"):
                cu_seqlens = cu_seqlens.detach().to("cpu").numpy()
            cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        nseq = cu.shape[0] - 1
        if nseq < 1 or cu[0] != 0 or cu[-1] != N or np.any(np.diff(cu) < 0):
            raise ValueError("oracle.prefill: bad cu_seqlens")
        init = None
        if init_state is not None:
            init = _as_f64(init_state)
            if init.shape != (nseq, H, dk, dv):
                raise ValueError("oracle.prefill: init_state must be [nseq, H, dk, dv]")
        o = np.zeros((N, H, dv), dtype=np.float64)
        fin = np.zeros((nseq, H, dk, dv), dtype=np.float64)
        rc = self._lib.kda_oracle_prefill_f64(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(init),
            cu.ctypes.data_as(_i64p), nseq, H, dk, dv, _ptr(o), _ptr(fin), int(nthreads))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_prefill_f64 failed with code {rc}")
        return o, fin

    def decode(self, q, k, v, log_alpha, beta, state, nthreads: int = 0, inplace: bool = False):
        """One token for each of B x H heads.

        q, k, log_alpha: [B, H, dk]; v: [B, H, dv]; beta: [B, H];
        state: [B, H, dk, dv].  Returns (o [B, H, dv], new_state) in float64;
        the input array is not modified, unless inplace=True and it is a C-contiguous
        float64 numpy array (then it is advanced in place and returned).
        """
        q, k, v, g, b = (_as_f64(t) for t in (q, k, v, log_alpha, beta))
        if inplace and isinstance(state, np.ndarray) and state.dtype == np.float64 and state.flags.c_contiguous:
            st = state
        else:
            st = _as_f64(state).copy()
        B, H, dk = q.shape
        dv = v.shape[2]
        if st.shape != (B, H, dk, dv) or b.shape != (B, H):
            raise ValueError("oracle.decode: inconsistent shapes")
        o = np.zeros((B, H, dv), dtype=np.float64)
        rc = self._lib.kda_oracle_decode_f64(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(st), B, H, dk, dv, _ptr(o), int(nthreads))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_decode_f64 failed with code {rc}")
        return o, st


    def backward(self, q, k, v, log_alpha, beta, dO, cu_seqlens=None, init_state=None, dfinal=None):
        """Gradients of a loss L with dL/do = dO and dL/dfinal_state = dfinal (None = 0).

        Returns a dict with dq, dk, dlog_alpha [N, H, dk], dv [N, H, dv], dbeta [N, H] and
        dinit [nseq, H, dk, dv] (float64).  Single-threaded; meant for small cases.
        """
        q, k, v, g, b, do = (_as_f64(t) for t in (q, k, v, log_alpha, beta, dO))
        N, H, dk = q.shape
        dv = v.shape[2]
        cu = np.array([0, N], dtype=np.int64) if cu_seqlens is None else \
            np.ascontiguousarray(np.asarray(_as_f64(cu_seqlens), dtype=np.int64))
        nseq = cu.shape[0] - 1
        init = None if init_state is None else _as_f64(init_state)
        dfin = None if dfinal is None else _as_f64(dfinal)
        out = {"dq": np.zeros((N, H, dk)), "dk": np.zeros((N, H, dk)), "dv": np.zeros((N, H, dv)),
               "dlog_alpha": np.zeros((N, H, dk)), "dbeta": np.zeros((N, H)), "dinit": np.zeros((nseq, H, dk, dv))}
        rc = self._lib.kda_oracle_backward_f64(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(init), cu.ctypes.data_as(_i64p), nseq, H, dk, dv,
            _ptr(do), _ptr(dfin), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]),
            _ptr(out["dbeta"]), _ptr(out["dinit"]))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_backward_f64 failed with code {rc}")
        return out


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def prefill(*args, **kwargs):
    """Module-level shortcut for ``Oracle().prefill``."""
    return default().prefill(*args, **kwargs)


def decode(*args, **kwargs):
    """Module-level shortcut for ``Oracle().decode``."""
    return default().decode(*args, **kwargs)


def backward(*args, **kwargs):
    """Module-level shortcut for ``Oracle().backward``."""
    return default().backward(*args, **kwargs)
