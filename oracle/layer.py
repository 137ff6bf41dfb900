"""fp64 CPU oracle for the KDA layer's prologue and epilogue -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the GPU library shares no code with it.

The operations around the recurrence, as the Kimi K3 report digest
(discuss.pytorch.kr) describes the KDA layer:

* Decay gate (section on bounded decay): the log-decay of key channel c is
  g = g_min * Sigmoid(exp(A_h) * z), with z the decay logit, A_h a per-head log
  scale and g_min = -5 fixed, so alpha = exp(g) lies in (e^-5, 1).
* Prologue (section "Kimi Delta Attention", the paragraph after the update
  equation): the q, k and v projections each pass through a short convolution
  of kernel size 4 and then Swish; q and k are then L2-normalised.
* Epilogue (section on the full-rank output gate): the recurrent output of
  each head goes through a per-head RMSNorm and is multiplied elementwise by
  Sigmoid of a full-rank, input-dependent gate; W_o and W_g are the caller's
  projections.

Readings where the page leaves details open (the plain ones):

* ShortConv is depthwise (one 4-tap filter per channel and head), causal and
  without bias: y_t = sum_{j=0..3} w[j] x_{t-j}.  Inputs before a sequence's
  first token are taken from a per-sequence cache of the 3 preceding inputs
  (zeros when there is none); the cache after a sequence holds its last 3
  inputs, oldest first.
* Swish(x) = x * Sigmoid(x).
* L2 normalisation over the key channels: y / sqrt(sum y^2 + eps).
* RMSNorm over the dv channels of a head: o / sqrt(mean(o^2) + eps) * w, with a
  weight w of length dv.

Every function takes and returns float64 numpy arrays and evaluates the
definition directly (no blocking or fusion).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

G_MIN = -5.0
CONV_TAPS = 4


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # CPU torch tensor
        import torch

        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def gate(z, A_log, g_min: float = G_MIN) -> np.ndarray:
    """g = g_min * Sigmoid(exp(A_h) z); z [N, H, dk], A_log [H]."""
    z, A = _f64(z), _f64(A_log)
    return g_min * sigmoid(np.exp(A)[None, :, None] * z)


def swish(x):
    x = _f64(x)
    return x * sigmoid(x)


def short_conv(x, w, cu_seqlens=None, cache=None, l2norm: bool = False,
               eps: float = 1e-6) -> Tuple[np.ndarray, np.ndarray]:
    """Causal depthwise convolution (4 taps), Swish, optional L2 norm over channels.

    x: [N, H, d] packed sequences; w: [H, d, 4] with w[..., j] the tap on x_{t-j};
    cu_seqlens: [nseq + 1] (None = one sequence); cache: [nseq, H, d, 3], the 3
    inputs before each sequence, oldest first (None = zeros).
    Returns (y [N, H, d], cache_out [nseq, H, d, 3]).
    """
    x, w = _f64(x), _f64(w)
    N, H, d = x.shape
    cu = np.array([0, N]) if cu_seqlens is None else np.asarray(_f64(cu_seqlens), dtype=np.int64)
    nseq = len(cu) - 1
    c_in = np.zeros((nseq, H, d, 3)) if cache is None else _f64(cache)
    y = np.zeros_like(x)
    c_out = np.zeros((nseq, H, d, 3))
    for s in range(nseq):
        bos, eos = int(cu[s]), int(cu[s + 1])
        # the sequence's inputs preceded by its cache: hist[3 + i] = x_{bos + i}
        hist = np.concatenate([c_in[s].transpose(2, 0, 1), x[bos:eos]], axis=0)  # [3 + L, H, d]
        for t in range(eos - bos):
            acc = np.zeros((H, d))
            for j in range(CONV_TAPS):
                acc += w[:, :, j] * hist[3 + t - j]
            y[bos + t] = swish(acc)
        c_out[s] = hist[-3:].transpose(1, 2, 0)
    if l2norm:
        y = y / np.sqrt(np.sum(y * y, axis=-1, keepdims=True) + eps)
    return y, c_out


def out_norm_gate(o, u, w, eps: float) -> np.ndarray:
    """y = Sigmoid(u) * RMSNorm(o) * w over the last axis (dv); o, u [..., dv], w [dv]."""
    o, u, w = _f64(o), _f64(u), _f64(w)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return sigmoid(u) * (o / rms) * w
