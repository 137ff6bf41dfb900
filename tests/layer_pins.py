"""Checks that pin the layer oracle (``oracle.layer``: decay gate, ShortConv prologue,
RMSNorm + output-gate epilogue) to facts other than itself.

Each check takes the oracle module (or a mutated copy of it) and raises AssertionError
when it disagrees with a closed form, a symmetry, a library routine on a special case or
a value printed on the pages.  ``test_layer_oracle.py`` runs them on the real module and
on copies with a planted mistake.

Sources (Kimi K3 report digest, discuss.pytorch.kr): the bounded-decay section
(g = g_min Sigmoid(e^{A_h} z), g_min = -5, gate_lower_bound = -5.0 in the released
configuration), the paragraph after the KDA update equation (ShortConv of kernel size 4
and Swish on q, k, v; L2 normalisation of q and k) and the output-gate section
(per-head RMSNorm, Sigmoid gate).
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max|err| = {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------- decay gate

def pin_gate_closed_forms(L):
    """Sigmoid(0) = 1/2 and Sigmoid(ln 3) = 3/4, so with A = (0, ln 2, -ln 4) per head:
    z = 0 gives -2.5 on every head; z = ln 3 / e^{A_h} gives -3.75 on head h."""
    A = np.array([0.0, np.log(2.0), -np.log(4.0)])
    z0 = np.zeros((2, 3, 4))
    _close(L.gate(z0, A), np.full((2, 3, 4), -2.5), 1e-15, "gate(z = 0)")
    z = np.empty((1, 3, 4))
    for h in range(3):
        z[0, h] = np.log(3.0) / np.exp(A[h])
    _close(L.gate(z, A), np.full((1, 3, 4), -3.75), 1e-14, "gate(z = ln 3 e^-A)")


def pin_gate_bounds_and_limits(L):
    """g lies in (g_min, 0) and decreases with z; z -> +inf gives g_min = -5 (the page's
    gate_lower_bound, tests/golden/bounded_decay.json), z -> -inf gives 0."""
    with open(os.path.join(GOLDEN, "bounded_decay.json")) as f:
        gmin = json.load(f)["log_decay_lower_bound"]
    rng = np.random.default_rng(1)
    z = np.sort(rng.normal(0.0, 3.0, 64))[None, None, :]
    A = np.array([0.3])
    g = L.gate(z, A)
    assert np.all(g > gmin) and np.all(g < 0.0), "gate leaves (g_min, 0)"
    assert np.all(np.diff(g[0, 0]) <= 0.0), "gate not decreasing in z"
    _close(L.gate(np.full((1, 1, 1), 60.0), A), [[[gmin]]], 1e-12, "gate(z -> +inf)")
    _close(L.gate(np.full((1, 1, 1), -60.0), A), [[[0.0]]], 1e-12, "gate(z -> -inf)")


# ----------------------------------------------------------------- ShortConv prologue

def _rand_conv(seed, N=23, H=2, d=5):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(N, H, d)), rng.normal(size=(H, d, 4)) * 0.5


def _linear_part(L, x, w, cu=None, cache=None):
    """Swish(a) - Swish(-a) = a, so the convolution itself is y(x) - y(-x) (the cache is
    negated with the input)."""
    yp, _ = L.short_conv(x, w, cu, cache)
    yn, _ = L.short_conv(-x, w, cu, None if cache is None else -cache)
    return yp - yn


def pin_conv_matches_library_convolution(L):
    """Per channel the linear part is numpy's full convolution of the zero-preceded input
    with the 4 taps, truncated to the sequence: y_t = sum_j w[j] x_{t-j}."""
    x, w = _rand_conv(2)
    lin = _linear_part(L, x, w)
    N, H, d = x.shape
    for h in range(H):
        for c in range(d):
            ref = np.convolve(x[:, h, c], w[h, c])[:N]
            _close(lin[:, h, c], ref, 1e-12, f"conv channel ({h}, {c})")


def pin_conv_impulse_taps(L):
    """Tap 0 alone gives Swish(x); tap 2 alone gives Swish(x_{t-2}) with zeros before the
    sequence.  Swish(ln 3) = (3/4) ln 3."""
    x = np.full((6, 1, 1), np.log(3.0))
    w0 = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    y, _ = L.short_conv(x, w0)
    _close(y, np.full((6, 1, 1), 0.75 * np.log(3.0)), 1e-15, "tap 0 on ln 3")
    w2 = np.array([[[0.0, 0.0, 1.0, 0.0]]])
    y, _ = L.short_conv(x, w2)
    ref = np.full((6, 1, 1), 0.75 * np.log(3.0))
    ref[:2] = 0.0
    _close(y, ref, 1e-15, "tap 2 shift")


def pin_conv_cache_resume_and_varlen(L):
    """A sequence split in two calls (the second starting from the first's cache) equals
    one call; packed sequences equal separate calls; a sequence shorter than 3 tokens
    keeps the older cache entries, oldest first."""
    x, w = _rand_conv(3, N=17)
    y_full, c_full = L.short_conv(x, w)
    y1, c1 = L.short_conv(x[:5], w)
    y2, c2 = L.short_conv(x[5:], w, None, c1)
    _close(np.concatenate([y1, y2]), y_full, 1e-14, "resume y")
    _close(c2, c_full, 0.0, "resume cache")
    _close(c_full[0].transpose(2, 0, 1), x[-3:], 0.0, "cache = last 3 inputs, oldest first")
    cu = np.array([0, 4, 4, 6, 17])
    y_pack, c_pack = L.short_conv(x, w, cu)
    for s in range(4):
        ys, cs = L.short_conv(x[cu[s]:cu[s + 1]], w)
        _close(y_pack[cu[s]:cu[s + 1]], ys, 0.0, f"varlen sequence {s}")
        _close(c_pack[s], cs[0], 0.0, f"varlen cache {s}")
    rng = np.random.default_rng(4)
    cache = rng.normal(size=(1, 2, 5, 3))
    _, c_short = L.short_conv(x[:2], w, None, cache)
    ref = np.concatenate([cache[0][..., 2:], x[:2].transpose(1, 2, 0)], axis=-1)
    _close(c_short[0], ref, 0.0, "cache after a 2-token sequence")
    # the cache feeds the first outputs: tap 3 at t = 0 reads the oldest cache entry
    w3 = np.zeros((2, 5, 4))
    w3[..., 3] = 1.0
    lin = _linear_part(L, x[:1], w3, None, cache)
    _close(lin[0], cache[0][..., 0], 1e-15, "tap 3 reads the oldest cache entry")


def pin_conv_l2norm(L):
    """With L2 normalisation each (token, head) row has unit norm (eps tiny) and points
    along the unnormalised output."""
    x, w = _rand_conv(5)
    y, _ = L.short_conv(x, w)
    yn, _ = L.short_conv(x, w, l2norm=True, eps=1e-30)
    _close(np.linalg.norm(yn, axis=-1), np.ones(yn.shape[:2]), 1e-14, "unit rows")
    _close(yn * np.linalg.norm(y, axis=-1, keepdims=True), y, 1e-13, "same direction")


# ----------------------------------------------------------------- output epilogue

def pin_norm_gate_closed_forms(L):
    """A constant head output c normalises to sign(c); Sigmoid(0) = 1/2 and
    Sigmoid(ln 3) = 3/4 scale it; the weight multiplies per channel."""
    o = np.array([[[2.5] * 4, [-0.25] * 4]])
    u = np.zeros_like(o)
    w = np.array([1.0, 2.0, 3.0, 4.0])
    _close(L.out_norm_gate(o, u, w, 0.0), np.array([[[0.5, 1.0, 1.5, 2.0], [-0.5, -1.0, -1.5, -2.0]]]),
           1e-15, "constant rows")
    u3 = np.full_like(o, np.log(3.0))
    _close(L.out_norm_gate(o, u3, np.ones(4), 0.0), np.sign(o) * 0.75, 1e-15, "gate ln 3")


def pin_norm_scale_invariance_and_rms(L):
    """RMSNorm is invariant to positive scaling (eps = 0) and leaves unit mean square;
    eps keeps a zero row at zero."""
    rng = np.random.default_rng(6)
    o = rng.normal(size=(3, 2, 8))
    u = rng.normal(size=(3, 2, 8))
    w = rng.uniform(0.5, 1.5, 8)
    y = L.out_norm_gate(o, u, w, 0.0)
    _close(L.out_norm_gate(7.0 * o, u, w, 0.0), y, 1e-14, "scale invariance")
    big = L.out_norm_gate(o, np.full_like(u, 60.0), np.ones(8), 0.0)  # gate -> 1
    _close(np.mean(big * big, axis=-1), np.ones((3, 2)), 1e-13, "unit mean square")
    z = L.out_norm_gate(np.zeros((1, 1, 8)), u[:1, :1], w, 1e-6)
    _close(z, np.zeros((1, 1, 8)), 0.0, "zero row")


ALL_PINS = [
    pin_gate_closed_forms,
    pin_gate_bounds_and_limits,
    pin_conv_matches_library_convolution,
    pin_conv_impulse_taps,
    pin_conv_cache_resume_and_varlen,
    pin_conv_l2norm,
    pin_norm_gate_closed_forms,
    pin_norm_scale_invariance_and_rms,
]
