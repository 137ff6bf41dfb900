"""Seeded synthetic inputs for the KDA operator.

This module draws random numbers and builds shapes; it holds none of the
operator's arithmetic.  Both the fp64 oracle (via the tests) and the HIP path
consume what it produces, so it imports neither of them.

Value distributions follow the five workloads the library is measured on:

1. ``tiny_fp32``   B=1, H=1, T=64, dk=dv=16, fp32; q, v ~ N(0,1); k ~ N(0,1)
                   then L2-normalised; beta = sigmoid(N(0,1)); log alpha ~ U[-5, 0).
2. ``batched``     B=4, H=8, T=2048, dk=dv=128, bf16 inputs; log alpha =
                   max(-softplus(N(0,1)), -5); other tensors as in 1.
3. ``k3_layer``    B=1, H=96, T=65,536 (the K3 layer shape: 96 heads, 128x128
                   state), distributions as in 2.
4. ``decode``      B=256 x H=96 heads, 128 single-token steps, bf16 inputs as in 2,
                   fp32 initial state N(0,1) scaled to unit Frobenius norm per head.
5. ``varlen_1m``   1,048,576 packed tokens, sequence lengths log-uniform in
                   [512, 262,144], H=96, d=128, distributions as in 2.

Decode windows (speculative verification) regroup the decode workload's steps:
window i of T tokens holds steps i*T .. i*T+T-1, and the number of accepted
drafts per sequence is uniform on [lo, T].

Keys are L2-normalised by the caller in the Kimi K3 design (report digest,
"Kimi Delta Attention": q and k are L2-normalised after the short convolution),
so the generator normalises k in fp32 before rounding to the input dtype.
Rounding to bf16 is round-to-nearest-even (torch's conversion).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Sequence

import numpy as np
import torch

CHUNK = 16
GATE_LOWER_BOUND = -5.0
TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "g": 4, "beta": 5, "state": 6, "lengths": 7, "accept": 8,
              "z": 9, "A_log": 10, "x": 11, "conv_w": 12, "conv_cache": 13, "o": 14, "u": 15, "norm_w": 16}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.  ``seqlens`` lists the packed sequence lengths."""

    name: str
    index: int                      # 1-based position in the list of workloads
    H: int
    dk: int
    dv: int
    seqlens: Sequence[int]
    dtype: torch.dtype
    gate: str                       # "uniform" (U[-5,0)) or "neg_softplus"
    decode_steps: int = 0           # > 0 for the recurrent-decode workload
    notes: str = ""

    @property
    def nseq(self) -> int:
        return len(self.seqlens)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))


def _seed(seed: int, *stream: int) -> int:
    """A 63-bit seed for an independent stream (numpy SeedSequence hashing)."""
    ss = np.random.SeedSequence([int(seed), *[int(s) for s in stream]])
    return int(ss.generate_state(2, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(device, seed: int, *stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, *stream))
    return g


def varlen_1m_lengths(seed: int = 0, total: int = 1 << 20, lo: int = 512, hi: int = 262144) -> List[int]:
    """Log-uniform lengths in [lo, hi] summing to exactly ``total``.

    Draw L = floor(exp(U[ln lo, ln hi])) until the sum reaches ``total``; shorten
    the last length so the sum is exact; if that leaves it shorter than ``lo``,
    fold it into the previous sequence.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 5, TENSOR_IDS["lengths"]])))
    out: List[int] = []
    acc = 0
    while acc < total:
        L = int(np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi)))))
        L = max(lo, min(hi, L))
        out.append(L)
        acc += L
    out[-1] -= acc - total
    if out[-1] < lo and len(out) > 1:
        out[-2] += out.pop()
    assert sum(out) == total
    return out


def workload(index: int, seed: int = 0) -> Workload:
    """The five measured workloads, by 1-based index."""
    bf16 = torch.bfloat16
    if index == 1:
        return Workload("tiny_fp32", 1, 1, 16, 16, [64], torch.float32, "uniform",
                        notes="B=1 H=1 T=64 d=16 fp32")
    if index == 2:
        return Workload("batched", 2, 8, 128, 128, [2048] * 4, bf16, "neg_softplus",
                        notes="B=4 H=8 T=2048 d=128 bf16")
    if index == 3:
        return Workload("k3_layer", 3, 96, 128, 128, [65536], bf16, "neg_softplus",
                        notes="B=1 H=96 T=65536 d=128 bf16")
    if index == 4:
        return Workload("decode", 4, 96, 128, 128, [1] * 256, bf16, "neg_softplus",
                        decode_steps=128, notes="B=256 H=96 d=128, 128 steps")
    if index == 5:
        lens = varlen_1m_lengths(seed)
        return Workload("varlen_1m", 5, 96, 128, 128, lens, bf16, "neg_softplus",
                        notes=f"{len(lens)} sequences, 1,048,576 tokens, H=96 d=128")
    raise ValueError(f"no workload {index}")


def custom(seqlens: Sequence[int], H: int, dk: int, dv: int, dtype=torch.bfloat16,
           gate: str = "neg_softplus", name: str = "custom") -> Workload:
    return Workload(name, 0, H, dk, dv, list(seqlens), dtype, gate)


def cu_seqlens_of(seqlens: Sequence[int]) -> List[int]:
    cu = [0]
    for L in seqlens:
        cu.append(cu[-1] + int(L))
    return cu


def _fill(kind: str, shape, gen, device, dtype, slab_tokens: int, gate: str) -> torch.Tensor:
    N = shape[0]
    out = torch.empty(shape, dtype=dtype, device=device)
    for s in range(0, N, slab_tokens):
        e = min(N, s + slab_tokens)
        sub = (e - s, *shape[1:])
        if kind in ("q", "v"):
            x = torch.randn(sub, generator=gen, device=device, dtype=torch.float32)
        elif kind == "k":
            x = torch.randn(sub, generator=gen, device=device, dtype=torch.float32)
            x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        elif kind == "beta":
            x = torch.sigmoid(torch.randn(sub, generator=gen, device=device, dtype=torch.float32))
        elif kind == "g":
            if gate == "uniform":
                # U[-5, 0): 1 - U[0,1) lies in (0, 1]; times -5 gives [-5, 0).
                u = torch.rand(sub, generator=gen, device=device, dtype=torch.float32)
                x = -5.0 * (1.0 - u)
            elif gate == "neg_softplus":
                z = torch.randn(sub, generator=gen, device=device, dtype=torch.float32)
                x = torch.clamp(-torch.nn.functional.softplus(z), min=GATE_LOWER_BOUND)
            else:
                raise ValueError(gate)
        else:
            raise ValueError(kind)
        out[s:e] = x.to(dtype)
        del x
    return out


def prefill_inputs(w: Workload, device="cpu", seed: int = 0, slab_tokens: int = 65536) -> Dict[str, object]:
    """q, k, v, log_alpha, beta, cu_seqlens for a prefill workload.

    Tensors are [N, H, d] in ``w.dtype`` (beta: [N, H]); cu_seqlens is int32 on
    ``device``.  Each tensor has its own seeded stream.
    """
    N, H = w.total_tokens, w.H
    wid = w.index if w.index else 1000 + len(w.seqlens)
    out: Dict[str, object] = {}
    for kind, shape in (("q", (N, H, w.dk)), ("k", (N, H, w.dk)), ("v", (N, H, w.dv)),
                        ("g", (N, H, w.dk)), ("beta", (N, H))):
        gen = _gen(device, seed, wid, TENSOR_IDS[kind])
        out[kind] = _fill(kind, shape, gen, device, w.dtype, slab_tokens, w.gate)
    out["log_alpha"] = out.pop("g")
    out["cu_seqlens"] = torch.tensor(cu_seqlens_of(w.seqlens), dtype=torch.int32, device=device)
    out["seqlens"] = list(w.seqlens)
    return out


def decode_initial_state(B: int, H: int, dk: int, dv: int, device="cpu", seed: int = 0) -> torch.Tensor:
    """fp32 [B, H, dk, dv]: per head N(0,1) drawn in fp64, divided by its Frobenius norm."""
    gen = _gen(device, seed, 4, TENSOR_IDS["state"])
    out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=device)
    for b in range(B):
        x = torch.randn((H, dk, dv), generator=gen, device=device, dtype=torch.float64)
        x = x / x.flatten(1).norm(dim=1).view(H, 1, 1)
        out[b] = x.to(torch.float32)
    return out


def decode_step_inputs(w: Workload, step: int, device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    """Fresh q, k, v, log_alpha, beta ([B, H, d], beta [B, H]) for one decode step."""
    B, H = w.nseq, w.H
    out = {}
    for kind, shape in (("q", (B, H, w.dk)), ("k", (B, H, w.dk)), ("v", (B, H, w.dv)),
                        ("g", (B, H, w.dk)), ("beta", (B, H))):
        gen = _gen(device, seed, w.index or 4, 100 + step, TENSOR_IDS[kind])
        out[kind] = _fill(kind, shape, gen, device, w.dtype, max(B, 1), w.gate)
    out["log_alpha"] = out.pop("g")
    return out


def decode_window_inputs(w: Workload, T: int, window: int, device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    """q, k, v, log_alpha [B, T, H, d] and beta [B, T, H]: decode steps window*T .. window*T+T-1
    stacked along a window axis after B (the same values decode_step_inputs gives per step)."""
    steps = [decode_step_inputs(w, window * T + t, device=device, seed=seed) for t in range(T)]
    return {n: torch.stack([s[n] for s in steps], dim=1).contiguous() for n in steps[0]}


def window_accept(B: int, T: int, device="cpu", seed: int = 0, lo: int = 0) -> torch.Tensor:
    """int32 [B]: accepted drafts per sequence, uniform on [lo, T]."""
    gen = _gen("cpu", seed, 4, TENSOR_IDS["accept"])
    a = torch.randint(lo, T + 1, (B,), generator=gen, dtype=torch.int64)
    return a.to(dtype=torch.int32, device=device)


def layer_inputs(N: int, H: int, d: int, dtype=torch.bfloat16, nseq: int = 1, device="cpu",
                 seed: int = 0) -> Dict[str, torch.Tensor]:
    """Synthetic tensors for the layer's passes around the recurrence (random-init weights):
    z decay logits ~ N(0, 2^2) and A_log ~ U[-1, 1] per head; x pre-convolution activations
    ~ N(0, 1); conv_w ~ N(0, 0.5^2) [H, d, 4]; conv_cache ~ N(0, 1) [nseq, H, d, 3] (fp32);
    o ~ N(0, 1) fp32 (a recurrent output); u gate logits ~ N(0, 1); norm_w ~ 1 + N(0, 0.1^2)."""
    out: Dict[str, torch.Tensor] = {}
    for kind, shape, scale, shift, dt in (("z", (N, H, d), 2.0, 0.0, dtype), ("x", (N, H, d), 1.0, 0.0, dtype),
                                          ("conv_w", (H, d, 4), 0.5, 0.0, torch.float32),
                                          ("conv_cache", (nseq, H, d, 3), 1.0, 0.0, torch.float32),
                                          ("o", (N, H, d), 1.0, 0.0, torch.float32),
                                          ("u", (N, H, d), 1.0, 0.0, dtype),
                                          ("norm_w", (d,), 0.1, 1.0, torch.float32)):
        gen = _gen(device, seed, 50, TENSOR_IDS[kind])
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * scale + shift
        out[kind] = t.to(dt)
    gen = _gen(device, seed, 50, TENSOR_IDS["A_log"])
    out["A_log"] = torch.rand((H,), generator=gen, device=device, dtype=torch.float32) * 2.0 - 1.0
    return out


def random_state(nseq: int, H: int, dk: int, dv: int, device="cpu", seed: int = 0, scale: float = 1.0) -> torch.Tensor:
    """fp32 [nseq, H, dk, dv] initial state, N(0,1) * scale / sqrt(dk) (for resume tests)."""
    gen = _gen(device, seed, 77, TENSOR_IDS["state"])
    x = torch.randn((nseq, H, dk, dv), generator=gen, device=device, dtype=torch.float32)
    return x * (scale / float(np.sqrt(dk)))
