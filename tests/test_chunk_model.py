"""The chunkwise algebra the kernels implement, checked in fp64 against the oracle."""
import numpy as np
import pytest

import chunk_model
import oracle


def _inputs(T, H, dk, dv, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = np.maximum(-np.log1p(np.exp(rng.standard_normal((T, H, dk)))), -5.0)
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, b


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b)))


@pytest.mark.parametrize("T,dk,dv", [(64, 16, 16), (50, 32, 24), (16, 128, 128), (37, 128, 128), (1, 16, 32)])
def test_chunked_form_matches_oracle(T, dk, dv):
    q, k, v, g, b = _inputs(T, 2, dk, dv, seed=T + dk)
    init = np.random.default_rng(1).standard_normal((1, 2, dk, dv)) * 0.1
    o_ref, f_ref = oracle.prefill(q, k, v, g, b, init_state=init)
    o, f = chunk_model.prefill(q, k, v, g, b, init_state=init)
    assert _rel(o, o_ref) < 1e-12 and _rel(f, f_ref) < 1e-12


def test_chunked_form_varlen_and_gate_floor():
    lens = [17, 0, 33, 5, 16]
    q, k, v, g, b = _inputs(sum(lens), 3, 32, 16, seed=3)
    g[::3] = -5.0  # the lower bound itself: 16 tokens reach a cumulative -80
    cu = np.concatenate([[0], np.cumsum(lens)])
    o_ref, f_ref = oracle.prefill(q, k, v, g, b, cu_seqlens=cu)
    o, f = chunk_model.prefill(q, k, v, g, b, cu_seqlens=cu)
    assert _rel(o, o_ref) < 1e-11 and _rel(f, f_ref) < 1e-11


@pytest.mark.parametrize("lens,init", [([64], True), ([50, 0, 17, 33, 1, 16], True), ([37, 80], False)])
def test_lookahead_form_matches_oracle(lens, init):
    """Lookahead form: the next chunk's K+ S from the state entering the current chunk plus one
    16 x 16 product with the current Delta (gate floor included)."""
    q, k, v, g, b = _inputs(sum(lens), 2, 32, 24, seed=len(lens) + 7)
    g[::5] = -5.0
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0 = np.random.default_rng(2).standard_normal((len(lens), 2, 32, 24)) * 0.1 if init else None
    o_ref, f_ref = oracle.prefill(q, k, v, g, b, cu_seqlens=cu, init_state=S0)
    o, f = chunk_model.prefill_lookahead(q, k, v, g, b, cu_seqlens=cu, init_state=S0)
    assert _rel(o, o_ref) < 1e-11 and _rel(f, f_ref) < 1e-11


def test_unit_lower_inverse_is_nilpotent_product():
    """A_kk is strictly lower triangular (A^16 = 0), so (I + A)^{-1} equals
    (I - A)(I + A^2)(I + A^4)(I + A^8)."""
    q, k, v, g, b = _inputs(16, 1, 128, 8, seed=5)
    loc = chunk_model.chunk_local(q[:, 0], k[:, 0], g[:, 0], b[:, 0])
    A = loc["A"]
    I = np.eye(16)
    A2 = A @ A
    A4 = A2 @ A2
    P = (I - A) @ (I + A2) @ (I + A4) @ (I + A4 @ A4)
    assert np.max(np.abs(P - loc["T"])) < 1e-13
    assert np.max(np.abs(np.linalg.matrix_power(A, 16))) < 1e-30


def test_chunk_factors_stay_in_range_at_gate_floor():
    """With g = -5 on all 16 tokens, e^{-G} reaches e^80 < fp32/bf16 max and e^{G} reaches
    e^-80 > the smallest normal: the factored K+ K-^T products are representable."""
    G = np.cumsum(np.full(16, -5.0))
    assert np.exp(-G).max() < np.finfo(np.float32).max
    assert np.exp(G).min() > np.finfo(np.float32).tiny


@pytest.mark.parametrize("seqlens,init,dfin", [([40, 0, 17, 16, 1], True, True), ([33], False, False),
                                               ([5, 48], True, False)])
def test_chunked_backward_matches_oracle_reverse_mode(seqlens, init, dfin):
    """The chunk-form gradients (the GPU backward's algebra) against the oracle's reverse mode."""
    rng = np.random.default_rng(len(seqlens) + sum(seqlens))
    N, H, dk, dv = sum(seqlens), 2, 16, 8
    q = rng.standard_normal((N, H, dk))
    k = rng.standard_normal((N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, H, dv))
    g = rng.uniform(-5.0, 0.0, (N, H, dk))
    b = rng.uniform(0.0, 1.0, (N, H))
    dO = rng.standard_normal((N, H, dv))
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    S0 = rng.standard_normal((len(seqlens), H, dk, dv)) if init else None
    dF = rng.standard_normal((len(seqlens), H, dk, dv)) if dfin else None
    ref = oracle.backward(q, k, v, g, b, dO, cu_seqlens=cu, init_state=S0, dfinal=dF)
    for form in ("checkpoint", "scan"):
        got = chunk_model.backward(q, k, v, g, b, dO, cu_seqlens=cu, init_state=S0, dfinal=dF, dg_form=form)
        for name in ref:
            r = ref[name]
            scale = max(1e-300, float(np.sqrt(np.mean(r * r)))) if r.size else 1.0
            err = float(np.max(np.abs(got[name] - r))) if r.size else 0.0
            assert err <= 1e-9 * max(scale, 1.0), f"{form} {name}: max|err| = {err:.3e} (rms {scale:.3e})"
