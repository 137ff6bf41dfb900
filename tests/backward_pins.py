"""Checks that pin the oracle's reverse mode (``Oracle.backward``) to facts other than
itself: central finite differences of the forward oracle, closed forms of a special case,
and identities that hold for any parameters (Euler's theorem for the parts of the loss
that are homogeneous in an input).  The loss is L = sum(dO * o) + sum(dfinal * final).
"""
from __future__ import annotations

import numpy as np


def _case(seed, seqlens=(5, 3), H=2, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    N = sum(seqlens)
    q = rng.standard_normal((N, H, dk))
    k = rng.standard_normal((N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, H, dv))
    g = rng.uniform(-2.0, 0.0, (N, H, dk))
    b = rng.uniform(0.1, 0.9, (N, H))
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    init = rng.standard_normal((len(seqlens), H, dk, dv)) * 0.5
    dO = rng.standard_normal((N, H, dv))
    dfin = rng.standard_normal((len(seqlens), H, dk, dv))
    return dict(q=q, k=k, v=v, log_alpha=g, beta=b, cu=cu, init=init, dO=dO, dfinal=dfin)


def _loss(orc, c):
    o, fin = orc.prefill(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], cu_seqlens=c["cu"],
                         init_state=c["init"], nthreads=1)
    return float(np.sum(c["dO"] * o) + np.sum(c["dfinal"] * fin)), o, fin


def _grads(orc, c):
    return orc.backward(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], c["dO"], cu_seqlens=c["cu"],
                        init_state=c["init"], dfinal=c["dfinal"])


def pin_backward_finite_differences(orc):
    """Every gradient entry against a central difference of the forward oracle (h = 1e-5;
    the truncation error is O(h^2) ~ 1e-10 relative)."""
    c = _case(1)
    gr = _grads(orc, c)
    names = {"q": "dq", "k": "dk", "v": "dv", "log_alpha": "dlog_alpha", "beta": "dbeta", "init": "dinit"}
    h = 1e-5
    for name, gname in names.items():
        x = c[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = _loss(orc, c)[0]
            x[idx] = old - h
            lm = _loss(orc, c)[0]
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = float(np.max(np.abs(gr[gname] - fd)))
        scale = max(1.0, float(np.max(np.abs(fd))))
        assert err <= 1e-7 * scale, f"{gname}: max|analytic - finite difference| = {err:.3e}"


def pin_backward_homogeneity(orc):
    """o is linear in q, so sum(q * dq) = sum(dO * o); o and the final state are linear in
    (v, initial state) jointly, so sum(v * dv) + sum(init * dinit) = L."""
    c = _case(2, seqlens=(7, 0, 4))
    L, o, _ = _loss(orc, c)
    gr = _grads(orc, c)
    lhs_q = float(np.sum(c["q"] * gr["dq"]))
    rhs_q = float(np.sum(c["dO"] * o))
    assert abs(lhs_q - rhs_q) <= 1e-10 * max(1.0, abs(rhs_q)), f"q homogeneity: {lhs_q} vs {rhs_q}"
    lhs_v = float(np.sum(c["v"] * gr["dv"]) + np.sum(c["init"] * gr["dinit"]))
    assert abs(lhs_v - L) <= 1e-10 * max(1.0, abs(L)), f"(v, init) homogeneity: {lhs_v} vs {L}"


def pin_backward_no_decay_no_write(orc):
    """alpha = 1, beta = 0: every state equals the initial one and o_t = S_0^T q_t, so
    dq_t = S_0 dO_t, dinit = dfinal + sum_t q_t dO_t^T, dk = dv = 0, and with the adjoint
    A_t = dfinal + sum_{s >= t} q_s dO_s^T: dbeta_t = (A_t^T k_t).(v_t - S_0^T k_t) and
    dlog_alpha_t = rowsum(A_t * S_0)."""
    c = _case(3, seqlens=(6,), H=1)
    c["log_alpha"][:] = 0.0
    c["beta"][:] = 0.0
    gr = _grads(orc, c)
    S0, dfin = c["init"][0, 0], c["dfinal"][0, 0]
    q, k, v, dO = c["q"][:, 0], c["k"][:, 0], c["v"][:, 0], c["dO"][:, 0]
    T = q.shape[0]
    np.testing.assert_allclose(gr["dq"][:, 0], dO @ S0.T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(gr["dinit"][0, 0], dfin + q.T @ dO, rtol=0, atol=1e-12)
    assert np.max(np.abs(gr["dk"])) == 0.0 and np.max(np.abs(gr["dv"])) == 0.0
    for t in range(T):
        A = dfin + q[t:].T @ dO[t:]
        e = A.T @ k[t]
        np.testing.assert_allclose(gr["dbeta"][t, 0], e @ (v[t] - S0.T @ k[t]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(gr["dlog_alpha"][t, 0], np.sum(A * S0, axis=1), rtol=0, atol=1e-12)


ALL_PINS = [pin_backward_finite_differences, pin_backward_homogeneity, pin_backward_no_decay_no_write]
