"""Checks that pin the fp64 oracle to facts other than itself.

Every check takes an ``oracle.Oracle`` handle and raises AssertionError when the
oracle disagrees with a closed form, an invariant, a brute-force product or a
value printed on the pages.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on copies with a planted mistake and
expects each mutant to fail at least one.

Sources (Kimi K3 technical-report digest, discuss.pytorch.kr):
  * "Kimi Delta Attention": the update S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T,
    o_t = S_t^T q_t; alpha is per key channel, beta a scalar write strength.
  * "KDA context parallelism (KCP)": S_t = M_t S_{t-1} + b_t k_t v_t^T with
    M_t = (I - b_t k_t k_t^T) Diag(a_t); a segment's end state is the state it
    generates from zero plus the accumulated transition applied to the incoming
    state.
  * "Bounded decay": g >= -5, so alpha > e^-5 ~ 6.7e-3 and a 16-token tile's
    cumulative log-decay lies in (-80, 0).
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _orthonormal(rng, n, d):
    """n <= d mutually orthonormal rows in R^d."""
    qmat, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return qmat[:, :n].T.copy()


def _single(T, dk, dv, rng):
    """Random single-sequence, single-head inputs as [T, 1, d] arrays."""
    q = rng.standard_normal((T, 1, dk))
    k = _unit_rows(rng.standard_normal((T, 1, dk)))
    v = rng.standard_normal((T, 1, dv))
    g = rng.uniform(-5.0, 0.0, (T, 1, dk))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, 1))))
    return q, k, v, g, b


def _close(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max|err| = {err:.3e} > {tol:.1e} * {scale:.3e}"


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def pin_state_carried(orc):
    """alpha = 1, beta = 0: no forgetting and no write, so S_t = S_0 for every t and
    o_t = S_0^T q_t (the literal reading of the update with g = 0 and b = 0)."""
    rng = _rng(1)
    T, dk, dv = 12, 8, 6
    q, k, v, g, b = _single(T, dk, dv, rng)
    g[:] = 0.0
    b[:] = 0.0
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, fin = orc.prefill(q, k, v, g, b, init_state=S0)
    assert np.array_equal(fin, S0), "state changed although alpha = 1 and beta = 0"
    _close(o[:, 0, :], q[:, 0, :] @ S0[0, 0], 1e-13, "o_t = S_0^T q_t")


def pin_additive_orthogonal_keys(orc):
    """alpha = 1, S_0 = 0, mutually orthogonal unit keys: the erase term k k^T S
    vanishes, so the state is the additive outer-product sum sum_t b_t k_t v_t^T
    (vanilla linear attention, the additive recurrence the KCP section contrasts)."""
    rng = _rng(2)
    T, dk, dv = 7, 9, 5
    q, _, v, g, b = _single(T, dk, dv, rng)
    k = _orthonormal(rng, T, dk)[:, None, :]
    g[:] = 0.0
    o, fin = orc.prefill(q, k, v, g, b)
    S = np.zeros((dk, dv))
    for t in range(T):
        S = S + b[t, 0] * np.outer(k[t, 0], v[t, 0])
        _close(o[t, 0], S.T @ q[t, 0], 1e-13, f"o_{t}")
    _close(fin[0, 0], S, 1e-13, "S_T = sum b k v^T")


def pin_first_order_small_beta(orc):
    """alpha = 1, S_0 = 0, beta = eps for every token: S_T / eps = sum_t k_t v_t^T + O(eps)
    for arbitrary (non-orthogonal) unit keys.  The error must shrink linearly in eps."""
    rng = _rng(3)
    T, dk, dv = 24, 6, 4
    q, k, v, g, b = _single(T, dk, dv, rng)
    g[:] = 0.0
    ref = np.einsum("ti,tj->ij", k[:, 0], v[:, 0])
    errs = []
    for eps in (1e-4, 1e-6):
        b[:] = eps
        _, fin = orc.prefill(q, k, v, g, b)
        errs.append(float(np.max(np.abs(fin[0, 0] / eps - ref))))
    assert errs[0] < 1e-2 * np.max(np.abs(ref)), f"first-order term wrong: {errs}"
    assert errs[1] < errs[0] * 1e-1, f"error does not shrink with eps: {errs}"


def pin_exact_recall(orc):
    """beta = 1, alpha = 1, S_0 = 0, orthonormal keys (T <= dk): writing v_i under k_i
    clears the slot and stores the value, so querying with q = k_i returns v_i, for
    every earlier i, after the last token; and o_t with q_t = k_t returns v_t."""
    rng = _rng(4)
    dk, dv = 8, 5
    T = dk
    _, _, v, g, b = _single(T, dk, dv, rng)
    k = _orthonormal(rng, T, dk)[:, None, :]
    g[:] = 0.0
    b[:] = 1.0
    o, fin = orc.prefill(k, k, v, g, b)
    _close(k[:, 0, :] @ fin[0, 0], v[:, 0, :], 1e-13, "k_i^T S_T = v_i^T")
    _close(o[:, 0, :], v[:, 0, :], 1e-13, "o_t(q=k_t) = v_t")


def pin_decay_only(orc):
    """beta = 0: only the forget stage acts, S_T = Diag(exp(sum_t g_t)) S_0 -- row i
    (key channel i) is scaled by the product of its retentions alpha_{t,i}."""
    rng = _rng(5)
    T, dk, dv = 10, 7, 4
    q, k, v, g, b = _single(T, dk, dv, rng)
    b[:] = 0.0
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, fin = orc.prefill(q, k, v, g, b, init_state=S0)
    G = np.cumsum(g[:, 0, :], axis=0)
    _close(fin[0, 0], np.exp(G[-1])[:, None] * S0[0, 0], 1e-13, "S_T = Diag(exp(sum g)) S_0")
    for t in range(T):
        _close(o[t, 0], (np.exp(G[t])[:, None] * S0[0, 0]).T @ q[t, 0], 1e-13, f"o_{t}")


# --------------------------------------------------------------------------
# Per-step identities (stepped through the decode entry point)
# --------------------------------------------------------------------------

def _step_states(orc, T=40, dk=8, dv=6, seed=6):
    rng = _rng(seed)
    q, k, v, g, b = _single(T, dk, dv, rng)
    S = rng.standard_normal((1, 1, dk, dv))
    states = [S[0, 0].copy()]
    for t in range(T):
        _, S = orc.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], S)
        states.append(S[0, 0].copy())
    return q, k, v, g, b, states


def pin_convex_blend(orc):
    """For a unit key, k_t^T S_t = (1 - b_t) k_t^T Diag(a_t) S_{t-1} + b_t v_t^T: the
    read-out along k is a blend of the decayed old read-out and the new value
    ("clear the slot, then write the value")."""
    q, k, v, g, b, states = _step_states(orc)
    for t in range(len(states) - 1):
        kt, bt = k[t, 0], b[t, 0]
        lhs = kt @ states[t + 1]
        rhs = (1 - bt) * (kt @ (np.exp(g[t, 0])[:, None] * states[t])) + bt * v[t, 0]
        _close(lhs, rhs, 1e-12, f"convex blend at t={t}")


def pin_norm_bound(orc):
    """For a unit key and b in (0,1): ||S_t||_F^2 <= ||Diag(a_t) S_{t-1}||_F^2 + b/(2-b) ||v_t||^2.
    (Split Diag(a)S into its component along k and the rest; the update keeps the rest
    and maps the k-row p to (1-b)p + b v, whose squared norm exceeds ||p||^2 by at most
    b||v||^2/(2-b).)  So with decay the state stays bounded."""
    q, k, v, g, b, states = _step_states(orc, seed=7)
    for t in range(len(states) - 1):
        P = np.exp(g[t, 0])[:, None] * states[t]
        bound = np.sum(P * P) + b[t, 0] / (2 - b[t, 0]) * np.sum(v[t, 0] ** 2)
        assert np.sum(states[t + 1] ** 2) <= bound * (1 + 1e-12) + 1e-300, f"norm bound broken at t={t}"


# --------------------------------------------------------------------------
# Brute force: explicit transition matrices (the KCP form)
# --------------------------------------------------------------------------

def pin_bruteforce_products(orc):
    """T <= 8, non-unit keys, dk != dv: build M_t = (I - b_t k_t k_t^T) Diag(a_t) as explicit
    dk x dk matrices and evaluate S_T = M_T...M_1 S_0 + sum_t M_T...M_{t+1} b_t k_t v_t^T and
    o_t = S_t^T q_t by plain matrix products."""
    for seed, (T, dk, dv) in ((8, (8, 5, 3)), (9, (5, 4, 7)), (10, (1, 3, 2))):
        rng = _rng(seed)
        q = rng.standard_normal((T, 1, dk))
        k = rng.standard_normal((T, 1, dk)) * 0.7
        v = rng.standard_normal((T, 1, dv))
        g = rng.uniform(-5.0, 0.0, (T, 1, dk))
        b = rng.uniform(0.0, 1.0, (T, 1))
        S0 = rng.standard_normal((1, 1, dk, dv))
        o, fin = orc.prefill(q, k, v, g, b, init_state=S0)
        I = np.eye(dk)
        M = [(I - b[t, 0] * np.outer(k[t, 0], k[t, 0])) @ np.diag(np.exp(g[t, 0])) for t in range(T)]
        for t in range(T):
            acc = S0[0, 0].copy()
            for u in range(t + 1):
                acc = M[u] @ acc
            for s in range(t + 1):
                term = b[s, 0] * np.outer(k[s, 0], v[s, 0])
                for u in range(s + 1, t + 1):
                    term = M[u] @ term
                acc = acc + term
            _close(o[t, 0], acc.T @ q[t, 0], 1e-12, f"brute-force o_{t} (T={T},dk={dk},dv={dv})")
            if t == T - 1:
                _close(fin[0, 0], acc, 1e-12, f"brute-force S_T (T={T},dk={dk},dv={dv})")


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def pin_padding_noop(orc):
    """A token with g = 0, b = 0, k = 0, v = 0 is an exact no-op on the state."""
    rng = _rng(11)
    T, dk, dv = 9, 6, 5
    q, k, v, g, b = _single(T, dk, dv, rng)
    S0 = rng.standard_normal((1, 1, dk, dv))
    _, fin = orc.prefill(q, k, v, g, b, init_state=S0)
    z = np.zeros
    q2 = np.concatenate([q, rng.standard_normal((4, 1, dk))])
    k2 = np.concatenate([k, z((4, 1, dk))])
    v2 = np.concatenate([v, z((4, 1, dv))])
    g2 = np.concatenate([g, z((4, 1, dk))])
    b2 = np.concatenate([b, z((4, 1))])
    _, fin2 = orc.prefill(q2, k2, v2, g2, b2, init_state=S0)
    assert np.array_equal(fin, fin2), "padding tokens changed the state"


def pin_split_resume(orc):
    """Prefill of tokens [0, t1) then [t1, T) from the first call's final state equals
    one prefill of [0, T) (resuming from a stored state)."""
    rng = _rng(12)
    T, dk, dv = 30, 6, 4
    q, k, v, g, b = _single(T, dk, dv, rng)
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, fin = orc.prefill(q, k, v, g, b, init_state=S0)
    t1 = 13
    o1, f1 = orc.prefill(q[:t1], k[:t1], v[:t1], g[:t1], b[:t1], init_state=S0)
    o2, f2 = orc.prefill(q[t1:], k[t1:], v[t1:], g[t1:], b[t1:], init_state=f1)
    assert np.array_equal(np.concatenate([o1, o2]), o) and np.array_equal(f2, fin), "split != whole"


def pin_affine_in_initial_state(orc):
    """For fixed tokens the final state and outputs are affine in the initial state
    (the KCP decomposition: end state = zero-start state + transition x incoming state)."""
    rng = _rng(13)
    T, dk, dv = 20, 6, 5
    q, k, v, g, b = _single(T, dk, dv, rng)
    S1 = rng.standard_normal((1, 1, dk, dv))
    S2 = rng.standard_normal((1, 1, dk, dv))
    a = 0.3
    o1, f1 = orc.prefill(q, k, v, g, b, init_state=S1)
    o2, f2 = orc.prefill(q, k, v, g, b, init_state=S2)
    o3, f3 = orc.prefill(q, k, v, g, b, init_state=a * S1 + (1 - a) * S2)
    _close(f3, a * f1 + (1 - a) * f2, 1e-13, "final state affine in S_0")
    _close(o3, a * o1 + (1 - a) * o2, 1e-13, "outputs affine in S_0")
    # and the zero-start state plus transition: f(S) - f(0) is linear in S
    _, f0 = orc.prefill(q, k, v, g, b)
    _, f12 = orc.prefill(q, k, v, g, b, init_state=S1 + S2)
    _close(f12 - f0, (f1 - f0) + (f2 - f0), 1e-12, "f(S1+S2) - f(0) = (f(S1)-f(0)) + (f(S2)-f(0))")


def pin_varlen_equals_separate(orc):
    """Packed sequences (cu_seqlens) give exactly the results of separate calls: the
    state restarts at every sequence boundary."""
    rng = _rng(14)
    lens = [5, 0, 17, 1, 9]
    H, dk, dv = 3, 6, 4
    N = sum(lens)
    q = rng.standard_normal((N, H, dk))
    k = _unit_rows(rng.standard_normal((N, H, dk)))
    v = rng.standard_normal((N, H, dv))
    g = rng.uniform(-5, 0, (N, H, dk))
    b = rng.uniform(0, 1, (N, H))
    init = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    for use_init in (True, False):
        o, fin = orc.prefill(q, k, v, g, b, cu_seqlens=cu, init_state=init if use_init else None, nthreads=2)
        for s, L in enumerate(lens):
            a, e = cu[s], cu[s + 1]
            start = init[s:s + 1] if use_init else np.zeros((1, H, dk, dv))
            if L == 0:
                assert np.array_equal(fin[s], start[0]), "empty sequence must return its initial state"
                continue
            os_, fs = orc.prefill(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], init_state=start)
            assert np.array_equal(o[a:e], os_) and np.array_equal(fin[s], fs[0]), f"sequence {s} differs"


def pin_heads_independent(orc):
    """Heads do not interact: permuting the head axis of every input permutes the outputs."""
    rng = _rng(15)
    N, H, dk, dv = 11, 4, 5, 3
    q = rng.standard_normal((N, H, dk))
    k = _unit_rows(rng.standard_normal((N, H, dk)))
    v = rng.standard_normal((N, H, dv))
    g = rng.uniform(-5, 0, (N, H, dk))
    b = rng.uniform(0, 1, (N, H))
    o, fin = orc.prefill(q, k, v, g, b)
    p = np.array([2, 0, 3, 1])
    o2, fin2 = orc.prefill(q[:, p], k[:, p], v[:, p], g[:, p], b[:, p])
    assert np.array_equal(o2, o[:, p]) and np.array_equal(fin2, fin[:, p]), "head permutation"


def pin_decode_matches_prefill(orc):
    """Stepping the decode entry point T times equals one prefill of T tokens."""
    rng = _rng(16)
    T, dk, dv = 14, 5, 6
    q, k, v, g, b = _single(T, dk, dv, rng)
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, fin = orc.prefill(q, k, v, g, b, init_state=S0)
    S = S0
    for t in range(T):
        ot, S = orc.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], S)
        assert np.array_equal(ot[0], o[t]), f"decode o_{t}"
    assert np.array_equal(S, fin), "decode state"


# --------------------------------------------------------------------------
# Printed values (tests/golden/bounded_decay.json)
# --------------------------------------------------------------------------

def pin_bounded_decay_golden(orc):
    """The bounded-decay section prints: alpha > e^-5 ~ 6.7e-3, a 16-token tile's
    cumulative log-decay in (-80, 0), and an inverse scale below e^80 that stays in the
    BF16 range.  With b = 0 and g = -5 on every channel, 16 tokens must scale the state
    by exactly e^-80, and one token by e^-5 ~ 6.7e-3."""
    with open(os.path.join(GOLDEN, "bounded_decay.json")) as f:
        gold = json.load(f)
    C = gold["tile_tokens"]
    dk, dv = 4, 3
    rng = _rng(17)
    q, k, v, g, b = _single(C, dk, dv, rng)
    g[:] = gold["log_decay_lower_bound"]
    b[:] = 0.0
    S0 = np.ones((1, 1, dk, dv))
    o, fin = orc.prefill(q, k, v, g, b, init_state=S0)
    lo = gold["tile_cumulative_log_decay_range"][0]
    _close(fin[0, 0], np.full((dk, dv), np.exp(lo)) , 1e-15, "16 tokens at g=-5 scale by e^-80")
    ratio = float(fin[0, 0, 0, 0] / S0[0, 0, 0, 0])
    assert ratio > 0 and abs(np.log(ratio) - lo) < 1e-9, "tile decay must be e^-80"
    alpha_min = float(np.exp(gold["log_decay_lower_bound"]))
    digits = gold["alpha_min_printed_sig_digits"]
    assert float(f"{alpha_min:.{digits}g}") == gold["alpha_min_printed"]
    _, one = orc.prefill(q[:1], k[:1], v[:1], g[:1], b[:1], init_state=S0)
    assert abs(float(one[0, 0, 0, 0]) - alpha_min) < 1e-15
    assert np.exp(-lo) < gold["bf16_max"], "inverse scale must stay inside the BF16 range"


ALL_PINS = [
    pin_state_carried,
    pin_additive_orthogonal_keys,
    pin_first_order_small_beta,
    pin_exact_recall,
    pin_decay_only,
    pin_convex_blend,
    pin_norm_bound,
    pin_bruteforce_products,
    pin_padding_noop,
    pin_split_resume,
    pin_affine_in_initial_state,
    pin_varlen_equals_separate,
    pin_heads_independent,
    pin_decode_matches_prefill,
    pin_bounded_decay_golden,
]
