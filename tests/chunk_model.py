"""fp64 numpy model of the chunkwise (16-token) evaluation of the KDA recurrence.

Test-only.  It is NOT the oracle: it models the algebra the HIP kernels implement
so that the derivation can be checked against the oracle on the CPU, and so the
chunk-local kernel's intermediates (T' = (I + A_kk)^-1 diag(beta) and A_qk) have
something to be compared with.  Derivation, for a chunk of n <= 16 tokens with
incoming state S (report digest, "Kimi Delta Attention": the chunked output is an
inter-chunk term (Gamma (.) Q) S plus an intra-chunk term A V~):

    G_r  = sum_{i<=r} g_i                        (per key channel)
    K+   = K (.) e^{G},   K- = K (.) e^{-G},   Q+ = Q (.) e^{G},   K~ = K (.) e^{G_n - G}
    A_kk = diag(beta) strictly_lower(K+ K-^T)     T' = (I + A_kk)^{-1} diag(beta)
    W    = T' K+,   U = T' V,   A_qk = lower_incl_diag(Q+ K-^T)
    Delta = U - W S
    O     = Q+ S + A_qk Delta
    S_out = Diag(e^{G_n}) S + K~^T Delta
"""
import numpy as np

C = 16


def chunk_local(q, k, g, beta):
    """Per-chunk quantities for one head: q, k, g are [n, dk], beta [n].
    Returns dict with G, Kp, Km, Qp, Kt, Tp (T'), Aqk."""
    n = q.shape[0]
    G = np.cumsum(g, axis=0)
    Kp, Km = k * np.exp(G), k * np.exp(-G)
    Qp = q * np.exp(G)
    Kt = k * np.exp(G[-1] - G)
    A = np.diag(beta) @ np.tril(Kp @ Km.T, -1)
    T = np.linalg.inv(np.eye(n) + A)
    return dict(G=G, Kp=Kp, Km=Km, Qp=Qp, Kt=Kt, A=A, T=T, Tp=T @ np.diag(beta),
                Aqk=np.tril(Qp @ Km.T))


def prefill(q, k, v, g, beta, cu_seqlens=None, init_state=None, chunk=C, keep=False):
    """Same interface as the oracle's prefill; optionally keeps per-chunk (Tp, Aqk)."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    N, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, N]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    nseq = len(cu) - 1
    o = np.zeros((N, H, dv))
    fin = np.zeros((nseq, H, dk, dv))
    kept = {}
    for s in range(nseq):
        for h in range(H):
            S = np.zeros((dk, dv)) if init_state is None else np.array(init_state[s, h], dtype=np.float64)
            for c0 in range(cu[s], cu[s + 1], chunk):
                c1 = min(cu[s + 1], c0 + chunk)
                loc = chunk_local(q[c0:c1, h], k[c0:c1, h], g[c0:c1, h], beta[c0:c1, h])
                W = loc["Tp"] @ loc["Kp"]
                U = loc["Tp"] @ v[c0:c1, h]
                D = U - W @ S
                o[c0:c1, h] = loc["Qp"] @ S + loc["Aqk"] @ D
                S = np.exp(loc["G"][-1])[:, None] * S + loc["Kt"].T @ D
                if keep:
                    kept[(s, h, (c0 - cu[s]) // chunk)] = loc
            fin[s, h] = S
    return (o, fin, kept) if keep else (o, fin)


def prefill_lookahead(q, k, v, g, beta, cu_seqlens=None, init_state=None, chunk=C):
    """The chunk recurrence with one chunk of lookahead (a way to take the state update off the
    serial chain between two chunks; a single-pass kernel built on it was slower than the plain
    form on gfx950, because forming C moves work onto the producer waves).  With S_c the state entering chunk c, Gamma_c = e^{G_n} of chunk c and
    K~_c = K-_c (.) Gamma_c, the next chunk's K+ S is split into a part known from the state
    entering the current chunk and a 16 x 16 product with the current Delta:
        K+_{c+1} S_{c+1} = (K+_{c+1} Diag(Gamma_c)) S_c + (K+_{c+1} K~_c^T) Delta_c
                         = W'_{c+1} S_c + C_{c+1} Delta_c,     C_{c+1} = W'_{c+1} K-_c^T
    so only C Delta lies on the serial chain between two chunks' Delta."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    N, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, N]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    nseq = len(cu) - 1
    o = np.zeros((N, H, dv))
    fin = np.zeros((nseq, H, dk, dv))
    for s in range(nseq):
        for h in range(H):
            S = np.zeros((dk, dv)) if init_state is None else np.array(init_state[s, h], dtype=np.float64)
            gam_prev = np.ones(dk)                 # no chunk before the first
            km_prev, d_prev = np.zeros((chunk, dk)), np.zeros((chunk, dv))
            S_prev = S                             # state entering the (virtual) previous chunk
            for c0 in range(cu[s], cu[s + 1], chunk):
                c1 = min(cu[s + 1], c0 + chunk)
                loc = chunk_local(q[c0:c1, h], k[c0:c1, h], g[c0:c1, h], beta[c0:c1, h])
                Wp = loc["Kp"] * gam_prev[None, :]
                Cm = Wp @ km_prev[:d_prev.shape[0]].T
                X = Wp @ S_prev + Cm @ d_prev       # = K+ S
                D = loc["Tp"] @ (v[c0:c1, h] - X)
                o[c0:c1, h] = loc["Qp"] @ S + loc["Aqk"] @ D
                gam = np.exp(loc["G"][-1])
                S_prev, S = S, gam[:, None] * S + loc["Kt"].T @ D
                gam_prev, km_prev, d_prev = gam, loc["Km"], D
            fin[s, h] = S
    return o, fin


def backward(q, k, v, g, beta, dO, cu_seqlens=None, init_state=None, dfinal=None, chunk=C, dg_form="checkpoint"):
    """Gradients in chunk form (the algebra of the GPU backward), same outputs as the oracle's
    reverse mode.  Per chunk with incoming state S0, its Delta, and the adjoint S^ of the
    state after the chunk (dO of later chunks and dfinal included):

        X  = A_qk^T dO + K~ S^            E = T^T X   (rows eps_r = S^_r^T k_r)
        dV = diag(beta) E                  S^ <- Diag(e^{G_n}) S^ + Q+^T dO - K+^T dV
        dQ = e^{G} (.) (dO S0^T + tril(dO Delta^T) K-)
        a  = e^{-G} (.) (triu(Delta dO^T) Q+ - striu(Delta dV^T) K+ + e^{G_n} (.) (Delta S^^T))
        b  = diag(beta) e^{G} (.) (E S0^T + stril(E Delta^T) K-)
        dK = a - b,   U = K+ S0 + stril(K+ K-^T) Delta,   dbeta_r = eps_r . (v_r - u_r)
        dg_t = rowsum(dfinal (.) S_T) + sum_{s >= t} (q_s (.) dq_s - k_s (.) (a_s + b_s))

    dg_form="scan" evaluates the last line as written (one reverse cumulative sum over the
    sequence); "checkpoint" (the GPU kernel's form) sums only within the chunk and takes the
    part from every later token as rowsum(S^ (.) S_tau), S_tau the state after the chunk:
        rowsum(S^ (.) S_tau) = e^{G_n} (.) rowsum(S^ (.) S0) + sum_r K~_r (.) (Delta S^^T)_r.
    """
    assert dg_form in ("checkpoint", "scan")
    q, k, v, g, beta, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta, dO))
    N, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, N]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    nseq = len(cu) - 1
    out = {"dq": np.zeros((N, H, dk)), "dk": np.zeros((N, H, dk)), "dv": np.zeros((N, H, dv)),
           "dlog_alpha": np.zeros((N, H, dk)), "dbeta": np.zeros((N, H)), "dinit": np.zeros((nseq, H, dk, dv))}
    for s in range(nseq):
        for h in range(H):
            S = np.zeros((dk, dv)) if init_state is None else np.array(init_state[s, h], dtype=np.float64)
            saved = []
            for c0 in range(cu[s], cu[s + 1], chunk):
                c1 = min(cu[s + 1], c0 + chunk)
                loc = chunk_local(q[c0:c1, h], k[c0:c1, h], g[c0:c1, h], beta[c0:c1, h])
                D = loc["Tp"] @ (v[c0:c1, h] - loc["Kp"] @ S)
                saved.append((c0, c1, loc, S.copy(), D))
                S = np.exp(loc["G"][-1])[:, None] * S + loc["Kt"].T @ D
            Sh = np.zeros((dk, dv)) if dfinal is None else np.array(dfinal[s, h], dtype=np.float64)
            incr = np.zeros((cu[s + 1] - cu[s], dk))
            boundary = np.sum(Sh * S, axis=1)
            for c0, c1, loc, S0, D in reversed(saved):
                b = beta[c0:c1, h]
                Ob = dO[c0:c1, h]
                eG, emG, eGn = np.exp(loc["G"]), np.exp(-loc["G"]), np.exp(loc["G"][-1])
                X = loc["Aqk"].T @ Ob + loc["Kt"] @ Sh
                E = loc["T"].T @ X
                dV = b[:, None] * E
                dQ = eG * (Ob @ S0.T + np.tril(Ob @ D.T) @ loc["Km"])
                a = emG * (np.triu(D @ Ob.T) @ loc["Qp"] - np.triu(D @ dV.T, 1) @ loc["Kp"]
                           + eGn[None, :] * (D @ Sh.T))
                bb = b[:, None] * eG * (E @ S0.T + np.tril(E @ D.T, -1) @ loc["Km"])
                U = loc["Kp"] @ S0 + np.tril(loc["Kp"] @ loc["Km"].T, -1) @ D
                out["dq"][c0:c1, h] = dQ
                out["dk"][c0:c1, h] = a - bb
                out["dv"][c0:c1, h] = dV
                out["dbeta"][c0:c1, h] = np.sum(E * (v[c0:c1, h] - U), axis=1)
                inc = q[c0:c1, h] * dQ - k[c0:c1, h] * (a + bb)
                incr[c0 - cu[s]:c1 - cu[s]] = inc
                if dg_form == "checkpoint":
                    later = eGn * np.sum(Sh * S0, axis=1) + np.sum(loc["Kt"] * (D @ Sh.T), axis=0)
                    out["dlog_alpha"][c0:c1, h] = np.cumsum(inc[::-1], axis=0)[::-1] + later[None, :]
                Sh = eGn[:, None] * Sh + loc["Qp"].T @ Ob - loc["Kp"].T @ dV
            out["dinit"][s, h] = Sh
            if dg_form == "scan":
                out["dlog_alpha"][cu[s]:cu[s + 1], h] = boundary[None, :] + np.cumsum(incr[::-1], axis=0)[::-1]
    return out
