"""numpy fp64 model of the chunked (UT / WY) form that the HIP kernels use.

Not the oracle and not GPU code: a second CPU model that checks the algebra
of the chunk form against the token-by-token oracle, so that a kernel bug and
an algebra bug can be told apart.

Within a chunk of c tokens with chunk-local cumulative log-decays
Gam_t = sum_{i<=t} g_i (per channel):
    K_L  rows exp(Gam_t) * k_t            Kt  rows exp(Gam_c - Gam_t) * k_t
    G_ti = sum_ch k_t,ch k_i,ch exp(Gam_t,ch - Gam_i,ch)      (t > i)
    A    = (I + diag(beta) tril(G, -1))^-1 diag(beta)
    W = A K_L,  U = A V
    [T | S] <- diag(exp(Gam_c)) [T | S] + Kt^T ([0 | U] - W [T | S])
Families without erasure drop W and use U = diag(beta) V.
Outputs of a chunk read from S0:
    X = A (V - K_L S0);   o_t = S0^T (exp(Gam_t) * q_t) + sum_{i<=t} ((exp(Gam_t - Gam_i) * q_t) . k_i) x_i
"""
import numpy as np

DELTA = ("deltanet", "gdn", "kda")


def _logdecay(fam, g, gamma, n, dk):
    if fam in ("linear", "deltanet"):
        return np.zeros((n, dk))
    if fam == "retnet":
        return np.full((n, dk), np.log(gamma))
    if fam in ("mamba2", "gdn"):
        return np.repeat(np.asarray(g, dtype=np.float64).reshape(n, 1), dk, axis=1)
    return np.asarray(g, dtype=np.float64).reshape(n, dk)


def _chunk_factors(fam, K, V, Gm, b):
    L, dk = K.shape
    Kl = np.exp(Gm) * K
    Kt = np.exp(Gm[-1] - Gm) * K
    if fam in DELTA:
        G = np.zeros((L, L))
        for t in range(L):
            for i in range(t):
                G[t, i] = np.sum(K[t] * K[i] * np.exp(Gm[t] - Gm[i]))
        A = np.linalg.solve(np.eye(L) + np.diag(b) @ G, np.diag(b))
        return Kl, Kt, A
    return Kl, Kt, np.diag(b)


def chunk_pair(fam, k, v, g=None, beta=None, gamma=1.0, c=64):
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    n, dk = k.shape
    dv = v.shape[1]
    lg = _logdecay(fam, g, gamma, n, dk)
    bb = np.ones(n) if beta is None or fam not in DELTA else np.asarray(beta, np.float64)
    X = np.concatenate([np.eye(dk), np.zeros((dk, dv))], axis=1)
    for s in range(0, n, c):
        e = min(n, s + c)
        K, V = k[s:e], v[s:e]
        Gm = np.cumsum(lg[s:e], axis=0)
        Kl, Kt, A = _chunk_factors(fam, K, V, Gm, bb[s:e])
        Y = np.concatenate([np.zeros((e - s, dk)), A @ V], axis=1)
        M = A @ Kl @ X if fam in DELTA else 0.0
        X = np.exp(Gm[-1])[:, None] * X + Kt.T @ (Y - M)
    return X[:, :dk], X[:, dk:]


def chunk_run(fam, q, k, v, g=None, beta=None, gamma=1.0, S0=None, c=64):
    """Outputs and final state of the recurrence read in chunks from S0."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    n, dk = k.shape
    dv = v.shape[1]
    lg = _logdecay(fam, g, gamma, n, dk)
    bb = np.ones(n) if beta is None or fam not in DELTA else np.asarray(beta, np.float64)
    S = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64).copy()
    O = np.zeros((n, dv))
    for s in range(0, n, c):
        e = min(n, s + c)
        K, V, Q = k[s:e], v[s:e], q[s:e]
        Gm = np.cumsum(lg[s:e], axis=0)
        Kl, Kt, A = _chunk_factors(fam, K, V, Gm, bb[s:e])
        X = A @ (V - Kl @ S) if fam in DELTA else A @ V
        for t in range(e - s):
            o = S.T @ (np.exp(Gm[t]) * Q[t])
            for i in range(t + 1):
                o += np.dot(np.exp(Gm[t] - Gm[i]) * Q[t], K[i]) * X[i]
            O[s + t] = o
        S = np.exp(Gm[-1])[:, None] * S + Kt.T @ X
    return S, O


def chunk_pair_folded(fam, k, v, g=None, beta=None, c=64, blk=16):
    """The dense-build form with the scalar decay folded out of the chunk
    system (DeltaNet, Gated DeltaNet).  With E = diag(exp(Gam_c - Gam_t)) the
    decayed system is a similarity transform of the undecayed one,
    I + diag(beta) tril(G o exp(Gam_t - Gam_i), -1) = E^-1 (I + N0) E with
    N0 = diag(beta) tril(K K^T, -1), so R' = E R solves
        (I + N0) R' = diag(beta) ([0 | E V] - exp(Gam_c) K X)
    and X <- exp(Gam_c) X + K^T R'.  R' is found block by block:
        R'_b = Inv_b diag(beta_b) Y'_b - sum_{c<b} Inv_b N0_bc R'_c,
    Inv_b = (I + N0_bb)^-1, which is how the bf16 kernel splits the work."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    n, dk = k.shape
    dv = v.shape[1]
    lg = np.zeros(n) if fam == "deltanet" else np.asarray(g, np.float64).reshape(n)
    bb = np.asarray(beta, np.float64)
    X = np.concatenate([np.eye(dk), np.zeros((dk, dv))], axis=1)
    for s in range(0, n, c):
        e = min(n, s + c)
        L = e - s
        K, V, b = k[s:e], v[s:e], bb[s:e]
        Gm = np.cumsum(lg[s:e])
        lam = np.exp(Gm[-1])
        ec = np.exp(Gm[-1] - Gm)
        N0 = np.diag(b) @ np.tril(K @ K.T, -1)
        Y = np.concatenate([np.zeros((L, dk)), ec[:, None] * V], axis=1) - lam * (K @ X)
        R = np.zeros_like(Y)
        for b0 in range(0, L, blk):
            b1 = min(L, b0 + blk)
            inv = np.linalg.inv(np.eye(b1 - b0) + N0[b0:b1, b0:b1])
            acc = inv @ np.diag(b[b0:b1]) @ Y[b0:b1]
            acc -= inv @ N0[b0:b1, :b0] @ R[:b0]
            R[b0:b1] = acc
        X = lam * X + K.T @ R
    return X[:, :dk], X[:, dk:]


def chunk_pair_kda_inv(k, v, g, beta, c=32):
    """The per-channel form of the bf16 KDA build: with K_L rows
    exp(Gam_t) * k_t and K_i rows exp(-Gam_t) * k_t (per channel),
        G = tril(K_L K_i^T, -1)       (no per-block reference token)
        A = (I + diag(beta) G)^-1 diag(beta)
        R = A ([0 | V] - K_L X)
        X <- diag(exp(Gam_c)) (X + K_i^T R)
    which is diag(exp Gam_c) X + Kt^T R with Kt = diag-scaled K_i."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    n, dk = k.shape
    dv = v.shape[1]
    lg = np.asarray(g, np.float64).reshape(n, dk)
    bb = np.asarray(beta, np.float64)
    X = np.concatenate([np.eye(dk), np.zeros((dk, dv))], axis=1)
    for s in range(0, n, c):
        e = min(n, s + c)
        L = e - s
        K, V, b = k[s:e], v[s:e], bb[s:e]
        Gm = np.cumsum(lg[s:e], axis=0)
        Kl, Ki = np.exp(Gm) * K, np.exp(-Gm) * K
        G = np.tril(Kl @ Ki.T, -1)
        A = np.linalg.solve(np.eye(L) + np.diag(b) @ G, np.diag(b))
        R = A @ (np.concatenate([np.zeros((L, dk)), V], axis=1) - Kl @ X)
        X = np.exp(Gm[-1])[:, None] * (X + Ki.T @ R)
    return X[:, :dk], X[:, dk:]
