"""Chunk-parallel form of the gated delta rule and its reverse mode, fp64
numpy, for tests only.

TEST INFRASTRUCTURE ONLY (part of the oracle; the HIP library never imports
it).  This is the second, independent route to the same result as the
token-by-token oracle in gdn_oracle.c.  The pages name it as the
"chunk-parallel" implementation next to the token-by-token reference
(jax-linear-attention page, "How it works"); they do not print its algebra, so
the equations below are derived here from the recurrence (the closed-form
S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t).

With M = S^T (dk x dv), a chunk of L tokens starting from state M0, and
gamma_r = g_1 + ... + g_r (the cumulative log-decay inside the chunk):

    A[r, s] = beta_r exp(gamma_r - gamma_s) (k_r . k_s)        for s < r, else 0
    (I + A) Delta = diag(beta) V - diag(beta exp(gamma)) K M0     (one row per token:
                                                                   delta_r of the
                                                                   token form)
    O   = diag(exp(gamma)) Q M0 + (Q K^T * D) Delta,  D[r, s] = exp(gamma_r - gamma_s), s <= r
    M_L = exp(gamma_L) M0 + K^T diag(exp(gamma_L - gamma)) Delta

The triangular system is solved explicitly (numpy.linalg.solve on I + A), with
no blocking or fusion, so the code can be checked against these lines by eye.
The chunk size C is a free parameter: C = 1 is the token rule itself.
"""
import numpy as np


def chunk_step(Q, K, V, g, beta, M0):
    """One chunk.  Q, K: [L, dk]; V: [L, dv]; g, beta: [L]; M0: [dk, dv].

    Returns (O [L, dv], M_L [dk, dv], pieces) where pieces holds the
    intermediate gamma, A, Delta for tests that look inside the chunk."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    L = K.shape[0]
    gamma = np.cumsum(g)
    diff = gamma[:, None] - gamma[None, :]
    lower_incl = np.tril(np.ones((L, L), dtype=bool))
    lower_strict = np.tril(np.ones((L, L), dtype=bool), -1)
    # exp only where the mask keeps the entry: gamma_r - gamma_s <= 0 there.
    D = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
    A = np.where(lower_strict, beta[:, None] * D * (K @ K.T), 0.0)
    rhs = beta[:, None] * V - (beta * np.exp(gamma))[:, None] * (K @ M0)
    Delta = np.linalg.solve(np.eye(L) + A, rhs)
    O = np.exp(gamma)[:, None] * (Q @ M0) + ((Q @ K.T) * D) @ Delta
    gL = gamma[-1]
    ML = np.exp(gL) * M0 + K.T @ (np.exp(gL - gamma)[:, None] * Delta)
    return O, ML, {"gamma": gamma, "A": A, "Delta": Delta}


def fwd(q, k, v, g, beta, chunk, scale=1.0, h0=None, cu_seqlens=None):
    """Whole forward in chunks of `chunk` tokens, chunks restarting at every
    sequence start (a sequence's last chunk may be shorter).

    Same shapes and meaning as oracle.gdn_fwd; returns (o, ht) in fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    G = Hv // Hqk
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        cu = [int(x) for x in cu_seqlens]
        seqs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    o = np.zeros((B, T, Hv, dv))
    ht = np.zeros((len(seqs), Hv, dk, dv))
    for n, (b, t0, t1) in enumerate(seqs):
        for j in range(Hv):
            hk = j // G
            M = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, j], np.float64)
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                O, M, _ = chunk_step(q[b, c0:c1, hk], k[b, c0:c1, hk], v[b, c0:c1, j],
                                     g[b, c0:c1, j], beta[b, c0:c1, j], M)
                o[b, c0:c1, j] = scale * O
            ht[n, j] = M
    return o, ht


def chunk_step_bwd(Q, K, V, g, beta, M0, dO, dML):
    """Reverse mode of chunk_step: given the gradients dO [L, dv] of its O and
    dML [dk, dv] of its M_L, returns (dQ, dK, dV, dg, dbeta, dM0).

    The chain rule is applied to the five lines in the module docstring in
    reverse order; with X = K M0, rhs the right-hand side of the solve,
    e = exp(gamma), l = exp(gamma_L - gamma), P = (Q K^T) * D:

        M_L = exp(gamma_L) M0 + K^T diag(l) Delta
        O   = diag(e) Q M0 + P Delta
        Delta = (I + A)^-1 rhs      ->  drhs = (I + A)^-T dDelta,  dA = -drhs Delta^T
        rhs = diag(beta) V - diag(beta e) X
        A   = beta_r D (K K^T) below the diagonal

    and the decay factors e, l, exp(gamma_L) and D all differentiate through
    gamma, whose gradient becomes dg by a reverse cumulative sum."""
    Q, K, V, g, beta, M0, dO, dML = (np.asarray(x, np.float64)
                                     for x in (Q, K, V, g, beta, M0, dO, dML))
    L = K.shape[0]
    gamma = np.cumsum(g)
    gL = gamma[-1]
    e = np.exp(gamma)
    el = np.exp(gL - gamma)
    eL = np.exp(gL)
    lower_incl = np.tril(np.ones((L, L), dtype=bool))
    lower_strict = np.tril(np.ones((L, L), dtype=bool), -1)
    diff = gamma[:, None] - gamma[None, :]
    D = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
    KK = K @ K.T
    QK = Q @ K.T
    A = np.where(lower_strict, beta[:, None] * D * KK, 0.0)
    X = K @ M0
    rhs = beta[:, None] * V - (beta * e)[:, None] * X
    Delta = np.linalg.solve(np.eye(L) + A, rhs)
    P = np.where(lower_incl, QK * D, 0.0)
    Y = Q @ M0

    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dM0 = np.zeros_like(M0)
    dgamma = np.zeros(L)
    dgL = 0.0
    dD = np.zeros((L, L))
    # M_L = exp(gamma_L) M0 + K^T W, W = diag(l) Delta
    dM0 += eL * dML
    dgL += eL * np.sum(dML * M0)
    W = el[:, None] * Delta
    dW = K @ dML
    dK += W @ dML.T
    dDelta = el[:, None] * dW
    dl = np.sum(Delta * dW, axis=1)
    dgamma -= el * dl
    dgL += np.sum(el * dl)
    # O = diag(e) Y + P Delta, Y = Q M0
    dY = e[:, None] * dO
    dgamma += e * np.sum(dO * Y, axis=1)
    dQ += dY @ M0.T
    dM0 += Q.T @ dY
    dDelta += P.T @ dO
    dP = np.where(lower_incl, dO @ Delta.T, 0.0)
    dQK = dP * D
    dQ += dQK @ K
    dK += dQK.T @ Q
    dD += dP * QK
    # Delta = (I + A)^-1 rhs
    drhs = np.linalg.solve((np.eye(L) + A).T, dDelta)
    dA = np.where(lower_strict, -drhs @ Delta.T, 0.0)
    # rhs = diag(beta) V - diag(beta e) X, X = K M0
    dV = beta[:, None] * drhs
    dbeta = np.sum(drhs * (V - e[:, None] * X), axis=1)
    dgamma -= beta * e * np.sum(drhs * X, axis=1)
    dX = -(beta * e)[:, None] * drhs
    dK += dX @ M0.T
    dM0 += K.T @ dX
    # A = beta_r D[r, s] KK[r, s], s < r
    dbeta += np.sum(dA * D * KK, axis=1)
    dKK = beta[:, None] * dA * D
    dK += (dKK + dKK.T) @ K
    dD += beta[:, None] * dA * KK
    # D[r, s] = exp(gamma_r - gamma_s)
    dDD = dD * D
    dgamma += np.sum(dDD, axis=1) - np.sum(dDD, axis=0)
    dgamma[-1] += dgL
    dg = np.cumsum(dgamma[::-1])[::-1]
    return dQ, dK, dV, dg, dbeta, dM0


def bwd(q, k, v, g, beta, do, chunk, scale=1.0, h0=None, dht=None, cu_seqlens=None):
    """Whole reverse mode in chunks of `chunk` tokens: the chunk states of the
    forward, then the chunks in reverse with the state gradient carried from
    each chunk's end to its start.  Same shapes and meaning as oracle.gdn_bwd;
    returns (dq, dk, dv, dg, dbeta, dh0) in fp64."""
    q, k, v, g, beta, do = (np.asarray(x, np.float64) for x in (q, k, v, g, beta, do))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    G = Hv // Hqk
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        cu = [int(x) for x in cu_seqlens]
        seqs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    dq = np.zeros((B, T, Hqk, dk))
    dk_ = np.zeros((B, T, Hqk, dk))
    dv_ = np.zeros((B, T, Hv, dv))
    dg = np.zeros((B, T, Hv))
    dbeta = np.zeros((B, T, Hv))
    dh0 = np.zeros((len(seqs), Hv, dk, dv))
    for n, (b, t0, t1) in enumerate(seqs):
        for j in range(Hv):
            hk = j // G
            M = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, j], np.float64)
            starts = list(range(t0, t1, chunk))
            M0s = []
            for c0 in starts:
                c1 = min(c0 + chunk, t1)
                M0s.append(M)
                _, M, _ = chunk_step(q[b, c0:c1, hk], k[b, c0:c1, hk], v[b, c0:c1, j],
                                     g[b, c0:c1, j], beta[b, c0:c1, j], M)
            dM = np.zeros((dk, dv)) if dht is None else np.array(dht[n, j], np.float64)
            for c0, M0 in zip(reversed(starts), reversed(M0s)):
                c1 = min(c0 + chunk, t1)
                gq, gk, gv, gg, gb, dM = chunk_step_bwd(
                    q[b, c0:c1, hk], k[b, c0:c1, hk], v[b, c0:c1, j], g[b, c0:c1, j],
                    beta[b, c0:c1, j], M0, scale * do[b, c0:c1, j], dM)
                dq[b, c0:c1, hk] += gq
                dk_[b, c0:c1, hk] += gk
                dv_[b, c0:c1, j] = gv
                dg[b, c0:c1, j] = gg
                dbeta[b, c0:c1, j] = gb
            dh0[n, j] = dM
    return dq, dk_, dv_, dg, dbeta, dh0
