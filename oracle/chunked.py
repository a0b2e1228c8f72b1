"""Chunk-parallel form of the gated delta rule, fp64 numpy, for tests only.

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
