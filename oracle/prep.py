"""Input preparation and the single-token step of the gated delta rule, fp64.

TEST INFRASTRUCTURE ONLY (part of the oracle; the HIP library never imports
it).

  * l2_normalize -- each row divided by its Euclidean norm: the in-op q/k
    normalisation the jax-linear-attention page's "Quick start" call switches
    on (use_qk_l2norm).  The pages give no epsilon, so the norm is exact; a
    row of zeros, whose direction is undefined, is mapped to zeros.
  * logsigmoid, sigmoid -- the gate activations the same example applies to
    raw values: g = logsigmoid(raw) is the natural-log decay (so a = exp(g) =
    sigmoid(raw) lies in (0, 1)) and beta = sigmoid(raw) the write strength.
  * step -- one token of the recurrence for a batch of sequences whose states
    live in a cache: the token-by-token form of "How it works" on the same
    page, one token per call.  With M = S^T the [dk, dv] state of the
    sequence's slot and a = exp(g), the closed form
    S <- a S (I - beta k k^T) + beta v k^T, o = scale S q reads
        y = M^T k,  delta = beta (v - a y),  M <- a M + k delta^T,  o = scale M^T q.
    Chaining it over a sequence is pinned against gdn_fwd, the token-by-token
    oracle in C.
  * l2_normalize_bwd, logsigmoid_bwd, sigmoid_bwd, chain_options -- the
    reverse mode of the preparation (derivatives of the three maps, which the
    pages do not print), so that the gradient of a forward that prepares its
    inputs in-op can be taken with respect to the raw inputs.
"""
import numpy as np


def l2_normalize(x):
    """x / ||x||_2 over the last axis, in fp64; zero rows stay zero."""
    x = np.asarray(x, np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    safe = np.where(n > 0.0, n, 1.0)
    return np.where(n > 0.0, x / safe, 0.0)


def logsigmoid(x):
    """log(1 / (1 + exp(-x))) in fp64, in a form that neither overflows nor
    cancels: -log1p(exp(-x)) for x >= 0 and x - log1p(exp(x)) for x < 0 (the
    same value, multiplied through by exp(x))."""
    x = np.asarray(x, np.float64)
    pos = -np.log1p(np.exp(-np.abs(x)))
    return np.where(x >= 0.0, pos, x + pos)


def sigmoid(x):
    """1 / (1 + exp(-x)) in fp64 (exp(x) / (1 + exp(x)) for x < 0)."""
    x = np.asarray(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0.0, 1.0 / (1.0 + e), e / (1.0 + e))


def step(q, k, v, g, beta, state, slots=None, scale=1.0, use_qk_l2norm=False,
         gate_activation=False):
    """One decode token for N sequences.

    q, k: [N, Hqk, dk]; v: [N, Hv, dv]; g, beta: [N, Hv]; state: [S, Hv, dk, dv]
    cache (not modified); slots: [N] ints or None (slot n).  A slot outside
    [0, S) is padding: zero initial state, nothing written back.  Returns
    (o [N, Hv, dv], new cache [S, Hv, dk, dv]), fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    if use_qk_l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    if gate_activation:
        g, beta = logsigmoid(g), sigmoid(beta)
    state = np.asarray(state, np.float64)
    N, Hqk = q.shape[0], q.shape[1]
    Hv, dv = v.shape[1], v.shape[2]
    G = Hv // Hqk
    S = state.shape[0]
    slots = np.arange(N) if slots is None else np.asarray(slots, np.int64)
    new = state.copy()
    o = np.zeros((N, Hv, dv))
    for n in range(N):
        s = int(slots[n])
        cached = 0 <= s < S
        for j in range(Hv):
            kv, qv = k[n, j // G], q[n, j // G]
            M = state[s, j] if cached else np.zeros((k.shape[2], dv))
            a = np.exp(g[n, j])
            y = M.T @ kv
            delta = beta[n, j] * (v[n, j] - a * y)
            M = a * M + np.outer(kv, delta)
            o[n, j] = scale * (M.T @ qv)
            if cached:
                new[s, j] = M
    return o, new


# ---------------------------------------------------------------------------
# Reverse mode of the preparation.  The pages state no gradients; these are
# the derivatives of the three maps above, written out: each takes the raw
# input x and the gradient dy of a loss with respect to the prepared value,
# and returns the gradient with respect to x.

def l2_normalize_bwd(x, dy):
    """Through y = x / n, n = ||x||: the Jacobian is (I - y y^T) / n, so
    dx = (dy - (dy . y) y) / n, row by row over the last axis.  A zero row,
    mapped to the constant zero, gets a zero gradient."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    safe = np.where(n > 0.0, n, 1.0)
    y = x / safe
    proj = np.sum(dy * y, axis=-1, keepdims=True)
    return np.where(n > 0.0, (dy - proj * y) / safe, 0.0)


def logsigmoid_bwd(x, dy):
    """d logsigmoid(x) / dx = 1 - sigmoid(x) = sigmoid(-x)."""
    return np.asarray(dy, np.float64) * sigmoid(-np.asarray(x, np.float64))


def sigmoid_bwd(x, dy):
    """d sigmoid(x) / dx = sigmoid(x) (1 - sigmoid(x)) = sigmoid(x) sigmoid(-x)."""
    x = np.asarray(x, np.float64)
    return np.asarray(dy, np.float64) * sigmoid(x) * sigmoid(-x)


def chain_options(q, k, g, beta, dq, dk, dg, dbeta, use_qk_l2norm=False,
                  gate_activation=False):
    """Gradients with respect to the raw q, k, g, beta of a forward that
    prepares its inputs in-op, from the gradients (dq, dk, dg, dbeta) with
    respect to the prepared inputs the recurrence consumed.  An option that
    is off passes its gradients through unchanged."""
    dq, dk = np.asarray(dq, np.float64), np.asarray(dk, np.float64)
    dg, dbeta = np.asarray(dg, np.float64), np.asarray(dbeta, np.float64)
    if use_qk_l2norm:
        dq, dk = l2_normalize_bwd(q, dq), l2_normalize_bwd(k, dk)
    if gate_activation:
        dg, dbeta = logsigmoid_bwd(g, dg), sigmoid_bwd(beta, dbeta)
    return dq, dk, dg, dbeta
