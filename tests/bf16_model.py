"""A CPU model of where the bf16 forward rounds, to predict its error.

Test-side tool (not part of the oracle: it copies the kernel's rounding
points, which the oracle must not know about).  It runs the chunk equations
of the gated delta rule in fp64 and rounds exactly where the HIP forward
takes an operand into the MFMA in bf16 without a low part:

  * Q M0 reads the state M0 as bf16(M0) (hi part only), and so does K M0 at
    dk = 128 and 256; at dk = 64 K M0 reads M0 as hi + lo;
  * P Delta reads bf16(P) and bf16(Delta);

and stores the state as fp32 between chunks.  Everything else the kernel
carries as split hi + lo bf16 pairs (about 16 significant bits) or in fp32,
which the model takes as exact.  Chunks are 64 tokens (32 for dk = 256), as
in the kernel.  With `rounding=False` the model is the plain chunk form and
must equal oracle.chunked.fwd.

The chunk form (derived from the recurrence S_t = a_t S_{t-1}(I - b_t k_t
k_t^T) + b_t v_t k_t^T, o_t = S_t q_t of Gated DeltaNet): with gamma the
in-chunk cumulative log-decay, D[r, s] = exp(gamma_r - gamma_s) for s <= r,
  A = strict lower part of diag(beta) D * (K K^T)
  Delta = (I + A)^-1 (diag(beta) V - diag(beta exp(gamma)) K M0)
  O = diag(exp(gamma)) Q M0 + (D * Q K^T) Delta
  M_L = exp(gamma_L) M0 + K^T diag(exp(gamma_L - gamma)) Delta
"""
import numpy as np


def bf16(x):
    """Round to the nearest bf16 (ties to even), returned as fp64."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = (u + (((u >> 16) & 1) + np.uint32(0x7FFF))) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def fp32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def chunk_len(dk):
    return 32 if dk == 256 else 64


def head(q, k, v, g, beta, h0=None, scale=1.0, rounding=True, km0_split=None):
    """One head of one sequence.  q, k: [T, dk]; v: [T, dv]; g, beta: [T];
    h0: [dk, dv] or None.  km0_split: K M0 with hi + lo parts of M0 (None:
    as the kernel does, at dk = 64 only).  Returns (o [T, dv], final state
    [dk, dv])."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    g, beta = np.asarray(g, np.float64), np.asarray(beta, np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    C = chunk_len(dk)
    if km0_split is None:
        km0_split = dk == 64
    M = np.zeros((dk, dv)) if h0 is None else np.asarray(h0, np.float64).copy()
    o = np.zeros((T, dv))
    rb = bf16 if rounding else (lambda x: np.asarray(x, np.float64))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        L = K.shape[0]
        gam = np.cumsum(g[sl])
        diff = gam[:, None] - gam[None, :]
        incl = np.tril(np.ones((L, L), dtype=bool))
        D = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
        A = np.where(np.tril(incl, -1), b[:, None] * D * (K @ K.T), 0.0)
        Mb = rb(M)
        Mk = (Mb + rb(M - Mb)) if km0_split else Mb
        rhs = b[:, None] * V - (b * np.exp(gam))[:, None] * (K @ Mk)
        Delta = np.linalg.solve(np.eye(L) + A, rhs)
        P = D * (Q @ K.T)
        o[sl] = scale * (np.exp(gam)[:, None] * (Q @ Mb) + rb(P) @ rb(Delta))
        M = np.exp(gam[-1]) * M + K.T @ (np.exp(gam[-1] - gam)[:, None] * Delta)
        if rounding:
            M = fp32(M)
    return o, M


def forward(q, k, v, g, beta, h0=None, scale=1.0, rounding=True, heads=None,
            km0_split=None):
    """Batch rows [B, T, H, ...] (no packing) over the value heads in `heads`
    (all by default); returns (o [B, T, H, dv], ht [B, H, dk, dv]) with the
    heads not modelled left at zero."""
    B, T, Hqk, dk = np.shape(q)
    Hv, dv = np.shape(v)[2], np.shape(v)[3]
    G = Hv // Hqk
    o = np.zeros((B, T, Hv, dv))
    ht = np.zeros((B, Hv, dk, dv))
    for bi in range(B):
        for h in (range(Hv) if heads is None else heads):
            o[bi, :, h], ht[bi, h] = head(
                q[bi, :, h // G], k[bi, :, h // G], v[bi, :, h], g[bi, :, h], beta[bi, :, h],
                None if h0 is None else h0[bi, h], scale, rounding, km0_split)
    return o, ht
