"""Pins for the CPU oracle: checks against facts that do not come from the
oracle itself.

Each pin takes `fwd`, a function with the signature of oracle.gdn_fwd, so the
same pins run against the oracle (test_oracle.py) and against deliberately
broken copies of it (test_oracle_mutants.py).  A pin raises AssertionError on
failure.

The recurrence being pinned is the gated delta rule of Gated DeltaNet (the
December 2024 paper by Yang, Kautz and Hatamizadeh that the Qwen FlashQLA
article names under "The bottleneck nobody wanted to talk about"):
S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t, with
a_t = exp(g_t) (g is a natural-log decay; jax-linear-attention page,
"Quick start") and the state returned as M = S^T of shape [dk, dv].
"""
import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_inputs(rng, B, T, Hqk, Hv, dk, dv, unit_keys=True):
    q = rng.standard_normal((B, T, Hqk, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, Hqk, dk)).astype(np.float32)
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True).astype(np.float32)
    v = rng.standard_normal((B, T, Hv, dv)).astype(np.float32)
    g = (-np.logaddexp(0, -rng.standard_normal((B, T, Hv))) / 4).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B, T, Hv))))).astype(np.float32)
    return q, k, v, g, beta


def _close(a, b, rtol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)
    assert err <= rtol, f"{what}: relative error {err:.3e} > {rtol:.1e}"


# --- closed forms -----------------------------------------------------------

def pin_single_token(fwd):
    """One token from a zero state: o = beta (k . q) v and M = beta k v^T."""
    rng = _rng(1)
    q, k, v, g, beta = _rand_inputs(rng, 2, 1, 3, 3, 5, 4)
    o, ht = fwd(q, k, v, g, beta)
    kq = np.einsum("bthd,bthd->bth", k.astype(np.float64), q.astype(np.float64))
    want_o = beta[..., None] * kq[..., None] * v
    _close(o, want_o, 1e-14, "single-token output")
    want_M = beta[:, 0, :, None, None] * k[:, 0, :, :, None].astype(np.float64) \
        * v[:, 0, :, None, :].astype(np.float64)
    _close(ht, want_M, 1e-14, "single-token state")


def pin_beta0_a1_state_unchanged(fwd):
    """beta = 0 and a = 1: the state never changes; o_t = M0^T q_t."""
    rng = _rng(2)
    q, k, v, g, beta = _rand_inputs(rng, 1, 9, 2, 2, 6, 3)
    g[:] = 0
    beta[:] = 0
    h0 = rng.standard_normal((1, 2, 6, 3))
    o, ht = fwd(q, k, v, g, beta, h0=h0)
    assert np.array_equal(ht, h0), "state changed with beta = 0, a = 1"
    want = np.einsum("bthi,bhic->bthc", q.astype(np.float64), h0)
    _close(o, want, 1e-14, "read-only output")


def pin_beta0_decay_product(fwd):
    """beta = 0: M_t = (a_1 ... a_t) M0, so o_t = exp(g_1 + ... + g_t) M0^T q_t."""
    rng = _rng(3)
    q, k, v, g, beta = _rand_inputs(rng, 1, 11, 1, 1, 4, 5)
    beta[:] = 0
    h0 = rng.standard_normal((1, 1, 4, 5))
    o, ht = fwd(q, k, v, g, beta, h0=h0)
    cum = np.cumsum(g[0, :, 0].astype(np.float64))
    want = np.exp(cum)[:, None] * (q[0, :, 0].astype(np.float64) @ h0[0, 0])
    _close(o[0, :, 0], want, 1e-13, "decay-only output")
    _close(ht, np.exp(cum[-1]) * h0, 1e-13, "decay-only state")


def pin_full_forgetting(fwd):
    """g = -100 (a = e^-100): each token sees only itself, o_t = beta_t (k_t . q_t) v_t."""
    rng = _rng(4)
    q, k, v, g, beta = _rand_inputs(rng, 1, 7, 2, 4, 8, 3)
    g[:] = -100.0
    o, _ = fwd(q, k, v, g, beta)
    kq = np.einsum("bthd,bthd->bth", k.astype(np.float64), q.astype(np.float64))
    kq = np.repeat(kq, 2, axis=2)  # value head j reads q/k head j // 2
    want = beta[..., None] * kq[..., None] * v
    _close(o, want, 1e-13, "full-forgetting output")


def pin_exact_write(fwd):
    """beta = 1 with |k| = 1 exactly: the delta rule overwrites, M_t^T k_t = v_t.
    Keys have four entries of +-1/2 (so |k|^2 = 1 in binary) and q_t = k_t."""
    rng = _rng(5)
    T, dk, dv = 10, 12, 3
    k = np.zeros((1, T, 1, dk), np.float32)
    for t in range(T):
        idx = rng.choice(dk, 4, replace=False)
        k[0, t, 0, idx] = rng.choice([-0.5, 0.5], 4)
    q = k.copy()
    v = rng.standard_normal((1, T, 1, dv)).astype(np.float32)
    g = (-rng.random((1, T, 1)) * 0.3).astype(np.float32)
    beta = np.ones((1, T, 1), np.float32)
    h0 = rng.standard_normal((1, 1, dk, dv))
    o, _ = fwd(q, k, v, g, beta, h0=h0)
    _close(o, v, 1e-14, "exact overwrite")


def _hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def pin_orthonormal_keys_linear_attention(fwd):
    """Orthonormal keys, a = 1, beta = 1, zero state: every delta equals its v,
    so the output is causal linear attention o_t = sum_{s<=t} (k_s . q_t) v_s.
    Keys are distinct rows of the 16 x 16 Hadamard matrix over 4 (exact)."""
    rng = _rng(6)
    dk, dv, T = 16, 5, 12
    rows = rng.choice(dk, T, replace=False)
    K = (_hadamard(dk)[rows] / 4.0) * rng.choice([-1.0, 1.0], (T, 1))
    Q = rng.standard_normal((T, dk)).astype(np.float32)
    V = rng.standard_normal((T, dv)).astype(np.float32)
    q, k, v = Q[None, :, None], K.astype(np.float32)[None, :, None], V[None, :, None]
    g = np.zeros((1, T, 1), np.float32)
    beta = np.ones((1, T, 1), np.float32)
    o, ht = fwd(q, k, v, g, beta)
    scores = np.tril(Q.astype(np.float64) @ K.T)  # [t, s] = q_t . k_s for s <= t
    want = scores @ V.astype(np.float64)
    _close(o[0, :, 0], want, 1e-14, "linear-attention output")
    _close(ht[0, 0], K.T @ V.astype(np.float64), 1e-14, "linear-attention state")


def pin_linearity(fwd):
    """For fixed q, k, g, beta the map (v, h0) -> (o, ht) is linear, and o is
    homogeneous in q (ht does not depend on q); scale multiplies o only."""
    rng = _rng(7)
    q, k, v1, g, beta = _rand_inputs(rng, 2, 13, 2, 2, 6, 4)
    v2 = rng.standard_normal(v1.shape).astype(np.float32)
    h1 = rng.standard_normal((2, 2, 6, 4))
    h2 = rng.standard_normal((2, 2, 6, 4))
    o1, s1 = fwd(q, k, v1, g, beta, h0=h1)
    o2, s2 = fwd(q, k, v2, g, beta, h0=h2)
    o12, s12 = fwd(q, k, v1 + v2, g, beta, h0=h1 + h2)
    # v1 + v2 rounds to fp32; compare against the fp32 sum's own run.
    _close(o12, o1 + o2, 1e-6, "additivity (output)")
    _close(s12, s1 + s2, 1e-6, "additivity (state)")
    o4, s4 = fwd(q, k, 4 * v1, g, beta, h0=4 * h1)
    assert np.array_equal(o4, 4 * o1) and np.array_equal(s4, 4 * s1), "not homogeneous in (v, h0)"
    oq, sq = fwd(0.5 * q, k, v1, g, beta, h0=h1)
    assert np.array_equal(oq, 0.5 * o1) and np.array_equal(sq, s1), "not homogeneous in q"
    os_, ss = fwd(q, k, v1, g, beta, scale=0.125, h0=h1)
    assert np.array_equal(os_, 0.125 * o1) and np.array_equal(ss, s1), "scale misapplied"


def pin_exact_rational(fwd):
    """Brute force in exact rational arithmetic on a tiny case, written in the
    untransposed form S_t = a S_{t-1}(I - b k k^T) + b v k^T, o_t = S_t q_t.
    a is taken as the exact value of the fp64 exp(g) the oracle forms, so the
    only difference left is the oracle's fp64 rounding."""
    rng = _rng(8)
    T, dk, dv = 6, 3, 2
    pick = lambda *s: (rng.integers(-4, 5, s) / 4.0).astype(np.float32)
    q, k, v = pick(1, T, 1, dk), pick(1, T, 1, dk), pick(1, T, 1, dv)
    beta = (rng.integers(1, 5, (1, T, 1)) / 4.0).astype(np.float32)
    g = (-rng.random((1, T, 1))).astype(np.float32)
    h0 = pick(1, 1, dk, dv).astype(np.float64)
    F = Fraction
    S = [[F(float(h0[0, 0, i, c])) for i in range(dk)] for c in range(dv)]  # S = M^T
    want_o = np.zeros((T, dv))
    for t in range(T):
        a = F(math.exp(float(g[0, t, 0])))
        b = F(float(beta[0, t, 0]))
        kt = [F(float(x)) for x in k[0, t, 0]]
        vt = [F(float(x)) for x in v[0, t, 0]]
        qt = [F(float(x)) for x in q[0, t, 0]]
        P = [[(1 if i == j else 0) - b * kt[i] * kt[j] for j in range(dk)] for i in range(dk)]
        S = [[a * sum(S[c][m] * P[m][i] for m in range(dk)) + b * vt[c] * kt[i]
              for i in range(dk)] for c in range(dv)]
        for c in range(dv):
            want_o[t, c] = float(sum(S[c][i] * qt[i] for i in range(dk)))
    want_M = np.array([[float(S[c][i]) for c in range(dv)] for i in range(dk)])
    o, ht = fwd(q, k, v, g, beta, h0=h0)
    _close(o[0, :, 0], want_o, 1e-14, "rational brute force (output)")
    _close(ht[0, 0], want_M, 1e-14, "rational brute force (state)")


def pin_hand_worked(fwd):
    """The two-token example worked by hand in tests/golden."""
    with open(os.path.join(GOLDEN, "two_tokens_by_hand.json")) as f:
        ex = json.load(f)
    arr = lambda name: np.asarray(ex[name], np.float32)
    o, ht = fwd(arr("q"), arr("k"), arr("v"), arr("g"), arr("beta"))
    np.testing.assert_allclose(o, np.asarray(ex["o"]), rtol=0, atol=1e-6)
    np.testing.assert_allclose(ht, np.asarray(ex["state"]), rtol=0, atol=1e-6)


# --- invariants and the independent chunked route ---------------------------

def pin_chunked_route(fwd):
    """The chunk-parallel algebra (oracle/chunked.py: explicit solve of
    I + A, no blocking) equals the token recurrence for chunk sizes
    1, 2, 3, 8 and 64, T not a multiple of the chunk, grouped value heads, a
    random initial state, a scale, and a packed batch."""
    from oracle import chunked
    rng = _rng(9)
    q, k, v, g, beta = _rand_inputs(rng, 2, 70, 2, 4, 8, 5)
    h0 = rng.standard_normal((2, 4, 8, 5))
    o, ht = fwd(q, k, v, g, beta, scale=0.7, h0=h0)
    for C in (1, 2, 3, 8, 64):
        oc, hc = chunked.fwd(q, k, v, g, beta, C, scale=0.7, h0=h0)
        _close(o, oc, 1e-12, f"chunked C={C} output")
        _close(ht, hc, 1e-12, f"chunked C={C} state")
    cu = np.array([0, 5, 5, 38, 70])
    qp, kp, vp, gp, bp = (x[:1] for x in (q, k, v, g, beta))
    hp = rng.standard_normal((4, 4, 8, 5))
    o, ht = fwd(qp, kp, vp, gp, bp, h0=hp, cu_seqlens=cu)
    oc, hc = chunked.fwd(qp, kp, vp, gp, bp, 16, h0=hp, cu_seqlens=cu)
    _close(o, oc, 1e-12, "chunked packed output")
    _close(ht, hc, 1e-12, "chunked packed state")


def pin_packed_equals_separate(fwd):
    """A packed row with cu_seqlens gives, bit for bit, the per-document calls
    (the per-document reset, jax-linear-attention page, "How it works"); an
    empty document returns its initial state."""
    rng = _rng(10)
    lengths = [7, 0, 1, 19, 4]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k, v, g, beta = _rand_inputs(rng, 1, T, 2, 4, 6, 3)
    h0 = rng.standard_normal((len(lengths), 4, 6, 3))
    o, ht = fwd(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        if a == b:
            assert np.array_equal(ht[n], h0[n]), "empty document changed its state"
            continue
        on, hn = fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], h0=h0[n:n + 1])
        assert np.array_equal(o[:, a:b], on), f"document {n}: output differs"
        assert np.array_equal(ht[n:n + 1], hn), f"document {n}: state differs"


def pin_chained_halves(fwd):
    """One call over T tokens equals two calls over the halves with the first
    half's final state passed as the second half's initial state, bit for bit
    (the chained-halves property in the jax-linear-attention page's
    "Highlights")."""
    rng = _rng(11)
    q, k, v, g, beta = _rand_inputs(rng, 2, 30, 1, 2, 5, 4)
    h0 = rng.standard_normal((2, 2, 5, 4))
    o, ht = fwd(q, k, v, g, beta, h0=h0)
    s = 13
    o1, h1 = fwd(q[:, :s], k[:, :s], v[:, :s], g[:, :s], beta[:, :s], h0=h0)
    o2, h2 = fwd(q[:, s:], k[:, s:], v[:, s:], g[:, s:], beta[:, s:], h0=h1)
    assert np.array_equal(o, np.concatenate([o1, o2], axis=1)), "halves: output differs"
    assert np.array_equal(ht, h2), "halves: state differs"


def pin_grouped_heads(fwd):
    """Grouped value heads: value head j reads q/k head j // G (consecutive value
    heads share), so a call with Hv = 3 Hqk equals single-head calls."""
    rng = _rng(12)
    q, k, v, g, beta = _rand_inputs(rng, 1, 9, 2, 6, 4, 3)
    o, ht = fwd(q, k, v, g, beta)
    for j in range(6):
        hk = j // 3
        oj, hj = fwd(q[:, :, hk:hk + 1], k[:, :, hk:hk + 1], v[:, :, j:j + 1],
                     g[:, :, j:j + 1], beta[:, :, j:j + 1])
        assert np.array_equal(o[:, :, j:j + 1], oj) and np.array_equal(ht[:, j:j + 1], hj), \
            f"value head {j} does not read q/k head {hk}"


def pin_thread_invariance(fwd):
    """The result does not depend on the number of host threads."""
    rng = _rng(13)
    q, k, v, g, beta = _rand_inputs(rng, 3, 17, 2, 2, 8, 70)
    o1, h1 = fwd(q, k, v, g, beta, nthreads=1)
    o7, h7 = fwd(q, k, v, g, beta, nthreads=7)
    assert np.array_equal(o1, o7) and np.array_equal(h1, h7), "thread count changes the result"


ALL_PINS = [
    pin_single_token, pin_beta0_a1_state_unchanged, pin_beta0_decay_product,
    pin_full_forgetting, pin_exact_write, pin_orthonormal_keys_linear_attention,
    pin_linearity, pin_exact_rational, pin_hand_worked, pin_chunked_route,
    pin_packed_equals_separate, pin_chained_halves, pin_grouped_heads,
    pin_thread_invariance,
]


# ---------------------------------------------------------------------------
# Reverse mode.  Each pin takes `fwd` and `bwd` (the signatures of
# oracle.gdn_fwd and oracle.gdn_bwd); the loss is L = sum(do * o) + sum(dht * ht).

def _bwd_case(rng, B, T, Hqk, Hv, dk, dv, N):
    q, k, v, g, beta = _rand_inputs(rng, B, T, Hqk, Hv, dk, dv)
    q /= np.linalg.norm(q, axis=-1, keepdims=True).astype(np.float32)
    do = rng.standard_normal((B, T, Hv, dv)).astype(np.float32)
    h0 = rng.standard_normal((N, Hv, dk, dv)) * 0.3
    dht = rng.standard_normal((N, Hv, dk, dv))
    return q, k, v, g, beta, do, h0, dht


def pin_bwd_finite_differences(fwd, bwd):
    """Every gradient equals the central difference of the forward loss.  A
    packed batch of two documents with grouped value heads, an initial state,
    a loss on the final state and a scale.  fp32 inputs move by 2^-12, which
    fp32 holds exactly at these magnitudes; the difference quotient is then
    accurate to about 1e-8 (its error is second order in the step)."""
    rng = _rng(101)
    cu = np.array([0, 7, 16])
    q, k, v, g, beta, do, h0, dht = _bwd_case(rng, 1, 16, 1, 2, 8, 8, 2)
    scale = 0.7

    def loss(args, h0_):
        o, ht = fwd(*args, scale=scale, h0=h0_, cu_seqlens=cu)
        return float(np.sum(do.astype(np.float64) * o) + np.sum(dht * ht))

    grads = bwd(q, k, v, g, beta, do, scale=scale, h0=h0, dht=dht, cu_seqlens=cu)
    base = [q, k, v, g, beta]
    h = 2.0 ** -12
    for gi, name in enumerate(("q", "k", "v", "g", "beta")):
        x = base[gi]
        fd = np.zeros(x.shape)
        for idx in np.ndindex(x.shape):
            args = list(base)
            xp = x.copy(); xp[idx] += np.float32(h); args[gi] = xp
            lp = loss(args, h0)
            xm = x.copy(); xm[idx] -= np.float32(h); args[gi] = xm
            lm = loss(args, h0)
            fd[idx] = (lp - lm) / (2 * h)
        _close(grads[gi], fd, 1e-6, f"d{name} against finite differences")
    fd = np.zeros(h0.shape)
    for idx in np.ndindex(h0.shape):
        hp = h0.copy(); hp[idx] += 1e-6
        hm = h0.copy(); hm[idx] -= 1e-6
        fd[idx] = (loss(base, hp) - loss(base, hm)) / 2e-6
    _close(grads[5], fd, 1e-6, "dh0 against finite differences")


def pin_bwd_single_token(fwd, bwd):
    """One token from a zero state: o = scale b (k.q) v and ht = b k v^T, so
    with u = v.do and w = k^T dht v:
    dq = scale b u k, dk = scale b u q + b dht v, dv = scale b (k.q) do + b dht^T k,
    db = scale (k.q) u + w, dg = 0, dh0 = a (I - b k k^T)(scale q do^T + dht)."""
    rng = _rng(102)
    q, k, v, g, beta, do, _, dht = _bwd_case(rng, 1, 1, 1, 1, 6, 5, 1)
    scale = 1.3
    dq, dk, dv, dg, db, dh0 = bwd(q, k, v, g, beta, do, scale=scale, dht=dht)
    q_, k_, v_, o_ = (x[0, 0, 0].astype(np.float64) for x in (q, k, v, do))
    a, b = math.exp(float(g[0, 0, 0])), float(beta[0, 0, 0])
    D = dht[0, 0]
    u, kq = float(v_ @ o_), float(k_ @ q_)
    _close(dq[0, 0, 0], scale * b * u * k_, 1e-13, "dq")
    _close(dk[0, 0, 0], scale * b * u * q_ + b * (D @ v_), 1e-13, "dk")
    _close(dv[0, 0, 0], scale * b * kq * o_ + b * (D.T @ k_), 1e-13, "dv")
    _close(db[0, 0, 0], scale * kq * u + float(k_ @ D @ v_), 1e-13, "dbeta")
    assert dg[0, 0, 0] == 0.0, "dg from a zero state"
    dM = scale * np.outer(q_, o_) + D
    _close(dh0[0, 0], a * (dM - b * np.outer(k_, k_ @ dM)), 1e-13, "dh0")


def pin_bwd_linear_in_upstream(fwd, bwd):
    """The gradients are linear in the upstream gradients (do, dht) jointly."""
    rng = _rng(103)
    q, k, v, g, beta, do1, h0, dht1 = _bwd_case(rng, 2, 11, 2, 4, 5, 3, 2)
    # upstream values on a 2^-8 grid, so alpha * do1 + do2 is exact in fp32
    do1 = (np.round(do1 * 256) / 256).astype(np.float32)
    do2 = (np.round(rng.standard_normal(do1.shape) * 256) / 256).astype(np.float32)
    dht2 = rng.standard_normal(dht1.shape)
    alpha = 0.5
    g1 = bwd(q, k, v, g, beta, do1, h0=h0, dht=dht1)
    g2 = bwd(q, k, v, g, beta, do2, h0=h0, dht=dht2)
    g3 = bwd(q, k, v, g, beta, (alpha * do1 + do2).astype(np.float32), h0=h0,
             dht=alpha * dht1 + dht2)
    for a_, b_, c_, name in zip(g1, g2, g3, ("dq", "dk", "dv", "dg", "dbeta", "dh0")):
        _close(c_, alpha * a_ + b_, 1e-11, f"{name} linear in the upstream gradient")


def pin_bwd_packed_equals_separate(fwd, bwd):
    """A packed call's gradients equal per-document calls', bitwise."""
    rng = _rng(104)
    lengths = [5, 0, 9, 1]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    q, k, v, g, beta, do, h0, dht = _bwd_case(rng, 1, T, 1, 2, 4, 3, len(lengths))
    packed = bwd(q, k, v, g, beta, do, h0=h0, dht=dht, cu_seqlens=cu)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        if a == b:
            assert np.array_equal(packed[5][n], h0[n] * 0 + dht[n]), "empty document: dh0 = dht"
            continue
        sl = slice(a, b)
        sep = bwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], do[:, sl],
                  h0=h0[n:n + 1], dht=dht[n:n + 1])
        for x, y in zip(packed[:5], sep[:5]):
            assert np.array_equal(x[:, sl], y), f"document {n} differs when packed"
        assert np.array_equal(packed[5][n], sep[5][0]), f"dh0 of document {n}"


def pin_bwd_chunked_route(fwd, bwd):
    """The chunk-parallel reverse mode (numpy, explicit solves; the algebra the
    GPU backward uses) equals the token-by-token reverse mode at several chunk
    sizes, with documents, grouped heads, initial states and a state loss."""
    import oracle
    rng = _rng(105)
    cu = np.array([0, 5, 70, 70, 131])
    q, k, v, g, beta, do, h0, dht = _bwd_case(rng, 1, 131, 2, 4, 8, 6, 4)
    ref = bwd(q, k, v, g, beta, do, scale=0.8, h0=h0, dht=dht, cu_seqlens=cu)
    for C in (1, 3, 8, 64):
        out = oracle.chunked.bwd(q, k, v, g, beta, do, C, scale=0.8, h0=h0, dht=dht,
                                 cu_seqlens=cu)
        for x, y, name in zip(out, ref, ("dq", "dk", "dv", "dg", "dbeta", "dh0")):
            _close(x, y, 1e-12, f"chunked {name} at C={C}")


BWD_PINS = [
    pin_bwd_finite_differences, pin_bwd_single_token, pin_bwd_linear_in_upstream,
    pin_bwd_packed_equals_separate, pin_bwd_chunked_route,
]


# ---------------------------------------------------------------------------
# Input preparation and the decode step (oracle/prep.py).  Each pin takes `P`,
# an object with the functions l2_normalize, logsigmoid, sigmoid and step, and
# `fwd` (the token-by-token C oracle, pinned above), which the step is checked
# against.

def pin_l2_known_rows(P, fwd):
    """Rows whose norms are exact: (3, 4) has norm 5, (1, 1, 1, 1) norm 2."""
    x = np.array([[3.0, 4.0, 0.0, 0.0], [0.0, 0.0, 0.0, -5.0], [1.0, 1.0, 1.0, 1.0],
                  [0.0, 0.0, 0.0, 0.0], [0.0, -2.0, 0.0, 0.0]])
    want = np.array([[0.6, 0.8, 0, 0], [0, 0, 0, -1.0], [0.5] * 4, [0.0] * 4, [0, -1.0, 0, 0]])
    got = P.l2_normalize(x)
    assert np.allclose(got, want, rtol=0, atol=1e-15), f"normalised rows {got}"


def pin_l2_unit_direction_scale(P, fwd):
    """Random rows: unit norm, the same direction (x . x/|x| = |x|), and
    invariance under a positive scale; batched over leading axes."""
    rng = _rng(40)
    x = rng.standard_normal((3, 5, 2, 64))
    n = P.l2_normalize(x)
    assert n.shape == x.shape
    assert np.allclose(np.linalg.norm(n, axis=-1), 1.0, rtol=0, atol=1e-14), "not unit"
    assert np.allclose(np.sum(x * n, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14), \
        "direction changed"
    assert np.allclose(P.l2_normalize(3.7 * x), n, rtol=0, atol=1e-15), "scale changes it"


def pin_gate_functions(P, fwd):
    """Closed forms (logsigmoid(0) = -ln 2, sigmoid(ln 3) = 3/4), the identities
    logsigmoid(x) - logsigmoid(-x) = x and sigmoid(x) + sigmoid(-x) = 1, the
    link exp(logsigmoid) = sigmoid, no overflow at |x| = 800, and scipy's
    expit and log_expit."""
    from scipy.special import expit, log_expit
    assert abs(P.logsigmoid(0.0) + math.log(2.0)) < 1e-16
    assert abs(P.sigmoid(math.log(3.0)) - 0.75) < 1e-16
    x = np.linspace(-30.0, 30.0, 601)
    ls, s = P.logsigmoid(x), P.sigmoid(x)
    assert np.allclose(ls - P.logsigmoid(-x), x, rtol=0, atol=1e-13), "logsigmoid identity"
    assert np.allclose(s + P.sigmoid(-x), 1.0, rtol=0, atol=1e-15), "sigmoid identity"
    assert np.allclose(np.exp(ls), s, rtol=1e-14, atol=0), "exp(logsigmoid) != sigmoid"
    assert np.allclose(ls, log_expit(x), rtol=1e-14, atol=1e-300), "logsigmoid vs scipy"
    assert np.allclose(s, expit(x), rtol=1e-14, atol=1e-300), "sigmoid vs scipy"
    big = np.array([-800.0, 800.0])
    assert np.allclose(P.logsigmoid(big), [-800.0, 0.0], rtol=1e-15, atol=1e-300)
    assert np.array_equal(P.sigmoid(big) > 0.5, [False, True])


def pin_step_hand_worked(P, fwd):
    """dk = dv = 2 by hand: M = [[1, 0], [0, 2]], k = (1, 0), v = (3, 1),
    q = (1, 1), a = 1/2, beta = 1/2, scale 2.  y = M^T k = (1, 0);
    delta = (1/2)((3, 1) - (1/2)(1, 0)) = (1.25, 0.5);
    M' = M/2 + k delta^T = [[1.75, 0.5], [0, 1]]; o = 2 M'^T q = (3.5, 3)."""
    M = np.array([[[[1.0, 0.0], [0.0, 2.0]]]])
    o, new = P.step(np.array([[[1.0, 1.0]]]), np.array([[[1.0, 0.0]]]),
                    np.array([[[3.0, 1.0]]]), np.array([[math.log(0.5)]]),
                    np.array([[0.5]]), M, scale=2.0)
    assert np.allclose(new[0, 0], [[1.75, 0.5], [0.0, 1.0]], rtol=0, atol=1e-15), new[0, 0]
    assert np.allclose(o[0, 0], [3.5, 3.0], rtol=0, atol=1e-15), o[0, 0]
    assert np.array_equal(M[0, 0], [[1.0, 0.0], [0.0, 2.0]]), "the input cache was modified"


def pin_step_chained_equals_token_oracle(P, fwd):
    """Steps chained over T tokens from h0 (grouped heads) give the outputs
    and final states of the token-by-token C oracle over the whole rows."""
    rng = _rng(41)
    B, T, Hqk, Hv, dk, dv = 3, 7, 2, 4, 8, 6
    q, k, v, g, beta = _rand_inputs(rng, B, T, Hqk, Hv, dk, dv)
    h0 = rng.standard_normal((B, Hv, dk, dv)).astype(np.float32)
    o_ref, h_ref = fwd(q, k, v, g, beta, scale=0.8, h0=h0)
    cache = h0.astype(np.float64)
    for t in range(T):
        o, cache = P.step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], cache, scale=0.8)
        _close(o, o_ref[:, t], 1e-13, f"step output at token {t}")
    _close(cache, h_ref, 1e-13, "chained final state")


def pin_step_slots_and_padding(P, fwd):
    """Slots address the cache: a permuted slot list gives each sequence the
    state of its slot, a padding slot (negative or past the end) starts from
    zero and writes nothing, and slots not named keep their state."""
    rng = _rng(42)
    N, Hqk, Hv, dk, dv, S = 4, 2, 2, 4, 3, 6
    q, k, v, g, beta = (x[:, 0] for x in _rand_inputs(rng, N, 1, Hqk, Hv, dk, dv))
    cache = rng.standard_normal((S, Hv, dk, dv))
    slots = np.array([4, -1, 0, S])
    o, new = P.step(q, k, v, g, beta, cache, slots=slots)
    h0 = np.stack([cache[4], np.zeros((Hv, dk, dv)), cache[0], np.zeros((Hv, dk, dv))])
    o_ref, h_ref = P.step(q, k, v, g, beta, h0)
    _close(o, o_ref, 1e-15, "slot outputs")
    _close(new[4], h_ref[0], 1e-15, "slot 4 state")
    _close(new[0], h_ref[2], 1e-15, "slot 0 state")
    for s in (1, 2, 3, 5):
        assert np.array_equal(new[s], cache[s]), f"slot {s} changed"
    # With a zero state the step is closed form: o = beta (q . k) v, M = beta k v^T.
    q1, k1, v1, b1 = (np.asarray(x[1], np.float64) for x in (q, k, v, beta))
    want = b1[:, None] * np.einsum("hd,hd->h", q1, k1)[:, None] * v1
    _close(o[1], want, 1e-14, "zero-state closed form")


def pin_step_options(P, fwd):
    """The options act on the inputs: raw gates of 0 are a = beta = 1/2; rows
    scaled by powers of two normalise back to the given unit rows."""
    rng = _rng(43)
    N, Hqk, Hv, dk, dv = 2, 1, 1, 16, 4
    K = _hadamard(dk)[[3, 9]] / 4.0
    Q = _hadamard(dk)[[5, 12]] / 4.0
    v = rng.standard_normal((N, Hv, dv))
    cache = rng.standard_normal((N, Hv, dk, dv))
    o_ref, h_ref = P.step(Q[:, None], K[:, None], v, np.full((N, Hv), math.log(0.5)),
                          np.full((N, Hv), 0.5), cache)
    o, h = P.step(8.0 * Q[:, None], 0.25 * K[:, None], v, np.zeros((N, Hv)),
                  np.zeros((N, Hv)), cache, use_qk_l2norm=True, gate_activation=True)
    _close(o, o_ref, 1e-15, "options output")
    _close(h, h_ref, 1e-15, "options state")


PREP_PINS = [
    pin_l2_known_rows, pin_l2_unit_direction_scale, pin_gate_functions, pin_step_hand_worked,
    pin_step_chained_equals_token_oracle, pin_step_slots_and_padding, pin_step_options,
]


# ---------------------------------------------------------------------------
# Reverse mode of the preparation (oracle/prep.py).  Same signature as the
# preparation pins above.

def pin_prep_bwd_closed_forms(P, fwd):
    """Values by hand.  x = (3, 4), dy = (1, 0): y = (0.6, 0.8), dy . y = 0.6,
    dx = ((1, 0) - 0.6 (0.6, 0.8)) / 5 = (0.128, -0.096).  logsigmoid'(0) =
    1/2, sigmoid'(0) = 1/4, sigmoid'(ln 3) = (3/4)(1/4) = 3/16,
    logsigmoid'(ln 3) = 1/4.  A zero row has a zero gradient."""
    dx = P.l2_normalize_bwd(np.array([[3.0, 4.0], [0.0, 0.0]]), np.array([[1.0, 0.0], [1.0, 2.0]]))
    assert np.allclose(dx, [[0.128, -0.096], [0.0, 0.0]], rtol=0, atol=1e-16), dx
    assert abs(P.logsigmoid_bwd(0.0, 1.0) - 0.5) < 1e-16
    assert abs(P.sigmoid_bwd(0.0, 1.0) - 0.25) < 1e-16
    assert abs(P.sigmoid_bwd(math.log(3.0), 2.0) - 0.375) < 1e-16
    assert abs(P.logsigmoid_bwd(math.log(3.0), 1.0) - 0.25) < 1e-16


def pin_prep_bwd_invariants(P, fwd):
    """The normalisation's gradient is orthogonal to x (moving along x does not
    change x / |x|), scales as 1 / c under x -> c x, is linear in dy, and a dy
    along x gives zero; sigmoid'(x) = sigmoid'(-x) and logsigmoid'(x) +
    logsigmoid'(-x) = 1."""
    rng = _rng(44)
    x = rng.standard_normal((4, 3, 32))
    dy = rng.standard_normal(x.shape)
    dx = P.l2_normalize_bwd(x, dy)
    assert np.allclose(np.sum(dx * x, axis=-1), 0.0, rtol=0, atol=1e-14), "not orthogonal to x"
    assert np.allclose(P.l2_normalize_bwd(2.5 * x, dy), dx / 2.5, rtol=1e-14, atol=1e-16)
    dy2 = rng.standard_normal(x.shape)
    assert np.allclose(P.l2_normalize_bwd(x, dy + 3.0 * dy2),
                       dx + 3.0 * P.l2_normalize_bwd(x, dy2), rtol=1e-13, atol=1e-14)
    assert np.allclose(P.l2_normalize_bwd(x, 0.7 * x), 0.0, rtol=0, atol=1e-14)
    t = np.linspace(-25.0, 25.0, 501)
    one = np.ones_like(t)
    assert np.allclose(P.sigmoid_bwd(t, one), P.sigmoid_bwd(-t, one), rtol=1e-14, atol=1e-300)
    assert np.allclose(P.logsigmoid_bwd(t, one) + P.logsigmoid_bwd(-t, one), 1.0,
                       rtol=0, atol=1e-15)


def pin_prep_bwd_finite_differences(P, fwd):
    """Each gradient equals the central difference of the forward map it
    reverses (fp64, step 1e-6: truncation error ~1e-12, rounding ~1e-10)."""
    rng = _rng(45)
    x = rng.standard_normal((3, 12))
    dy = rng.standard_normal(x.shape)
    got = P.l2_normalize_bwd(x, dy)
    h = 1e-6
    fd = np.zeros(x.shape)
    for idx in np.ndindex(x.shape):
        xp = x.copy(); xp[idx] += h
        xm = x.copy(); xm[idx] -= h
        fd[idx] = (np.sum(dy * P.l2_normalize(xp)) - np.sum(dy * P.l2_normalize(xm))) / (2 * h)
    _close(got, fd, 1e-8, "l2 normalisation gradient")
    t = np.linspace(-12.0, 12.0, 97)
    w = rng.standard_normal(t.shape)
    for f, b, name in ((P.logsigmoid, P.logsigmoid_bwd, "logsigmoid"),
                       (P.sigmoid, P.sigmoid_bwd, "sigmoid")):
        fd = w * (f(t + h) - f(t - h)) / (2 * h)
        _close(b(t, w), fd, 1e-8, f"{name} gradient")


def pin_prep_bwd_chain_through_forward(P, fwd):
    """The gradient of a forward that normalises q, k and activates raw gates
    in-op, with respect to the raw inputs: the C oracle's reverse mode on the
    prepared inputs, chained through chain_options, equals the central
    difference of the whole composition (raw inputs -> preparation -> forward
    -> loss).  The prepared values are not fp32 numbers, which the C oracle
    takes, so both sides run the chunk-parallel numpy route (pinned to the C
    oracle above) in fp64."""
    from oracle import chunked
    rng = _rng(46)
    B, T, Hqk, Hv, dk, dv = 1, 9, 1, 2, 6, 4
    q = rng.standard_normal((B, T, Hqk, dk)) * 2.0
    k = rng.standard_normal((B, T, Hqk, dk)) * 0.5
    v = rng.standard_normal((B, T, Hv, dv))
    gr = rng.standard_normal((B, T, Hv)) + 2.0
    br = rng.standard_normal((B, T, Hv))
    do = rng.standard_normal((B, T, Hv, dv))
    h0 = rng.standard_normal((B, Hv, dk, dv)) * 0.3
    dht = rng.standard_normal((B, Hv, dk, dv))

    def prepared(q_, k_, g_, b_):
        return P.l2_normalize(q_), P.l2_normalize(k_), P.logsigmoid(g_), P.sigmoid(b_)

    def loss(q_, k_, g_, b_):
        qn, kn, gn, bn = prepared(q_, k_, g_, b_)
        o, ht = chunked.fwd(qn, kn, v, gn, bn, 4, scale=0.9, h0=h0)
        return float(np.sum(do * o) + np.sum(dht * ht))

    qn, kn, gn, bn = prepared(q, k, gr, br)
    dqn, dkn, _, dgn, dbn, _ = chunked.bwd(qn, kn, v, gn, bn, do, 4, scale=0.9, h0=h0, dht=dht)
    got = P.chain_options(q, k, gr, br, dqn, dkn, dgn, dbn, use_qk_l2norm=True,
                          gate_activation=True)
    base = [q, k, gr, br]
    h = 1e-6
    for i, name in enumerate(("q", "k", "g", "beta")):
        fd = np.zeros(base[i].shape)
        for idx in np.ndindex(base[i].shape):
            args = list(base)
            xp = base[i].copy(); xp[idx] += h; args[i] = xp
            lp = loss(*args)
            xm = base[i].copy(); xm[idx] -= h; args[i] = xm
            fd[idx] = (lp - loss(*args)) / (2 * h)
        _close(got[i], fd, 1e-7, f"d{name} through the preparation")


PREP_BWD_PINS = [
    pin_prep_bwd_closed_forms, pin_prep_bwd_invariants, pin_prep_bwd_finite_differences,
    pin_prep_bwd_chain_through_forward,
]
