"""CPU oracle for the gated delta rule, forward and reverse mode.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library and imports nothing from it.

Two independent routes to the same fp64 result:
  * gdn_fwd   -- the token-by-token recurrence in plain C (gdn_oracle.c),
                 threaded over independent (sequence, head, column block) units;
  * gdn_bwd   -- its reverse mode, token by token in plain C, threaded over
                 (sequence, head) units;
  * chunked   -- the chunk-parallel algebra in numpy (chunked.py).
And beside them (prep.py): the in-op L2 normalisation, the gate activations
and the single-token decode step over a cache of states, in fp64 numpy.

Every function here is pinned by the CPU tests (closed forms, invariants,
exact rational brute force, and the two routes against each other).
"""
import ctypes
import os

import numpy as np

from . import chunked  # noqa: F401  (re-exported for tests)
from . import prep  # noqa: F401  (re-exported for tests)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load(path=None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    f = lib.gdn_oracle_fwd
    f.restype = ctypes.c_int
    P = ctypes.c_void_p
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, ctypes.c_double,
                  P, P, ctypes.c_int64, P, P, ctypes.c_int32]
    f = lib.gdn_oracle_bwd
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, ctypes.c_double,
                  P, P, P, ctypes.c_int64, P, P, P, P, P, P, ctypes.c_int32]
    return lib


def default_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f32(x):
    """Exact fp32 copy.  bf16 and fp32 input values are fp32-representable;
    a value that is not would silently round, so that is refused."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    if np.asarray(x).dtype not in (np.float32,):
        back = a.astype(np.float64)
        if not np.array_equal(back, np.asarray(x, dtype=np.float64), equal_nan=True):
            raise ValueError("oracle inputs must be exactly representable in fp32")
    return a


def gdn_fwd(q, k, v, g, beta, scale=1.0, h0=None, cu_seqlens=None, nthreads=None,
            lib_path=None):
    """Token-by-token fp64 forward.

    q, k: [B, T, Hqk, dk]; v: [B, T, Hv, dv]; g (natural-log decay), beta:
    [B, T, Hv]; h0: [N, Hv, dk, dv] or None (zero state); cu_seqlens: [N + 1]
    token offsets into the single row of a packed batch (B must be 1), or None
    (then sequence n is batch row n and N = B).  Returns (o [B, T, Hv, dv],
    ht [N, Hv, dk, dv]), both fp64.  `lib_path` loads another build of the
    same C source (the mutation tests use it)."""
    lib = _load(lib_path)
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, Hv) \
            or beta.shape != (B, T, Hv):
        raise ValueError("shape mismatch")
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = cu.shape[0] - 1
        cu_p = cu.ctypes.data
    else:
        cu = None
        N = B
        cu_p = None
    if h0 is not None:
        h0 = np.ascontiguousarray(h0, dtype=np.float64)
        if h0.shape != (N, Hv, dk, dv):
            raise ValueError("h0 shape mismatch")
    o = np.zeros((B, T, Hv, dv), dtype=np.float64)
    ht = np.zeros((N, Hv, dk, dv), dtype=np.float64)
    rc = lib.gdn_oracle_fwd(B, T, Hqk, Hv, dk, dv, q.ctypes.data, k.ctypes.data,
                            v.ctypes.data, g.ctypes.data, beta.ctypes.data, float(scale),
                            None if h0 is None else h0.ctypes.data, cu_p, N,
                            o.ctypes.data, ht.ctypes.data,
                            int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_fwd failed with code {rc}")
    return o, ht


def gdn_bwd(q, k, v, g, beta, do, scale=1.0, h0=None, dht=None, cu_seqlens=None,
            nthreads=None, lib_path=None):
    """Token-by-token fp64 reverse mode: the gradients of
    L = sum(do * o) + sum(dht * ht) for the forward of `gdn_fwd` with the same
    arguments.  do: [B, T, Hv, dv]; dht: [N, Hv, dk, dv] or None.  Returns
    (dq, dk [B, T, Hqk, dk], dv [B, T, Hv, dv], dg, dbeta [B, T, Hv],
    dh0 [N, Hv, dk, dv]), all fp64."""
    lib = _load(lib_path)
    q, k, v, g, beta, do = (_f32(x) for x in (q, k, v, g, beta, do))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, Hv) \
            or beta.shape != (B, T, Hv) or do.shape != v.shape:
        raise ValueError("shape mismatch")
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = cu.shape[0] - 1
        cu_p = cu.ctypes.data
    else:
        cu = None
        N = B
        cu_p = None
    for name, x in (("h0", h0), ("dht", dht)):
        if x is not None and np.shape(x) != (N, Hv, dk, dv):
            raise ValueError(f"{name} shape mismatch")
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    dht = None if dht is None else np.ascontiguousarray(dht, dtype=np.float64)
    dq = np.zeros((B, T, Hqk, dk), dtype=np.float64)
    dk_ = np.zeros((B, T, Hqk, dk), dtype=np.float64)
    dv_ = np.zeros((B, T, Hv, dv), dtype=np.float64)
    dg = np.zeros((B, T, Hv), dtype=np.float64)
    dbeta = np.zeros((B, T, Hv), dtype=np.float64)
    dh0 = np.zeros((N, Hv, dk, dv), dtype=np.float64)
    rc = lib.gdn_oracle_bwd(B, T, Hqk, Hv, dk, dv, q.ctypes.data, k.ctypes.data,
                            v.ctypes.data, g.ctypes.data, beta.ctypes.data, do.ctypes.data,
                            float(scale), None if h0 is None else h0.ctypes.data,
                            None if dht is None else dht.ctypes.data, cu_p, N,
                            dq.ctypes.data, dk_.ctypes.data, dv_.ctypes.data, dg.ctypes.data,
                            dbeta.ctypes.data, dh0.ctypes.data,
                            int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_bwd failed with code {rc}")
    return dq, dk_, dv_, dg, dbeta, dh0
