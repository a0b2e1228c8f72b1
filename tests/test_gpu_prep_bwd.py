"""Gradients through the in-op preparation on the GPU, against the oracle.

* gdn_prepare_inputs_bwd (the reverse of the row normalisation and the gate
  activations) against oracle/prep.py's fp64 derivatives, row by row, for
  bf16 and fp32 rows on the vector path (16-byte pieces) and the one-wave
  path, zero rows and extreme gate values included.
* gdn_chunk_bwd with use_qk_l2norm / gate_activation on raw inputs against the
  fp64 chain: the oracle's chunk-parallel reverse mode (pinned to the
  token-by-token one) on the exactly prepared inputs, then
  oracle.prep.chain_options.  Also bitwise equal to the three calls made by
  hand (prepare, backward on the prepared copies, prepare_bwd).
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gpu_util import rel_l2, to_device
from oracle import chunked, prep

pytestmark = pytest.mark.gpu

TOL_BWD = 1e-2   # as for the plain backward: bf16 inputs and bf16 dq, dk, dv


def _dev_rows(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def _host(x):
    return x.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("bf16", 64), ("bf16", 256),
                                      ("bf16", 40), ("f32", 128), ("f32", 256), ("f32", 7)])
def test_prepare_inputs_bwd_matches_oracle(dtype, dk):
    """Rows of random norm (a few zero rows), upstream gradients ~ N(0, 1), raw
    gates ~ N(0, 3) with +-30 at the ends.  Per row, relative L2 within 4e-3
    for bf16 results (their rounding is 2^-9) and 2e-6 for fp32; gates within
    2e-6 elementwise.  In place gives the same bits."""
    import gated_deltanet_chunked_chunk_amd as gdn
    seed = 7100 + dk + (0 if dtype == "bf16" else 1)
    print(f"[gpu prep bwd] dtype={dtype} dk={dk} seed={seed}", flush=True)
    rows = 1000
    d = gi.make_raw(1, rows, 1, 1, dk, 8, dtype, seed, qk_std=3.0)
    up = gi.make_raw(1, rows, 1, 1, dk, 8, dtype, seed + 50)
    q, k = d["q"].reshape(rows, dk), d["k"].reshape(rows, dk)
    dq, dk_ = up["q"].reshape(rows, dk), up["k"].reshape(rows, dk)
    q[[3, 500]] = 0
    k[[999]] = 0
    g = np.ascontiguousarray(d["g"].reshape(rows) * 3.0)
    b = np.ascontiguousarray(d["beta"].reshape(rows) * 3.0)
    g[0], g[-1], b[0], b[-1] = -30.0, 30.0, 30.0, -30.0
    dg, db = up["g"].reshape(rows), up["beta"].reshape(rows)
    t = [_dev_rows(np.ascontiguousarray(x)) for x in (q, k, dq, dk_)]
    tg = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (g, b, dg, db)]
    out = gdn.gdn_prepare_inputs_bwd(*t[:2], *tg[:2], t[2], t[3], tg[2], tg[3],
                                     use_qk_l2norm=True, gate_activation=True)
    torch.cuda.synchronize()
    got = [_host(x) for x in out]
    w = gi.widen
    ref = [prep.l2_normalize_bwd(w(q), w(dq)), prep.l2_normalize_bwd(w(k), w(dk_)),
           prep.logsigmoid_bwd(g, dg), prep.sigmoid_bwd(b, db)]
    tol = 4e-3 if dtype == "bf16" else 2e-6
    for name, x, y in zip(("dq", "dk"), got[:2], ref[:2]):
        assert np.all(np.isfinite(x)), name
        for r in range(rows):
            e = rel_l2(x[r], y[r])
            assert e <= tol, f"{name} row {r}: rel-L2 {e:.3e} > {tol}"
    assert not got[0][[3, 500]].any() and not got[1][999].any(), "zero rows get zero gradients"
    for name, x, y in zip(("dg", "dbeta"), got[2:], ref[2:]):
        err = np.abs(x - y) / np.maximum(np.abs(y), 1e-30)
        assert err.max() <= 2e-6, f"{name}: worst relative error {err.max():.3e}"
    # in place: the gradient buffers are overwritten with the same bits
    ip = [x.clone() for x in (t[2], t[3], tg[2], tg[3])]
    res = gdn.gdn_prepare_inputs_bwd(*t[:2], *tg[:2], *ip, use_qk_l2norm=True,
                                     gate_activation=True, in_place=True)
    torch.cuda.synchronize()
    for a, b_, c in zip(res, ip, out):
        assert a.data_ptr() == b_.data_ptr()
        assert torch.equal(a, c), "in place differs"


def _raw_case(B, T, Hqk, Hv, dk, dv, seed, lengths=None, l2=True, gate=True):
    # Rows the call normalises get norms near 2 sqrt(dk); rows it does not get
    # norms near 1, as the recurrence needs (beta |k|^2 < 2).  Gates the call
    # does not activate arrive activated (g <= 0, 0 < beta < 1).
    d = gi.make_raw(B, T, Hqk, Hv, dk, dv, "bf16", seed,
                    qk_std=2.0 if l2 else 1.0 / np.sqrt(dk))
    if not gate:
        zg, zb = d["g"].astype(np.float64), d["beta"].astype(np.float64)
        d["g"] = (-np.logaddexp(0.0, -zg)).astype(np.float32)
        d["beta"] = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    rng = np.random.default_rng(seed)
    if lengths is not None:
        d["cu_seqlens"] = gi.cu_from_lengths(lengths)
        d["N"] = len(lengths)
    d["h0"] = (rng.standard_normal((d["N"], Hv, dk, dv)) * 0.1).astype(np.float32)
    return d


def _oracle_chain(d, do, dht, scale, l2, gate):
    """fp64: exact preparation, the chunk-parallel oracle reverse mode on the
    prepared inputs, the chain through the preparation."""
    q, k, v = (gi.widen(d[x]) for x in ("q", "k", "v"))
    g, b = d["g"].astype(np.float64), d["beta"].astype(np.float64)
    qn, kn = (prep.l2_normalize(q), prep.l2_normalize(k)) if l2 else (q, k)
    gn, bn = (prep.logsigmoid(g), prep.sigmoid(b)) if gate else (g, b)
    dq, dk, dv, dg, db, dh0 = chunked.bwd(qn, kn, v, gn, bn, gi.widen(do), 64, scale=scale,
                                          h0=d["h0"].astype(np.float64),
                                          dht=dht.astype(np.float64),
                                          cu_seqlens=d["cu_seqlens"])
    dq, dk, dg, db = prep.chain_options(q, k, g, b, dq, dk, dg, db, use_qk_l2norm=l2,
                                        gate_activation=gate)
    return dq, dk, dv, dg, db, dh0


OPTION_CASES = [
    # (label, B, T, Hqk, Hv, dk, dv, lengths, l2, gate)
    ("both, grouped heads", 2, 130, 1, 2, 128, 128, None, True, True),
    ("l2 only, dk64, packed", 1, 200, 2, 2, 64, 64, [70, 0, 129, 1], True, False),
    ("gates only, dv256", 1, 150, 1, 1, 128, 256, None, False, True),
    ("both, dk64, ragged", 2, 65, 2, 4, 64, 128, None, True, True),
    ("both, dk256, packed", 1, 90, 1, 2, 256, 64, [33, 0, 57], True, True),
]


@pytest.mark.parametrize("case", OPTION_CASES, ids=[c[0] for c in OPTION_CASES])
def test_bwd_with_options_against_oracle(case):
    import gated_deltanet_chunked_chunk_amd as gdn
    label, B, T, Hqk, Hv, dk, dv, lengths, l2, gate = case
    seed = 7300 + T + dk
    d = _raw_case(B, T, Hqk, Hv, dk, dv, seed, lengths, l2, gate)
    do, dht = gi.make_upstream(d, seed)
    print(f"[gpu bwd options] {label} B={B} T={T} Hqk={Hqk} Hv={Hv} dk={dk} dv={dv} "
          f"seed={seed}", flush=True)
    t = to_device(d)
    do_t = _dev_rows(do)
    dht_t = torch.from_numpy(dht).cuda()
    kw = dict(dht=dht_t, scale=0.8, initial_state=t["h0"], cu_seqlens=t["cu"],
              cu_seqlens_host=t["cu_host"])
    got = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], do_t,
                            use_qk_l2norm=l2, gate_activation=gate, **kw)
    torch.cuda.synchronize()
    ref = _oracle_chain(d, do, dht, 0.8, l2, gate)
    errs = {}
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, ref):
        x = _host(x)
        assert np.all(np.isfinite(x)), name
        errs[name] = rel_l2(x, y)
    print("  rel-L2 " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for name, e in errs.items():
        assert e <= TOL_BWD, f"{name} rel-L2 {e:.3e} > {TOL_BWD}"

    # The same three steps by hand give the same bits.
    qn, kn, gn, bn = gdn.gdn_prepare_inputs(t["q"], t["k"], t["g"], t["beta"],
                                            use_qk_l2norm=l2, gate_activation=gate)
    mid = gdn.gdn_chunk_bwd(qn, kn, t["v"], gn, bn, do_t, **kw)
    dq, dk_, dg, db = gdn.gdn_prepare_inputs_bwd(t["q"], t["k"], t["g"], t["beta"], mid[0],
                                                 mid[1], mid[3], mid[4], use_qk_l2norm=l2,
                                                 gate_activation=gate)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got,
                          (dq, dk_, mid[2], dg, db, mid[5])):
        assert torch.equal(a, b), f"{name}: the fused call differs from the three calls"


def test_bwd_with_options_matches_forward_gradient_direction():
    """With q normalised in-op, moving a raw q row along itself does not change
    the output, so every dq row is orthogonal to its raw q row (up to the
    bf16 rounding of dq): |dq . q| <= 1e-2 |dq| |q| for every row."""
    import gated_deltanet_chunked_chunk_amd as gdn
    d = _raw_case(1, 256, 2, 2, 128, 128, 7400)
    do, dht = gi.make_upstream(d, 7400)
    t = to_device(d)
    got = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], _dev_rows(do),
                            dht=torch.from_numpy(dht).cuda(), initial_state=t["h0"],
                            use_qk_l2norm=True, gate_activation=True)
    torch.cuda.synchronize()
    for name, x, gx in (("q", d["q"], got[0]), ("k", d["k"], got[1])):
        x = gi.widen(x).reshape(-1, 128)
        gx = _host(gx).reshape(-1, 128)
        dots = np.abs(np.sum(x * gx, axis=1))
        bound = 1e-2 * np.linalg.norm(x, axis=1) * np.linalg.norm(gx, axis=1) + 1e-30
        assert np.all(dots <= bound), f"d{name} not orthogonal to the raw {name} rows"
