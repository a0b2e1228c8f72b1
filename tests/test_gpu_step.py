"""Parity of the input preparation, the forward with in-op preparation and the
single-token decode step (HIP, through the C ABI) with the fp64 oracle.

Readings of the pages for the in-op preparation: the forward applies each
row's inverse norm (fp32) where the row enters the chunk equations, so its
normalised rows are never rounded; its oracle takes the fp64 normalisation
rounded to fp32.  The preparation pass stores normalised rows in the input
dtype, so a forward on its output is compared with the oracle on the
bf16-rounded normalisation.  The decode step normalises in fp32 without
rounding and is compared with the unrounded fp64 step.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_chunk_amd as gdn
import gdn_inputs as gi
import oracle
from gpu_util import TOL, rel_l2, to_device
from oracle import prep

pytestmark = pytest.mark.gpu


def _dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 128), ("f32", 64), ("bf16", 96),
                                      ("bf16", 256), ("f32", 256), ("bf16", 200)])
@pytest.mark.parametrize("in_place", [False, True])
def test_prepare_inputs(dtype, dk, in_place):
    seed = 6000 + dk
    d = gi.make_raw(2, 70, 3, 6, dk, 64, dtype, seed, qk_std=3.0)
    d["q"][1, 5, 2] = 0  # a zero row stays zero
    print(f"[gpu prep case] dtype={dtype} dk={dk} in_place={in_place}", flush=True)
    t = to_device(d)
    q0, k0 = _host(t["q"]), _host(t["k"])
    qn, kn, gn, bn = gdn.gdn_prepare_inputs(t["q"], t["k"], t["g"], t["beta"],
                                            use_qk_l2norm=True, gate_activation=True,
                                            in_place=in_place)
    torch.cuda.synchronize()
    if in_place:
        assert qn.data_ptr() == t["q"].data_ptr() and gn.data_ptr() == t["g"].data_ptr()
    else:
        assert np.array_equal(_host(t["q"]), q0) and np.array_equal(_host(t["k"]), k0)
    # bf16: one rounding to nearest (half an ulp, 2^-9) plus the fp32 norm;
    # fp32: a few ulps of the norm.
    rtol = 2.0 ** -8 if dtype == "bf16" else 1e-6
    for name, got, raw in (("q", qn, q0), ("k", kn, k0)):
        want = prep.l2_normalize(raw)
        err = np.abs(_host(got) - want)
        assert np.all(err <= rtol * np.abs(want)), f"{name}: max error {err.max():.3e}"
    assert np.all(_host(qn)[1, 5, 2] == 0)
    for name, got, want in (("g", gn, prep.logsigmoid(d["g"])),
                            ("beta", bn, prep.sigmoid(d["beta"]))):
        err = np.abs(_host(got) - want)
        assert np.all(err <= 2e-6 * np.abs(want)), f"{name}: max error {err.max():.3e}"


def _rounded_to(x64, dtype):
    """fp64 values rounded to the input dtype (the reading of the in-op
    normalisation: its rows are handed to the chunk pass in that dtype)."""
    x32 = np.asarray(x64, np.float64).astype(np.float32)
    return gi.widen(gi.bf16_bits(x32)) if dtype == "bf16" else x32


FUSED_CASES = [
    # dtype, B, T, Hqk, Hv, dk, dv, document lengths (None: B rows)
    ("bf16", 2, 200, 2, 4, 128, 128, None),
    ("bf16", 1, 65, 1, 1, 128, 64, None),
    ("bf16", 2, 130, 1, 2, 64, 128, None),
    ("bf16", 1, 300, 2, 2, 128, 128, [70, 0, 129, 101]),
    ("f32", 1, 100, 2, 2, 64, 64, None),
    ("f32", 1, 150, 1, 2, 128, 128, [1, 85, 64]),
    ("bf16", 2, 100, 1, 2, 256, 128, None),
    ("bf16", 1, 180, 2, 4, 256, 64, [33, 0, 100, 47]),
    ("f32", 1, 70, 1, 1, 256, 64, None),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: f"{c[0]}-T{c[2]}-cu{c[7] is not None}")
def test_fwd_with_in_op_preparation(case):
    dtype, B, T, Hqk, Hv, dk, dv, lengths = case
    seed = 6100 + T + dk
    d = gi.make_raw(B, T, Hqk, Hv, dk, dv, dtype, seed, qk_std=3.0)
    cu = None if lengths is None else gi.cu_from_lengths(lengths)
    h0 = None
    if cu is not None:
        h0 = np.random.default_rng(seed).standard_normal(
            (len(lengths), Hv, dk, dv)).astype(np.float32) * np.float32(0.1)
    print(f"[gpu fused-prep case] {case}", flush=True)
    t = to_device(d)
    q0, g0 = _host(t["q"]), t["g"].cpu().numpy()
    kw = {}
    if cu is not None:
        kw = dict(cu_seqlens=torch.from_numpy(cu).cuda(), cu_seqlens_host=[int(x) for x in cu],
                  initial_state=torch.from_numpy(h0).cuda())
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=0.5,
                              use_qk_l2norm=True, gate_activation=True, **kw)
    # The same call on inputs prepared by the separate pass.
    pq, pk, pg, pb = gdn.gdn_prepare_inputs(t["q"], t["k"], t["g"], t["beta"],
                                            use_qk_l2norm=True, gate_activation=True)
    o2, ht2 = gdn.gdn_chunk_fwd(pq, pk, t["v"], pg, pb, scale=0.5, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(_host(t["q"]), q0) and np.array_equal(t["g"].cpu().numpy(), g0), \
        "the call changed its inputs"
    g = prep.logsigmoid(d["g"]).astype(np.float32)
    beta = prep.sigmoid(d["beta"]).astype(np.float32)
    tol_o, tol_h = TOL[dtype]
    errs = []
    for got_o, got_h, rounding in ((o, ht, "f32"), (o2, ht2, dtype)):
        qn, kn = (_rounded_to(prep.l2_normalize(gi.widen(d[x])), rounding) for x in ("q", "k"))
        ro, rht = oracle.gdn_fwd(qn, kn, gi.widen(d["v"]), g, beta, scale=0.5, h0=h0,
                                 cu_seqlens=cu)
        errs.append((rel_l2(_host(got_o), ro), rel_l2(got_h.cpu().numpy(), rht)))
    print(f"  fused: rel-L2 output {errs[0][0]:.3e}, state {errs[0][1]:.3e}; separate pass: "
          f"{errs[1][0]:.3e}, {errs[1][1]:.3e}", flush=True)
    for eo, eh in errs:
        assert eo <= tol_o and eh <= tol_h


def _step_inputs(d, t_idx):
    """Token t_idx of every row of a generator dict, as device tensors."""
    out = {}
    for name in ("q", "k", "v", "g", "beta"):
        out[name] = _dev(np.ascontiguousarray(d[name][:, t_idx]))
    return out


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("f32", 128, 128), ("bf16", 128, 64),
                                         ("f32", 256, 256), ("bf16", 256, 128)])
def test_step_chain_matches_token_oracle(dtype, dk, dv):
    """40 decode steps from an initial state against the token-by-token
    oracle over the whole rows."""
    seed = 6200 + dk + dv
    d = gi.make(3, 40, 1, 2, dk, dv, dtype, seed, h0_std=0.5)
    print(f"[gpu step chain] dtype={dtype} dk={dk} dv={dv}", flush=True)
    cache = torch.from_numpy(d["h0"]).cuda()
    outs = []
    for t_idx in range(d["T"]):
        s = _step_inputs(d, t_idx)
        outs.append(_host(gdn.gdn_recurrent_step(s["q"], s["k"], s["v"], s["g"], s["beta"],
                                                 cache, scale=0.7)))
    torch.cuda.synchronize()
    o = np.stack(outs, axis=1)
    ro, rht = oracle.gdn_fwd(*(gi.widen(d[x]) for x in ("q", "k", "v")), d["g"], d["beta"],
                             scale=0.7, h0=d["h0"].astype(np.float64))
    eo, eh = rel_l2(o, ro), rel_l2(cache.cpu().numpy(), rht)
    print(f"  rel-L2 output {eo:.3e}, state {eh:.3e}", flush=True)
    tol_o, tol_h = TOL[dtype] if dtype == "f32" else (TOL["bf16"][0], TOL["f32"][1])
    assert eo <= tol_o and eh <= tol_h


def test_decode_after_prefill():
    """A chunked prefill's final states seed the cache; 24 decode steps then
    continue the rows (packed-free, B = 2)."""
    T0, S = 100, 24
    d = gi.make(2, T0 + S, 2, 2, 128, 128, "bf16", 6300, h0_std=0.1)
    print("[gpu prefill+decode]", flush=True)
    pre = {x: _dev(np.ascontiguousarray(d[x][:, :T0])) for x in ("q", "k", "v", "g", "beta")}
    _, cache = gdn.gdn_chunk_fwd(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"],
                                 initial_state=torch.from_numpy(d["h0"]).cuda())
    outs = []
    for t_idx in range(T0, T0 + S):
        s = _step_inputs(d, t_idx)
        outs.append(_host(gdn.gdn_recurrent_step(s["q"], s["k"], s["v"], s["g"], s["beta"],
                                                 cache)))
    torch.cuda.synchronize()
    ro, rht = oracle.gdn_fwd(*(gi.widen(d[x]) for x in ("q", "k", "v")), d["g"], d["beta"],
                             h0=d["h0"].astype(np.float64))
    eo = rel_l2(np.stack(outs, axis=1), ro[:, T0:])
    eh = rel_l2(cache.cpu().numpy(), rht)
    print(f"  rel-L2 decode output {eo:.3e}, state {eh:.3e}", flush=True)
    tol_o, tol_h = TOL["bf16"]
    assert eo <= tol_o and eh <= tol_h


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_slots_padding_options(dtype):
    """Cache slots (permuted, with padding past the end and negative), grouped
    heads, in-op L2 norm and gate activations, against the fp64 step."""
    N, Hqk, Hv, dk, dv, S = 6, 2, 4, 64, 128, 5
    seed = 6400 + (dtype == "f32")
    d = gi.make_raw(N, 1, Hqk, Hv, dk, dv, dtype, seed, qk_std=2.0)
    cache0 = np.random.default_rng(seed).standard_normal((S, Hv, dk, dv)).astype(np.float32)
    slots = np.array([3, -1, 0, 5, 1, 7], np.int32)
    print(f"[gpu step slots] dtype={dtype}", flush=True)
    s = _step_inputs(d, 0)
    cache = torch.from_numpy(cache0).cuda()
    o = gdn.gdn_recurrent_step(s["q"], s["k"], s["v"], s["g"], s["beta"], cache, scale=0.9,
                               slots=torch.from_numpy(slots).cuda(), use_qk_l2norm=True,
                               gate_activation=True)
    torch.cuda.synchronize()
    ro, rcache = prep.step(*(gi.widen(d[x][:, 0]) for x in ("q", "k", "v")), d["g"][:, 0],
                           d["beta"][:, 0], cache0, slots=slots, scale=0.9,
                           use_qk_l2norm=True, gate_activation=True)
    got = cache.cpu().numpy()
    for untouched in (2, 4):
        assert np.array_equal(got[untouched], cache0[untouched]), f"slot {untouched} changed"
    eo, eh = rel_l2(_host(o), ro), rel_l2(got, rcache)
    print(f"  rel-L2 output {eo:.3e}, cache {eh:.3e}", flush=True)
    assert eo <= TOL[dtype][0] and eh <= TOL["f32"][1]


def test_step_decode_workload_full_size():
    """The decode workload: 256 sequences x 16 heads, dk = dv = 128, bf16,
    a 256-slot fp32 cache (256 MiB), every output and state compared."""
    d = gi.make_config("decode_bf16")
    print("[gpu step] decode_bf16 full size", flush=True)
    s = _step_inputs(d, 0)
    cache = torch.from_numpy(d["h0"]).cuda()
    o = gdn.gdn_recurrent_step(s["q"], s["k"], s["v"], s["g"], s["beta"], cache)
    torch.cuda.synchronize()
    ro, rcache = prep.step(*(gi.widen(d[x][:, 0]) for x in ("q", "k", "v")), d["g"][:, 0],
                           d["beta"][:, 0], d["h0"])
    eo, eh = rel_l2(_host(o), ro), rel_l2(cache.cpu().numpy(), rcache)
    print(f"  rel-L2 output {eo:.3e}, cache {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"][0] and eh <= TOL["f32"][1]


def test_step_empty_batch():
    z = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    gb = torch.zeros((0, 2), device="cuda")
    cache = torch.ones((1, 2, 128, 64), device="cuda")
    o = gdn.gdn_recurrent_step(z, z, v, gb, gb, cache)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 64) and bool(torch.all(cache == 1))
