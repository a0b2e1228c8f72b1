"""Parity over seeded random configurations (forward and backward) with the
fp64 oracle: head dimensions, grouped-head ratios, ragged and packed lengths
(with empty documents), initial states, scales and the in-op options drawn
together, so that combinations no hand-written case names are exercised.
The configurations are fixed by the seed; each prints before it runs."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from oracle import prep
from gpu_util import TOL, rel_l2, to_device

pytestmark = pytest.mark.gpu


def _fwd_configs(n=40, seed=7100):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        dk = int(rng.choice([64, 128, 256]))
        dv = int(rng.choice([64, 128, 256]))
        G = int(rng.choice([1, 2, 4]))
        Hqk = int(rng.integers(1, 3))
        packed = rng.random() < 0.4
        if packed:
            lengths = [int(x) for x in rng.integers(0, 160, size=int(rng.integers(1, 5)))]
            if sum(lengths) == 0:
                lengths[0] = 1
            B, T = 1, sum(lengths)
        else:
            lengths, B, T = None, int(rng.integers(1, 3)), int(rng.integers(1, 300))
        out.append(dict(i=i, dtype=dtype, dk=dk, dv=dv, Hqk=Hqk, Hv=Hqk * G, B=B, T=T,
                        lengths=lengths, h0=rng.random() < 0.5,
                        scale=float(rng.choice([1.0, 0.5, 0.125])),
                        l2=rng.random() < 0.3, gate=rng.random() < 0.3,
                        seed=int(seed + 10 * i)))
    return out


FWD = _fwd_configs()


@pytest.mark.parametrize("c", FWD, ids=lambda c: f"{c['i']}-{c['dtype']}-k{c['dk']}-v{c['dv']}")
def test_forward_random_configuration(c):
    import gated_deltanet_chunked_chunk_amd as gdn
    print(f"[gpu random fwd] {c}", flush=True)
    cu = None if c["lengths"] is None else gi.cu_from_lengths(c["lengths"])
    N = c["B"] if cu is None else len(c["lengths"])
    d = gi.make(c["B"], c["T"], c["Hqk"], c["Hv"], c["dk"], c["dv"], c["dtype"], c["seed"],
                cu_seqlens=cu)
    # Each option's inputs are raw only when the option is on: q, k rows off
    # unit length (each row scaled by a factor in [0.5, 3)) for the in-op
    # L2 norm; raw N(0, 1) gate values for the gate activations.
    raw = gi.make_raw(c["B"], c["T"], c["Hqk"], c["Hv"], c["dk"], c["dv"], c["dtype"],
                      c["seed"] + 5)
    if c["l2"]:
        rs = np.random.default_rng(c["seed"] + 2)
        for x in ("q", "k"):
            f = gi.widen(d[x]) * rs.uniform(0.5, 3.0, size=d[x].shape[:-1] + (1,)).astype(np.float32)
            d[x] = gi.bf16_bits(f) if c["dtype"] == "bf16" else f.astype(np.float32)
    if c["gate"]:
        d["g"], d["beta"] = raw["g"], raw["beta"]
    h0 = None
    if c["h0"]:
        h0 = (np.random.default_rng(c["seed"] + 1).standard_normal(
            (N, c["Hv"], c["dk"], c["dv"])) * 0.1).astype(np.float32)
    t = to_device(d)
    kw = dict(scale=c["scale"], use_qk_l2norm=c["l2"], gate_activation=c["gate"])
    if cu is not None:
        kw.update(cu_seqlens=t["cu"], cu_seqlens_host=t["cu_host"])
    if h0 is not None:
        kw["initial_state"] = torch.from_numpy(h0).cuda()
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], **kw)
    torch.cuda.synchronize()
    q, k = gi.widen(d["q"]), gi.widen(d["k"])
    g, beta = d["g"], d["beta"]
    if c["l2"]:  # the fused normalisation applies its fp32 factors to the rows
        q, k = (prep.l2_normalize(x).astype(np.float32) for x in (q, k))
    if c["gate"]:
        g, beta = prep.logsigmoid(g).astype(np.float32), prep.sigmoid(beta).astype(np.float32)
    ro, rht = oracle.gdn_fwd(q, k, gi.widen(d["v"]), g, beta, scale=c["scale"],
                             h0=None if h0 is None else h0.astype(np.float64), cu_seqlens=cu)
    eo = rel_l2(o.float().cpu().numpy(), ro)
    eh = rel_l2(ht.cpu().numpy(), rht)
    tol_o, tol_h = TOL[c["dtype"]]
    print(f"  rel-L2 output {eo:.3e}, state {eh:.3e}", flush=True)
    assert np.all(np.isfinite(o.float().cpu().numpy()))
    assert eo <= tol_o and eh <= tol_h


def _bwd_configs(n=16, seed=7600):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dk = int(rng.choice([64, 128]))
        dv = int(rng.choice([64, 128, 256]))
        G = int(rng.choice([1, 2, 4]))
        Hqk = int(rng.integers(1, 3))
        packed = rng.random() < 0.4
        if packed:
            lengths = [int(x) for x in rng.integers(0, 140, size=int(rng.integers(1, 4)))]
            if sum(lengths) == 0:
                lengths[0] = 1
            B, T = 1, sum(lengths)
        else:
            lengths, B, T = None, int(rng.integers(1, 3)), int(rng.integers(1, 260))
        out.append(dict(i=i, dk=dk, dv=dv, Hqk=Hqk, Hv=Hqk * G, B=B, T=T, lengths=lengths,
                        h0=rng.random() < 0.5, dht=rng.random() < 0.7,
                        scale=float(rng.choice([1.0, 0.5])), seed=int(seed + 10 * i)))
    return out


BWD = _bwd_configs()


@pytest.mark.parametrize("c", BWD, ids=lambda c: f"{c['i']}-k{c['dk']}-v{c['dv']}")
def test_backward_random_configuration(c):
    import gated_deltanet_chunked_chunk_amd as gdn
    print(f"[gpu random bwd] {c}", flush=True)
    cu = None if c["lengths"] is None else gi.cu_from_lengths(c["lengths"])
    d = gi.make(c["B"], c["T"], c["Hqk"], c["Hv"], c["dk"], c["dv"], "bf16", c["seed"],
                h0_std=0.1 if c["h0"] else None, cu_seqlens=cu)
    do, dht = gi.make_upstream(d, c["seed"])
    if not c["dht"]:
        dht = None
    t = to_device(d)
    do_t = torch.from_numpy(do.view(np.int16)).cuda().view(torch.bfloat16)
    got = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], do_t,
                            dht=None if dht is None else torch.from_numpy(dht).cuda(),
                            scale=c["scale"], initial_state=t["h0"], cu_seqlens=t["cu"],
                            cu_seqlens_host=t["cu_host"])
    torch.cuda.synchronize()
    ref = oracle.gdn_bwd(gi.widen(d["q"]), gi.widen(d["k"]), gi.widen(d["v"]), d["g"], d["beta"],
                         gi.widen(do), scale=c["scale"],
                         h0=None if d["h0"] is None else d["h0"].astype(np.float64),
                         dht=None if dht is None else dht.astype(np.float64), cu_seqlens=cu)
    errs = [rel_l2(x.float().cpu().numpy(), r) for x, r in zip(got, ref)]
    print("  rel-L2 " + ", ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs[:5]) <= 1e-2
    assert errs[5] <= 1e-3, "dh0: a state gradient, held to the state tolerance"
