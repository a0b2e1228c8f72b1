"""Helpers for the GPU tests: move generator inputs to the device, run the HIP
path through the binding, and compare with the oracle."""
import numpy as np
import torch

import gated_deltanet_chunked_chunk_amd as gdn
import gdn_inputs as gi
import oracle

# Tolerances on relative L2 error against the fp64 oracle (whole tensor):
# bf16 inputs: output <= 1e-2, final state <= 1e-3; fp32 inputs: 1e-5 / 1e-6.
TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-5, 1e-6)}


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((x - ref).ravel()) / (den if den > 0 else 1.0))


def to_device(d, dev="cuda"):
    """Device tensors for a generator dict (bf16 bits become bf16 tensors)."""
    out = {}
    for name in ("q", "k", "v"):
        x = d[name]
        if x.dtype == np.uint16:
            out[name] = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            out[name] = torch.from_numpy(x).to(dev)
    out["g"] = torch.from_numpy(d["g"]).to(dev)
    out["beta"] = torch.from_numpy(d["beta"]).to(dev)
    out["h0"] = None if d["h0"] is None else torch.from_numpy(d["h0"]).to(dev)
    cu = d["cu_seqlens"]
    out["cu"] = None if cu is None else torch.from_numpy(cu).to(dev)
    out["cu_host"] = None if cu is None else [int(x) for x in cu]
    return out


def run_gpu(d, scale=1.0, dev="cuda", host_cu=True):
    t = to_device(d, dev)
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=scale,
                              initial_state=t["h0"], cu_seqlens=t["cu"],
                              cu_seqlens_host=t["cu_host"] if host_cu else None)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


def run_oracle(d, scale=1.0):
    q, k, v = (gi.widen(d[x]) for x in ("q", "k", "v"))
    h0 = None if d["h0"] is None else d["h0"].astype(np.float64)
    return oracle.gdn_fwd(q, k, v, d["g"], d["beta"], scale=scale, h0=h0,
                          cu_seqlens=d["cu_seqlens"])


def per_unit_max(o, ro, ht, rht, cu):
    """The largest relative L2 error over (sequence, value head) units: the
    output rows of each document (or batch row) and head, and each final
    state.  Returns (output max, its unit, state max, its unit)."""
    B, T, Hv = o.shape[:3]
    spans = ([(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)] if cu is not None
             else [(b, 0, T) for b in range(B)])
    wo, uo = 0.0, None
    for n, (b, t0, t1) in enumerate(spans):
        if t1 <= t0:
            continue
        for j in range(Hv):
            e = rel_l2(o[b, t0:t1, j], ro[b, t0:t1, j])
            if e > wo:
                wo, uo = e, (n, j)
    wh, uh = 0.0, None
    for n in range(ht.shape[0]):
        for j in range(Hv):
            e = rel_l2(ht[n, j], rht[n, j])
            if e > wh:
                wh, uh = e, (n, j)
    return wo, uo, wh, uh


def check(d, scale=1.0, label=""):
    """Run both sides, assert the tolerances on the whole tensors and on every
    (sequence, value head) unit, return the two whole-tensor errors."""
    print(f"[gpu case] {label} B={d['B']} T={d['T']} Hqk={d['Hqk']} Hv={d['Hv']} "
          f"dk={d['dk']} dv={d['dv']} dtype={d['dtype']} N={d['N']}", flush=True)
    o, ht = run_gpu(d, scale)
    ro, rht = run_oracle(d, scale)
    eo, eh = rel_l2(o, ro), rel_l2(ht, rht)
    tol_o, tol_h = TOL[d["dtype"]]
    wo, uo, wh, uh = per_unit_max(o, ro, ht, rht, d["cu_seqlens"])
    print(f"  rel-L2 output {eo:.3e} (tol {tol_o:.0e}), state {eh:.3e} (tol {tol_h:.0e}); "
          f"worst (sequence, head): output {wo:.3e} at {uo}, state {wh:.3e} at {uh}",
          flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    assert eo <= tol_o, f"output rel-L2 {eo:.3e} > {tol_o}"
    assert eh <= tol_h, f"state rel-L2 {eh:.3e} > {tol_h}"
    assert wo <= tol_o, f"output rel-L2 {wo:.3e} > {tol_o} for (sequence, head) {uo}"
    assert wh <= tol_h, f"state rel-L2 {wh:.3e} > {tol_h} for (sequence, head) {uh}"
    return eo, eh
