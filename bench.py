"""Benchmark of gdn_chunk_fwd on one MI355X.

A step is one forward call over the headline workload: B=8 rows of T=2048
tokens, H=16 heads, dk=dv=128, bf16 q/k/v, fp32 gates, zero initial state,
output and fp32 final state (synthetic inputs, seeded; the recipe is in
gdn_inputs.py).  Inputs are resident in HBM before timing starts.

Prints one JSON line with the throughput (tokens/s), the roofline of the
kernel (HBM-bound: algorithmic bytes per launch over the measured launch
time, against the 8 TB/s HBM3E peak), and the CPU oracle timed on this host.
Further entries of the same line time the other calls on their own
workloads: the backward (d = 128 and d = 64, the latter with its forward),
the preparation pass and the fused preparation, the decode step, head
dimension 256, the long rows with and without the piece scan, the packed
workload with grouped heads, and the tiny fp32 workload; each is checked
against the oracle on a sample.  Before the warm-up steps the step runs back
to back, untimed, for --settle-ms (clocks ramp up under load); the timed
region is exactly --steps steps.  Everything else goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0
WORKLOAD = "headline_bf16"
KERNEL_NAME = "gdn_fwd_bf16<false, 0, 128>"
KERNEL_SOURCES = ["gated_deltanet_chunked_chunk_amd/csrc/gdn_fwd_bf16.hip"]
BWD_KERNEL_SOURCES = KERNEL_SOURCES + ["gated_deltanet_chunked_chunk_amd/csrc/gdn_bwd_bf16.hip"]
K256_KERNEL_NAME = "gdn_fwd_bf16<false, 0, 256>"


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(B, T, Hqk, Hv, dk, dv, in_bytes=2, h0=False):
    """Each input read once, each output written once."""
    tokens = B * T
    qk = 2 * tokens * Hqk * dk * in_bytes
    v = tokens * Hv * dv * in_bytes
    gates = 2 * tokens * Hv * 4
    o = tokens * Hv * dv * in_bytes
    states = B * Hv * dk * dv * 4 * (2 if h0 else 1)
    return qk + v + gates + o + states


def chunked_flops(B, T, Hv, dk, dv, C=64):
    """Algorithmic flops of the chunk form, per chunk and value head:
    2 C^2 (3 dk + 2 dv) for K K^T, Q K^T and W = T' diag(e^gamma) K (the
    three C x C x dk products) and U = T' V, P Delta (the two C x C x dv
    ones); 6 C dk dv for W h, Q h and K^T Delta'; 2 C^3 / 3 for the
    triangular inverse."""
    chunks = B * Hv * (-(-T // C))
    per = 2 * C * C * (3 * dk + 2 * dv) + 6 * C * dk * dv + 2 * C ** 3 / 3
    return chunks * per


def bwd_algorithmic_bytes(B, T, Hqk, Hv, dk, dv, in_bytes=2):
    """Backward: q, k, v, do, g, beta and dht read once; dq, dk, dv, dg, dbeta
    and dh0 written once (no initial state)."""
    tokens = B * T
    reads = tokens * (2 * Hqk * dk + 2 * Hv * dv) * in_bytes + 2 * tokens * Hv * 4
    writes = tokens * (2 * Hqk * dk + Hv * dv) * in_bytes + 2 * tokens * Hv * 4
    states = 2 * B * Hv * dk * dv * 4
    return reads + writes + states


def measure_bwd(gdn, gi, torch, dev, steps, warmup, name="fwd_bwd_bf16", with_fwd=False):
    """The backward on a workload with upstream gradients do and dht
    (fwd_bwd_bf16: the headline shapes; fwd_bwd_dk64_bf16: head dimension 64):
    milliseconds per call over `steps` back-to-back calls, its HBM roofline
    fraction, and the oracle on one sampled head; with_fwd adds the forward's
    time on the same inputs and the forward + backward throughput."""
    import oracle
    d = gi.make_config(name)
    do, dht = gi.make_upstream(d, gi.CONFIGS[name]["seed"])
    B, T, Hqk, Hv, dk, dv = d["B"], d["T"], d["Hqk"], d["Hv"], d["dk"], d["dv"]
    up = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v, dO = up(d["q"]), up(d["k"]), up(d["v"]), up(do)
    g, beta = torch.from_numpy(d["g"]).to(dev), torch.from_numpy(d["beta"]).to(dev)
    dh = torch.from_numpy(dht).to(dev)
    ws = torch.empty(gdn.gdn_chunk_bwd_workspace_size(1, B, T, Hqk, Hv, dk, dv, B),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    call = lambda: gdn.gdn_chunk_bwd(q, k, v, g, beta, dO, dht=dh, workspace=ws,
                                     stream=stream.cuda_stream)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        out = call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = bwd_algorithmic_bytes(B, T, Hqk, Hv, dk, dv)
    fwd_ms = None
    if with_fwd:
        o = torch.empty_like(dO)
        ht = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
        fwd_ms = _time_calls(torch, stream, lambda: gdn.gdn_chunk_fwd(
            q, k, v, g, beta, out=o, final_state=ht, stream=stream.cuda_stream), steps, warmup)
    bs, hs = 2, 7 % Hv
    sl = lambda x: gi.widen(x[bs:bs + 1, :, hs:hs + 1])
    ref = oracle.gdn_bwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), d["g"][bs:bs + 1, :, hs:hs + 1],
                         d["beta"][bs:bs + 1, :, hs:hs + 1], sl(do),
                         dht=dht[bs:bs + 1, hs:hs + 1].astype(np.float64))
    got = [x[bs:bs + 1, :, hs:hs + 1] if x.dim() >= 3 and x.shape[0] == B and x.shape[1] == T
           else x[bs:bs + 1, hs:hs + 1] for x in out]
    errs = {}
    for nm, x, r in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, ref):
        x = x.float().cpu().numpy()
        errs[nm] = float(np.linalg.norm(x - r) / np.linalg.norm(r))
    log("[bench] backward (%s) %.4f ms/call; sampled head rel-L2 %s" %
        (name, ms, ", ".join(f"{n} {e:.2e}" for n, e in errs.items())))
    achieved = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": f"{name}: B={B} T={T} H={Hv} dk={dk} dv={dv}, do ~ N(0,1) bf16, "
                       f"dht ~ N(0,0.02) fp32",
           "ms_per_call": ms, "tokens_per_s": B * T / (ms * 1e-3), "steps": steps,
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                        "algorithmic_bytes_per_call": nbytes,
                        "kernels": [f"gdn_fwd_bf16<false, 3, {dk}>",
                                    f"gdn_fwd_bf16<false, 4, {dk}>", "bwd_grads"]},
           "check": {"sampled_head": [bs, hs], "rel_l2": errs}}
    # The same inputs taken as raw ones, with both in-op options: the
    # preparation into the workspace, the backward, the chain back through it.
    ws_opt = torch.empty(gdn.gdn_chunk_bwd_workspace_size(1, B, T, Hqk, Hv, dk, dv, B, 3),
                         dtype=torch.uint8, device=dev)
    opt_ms = _time_calls(torch, stream, lambda: gdn.gdn_chunk_bwd(
        q, k, v, g, beta, dO, dht=dh, workspace=ws_opt, stream=stream.cuda_stream,
        use_qk_l2norm=True, gate_activation=True), steps, warmup)
    del ws_opt
    log(f"[bench] backward ({name}) with both in-op options {opt_ms:.4f} ms/call")
    res["ms_per_call_with_options"] = opt_ms
    if with_fwd:
        log(f"[bench] forward ({name}) {fwd_ms * 1e3:.1f} us/call; forward + backward "
            f"{B * T / ((fwd_ms + ms) * 1e-3):.3g} tokens/s")
        res["fwd_ms_per_call"] = fwd_ms
        res["fwd_bwd_tokens_per_s"] = B * T / ((fwd_ms + ms) * 1e-3)
    return res


def measure_bwd_k256(gdn, gi, torch, dev, steps, warmup):
    """The backward at head dimension 256 on the k256 workload's shapes (B=8,
    T=2048, H=32, D=256: the FLA table's D = 256 row), inputs drawn on the
    device with the workload's recipe plus do ~ N(0, 1) and dht ~ N(0, 0.02):
    milliseconds per call, the forward on the same inputs, its HBM roofline
    fraction, and the oracle on one sampled head."""
    import oracle
    name = "k256_bf16"
    c = gi.CONFIGS[name]
    B, T, Hqk, Hv, dk, dv = c["B"], c["T"], c["Hqk"], c["Hv"], c["dk"], c["dv"]
    t = gi.make_device(B, T, Hqk, Hv, dk, dv, c["seed"], device=dev)
    gen = torch.Generator(device=dev).manual_seed(c["seed"] + 1)
    dO = torch.randn((B, T, Hv, dv), generator=gen, device=dev).to(torch.bfloat16)
    dh = 0.02 * torch.randn((B, Hv, dk, dv), generator=gen, device=dev)
    q, k, v, g, beta = (t[x] for x in ("q", "k", "v", "g", "beta"))
    ws = torch.empty(gdn.gdn_chunk_bwd_workspace_size(1, B, T, Hqk, Hv, dk, dv, B),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = None

    def call():
        nonlocal out
        out = gdn.gdn_chunk_bwd(q, k, v, g, beta, dO, dht=dh, workspace=ws,
                                stream=stream.cuda_stream)
    ms = _time_calls(torch, stream, call, steps, warmup)
    o = torch.empty_like(dO)
    ht = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    fwd_ms = _time_calls(torch, stream, lambda: gdn.gdn_chunk_fwd(
        q, k, v, g, beta, out=o, final_state=ht, stream=stream.cuda_stream), steps, warmup)
    bs, hs = 3, 21
    sl = lambda x: x[bs:bs + 1, :, hs:hs + 1].float().cpu().numpy()
    ref = oracle.gdn_bwd(sl(q), sl(k), sl(v), sl(g), sl(beta), sl(dO),
                         dht=dh[bs:bs + 1, hs:hs + 1].double().cpu().numpy())
    errs = {}
    for i, (nm, r) in enumerate(zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), ref)):
        x = out[i][bs:bs + 1, :, hs:hs + 1] if i < 5 else out[i][bs:bs + 1, hs:hs + 1]
        x = x.float().cpu().numpy()
        errs[nm] = float(np.linalg.norm(x - r) / np.linalg.norm(r))
    nbytes = bwd_algorithmic_bytes(B, T, Hqk, Hv, dk, dv)
    achieved = nbytes / (ms * 1e-3) / 1e9
    log("[bench] backward (%s) %.4f ms/call, forward %.1f us/call; sampled head rel-L2 %s" %
        (name, ms, fwd_ms * 1e3, ", ".join(f"{n} {e:.2e}" for n, e in errs.items())))
    return {"workload": f"{name}: B={B} T={T} H={Hv} dk={dk} dv={dv}, chunk=32, do ~ N(0,1) "
                        f"bf16, dht ~ N(0,0.02) fp32 (drawn on the device)",
            "ms_per_call": ms, "fwd_ms_per_call": fwd_ms,
            "tokens_per_s": B * T / (ms * 1e-3),
            "fwd_bwd_tokens_per_s": B * T / ((fwd_ms + ms) * 1e-3), "steps": steps,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                         "algorithmic_bytes_per_call": nbytes,
                         "kernels": ["gdn_fwd_bf16<false, 3, 256>",
                                     "gdn_fwd_bf16<false, 4, 256>", "bwd_grads_k256"]},
            "check": {"sampled_head": [bs, hs], "rel_l2": errs}}


def per_launch(torch, stream, call, n, flush=None):
    """Per-launch durations (ms) with HIP events on the launch stream; with
    `flush` (a device buffer) it is overwritten before every launch, outside
    the events, so each launch starts with cold caches (L2 and the 256 MB
    MALL).  Returns mean, median and minimum."""
    times = []
    for i in range(n):
        if flush is not None:
            flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        b.synchronize()
        times.append(a.elapsed_time(b))
    t = np.array(times)
    return {"mean": float(t.mean()), "median": float(np.median(t)), "min": float(t.min()),
            "n": n}


def settle_clocks(torch, call, ms):
    """Launches `call` back to back, untimed, for about `ms` of wall clock so
    the GPU's clocks have ramped up under this load; returns the count."""
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(20):
            call()
        n += 20
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return n


def _time_calls(torch, stream, call, steps, warmup):
    """Milliseconds per call over `steps` back-to-back calls on `stream`."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def decode_algorithmic_bytes(N, Hqk, Hv, dk, dv, in_bytes=2):
    """One decode step: the state read and written once; q, k, v, g, beta
    read and o written once."""
    return (N * Hv * dk * dv * 4 * 2 + N * (2 * Hqk * dk + 2 * Hv * dv) * in_bytes
            + 2 * N * Hv * 4)


def measure_decode(gdn, gi, torch, dev, steps, warmup):
    """The decode step on its workload (256 sequences, one token each, a
    256-slot fp32 cache): milliseconds per call, tokens/s, HBM roofline
    fraction, and a check of one call against the fp64 step on 4 sequences."""
    from oracle import prep
    name = "decode_bf16"
    d = gi.make_config(name)
    N, Hqk, Hv, dk, dv = d["B"], d["Hqk"], d["Hv"], d["dk"], d["dv"]
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x[:, 0]).view(np.int16)).to(dev) \
        .view(torch.bfloat16)
    q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
    g = torch.from_numpy(np.ascontiguousarray(d["g"][:, 0])).to(dev)
    beta = torch.from_numpy(np.ascontiguousarray(d["beta"][:, 0])).to(dev)
    cache = torch.from_numpy(d["h0"]).to(dev)
    o = torch.empty((N, Hv, dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    call = lambda: gdn.gdn_recurrent_step(q, k, v, g, beta, cache, out=o,
                                          stream=stream.cuda_stream)
    call()
    torch.cuda.synchronize()
    sel = [0, 77, 150, 255]
    ro, rc = prep.step(*(gi.widen(d[x][sel, 0]) for x in ("q", "k", "v")), d["g"][sel, 0],
                       d["beta"][sel, 0], d["h0"][sel])
    err_o = float(np.linalg.norm(o[sel].float().cpu().numpy() - ro) / np.linalg.norm(ro))
    err_c = float(np.linalg.norm(cache[sel].cpu().numpy() - rc) / np.linalg.norm(rc))
    ms = _time_calls(torch, stream, call, steps, warmup)
    flushed = per_launch(torch, stream, call, 50, flush=flush_buffer(torch, dev))
    nbytes = decode_algorithmic_bytes(N, Hqk, Hv, dk, dv)
    achieved = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] decode step {ms * 1e3:.1f} us/call back to back ({achieved:.0f} GB/s), "
        f"{flushed['median'] * 1e3:.1f} us flushed (median); "
        f"check rel-L2 output {err_o:.2e}, cache {err_c:.2e}")
    return {"workload": f"{name}: N={N} sequences x 1 token, H={Hv}, dk={dk}, dv={dv}, "
                        f"bf16 q/k/v/o, fp32 cache of {N} slots",
            "ms_per_call": ms, "tokens_per_s": N / (ms * 1e-3), "steps": steps,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                         "frac_flushed_median": nbytes / (flushed["median"] * 1e-3) / 1e9 /
                                                HBM_PEAK_GBPS,
                         "note": "the 272 MB working set fits the 256 MB MALL between "
                                 "back-to-back calls; the flushed figure is the HBM one",
                         "algorithmic_bytes_per_call": nbytes, "kernels": ["recurrent_step"]},
            "launch_ms_flushed": flushed,
            "check": {"sequences": sel, "rel_l2_output": err_o, "rel_l2_cache": err_c}}


def measure_prep(gdn, torch, q, k, vv, g, beta, fwd_ms, steps, warmup):
    """In-op preparation (q/k L2 norm and gate activations) on the headline
    tensors: the forward with both options fused into its staging, against
    the plain forward, and the separate preparation pass (out of place) with
    its HBM roofline fraction."""
    stream = torch.cuda.current_stream(q.device)
    qo, ko, go, bo = (torch.empty_like(x) for x in (q, k, g, beta))
    lib = gdn.load()
    dk = q.shape[-1]

    def call():
        st = lib.gdn_prepare_inputs(1, q.numel() // dk, dk, q.data_ptr(), k.data_ptr(),
                                    qo.data_ptr(), ko.data_ptr(), g.numel(), g.data_ptr(),
                                    beta.data_ptr(), go.data_ptr(), bo.data_ptr(),
                                    gdn.GDN_QK_L2NORM | gdn.GDN_GATE_ACT, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(gdn.gdn_status_string(st))
    ms = _time_calls(torch, stream, call, steps, warmup)
    flushed = per_launch(torch, stream, call, 50, flush=flush_buffer(torch, q.device))
    nbytes = 2 * (q.numel() + k.numel()) * q.element_size() + 2 * (g.numel() + beta.numel()) * 4
    achieved = nbytes / (ms * 1e-3) / 1e9
    o = torch.empty_like(vv)
    ht = torch.empty((q.shape[0], vv.shape[2], q.shape[3], vv.shape[3]), dtype=torch.float32,
                     device=q.device)
    fused = lambda: gdn.gdn_chunk_fwd(q, k, vv, g, beta, out=o, final_state=ht,
                                      stream=stream.cuda_stream, use_qk_l2norm=True,
                                      gate_activation=True)
    fused_ms = _time_calls(torch, stream, fused, 1000, 500)
    log(f"[bench] preparation pass {ms * 1e3:.1f} us/call back to back ({achieved:.0f} GB/s), "
        f"{flushed['median'] * 1e3:.1f} us flushed (median); forward with "
        f"fused preparation {fused_ms * 1e3:.1f} us (plain {fwd_ms * 1e3:.1f} us)")
    return {"ms_per_call": ms, "fwd_fused_prep_ms": fused_ms, "fwd_plain_ms": fwd_ms,
            "launch_ms_flushed": flushed,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                         "frac_flushed_median": nbytes / (flushed["median"] * 1e-3) / 1e9 /
                                                HBM_PEAK_GBPS,
                         "note": "back to back, the 273 MB working set largely stays in the "
                                 "256 MB MALL; the flushed figure is the HBM one",
                         "algorithmic_bytes_per_call": nbytes, "kernels": ["preprocess"]}}


def measure_long(gdn, gi, torch, dev, steps=3, name="long_bf16"):
    """A long-row workload (long_bf16: B=1, T=1,064,960, H=16, d=128;
    long_k256_bf16: B=1, T=65,536, H=8, d=256; bf16, inputs drawn on the
    device with the same recipe): milliseconds per forward with the piece
    scan and with whole rows, the HBM roofline fraction of each, and the
    agreement of the two routes' outputs and final states (their parity with
    the oracle is a GPU test)."""
    c = gi.CONFIGS[name]
    B, T, Hqk, Hv, dk, dv = c["B"], c["T"], c["Hqk"], c["Hv"], c["dk"], c["dv"]
    t = gi.make_device(B, T, Hqk, Hv, dk, dv, c["seed"], device=dev)
    q, k, v, g, beta = (t[x] for x in ("q", "k", "v", "g", "beta"))
    outs = {}
    ws = torch.empty(max(1, gdn.gdn_chunk_fwd_workspace_size(1, B, T, Hqk, Hv, dk, dv, B)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {"workload": f"{name}: B={B} T={T} H={Hv} dk={dk} dv={dv}, zero initial state"}
    nbytes = algorithmic_bytes(B, T, Hqk, Hv, dk, dv)
    for mode, kw in (("pieces", dict(workspace=ws)), ("whole_rows", dict(pieces=False))):
        o = torch.empty_like(v)
        ht = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
        call = lambda: gdn.gdn_chunk_fwd(q, k, v, g, beta, out=o, final_state=ht,
                                         stream=stream.cuda_stream, **kw)
        call()
        tm = per_launch(torch, stream, call, steps)
        ms = tm["median"]
        out[mode] = {"ms_per_call_median": ms, "ms_per_call_min": tm["min"],
                     "tokens_per_s": B * T / (ms * 1e-3),
                     "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        outs[mode] = (o, ht)
        log(f"[bench] {name}, {mode}: {ms:.2f} ms/call (median of {steps})")
    (o1, h1), (o2, h2) = outs["pieces"], outs["whole_rows"]
    rel = lambda a, b: float(torch.linalg.vector_norm((a.float() - b.float()).ravel()) /
                             torch.linalg.vector_norm(b.float().ravel()))
    out["pieces_vs_whole_rows_rel_l2"] = {"output": rel(o1, o2), "state": rel(h1, h2)}
    out["pieces"]["speedup_over_whole_rows"] = (out["whole_rows"]["ms_per_call_median"] /
                                                out["pieces"]["ms_per_call_median"])
    out["algorithmic_bytes_per_call"] = nbytes
    del q, k, v, g, beta, t, outs, o1, h1, o2, h2
    torch.cuda.empty_cache()
    return out


def measure_packed(gdn, gi, torch, dev, steps, warmup, name="packed_gva_bf16"):
    """A packed workload (packed_gva_bf16: 16,384 tokens in geometric
    documents of mean length 1024, H_qk=16, H_v=32, d=128, bf16, an initial
    state per document; packed_8h_bf16: the same at 8 heads): milliseconds
    per forward as planned from the host copy of cu_seqlens (documents
    longest first, long ones split into pieces where the plan says so) and
    as whole documents in index order (no workspace), back to back and
    flushed; tokens/s; the HBM roofline fraction (initial and final states
    counted); the oracle on two sampled (document, head) pairs."""
    import oracle
    d = gi.make_config(name)
    Hqk, Hv, dk, dv, T, N = d["Hqk"], d["Hv"], d["dk"], d["dv"], d["T"], d["N"]
    up = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
    g, beta = torch.from_numpy(d["g"]).to(dev), torch.from_numpy(d["beta"]).to(dev)
    h0 = torch.from_numpy(d["h0"]).to(dev)
    cu = d["cu_seqlens"]
    cu_dev = torch.from_numpy(cu).to(dev)
    cu_host = [int(x) for x in cu]
    o = torch.empty_like(v)
    ht = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    plan = gdn.gdn_chunk_fwd_plan(1, 1, T, Hqk, Hv, dk, dv, cu_host)
    nbytes = (2 * T * Hqk * dk * 2 + 2 * T * Hv * dv * 2 + 2 * T * Hv * 4 +
              2 * N * Hv * dk * dv * 4)
    cfg = gi.CONFIGS[name]
    docs = (f"lengths {cfg['lengths']}" if "lengths" in cfg else
            f"geometric, mean {cfg['mean_len']}")
    res = {"workload": f"{name}: {T} tokens in {N} documents ({docs}), "
                       f"H_qk={Hqk} H_v={Hv} dk={dk} dv={dv}, h0 ~ N(0, 0.02)",
           "plan": {"piece_len": plan[0], "slots": plan[1], "longest_first": plan[2]},
           "algorithmic_bytes_per_call": nbytes}
    for mode, kw in (("planned", {}), ("whole_documents_index_order", dict(pieces=False))):
        call = lambda: gdn.gdn_chunk_fwd(q, k, v, g, beta, initial_state=h0, cu_seqlens=cu_dev,
                                         cu_seqlens_host=cu_host, out=o, final_state=ht,
                                         stream=stream.cuda_stream, **kw)
        ms = _time_calls(torch, stream, call, steps, warmup)
        flushed = per_launch(torch, stream, call, 50, flush=flush_buffer(torch, dev))
        achieved = nbytes / (ms * 1e-3) / 1e9
        res[mode] = {"ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
                     "launch_ms_flushed": flushed,
                     "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                                  "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                                  "frac_flushed_median": nbytes / (flushed["median"] * 1e-3) /
                                                         1e9 / HBM_PEAK_GBPS}}
        log(f"[bench] {name} ({N} documents, {mode}): {ms * 1e3:.1f} us/call back to back, "
            f"{flushed['median'] * 1e3:.1f} us flushed (median)")
    # The planned call's output against the oracle on two (document, head)
    # pairs drawn with the workload seed.
    gdn.gdn_chunk_fwd(q, k, v, g, beta, initial_state=h0, cu_seqlens=cu_dev,
                      cu_seqlens_host=cu_host, out=o, final_state=ht, stream=stream.cuda_stream)
    torch.cuda.synchronize()
    seed = gi.CONFIGS[name]["seed"]
    rng = np.random.default_rng(seed)
    lens = np.diff(cu)
    docs = sorted(int(x) for x in rng.choice(np.flatnonzero(lens > 0), size=2, replace=False))
    heads = gi.sampled_heads(seed, Hv)
    errs = []
    G = Hv // Hqk
    for n, j in zip(docs, heads):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        sl = lambda x, hh: gi.widen(x[:, t0:t1, hh:hh + 1])
        ro, rh = oracle.gdn_fwd(sl(d["q"], j // G), sl(d["k"], j // G), sl(d["v"], j),
                                d["g"][:, t0:t1, j:j + 1], d["beta"][:, t0:t1, j:j + 1],
                                h0=d["h0"][n:n + 1, j:j + 1].astype(np.float64))
        go = o[:, t0:t1, j:j + 1].float().cpu().numpy()
        gh = ht[n:n + 1, j:j + 1].cpu().numpy()
        errs.append({"document": n, "tokens": t1 - t0, "head": j,
                     "rel_l2_output": float(np.linalg.norm(go - ro) / np.linalg.norm(ro)),
                     "rel_l2_state": float(np.linalg.norm(gh - rh) / np.linalg.norm(rh))})
    log(f"[bench] {name} checks {errs}")
    res["check"] = errs
    # The headline keys: the planned call.
    res["ms_per_call"] = res["planned"]["ms_per_call"]
    res["tokens_per_s"] = res["planned"]["tokens_per_s"]
    res["roofline"] = dict(res["planned"]["roofline"], algorithmic_bytes_per_call=nbytes,
                           kernel="gdn_fwd_bf16<false, 0, 128> (or <false, 1|2, 128> with pieces)")
    return res


def measure_tiny(gdn, gi, torch, dev):
    """The tiny fp32 workload (B=1, T=256, H=2, d=64): four workgroups (one
    per head and 32 value columns) walk four chunks each, so the time is the
    latency of one workgroup's chunk steps in fp32 vector arithmetic, not
    bandwidth; only its absolute time is reported (per-launch events, back to
    back), with the whole output checked against the oracle."""
    import oracle
    d = gi.make_config("tiny_f32")
    tt = {x: torch.from_numpy(d[x]).to(dev) for x in ("q", "k", "v", "g", "beta")}
    stream = torch.cuda.current_stream(dev)
    res = {}
    call = lambda: res.update(zip(("o", "ht"), gdn.gdn_chunk_fwd(
        tt["q"], tt["k"], tt["v"], tt["g"], tt["beta"], stream=stream.cuda_stream)))
    call()
    tm = per_launch(torch, stream, call, 200)
    ro, rh = oracle.gdn_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"])
    eo = float(np.linalg.norm(res["o"].cpu().numpy() - ro) / np.linalg.norm(ro))
    eh = float(np.linalg.norm(res["ht"].cpu().numpy() - rh) / np.linalg.norm(rh))
    log(f"[bench] tiny fp32: {tm['median'] * 1e3:.1f} us per launch (median); rel-L2 output "
        f"{eo:.2e}, state {eh:.2e}")
    return {"workload": "tiny_f32: B=1 T=256 H=2 dk=64 dv=64, fp32, zero initial state",
            "launch_ms": tm,
            "bound": "latency of 4 workgroups' fp32 chunk steps (absolute time only)",
            "check": {"rel_l2_output": eo, "rel_l2_state": eh}}


def flush_buffer(torch, dev, mb=512):
    return torch.empty(mb << 20, dtype=torch.uint8, device=dev)


def measure_k256(gdn, gi, torch, dev, steps, warmup):
    """Head dimension 256 (B=8, T=2048, H=32, dk=dv=256, bf16; inputs drawn
    on the device with the same recipe; chunks of 32 tokens): milliseconds
    per forward, tokens/s, HBM and MFMA fractions, and a check of one head
    against the fp64 oracle."""
    import oracle
    name = "k256_bf16"
    c = gi.CONFIGS[name]
    B, T, Hqk, Hv, dk, dv = c["B"], c["T"], c["Hqk"], c["Hv"], c["dk"], c["dv"]
    t = gi.make_device(B, T, Hqk, Hv, dk, dv, c["seed"], device=dev)
    q, k, v, g, beta = (t[x] for x in ("q", "k", "v", "g", "beta"))
    o = torch.empty_like(v)
    ht = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    call = lambda: gdn.gdn_chunk_fwd(q, k, v, g, beta, out=o, final_state=ht,
                                     stream=stream.cuda_stream)
    ms = _time_calls(torch, stream, call, steps, warmup)
    bs, hs = 3, 21
    sel = lambda x: x[bs:bs + 1, :, hs:hs + 1].float().cpu().numpy()
    ro, rh = oracle.gdn_fwd(sel(q), sel(k), sel(v), sel(g), sel(beta))
    err_o = float(np.linalg.norm(sel(o) - ro) / np.linalg.norm(ro))
    err_h = float(np.linalg.norm(ht[bs:bs + 1, hs:hs + 1].cpu().numpy() - rh) / np.linalg.norm(rh))
    nbytes = algorithmic_bytes(B, T, Hqk, Hv, dk, dv)
    flops = chunked_flops(B, T, Hv, dk, dv, C=32)
    achieved = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] dk=256: {ms * 1e3:.1f} us/call ({achieved:.0f} GB/s); check head "
        f"(b={bs}, h={hs}) rel-L2 output {err_o:.2e}, state {err_h:.2e}")
    del q, k, v, g, beta, o, t
    torch.cuda.empty_cache()
    return {"workload": f"{name}: B={B} T={T} H={Hv} dk={dk} dv={dv}, chunk=32, zero initial "
                        f"state, output + final state",
            "ms_per_call": ms, "tokens_per_s": B * T / (ms * 1e-3), "steps": steps,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                         "traffic": measured_traffic(name),
                         "algorithmic_bytes_per_call": nbytes,
                         "mfma_bf16_tflops": flops / (ms * 1e-3) / 1e12,
                         "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                         "kernel": K256_KERNEL_NAME},
            "check": {"head": [bs, hs], "rel_l2_output": err_o, "rel_l2_state": err_h}}


def kernel_source_hash(sources=None):
    """sha256 of the kernel's code: its source with // comments, trailing
    blanks and empty lines removed, so editing a comment does not count as a
    change of the kernel."""
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic(workload=WORKLOAD):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    the workload's kernel, or None if it is missing or was taken on another
    version of the kernel."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(d, target_s=10.0):
    """The fp64 oracle on this host: whole-workload runs, repeated until
    about target_s seconds of wall clock have passed (at least one run)."""
    import gdn_inputs as gi
    import oracle
    q, k, v = (gi.widen(d[x]) for x in ("q", "k", "v"))
    threads = oracle.default_threads()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.gdn_fwd(q, k, v, d["g"], d["beta"], nthreads=threads)
        runs += 1
        el = time.perf_counter() - t0
        if el >= target_s or runs >= 50:
            break
    tokens = d["B"] * d["T"] * runs
    return {"value": tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole workload (B={d['B']}, T={d['T']}, H={d['Hv']}, d={d['dk']}), "
                      f"{runs} run(s) in {el:.2f} s, fp64 token recurrence, "
                      f"{threads} threads"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=500)
    # The GPU's clocks take tens of milliseconds of load to ramp up: before
    # the warm-up steps the step is launched back to back, untimed, for this
    # long.  The timed region is still exactly --steps steps.
    ap.add_argument("--settle-ms", type=float, default=300.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-step and preparation measurements")
    ap.add_argument("--no-k256", action="store_true",
                    help="skip the head-dimension-256 measurement")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long rows (B=1, T=1,064,960, d=128; B=1, T=65,536, d=256)")
    ap.add_argument("--no-packed", action="store_true",
                    help="skip the packed workload and the tiny fp32 one")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="cache-flush write between the per-launch timings")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(--gpus {args.gpus} was asked for)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_chunked_chunk_amd as gdn
    import gdn_inputs as gi
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gdn.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    c = gi.CONFIGS[WORKLOAD]
    log(f"[bench] generating {WORKLOAD} inputs")
    d = gi.make_config(WORKLOAD)
    B, T, Hqk, Hv, dk, dv = d["B"], d["T"], d["Hqk"], d["Hv"], d["dk"], d["dv"]
    dt = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v = dt(d["q"]), dt(d["k"]), dt(d["v"])
    g = torch.from_numpy(d["g"]).to(dev)
    beta = torch.from_numpy(d["beta"]).to(dev)
    o = torch.empty((B, T, Hv, dv), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        gdn.gdn_chunk_fwd(q, k, v, g, beta, out=o, final_state=ht, stream=stream.cuda_stream)

    settle_n = settle_clocks(torch, step, args.settle_ms) if args.settle_ms > 0 else 0
    log(f"[bench] clocks settled over {settle_n} untimed launches; warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed region: exactly K back-to-back steps.
    log(f"[bench] timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    tokens = B * T
    value = tokens * args.steps / (ms_total * 1e-3)

    # Per-launch durations with HIP events on the launch stream: once back to
    # back, once with the caches flushed by a large write before each launch.
    n_launch = min(max(args.steps, 10), 100)
    t_b2b = per_launch(torch, stream, step, n_launch)
    t_fl = per_launch(torch, stream, step, n_launch, flush=flush_buffer(torch, dev, args.flush_mb))
    nbytes = algorithmic_bytes(B, T, Hqk, Hv, dk, dv)
    flops = chunked_flops(B, T, Hv, dk, dv)
    # One launch per step on `stream`: the timed region's events give the
    # kernel's average launch duration.
    launch_ms = ms_per_step
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    traffic = measured_traffic()

    # A device copy of the same byte count, for context (not the denominator).
    src = torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)
    dstb = torch.empty_like(src)
    dstb.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        dstb.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dstb

    # Spot check of the timed output against the oracle on one sampled head.
    import oracle
    import gdn_inputs as gi2
    bs, hs = 5, 11
    qq, kk, vv = (gi2.widen(d[x][bs:bs + 1, :, hs:hs + 1]) for x in ("q", "k", "v"))
    ro, rh = oracle.gdn_fwd(qq, kk, vv, d["g"][bs:bs + 1, :, hs:hs + 1],
                            d["beta"][bs:bs + 1, :, hs:hs + 1])
    go = o[bs:bs + 1, :, hs:hs + 1].float().cpu().numpy()
    gh = ht[bs:bs + 1, hs:hs + 1].cpu().numpy()
    err_o = float(np.linalg.norm(go - ro) / np.linalg.norm(ro))
    err_h = float(np.linalg.norm(gh - rh) / np.linalg.norm(rh))
    log(f"[bench] sampled head (b={bs}, h={hs}) rel-L2: output {err_o:.2e}, state {err_h:.2e}")

    bwd = bwd_dk64 = bwd_k256 = None
    if not args.no_bwd:
        log("[bench] backward")
        bwd = measure_bwd(gdn, gi, torch, dev, steps=50, warmup=20)
        bwd_dk64 = measure_bwd(gdn, gi, torch, dev, steps=50, warmup=20,
                               name="fwd_bwd_dk64_bf16", with_fwd=True)
        if not args.no_k256:
            bwd_k256 = measure_bwd_k256(gdn, gi, torch, dev, steps=10, warmup=3)

    decode = prep = None
    if not args.no_decode:
        log("[bench] preparation pass and decode step")
        prep = measure_prep(gdn, torch, q, k, v, g, beta, ms_per_step, steps=200, warmup=50)
        decode = measure_decode(gdn, gi, torch, dev, steps=200, warmup=100)

    k256 = None
    if not args.no_k256:
        log("[bench] head dimension 256")
        k256 = measure_k256(gdn, gi, torch, dev, steps=200, warmup=100)

    packed = packed_8h = packed_long_doc = tiny = None
    if not args.no_packed:
        log("[bench] packed documents and the tiny fp32 workload")
        packed = measure_packed(gdn, gi, torch, dev, steps=200, warmup=50)
        packed_8h = measure_packed(gdn, gi, torch, dev, steps=200, warmup=50,
                                   name="packed_8h_bf16")
        packed_long_doc = measure_packed(gdn, gi, torch, dev, steps=100, warmup=20,
                                         name="packed_long_doc_bf16")
        tiny = measure_tiny(gdn, gi, torch, dev)

    long_row = long_k256 = None
    if not args.no_long:
        log("[bench] long rows")
        long_row = measure_long(gdn, gi, torch, dev)
        long_k256 = measure_long(gdn, gi, torch, dev, steps=10, name="long_k256_bf16")

    baseline = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        baseline = cpu_baseline(d)
        baseline["cpu_model"] = cpu_model()

    result = {
        "metric": "GDN chunked fwd tokens/s (8x2K, H16, d128, bf16); % of roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"ms": args.settle_ms, "launches": settle_n,
                         "note": "untimed back-to-back launches before the warm-up steps"},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), "
                "beta=sigmoid(N(0,1)), g=logsigmoid(N(0,1))/16)",
        "config": {"workload": f"{WORKLOAD}: B={B} T={T} H_qk={Hqk} H_v={Hv} dk={dk} dv={dv} "
                               f"chunk=64, zero initial state, output + final state",
                   "B": B, "T": T, "H": Hv, "dk": dk, "dv": dv, "chunk": 64,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "kernel": KERNEL_NAME,
            "algorithmic_bytes_per_launch": nbytes,
            "launch_ms_mean": launch_ms,
            "launch_ms_back_to_back": t_b2b,
            "launch_ms_flushed": t_fl,
            "frac_flushed_median": nbytes / (t_fl["median"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "frac_flushed_min": nbytes / (t_fl["min"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "mfma_bf16_tflops": flops / (launch_ms * 1e-3) / 1e12,
            "mfma_frac": flops / (launch_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "copy_gbps": copy_gbps,
        },
        "cpu_baseline": baseline,
        "check": {"sampled_head": [bs, hs], "rel_l2_output": err_o, "rel_l2_state": err_h},
        "bwd": bwd,
        "bwd_dk64": bwd_dk64,
        "bwd_k256": bwd_k256,
        "prep": prep,
        "decode": decode,
        "k256": k256,
        "packed": packed,
        "packed_8h": packed_8h,
        "packed_long_doc": packed_long_doc,
        "tiny": tiny,
        "long_row": long_row,
        "long_k256": long_k256,
        "wall_s_timed_region": wall,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
