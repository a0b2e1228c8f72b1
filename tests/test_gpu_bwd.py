"""Parity of the HIP backward (through the C ABI) with the fp64 reverse-mode
oracle.

Each case draws seeded inputs with the workloads' recipe plus upstream
gradients do ~ N(0, 1) and dht ~ N(0, 0.02), runs gdn_chunk_bwd on the GPU and
oracle.gdn_bwd on the host, and compares all six gradients element by element
(relative L2 over each whole tensor).  Sizes span several chunks and ragged
tails; the forward-and-backward workload runs at full size.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_util import rel_l2, to_device

pytestmark = pytest.mark.gpu

# bf16 inputs: every gradient within 1e-2 relative L2 of the fp64 oracle (the
# bf16 rounding of dq, dk, dv alone is about 2e-3); dh0, a state gradient kept
# in fp32, within the forward's state tolerance of 1e-3.
TOL_BWD = 1e-2
TOL_DH0 = 1e-3
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def run_bwd_gpu(d, do, dht, scale=1.0):
    import gated_deltanet_chunked_chunk_amd as gdn
    t = to_device(d)
    do_t = torch.from_numpy(do.view(np.int16)).cuda().view(torch.bfloat16)
    dht_t = None if dht is None else torch.from_numpy(dht).cuda()
    out = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], do_t, dht=dht_t,
                            scale=scale, initial_state=t["h0"], cu_seqlens=t["cu"],
                            cu_seqlens_host=t["cu_host"])
    torch.cuda.synchronize()
    return [x.float().cpu().numpy() for x in out]


def run_bwd_oracle(d, do, dht, scale=1.0):
    q, k, v = (gi.widen(d[x]) for x in ("q", "k", "v"))
    return oracle.gdn_bwd(q, k, v, d["g"], d["beta"], gi.widen(do), scale=scale,
                          h0=None if d["h0"] is None else d["h0"].astype(np.float64),
                          dht=None if dht is None else dht.astype(np.float64),
                          cu_seqlens=d["cu_seqlens"])


def check_bwd(d, seed, scale=1.0, with_dht=True, label=""):
    do, dht = gi.make_upstream(d, seed)
    if not with_dht:
        dht = None
    print(f"[gpu bwd case] {label} B={d['B']} T={d['T']} Hqk={d['Hqk']} Hv={d['Hv']} "
          f"dv={d['dv']} N={d['N']} h0={d['h0'] is not None} dht={with_dht}", flush=True)
    got = run_bwd_gpu(d, do, dht, scale)
    ref = run_bwd_oracle(d, do, dht, scale)
    errs = {}
    for name, x, y in zip(NAMES, got, ref):
        assert np.all(np.isfinite(x)), f"{name} not finite"
        errs[name] = rel_l2(x, y)
    print("  rel-L2 " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for name, e in errs.items():
        tol = TOL_DH0 if name == "dh0" else TOL_BWD
        assert e <= tol, f"{name} rel-L2 {e:.3e} > {tol}"
    return errs


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_bwd_ragged(T):
    d = gi.make(2, T, 2, 2, 128, 128, "bf16", 5000 + T, h0_std=0.1)
    check_bwd(d, 5000 + T, scale=0.75, label=f"ragged T={T}")


def test_bwd_grouped_dv64():
    d = gi.make(1, 150, 1, 2, 128, 64, "bf16", 5100, h0_std=0.1)
    check_bwd(d, 5100, label="grouped heads, dv=64")


def test_bwd_grouped_dv128():
    """Two value heads of 128 columns per q/k head: four value steps per
    (chunk, q/k head) item of the gradient kernel."""
    d = gi.make(1, 200, 1, 2, 128, 128, "bf16", 5150, h0_std=0.1)
    check_bwd(d, 5150, scale=0.8, label="grouped heads, dv=128")


def test_bwd_more_items_than_workgroups():
    """260 (chunk, q/k head) items over 256 persistent workgroups: four walk
    two items (the next item's K, Q and first value step loaded during the
    first), the rest one (the loads for no next item read nothing), with a
    ragged last chunk in each sequence."""
    d = gi.make(2, 4100, 2, 2, 128, 128, "bf16", 5160, h0_std=0.05)
    check_bwd(d, 5160, label="260 items")


def test_bwd_packed_with_empty_document():
    cu = gi.cu_from_lengths([70, 0, 129, 1])
    d = gi.make(1, 200, 2, 4, 128, 128, "bf16", 5200, h0_std=0.05, cu_seqlens=cu)
    check_bwd(d, 5200, label="packed")


def test_bwd_no_state_gradient():
    d = gi.make(1, 130, 2, 2, 128, 128, "bf16", 5300)
    check_bwd(d, 5300, with_dht=False, label="no dht, no h0")


def test_bwd_workload_full_size():
    """The forward-and-backward workload: B=8, T=2048, H=16, dk=dv=128."""
    d = gi.make_config("fwd_bwd_bf16")
    check_bwd(d, gi.CONFIGS["fwd_bwd_bf16"]["seed"], label="fwd_bwd_bf16 full size")


def test_bwd_deterministic():
    d = gi.make(1, 190, 2, 2, 128, 128, "bf16", 5400, h0_std=0.1)
    do, dht = gi.make_upstream(d, 5400)
    a = run_bwd_gpu(d, do, dht)
    b = run_bwd_gpu(d, do, dht)
    for x, y, n in zip(a, b, NAMES):
        assert np.array_equal(x, y), f"{n} differs between runs"


@pytest.mark.parametrize("T,dv", [(1, 64), (65, 128), (200, 64)])
def test_bwd_dk64(T, dv):
    """dk = 64: q and k staged into the 128-wide tiles with zero upper halves
    (the chunk states kept 128 keys wide): ragged T, grouped heads, h0, scale."""
    d = gi.make(2, T, 1, 2, 64, dv, "bf16", 5500 + T, h0_std=0.1)
    check_bwd(d, 5500 + T, scale=0.8, label=f"dk64 T={T} dv={dv}")


def test_bwd_dk64_packed_no_dht():
    cu = gi.cu_from_lengths([90, 0, 64, 33])
    d = gi.make(1, 187, 2, 4, 64, 64, "bf16", 5600, h0_std=0.05, cu_seqlens=cu)
    check_bwd(d, 5600, with_dht=False, label="dk64 packed, no dht")


def test_bwd_dv256():
    d = gi.make(1, 150, 1, 1, 128, 256, "bf16", 5700, h0_std=0.1)
    check_bwd(d, 5700, label="dv=256")


def test_bwd_dk64_fla_shape():
    """Head dim 64 at the shape of the B=8, T=1024, H=8, D=64 row of the
    flash-linear-attention benchmark table, all heads against the oracle."""
    d = gi.make(8, 1024, 8, 8, 64, 64, "bf16", 5800, h0_std=0.02)
    check_bwd(d, 5800, label="dk64 8x1024x8")


@pytest.mark.parametrize("T,dv", [(1, 64), (31, 128), (33, 64), (100, 256)])
def test_bwd_dk256(T, dv):
    """dk = 256: chunks of 32 tokens (the forward's dk = 256 instance), ragged
    around the chunk, grouped heads, h0, dht and scale."""
    d = gi.make(2, T, 1, 2, 256, dv, "bf16", 5800 + T, h0_std=0.1)
    check_bwd(d, 5800 + T, scale=0.8, label=f"dk256 T={T} dv={dv}")


def test_bwd_dk256_packed_no_dht():
    cu = gi.cu_from_lengths([40, 0, 64, 17])
    d = gi.make(1, 121, 2, 4, 256, 64, "bf16", 5900, h0_std=0.05, cu_seqlens=cu)
    check_bwd(d, 5900, with_dht=False, label="dk256 packed, no dht")


def test_bwd_dk256_deterministic():
    d = gi.make(1, 90, 1, 1, 256, 128, "bf16", 5950, h0_std=0.1)
    do, dht = gi.make_upstream(d, 5950)
    a = run_bwd_gpu(d, do, dht)
    b = run_bwd_gpu(d, do, dht)
    for x, y, n in zip(a, b, NAMES):
        assert np.array_equal(x, y), f"{n} differs between runs"


def test_bwd_k256_workload_sampled_heads():
    """The head-dimension-256 shape of the FLA benchmark table (B=8, T=2048,
    H=32, D=256) at full size on the GPU; the oracle checks two sampled
    (row, head) pairs, all six gradients."""
    import gated_deltanet_chunked_chunk_amd as gdn
    name = "k256_bf16"
    c = gi.CONFIGS[name]
    B, T, H, D = c["B"], c["T"], c["Hv"], c["dk"]
    dev = torch.device("cuda")
    t = gi.make_device(B, T, c["Hqk"], H, D, c["dv"], c["seed"], device=dev)
    gen = torch.Generator(device=dev).manual_seed(c["seed"] + 1)
    do = torch.randn((B, T, H, c["dv"]), generator=gen, device=dev).to(torch.bfloat16)
    dht = 0.02 * torch.randn((B, H, D, c["dv"]), generator=gen, device=dev)
    print(f"[gpu bwd case] k256 workload B={B} T={T} H={H} D={D}", flush=True)
    got = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], do, dht=dht)
    torch.cuda.synchronize()
    for n in range(6):
        assert torch.isfinite(got[n]).all(), NAMES[n]
    for i, h in enumerate(gi.sampled_heads(c["seed"], H, n=2)):
        b = (3 + 4 * i) % B
        sl = lambda x: x[b:b + 1, :, h:h + 1].float().cpu().numpy()
        ref = oracle.gdn_bwd(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["g"]), sl(t["beta"]),
                             sl(do), dht=dht[b:b + 1, h:h + 1].double().cpu().numpy())
        for n, (x, y) in enumerate(zip(got, ref)):
            x = (x[b:b + 1, :, h:h + 1] if n < 5 else x[b:b + 1, h:h + 1]).float().cpu().numpy()
            e = rel_l2(x, y)
            tol = TOL_DH0 if NAMES[n] == "dh0" else TOL_BWD
            print(f"  (b={b}, h={h}) {NAMES[n]} rel-L2 {e:.2e}", flush=True)
            assert e <= tol, f"{NAMES[n]} (b={b}, h={h}) rel-L2 {e:.3e} > {tol}"
