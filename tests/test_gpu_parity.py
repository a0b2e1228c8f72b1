"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case uses the seeded generator with the workloads' recipe; sizes span
several chunks and a ragged tail, and the named workloads run at full size.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gpu_util import TOL, check, rel_l2, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu


def test_tiny_fp32_workload():
    """B=1, T=256, H=2, d=64, fp32: the whole workload."""
    check(gi.make_config("tiny_f32"), label="tiny fp32")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_fp32_ragged(T):
    d = gi.make(2, T, 2, 4, 64, 128, "f32", 2000 + T, h0_std=0.5)
    check(d, scale=0.75, label=f"fp32 ragged T={T}")


def test_fp32_dk128():
    check(gi.make(1, 130, 1, 2, 128, 64, "f32", 2100, h0_std=0.1), label="fp32 dk128 dv64")


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 200])
def test_bf16_ragged(T):
    """Several chunks and a ragged tail, grouped heads, an initial state, a scale."""
    d = gi.make(2, T, 2, 4, 128, 128, "bf16", 3000 + T, h0_std=0.3)
    check(d, scale=0.5, label=f"bf16 ragged T={T}")


def test_bf16_dv64():
    check(gi.make(2, 190, 3, 3, 128, 64, "bf16", 3300, h0_std=0.1), label="bf16 dv64")


def test_bf16_strong_decay_and_zero_beta():
    """Extremes of the gates: g = -30 (near-total forgetting) on some tokens,
    beta = 0 on others, g = 0 on the rest."""
    d = gi.make(1, 300, 2, 2, 128, 128, "bf16", 3400, h0_std=0.2)
    rng = np.random.default_rng(0)
    sel = rng.random(d["g"].shape)
    d["g"] = np.where(sel < 0.1, np.float32(-30.0), np.where(sel < 0.3, np.float32(0.0), d["g"]))
    d["beta"] = np.where(rng.random(d["beta"].shape) < 0.2, np.float32(0.0), d["beta"])
    check(d, label="bf16 gate extremes")


@pytest.mark.parametrize("g", [-0.1, -0.3, -1.0])
def test_bf16_steady_decay_rescaling(g):
    """Steady decays of about g per token: the state loses a factor of e^6 to
    e^64 per chunk, so the carried state ranges from mattering over several
    chunks to vanishing within one."""
    d = gi.make(1, 400, 2, 2, 128, 128, "bf16", 3500, h0_std=0.3)
    rng = np.random.default_rng(1)
    d["g"] = (g * (1.0 + 0.1 * rng.standard_normal(d["g"].shape))).astype(np.float32)
    check(d, label=f"bf16 steady decay {g}")


def test_bf16_negative_scale():
    """A negative attention scale."""
    d = gi.make(1, 150, 2, 2, 128, 128, "bf16", 3600, h0_std=0.2)
    check(d, scale=-0.25, label="bf16 negative scale")


def test_headline_workload_full_size():
    """B=8, T=2048, H=16, d=128, bf16, zero state: the benchmarked launch."""
    check(gi.make_config("headline_bf16"), label="headline 8x2048x16x128")


def test_packed_grouped_workload_full_size():
    """16,384 tokens in geometric documents, H_qk=16, H_v=32, h0 ~ N(0, 0.02)."""
    check(gi.make_config("packed_gva_bf16"), label="packed GVA 16384")


def test_packed_equals_separate_bitwise():
    """A packed row gives the per-document results bit for bit: each document
    starts its own chunks, so its arithmetic does not depend on its offset."""
    lengths = [1, 130, 0, 64, 77, 5]
    cu = gi.cu_from_lengths(lengths)
    d = gi.make(1, int(cu[-1]), 2, 4, 128, 128, "bf16", 3500, h0_std=0.1, cu_seqlens=cu)
    o, ht = run_gpu(d)
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            assert np.array_equal(ht[n], d["h0"][n]), "empty document changed its state"
            continue
        dn = dict(d, q=d["q"][:, a:b], k=d["k"][:, a:b], v=d["v"][:, a:b], g=d["g"][:, a:b],
                  beta=d["beta"][:, a:b], h0=d["h0"][n:n + 1], cu_seqlens=None, T=b - a, N=1)
        on, hn = run_gpu(dn)
        assert np.array_equal(o[:, a:b], on), f"document {n}: output differs"
        assert np.array_equal(ht[n:n + 1], hn), f"document {n}: state differs"


def test_packed_order_is_bitwise_neutral():
    """Scheduling the documents longest first (the workspace's order array)
    changes no arithmetic: with the order, without it (no workspace: index
    order), and planned from the host copy or not, the results are bitwise
    equal when the plan splits no document."""
    import gated_deltanet_chunked_chunk_amd as gdn
    d = gi.make_config("packed_gva_bf16", total=3000)
    cu = [int(x) for x in d["cu_seqlens"]]
    pl, _, ordered = gdn.gdn_chunk_fwd_plan(1, 1, d["T"], d["Hqk"], d["Hv"], 128, 128, cu)
    assert pl == 0 and ordered
    o1, h1 = run_gpu(d, host_cu=True)
    o2, h2 = run_gpu(d, host_cu=False)
    t = to_device(d)
    o3, h3 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"],
                               cu_seqlens=t["cu"], pieces=False)
    torch.cuda.synchronize()
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)
    assert np.array_equal(o1, o3.float().cpu().numpy()) and np.array_equal(h1, h3.cpu().numpy())


PACKED_PIECE_CASES = [
    # label, lengths (or a geometric draw), H_qk, H_v, dk, dv, h0 std, decay divisor
    ("one long document of eight x 8 heads", [8000, 700, 500, 1200, 300, 64, 0, 900], 8, 8,
     128, 128, 0.02, 1),
    ("one long document", [12000, 300, 0, 77, 1500], 2, 4, 128, 128, 0.3, 8),
    ("dk64", [9000, 0, 2500, 640, 1], 1, 2, 64, 128, 0.3, 8),
    ("dk256", [6000, 33, 0, 2100], 1, 2, 256, 128, 0.1, 8),
]


@pytest.mark.parametrize("case", PACKED_PIECE_CASES, ids=lambda c: c[0].replace(" ", "_"))
def test_packed_piece_scan(case):
    """Long documents of a packed call split into pieces (planned from the
    host copy of cu_seqlens): against the oracle on every (document, head)
    and against whole documents (no workspace)."""
    import gated_deltanet_chunked_chunk_amd as gdn
    label, lengths, Hqk, Hv, dk, dv, h0_std, div = case
    cu = gi.cu_from_lengths(lengths)
    T = int(cu[-1])
    d = gi.make(1, T, Hqk, Hv, dk, dv, "bf16", 5100 + T % 97, h0_std=h0_std, cu_seqlens=cu)
    d["g"] = (d["g"] / div).astype(np.float32)
    pl, slots, _ = gdn.gdn_chunk_fwd_plan(1, 1, T, Hqk, Hv, dk, dv, [int(x) for x in cu])
    print(f"[gpu case] packed pieces {label}: {len(lengths)} documents, piece length {pl}, "
          f"{slots} slots", flush=True)
    assert pl > 0 and slots > 0
    check(d, scale=0.9, label=f"packed pieces {label}")
    o1, h1 = run_gpu(d, scale=0.9)
    t = to_device(d)
    o2, h2 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=0.9,
                               initial_state=t["h0"], cu_seqlens=t["cu"], pieces=False)
    torch.cuda.synchronize()
    tol_o, tol_h = TOL["bf16"]
    assert rel_l2(o1, o2.float().cpu().numpy()) <= tol_o
    assert rel_l2(h1, h2.cpu().numpy()) <= tol_h


def test_packed_piece_scan_carries_state():
    """No decay and a weak write (g = 0, beta = 0.02) across the pieces of a
    long document, with a large initial state: the start states the scan
    hands over carry most of the result."""
    import gated_deltanet_chunked_chunk_amd as gdn
    cu = gi.cu_from_lengths([10000, 50, 3000, 0])
    T = int(cu[-1])
    d = gi.make(1, T, 1, 2, 128, 128, "bf16", 5200, h0_std=1.0, cu_seqlens=cu)
    d["g"] = np.zeros_like(d["g"])
    d["beta"] = np.full_like(d["beta"], 0.02)
    pl, slots, _ = gdn.gdn_chunk_fwd_plan(1, 1, T, 1, 2, 128, 128, [int(x) for x in cu])
    assert pl > 0 and slots > 0
    check(d, label="packed pieces, g = 0, beta = 0.02")


def test_chained_halves():
    """A long row run whole equals its two halves with the state passed on."""
    d = gi.make(1, 4096 + 37, 2, 2, 128, 128, "bf16", 3600)
    o, ht = run_gpu(d)
    s = 2048 + 13
    d1 = dict(d, q=d["q"][:, :s], k=d["k"][:, :s], v=d["v"][:, :s], g=d["g"][:, :s],
              beta=d["beta"][:, :s], T=s)
    o1, h1 = run_gpu(d1)
    d2 = dict(d, q=d["q"][:, s:], k=d["k"][:, s:], v=d["v"][:, s:], g=d["g"][:, s:],
              beta=d["beta"][:, s:], h0=h1, T=d["T"] - s)
    o2, h2 = run_gpu(d2)
    tol_o, tol_h = TOL["bf16"]
    assert rel_l2(np.concatenate([o1, o2], axis=1), o) <= tol_o
    assert rel_l2(h2, ht) <= tol_h
    ro, rht = run_oracle(d)
    assert rel_l2(o2, ro[:, s:]) <= tol_o and rel_l2(h2, rht) <= tol_h


def test_long_row_full_size():
    """The long row (T = 1,064,960; 16,640 chunks per head) at full size: run
    whole (the piece scan: 8 pieces per head) and as two chained halves (8
    pieces each), which agree within tolerance, and compared with the oracle
    on two sampled heads; the whole row without the piece scan agrees too."""
    import gated_deltanet_chunked_chunk_amd as gdn
    c = gi.CONFIGS["long_bf16"]
    B, T, H, dk, dv = c["B"], c["T"], c["Hv"], c["dk"], c["dv"]
    print(f"[gpu case] long row B={B} T={T} H={H} dk={dk} dv={dv} bf16 (device-drawn inputs)",
          flush=True)
    t = gi.make_device(B, T, c["Hqk"], H, dk, dv, c["seed"])
    q, k, v, g, beta = (t[x] for x in ("q", "k", "v", "g", "beta"))
    o, ht = gdn.gdn_chunk_fwd(q, k, v, g, beta)
    s = T // 2
    o1, h1 = gdn.gdn_chunk_fwd(q[:, :s], k[:, :s], v[:, :s], g[:, :s], beta[:, :s])
    o2, h2 = gdn.gdn_chunk_fwd(q[:, s:], k[:, s:], v[:, s:], g[:, s:], beta[:, s:],
                               initial_state=h1)
    o3, h3 = gdn.gdn_chunk_fwd(q, k, v, g, beta, pieces=False)
    torch.cuda.synchronize()
    tol_o, tol_h = TOL["bf16"]
    f = lambda x: x.float().cpu().numpy()
    e_halves = (rel_l2(f(torch.cat([o1, o2], dim=1)), f(o)), rel_l2(f(h2), f(ht)))
    e_serial = (rel_l2(f(o3), f(o)), rel_l2(f(h3), f(ht)))
    print(f"  halves vs whole {e_halves[0]:.2e} {e_halves[1]:.2e}; whole rows vs pieces "
          f"{e_serial[0]:.2e} {e_serial[1]:.2e}", flush=True)
    assert e_halves[0] <= tol_o and e_halves[1] <= tol_h
    assert e_serial[0] <= tol_o and e_serial[1] <= tol_h
    heads = gi.sampled_heads(c["seed"], H)
    sel = lambda x: x[:, :, heads].float().cpu().numpy()
    ro, rht = run_oracle({"q": sel(q), "k": sel(k), "v": sel(v), "g": sel(g), "beta": sel(beta),
                          "h0": None, "cu_seqlens": None})
    eo = rel_l2(sel(o), ro)
    eh = rel_l2(ht[:, heads].cpu().numpy(), rht)
    print(f"  heads {heads}: rel-L2 output {eo:.3e} (tol {tol_o:.0e}), state {eh:.3e} "
          f"(tol {tol_h:.0e})", flush=True)
    assert eo <= tol_o and eh <= tol_h


def test_deterministic():
    d = gi.make(2, 333, 2, 2, 128, 128, "bf16", 3700, h0_std=0.1)
    a = run_gpu(d)
    b = run_gpu(d)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_nan_stays_in_its_document():
    """A NaN in one document's values leaves every other document finite and
    unchanged."""
    cu = gi.cu_from_lengths([100, 100, 100])
    d = gi.make(1, 300, 1, 2, 128, 128, "bf16", 3800, h0_std=0.1, cu_seqlens=cu)
    o_ref, h_ref = run_gpu(d)
    v = d["v"].copy()
    v[0, 150, 0, 3] = 0x7FC0  # bf16 quiet NaN in document 1, value head 0
    o, ht = run_gpu(dict(d, v=v))
    assert np.array_equal(o[:, :100], o_ref[:, :100]) and np.array_equal(o[:, 200:], o_ref[:, 200:])
    assert np.array_equal(ht[0], h_ref[0]) and np.array_equal(ht[2], h_ref[2])
    assert not np.all(np.isfinite(o[:, 150:200, 0]))


def test_no_final_state_and_preallocated_output():
    import gated_deltanet_chunked_chunk_amd as gdn
    from gpu_util import to_device
    d = gi.make(1, 100, 1, 1, 128, 128, "bf16", 3900)
    t = to_device(d)
    out = torch.full((1, 100, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], out=out,
                              output_final_state=False)
    torch.cuda.synchronize()
    assert ht is None and o.data_ptr() == out.data_ptr()
    ro, _ = run_oracle(d)
    assert rel_l2(o.float().cpu().numpy(), ro) <= TOL["bf16"][0]


PIECE_CASES = [
    # B, T, Hqk, Hv, dv, h0 std, pieces the host plan picks
    (1, 4096 + 37, 1, 2, 128, 0.1, 6),  # ragged last piece, grouped heads
    (2, 6000, 1, 1, 64, 0.1, 8),        # two rows, dv = 64, a partial last chunk
    (1, 4096, 1, 1, 128, None, 6),      # 11-chunk pieces, a 9-chunk last piece
]


@pytest.mark.parametrize("case", PIECE_CASES, ids=lambda c: f"B{c[0]}-T{c[1]}-dv{c[4]}")
def test_piece_scan_matches_oracle(case):
    """The piece scan (zero-start ends and transitions, the scan of start
    states, the output pass) against the oracle and against whole rows."""
    import gated_deltanet_chunked_chunk_amd as gdn
    B, T, Hqk, Hv, dv, h0_std, pieces = case
    lib = gdn.load()
    need = lib.gdn_chunk_fwd_workspace_size(1, B, T, Hqk, Hv, 128, dv, B)
    per = B * (pieces - 1) * Hv * 128
    assert need == -(-per * (dv + 128) * 4 // 256) * 256 + per * dv * 4
    d = gi.make(B, T, Hqk, Hv, 128, dv, "bf16", 3900 + T, h0_std=h0_std)
    check(d, scale=0.8, label=f"piece scan, {pieces} pieces")
    o1, h1 = run_gpu(d, scale=0.8)
    from gpu_util import to_device
    t = to_device(d)
    o2, h2 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=0.8,
                               initial_state=t["h0"], pieces=False)
    tol_o, tol_h = TOL["bf16"]
    assert rel_l2(o1, o2.float().cpu().numpy()) <= tol_o
    assert rel_l2(h1, h2.cpu().numpy()) <= tol_h


def test_piece_scan_carries_state():
    """No decay and a weak write (g = 0, beta = 0.02): each piece's transition
    stays near the identity, so the start states the scan hands over carry
    most of the result; 6 pieces of 11 chunks, a large initial state."""
    d = gi.make(1, 4096 + 37, 1, 2, 128, 128, "bf16", 3950, h0_std=1.0)
    d["g"] = np.zeros_like(d["g"])
    d["beta"] = np.full_like(d["beta"], 0.02)
    check(d, label="piece scan, g = 0, beta = 0.02")


def test_piece_scan_with_in_op_preparation():
    import gated_deltanet_chunked_chunk_amd as gdn
    import oracle
    from oracle import prep
    from gpu_util import to_device
    d = gi.make_raw(1, 4096 + 37, 1, 2, 128, 128, "bf16", 3960, qk_std=2.0)
    print("[gpu case] piece scan with in-op preparation", flush=True)
    t = to_device(d)
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], use_qk_l2norm=True,
                              gate_activation=True)
    torch.cuda.synchronize()
    # The fused normalisation is applied in fp32 (rows never rounded to bf16).
    qn, kn = (prep.l2_normalize(gi.widen(d[x])).astype(np.float32) for x in ("q", "k"))
    ro, rht = oracle.gdn_fwd(qn, kn, gi.widen(d["v"]), prep.logsigmoid(d["g"]).astype(np.float32),
                             prep.sigmoid(d["beta"]).astype(np.float32))
    tol_o, tol_h = TOL["bf16"]
    eo, eh = rel_l2(o.float().cpu().numpy(), ro), rel_l2(ht.cpu().numpy(), rht)
    print(f"  rel-L2 output {eo:.3e}, state {eh:.3e}", flush=True)
    assert eo <= tol_o and eh <= tol_h


@pytest.mark.parametrize("T,dv", [(1, 128), (65, 64), (200, 128)])
def test_bf16_dk64(T, dv):
    """bf16 with dk = 64 (the key rows are staged into the 128-wide LDS
    layout with zero upper halves): ragged T, grouped heads, h0, scale."""
    d = gi.make(2, T, 1, 2, 64, dv, "bf16", 4100 + T, h0_std=0.1)
    check(d, scale=0.9, label=f"bf16 dk64 T={T} dv={dv}")


def test_bf16_dk64_packed_with_empty_document():
    cu = gi.cu_from_lengths([70, 0, 129, 1])
    d = gi.make(1, 200, 2, 4, 64, 64, "bf16", 4150, h0_std=0.05, cu_seqlens=cu)
    check(d, label="bf16 dk64 packed")


def test_bf16_dk64_piece_scan():
    """dk = 64 through the piece scan: 11 pieces of 6 chunks, one transition
    tile."""
    d = gi.make(1, 4096 + 37, 1, 2, 64, 128, "bf16", 4160, h0_std=0.5)
    d["g"] = (d["g"] / 8).astype(np.float32)  # slower decay: carried states matter
    eo, eh = check(d, label="bf16 dk64 piece scan")
    import gated_deltanet_chunked_chunk_amd as gdn
    from gpu_util import to_device
    t = to_device(d)
    o2, h2 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"],
                               pieces=False)
    ro, rht = run_oracle(d)
    ew = (rel_l2(o2.float().cpu().numpy(), ro), rel_l2(h2.cpu().numpy(), rht))
    print(f"  whole rows: rel-L2 output {ew[0]:.3e}, state {ew[1]:.3e}", flush=True)
    assert ew[0] <= TOL["bf16"][0] and ew[1] <= TOL["bf16"][1]


def test_many_short_documents():
    """1,000 packed documents of 0 to 20 tokens (most shorter than one
    chunk, some empty), with initial states, grouped heads (ratio 4): the
    call planned with the host copy of cu_seqlens and the one without agree
    bitwise (no document is split), and both match the oracle."""
    rng = np.random.default_rng(4200)
    lengths = [int(x) for x in rng.integers(0, 21, size=1000)]
    cu = gi.cu_from_lengths(lengths)
    d = gi.make(1, int(cu[-1]), 1, 4, 128, 64, "bf16", 4200, h0_std=0.1, cu_seqlens=cu)
    check(d, label="1000 short documents")
    o1, h1 = run_gpu(d)
    o2, h2 = run_gpu(d, host_cu=False)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


def test_grouped_heads_ratio_four_fp32():
    d = gi.make(2, 130, 1, 4, 64, 64, "f32", 4300, h0_std=0.2)
    check(d, scale=0.6, label="fp32 GVA ratio 4")


@pytest.mark.parametrize("T,dv", [(1, 128), (31, 64), (32, 256), (33, 128), (200, 128)])
def test_bf16_dk256(T, dv):
    """bf16 with dk = 256 (chunks of 32 tokens): ragged T around one chunk,
    grouped heads, h0, scale, dv in {64, 128, 256}."""
    d = gi.make(2, T, 1, 2, 256, dv, "bf16", 4400 + T, h0_std=0.1)
    check(d, scale=0.8, label=f"bf16 dk256 T={T} dv={dv}")


def test_bf16_dk256_packed_with_empty_document():
    cu = gi.cu_from_lengths([45, 0, 97, 1, 32])
    d = gi.make(1, 175, 2, 4, 256, 64, "bf16", 4450, h0_std=0.05, cu_seqlens=cu)
    check(d, label="bf16 dk256 packed")


def test_bf16_dk256_slow_decay():
    """Slower decay, so states carried over many chunks matter."""
    d = gi.make(1, 700, 1, 2, 256, 128, "bf16", 4460, h0_std=0.5)
    d["g"] = (d["g"] / 8).astype(np.float32)
    check(d, label="bf16 dk256 slow decay")


@pytest.mark.parametrize("T", [1, 31, 33, 100])
def test_fp32_dk256(T):
    d = gi.make(1, T, 1, 2, 256, 64, "f32", 4470 + T, h0_std=0.2)
    check(d, scale=0.7, label=f"fp32 dk256 T={T}")


def test_bf16_dv256():
    check(gi.make(1, 150, 2, 2, 128, 256, "bf16", 4480, h0_std=0.1), label="bf16 dk128 dv256")


def test_k256_workload_full_size():
    """B=8, T=2048, H=32, dk=dv=256 (device-drawn inputs), compared with the
    oracle on two sampled heads."""
    import gated_deltanet_chunked_chunk_amd as gdn
    c = gi.CONFIGS["k256_bf16"]
    B, T, H, dk, dv = c["B"], c["T"], c["Hv"], c["dk"], c["dv"]
    print(f"[gpu case] k256 B={B} T={T} H={H} dk={dk} dv={dv} bf16 (device-drawn inputs)",
          flush=True)
    t = gi.make_device(B, T, c["Hqk"], H, dk, dv, c["seed"])
    q, k, v, g, beta = (t[x] for x in ("q", "k", "v", "g", "beta"))
    o, ht = gdn.gdn_chunk_fwd(q, k, v, g, beta)
    torch.cuda.synchronize()
    heads = gi.sampled_heads(c["seed"], H)
    sel = lambda x: x[:, :, heads].float().cpu().numpy()
    ro, rht = run_oracle({"q": sel(q), "k": sel(k), "v": sel(v), "g": sel(g), "beta": sel(beta),
                          "h0": None, "cu_seqlens": None})
    eo = rel_l2(sel(o), ro)
    eh = rel_l2(ht[:, heads].cpu().numpy(), rht)
    tol_o, tol_h = TOL["bf16"]
    print(f"  heads {heads}: rel-L2 output {eo:.3e} (tol {tol_o:.0e}), state {eh:.3e} "
          f"(tol {tol_h:.0e})", flush=True)
    assert eo <= tol_o and eh <= tol_h


def _dk256_piece_check(d, pieces, label):
    """The piece scan at dk = 256 against the oracle and against whole rows."""
    import gated_deltanet_chunked_chunk_amd as gdn
    from gpu_util import to_device
    B, T, Hqk, Hv, dv = d["B"], d["T"], d["Hqk"], d["Hv"], d["dv"]
    per = B * (pieces - 1) * Hv * 256
    assert gdn.load().gdn_chunk_fwd_workspace_size(1, B, T, Hqk, Hv, 256, dv, B) == \
        -(-per * (dv + 256) * 4 // 256) * 256 + per * dv * 4
    check(d, label=f"{label}, {pieces} pieces")
    o1, h1 = run_gpu(d)
    t = to_device(d)
    o2, h2 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"],
                               pieces=False)
    e = (rel_l2(o1, o2.float().cpu().numpy()), rel_l2(h1, h2.cpu().numpy()))
    print(f"  pieces vs whole rows: output {e[0]:.3e}, state {e[1]:.3e}", flush=True)
    tol_o, tol_h = TOL["bf16"]
    assert e[0] <= tol_o and e[1] <= tol_h


def test_bf16_dk256_piece_scan():
    """dk = 256 through the piece scan (four transition tiles per piece, the
    scan staging Phi in 64-column blocks): 4 pieces of 1,088 tokens."""
    d = gi.make(1, 4096 + 37, 1, 2, 256, 128, "bf16", 4490, h0_std=0.5)
    d["g"] = (d["g"] / 8).astype(np.float32)
    _dk256_piece_check(d, 4, "bf16 dk256 piece scan")


def test_bf16_dk256_piece_scan_carries_state():
    """No decay and a weak write (g = 0, beta = 0.02) at dk = 256: every
    piece's transition stays near the identity, so the scanned start states
    (all four 64-column blocks of Phi) carry most of the result."""
    d = gi.make(1, 5000 + 37, 1, 2, 256, 64, "bf16", 4495, h0_std=1.0)
    d["g"] = np.zeros_like(d["g"])
    d["beta"] = np.full_like(d["beta"], 0.02)
    _dk256_piece_check(d, 4, "bf16 dk256 piece scan, g = 0, beta = 0.02")


def test_bf16_dk256_piece_scan_with_in_op_preparation():
    import gated_deltanet_chunked_chunk_amd as gdn
    import oracle
    from oracle import prep
    from gpu_util import to_device
    d = gi.make_raw(1, 4096 + 37, 1, 2, 256, 128, "bf16", 4497, qk_std=2.0)
    print("[gpu case] dk256 piece scan with in-op preparation", flush=True)
    t = to_device(d)
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], use_qk_l2norm=True,
                              gate_activation=True)
    torch.cuda.synchronize()
    qn, kn = (prep.l2_normalize(gi.widen(d[x])).astype(np.float32) for x in ("q", "k"))
    ro, rht = oracle.gdn_fwd(qn, kn, gi.widen(d["v"]), prep.logsigmoid(d["g"]).astype(np.float32),
                             prep.sigmoid(d["beta"]).astype(np.float32))
    tol_o, tol_h = TOL["bf16"]
    eo, eh = rel_l2(o.float().cpu().numpy(), ro), rel_l2(ht.cpu().numpy(), rht)
    print(f"  rel-L2 output {eo:.3e}, state {eh:.3e}", flush=True)
    assert eo <= tol_o and eh <= tol_h


def test_long_k256_row_full_size():
    """One row of 65,536 tokens at dk = dv = 256, 8 heads (device-drawn): the
    piece scan against whole rows, and both against the oracle on two sampled
    heads."""
    import gated_deltanet_chunked_chunk_amd as gdn
    c = gi.CONFIGS["long_k256_bf16"]
    B, T, H, dk, dv = c["B"], c["T"], c["Hv"], c["dk"], c["dv"]
    print(f"[gpu case] long row B={B} T={T} H={H} dk={dk} dv={dv} bf16 (device-drawn inputs)",
          flush=True)
    t = gi.make_device(B, T, c["Hqk"], H, dk, dv, c["seed"])
    q, k, v, g, beta = (t[x] for x in ("q", "k", "v", "g", "beta"))
    assert gdn.gdn_chunk_fwd_workspace_size(1, B, T, H, H, dk, dv, B) > 0
    o, ht = gdn.gdn_chunk_fwd(q, k, v, g, beta)
    o2, h2 = gdn.gdn_chunk_fwd(q, k, v, g, beta, pieces=False)
    torch.cuda.synchronize()
    tol_o, tol_h = TOL["bf16"]
    f = lambda x: x.float().cpu().numpy()
    e = (rel_l2(f(o2), f(o)), rel_l2(f(h2), f(ht)))
    print(f"  whole rows vs pieces {e[0]:.2e} {e[1]:.2e}", flush=True)
    assert e[0] <= tol_o and e[1] <= tol_h
    heads = gi.sampled_heads(c["seed"], H)
    sel = lambda x: x[:, :, heads].float().cpu().numpy()
    ro, rht = run_oracle({"q": sel(q), "k": sel(k), "v": sel(v), "g": sel(g), "beta": sel(beta),
                          "h0": None, "cu_seqlens": None})
    eo, eh = rel_l2(sel(o), ro), rel_l2(ht[:, heads].cpu().numpy(), rht)
    print(f"  heads {heads}: rel-L2 output {eo:.3e} (tol {tol_o:.0e}), state {eh:.3e} "
          f"(tol {tol_h:.0e})", flush=True)
    assert eo <= tol_o and eh <= tol_h
