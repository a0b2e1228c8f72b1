"""Seeded synthetic inputs for the gated delta rule forward.

This module is shared by the CPU oracle's tests and the HIP library's tests
and benchmark, and holds none of the method's arithmetic: it only draws
random tensors, shapes them, and rounds them to the input precision.

Recipe (the distributions come from the workloads the library is measured on;
the pages give q, k, v, a log-decay g and a write strength beta in the
jax-linear-attention page's "Quick start", where g = logsigmoid(noise)/4 and
beta = sigmoid(noise); the workloads here use /16 for g):

  * q, k ~ N(0, 1) per element, each (token, head) row L2-normalised in fp32;
  * v ~ N(0, 1);
  * beta = sigmoid(N(0, 1)), g = logsigmoid(N(0, 1)) / 16, both fp32;
  * bf16 inputs are the fp32 values rounded to nearest-even;
  * h0, when asked for, ~ N(0, std) in fp32 (std = 0.02 for packed batches);
  * packed lengths are geometric on {1, 2, ...} with the given mean, drawn
    until they cover the total, the last one clipped so the sum is exact;
  * for the backward, the upstream gradients: do ~ N(0, 1) in the input
    dtype and dht ~ N(0, 0.02) in fp32;
  * for the in-op preparation (make_raw), q and k rows ~ N(0, qk_std) left
    unnormalised and the raw gate values z ~ N(0, 1) in fp32, before
    logsigmoid and sigmoid;
  * for a decode step, one token per sequence of the same recipe and a state
    cache ~ N(0, 0.5) in fp32 (the scale of a state after a long prefill).

Every tensor draws from its own PCG64 stream spawned from the config seed, so
a tensor can be drawn in blocks of tokens (and the blocked draw equals the
whole draw; tested).  bf16 tensors are returned as uint16 bit patterns; use
`widen` for the exact fp32 values.
"""
import numpy as np

_STREAMS = ("q", "k", "v", "g", "beta", "h0", "lengths", "do", "dht")

# Elements drawn per block (bounds peak host memory for very long inputs).
_BLOCK_ELEMS = 1 << 24


def _streams(seed):
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(_STREAMS, children)}


def bf16_bits(x32):
    """Round fp32 values to bf16, nearest-even, as uint16 bit patterns.
    (Inputs here are finite and far from the fp32 range limits.)"""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    u = u + (((u >> 16) & 1) + np.uint32(0x7FFF))
    return (u >> 16).astype(np.uint16)


def widen(x):
    """Exact fp32 values of an input tensor (uint16 bf16 bits, or fp32)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return np.asarray(x, dtype=np.float32)


def _normal_rows(rng, rows, width, std=1.0, normalise=False, out_dtype="f32"):
    """rows x width N(0, std) draws, drawn in blocks of rows; optionally each
    row divided by its fp32 L2 norm; returned as fp32 or bf16 bits."""
    dt = np.uint16 if out_dtype == "bf16" else np.float32
    out = np.empty((rows, width), dtype=dt)
    step = max(1, _BLOCK_ELEMS // max(width, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = rng.standard_normal((r1 - r0, width), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if normalise:
            x /= np.sqrt(np.sum(x * x, axis=1, dtype=np.float32, keepdims=True))
        out[r0:r1] = bf16_bits(x) if out_dtype == "bf16" else x
    return out


def geometric_lengths(total, mean, seed):
    """Document lengths on {1, 2, ...}, geometric with the given mean, drawn
    until they cover `total` tokens; the last is clipped so they sum to it."""
    rng = _streams(seed)["lengths"]
    lengths = []
    s = 0
    while s < total:
        n = int(rng.geometric(1.0 / mean))
        n = min(n, total - s)
        lengths.append(n)
        s += n
    return lengths


def cu_from_lengths(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def make(B, T, Hqk, Hv, dk, dv, dtype, seed, h0_std=None, cu_seqlens=None):
    """Inputs for one forward call.

    Returns a dict with q, k [B, T, Hqk, dk], v [B, T, Hv, dv] (uint16 bf16
    bits, or fp32), g, beta [B, T, Hv] fp32, h0 [N, Hv, dk, dv] fp32 or None,
    cu_seqlens int32 [N + 1] or None, and the sizes."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    rs = _streams(seed)
    q = _normal_rows(rs["q"], B * T * Hqk, dk, normalise=True, out_dtype=dtype)
    k = _normal_rows(rs["k"], B * T * Hqk, dk, normalise=True, out_dtype=dtype)
    v = _normal_rows(rs["v"], B * T * Hv, dv, out_dtype=dtype)
    zg = rs["g"].standard_normal(B * T * Hv, dtype=np.float32).astype(np.float64)
    zb = rs["beta"].standard_normal(B * T * Hv, dtype=np.float32).astype(np.float64)
    # logsigmoid(z) = -log(1 + exp(-z)), sigmoid(z) = 1 / (1 + exp(-z))
    g = (-np.logaddexp(0.0, -zg) / 16.0).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    h0 = None
    if h0_std is not None:
        h0 = _normal_rows(rs["h0"], N * Hv * dk, dv, std=h0_std).reshape(N, Hv, dk, dv)
    return {
        "q": q.reshape(B, T, Hqk, dk), "k": k.reshape(B, T, Hqk, dk),
        "v": v.reshape(B, T, Hv, dv),
        "g": g.reshape(B, T, Hv), "beta": beta.reshape(B, T, Hv),
        "h0": h0,
        "cu_seqlens": None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int32),
        "dtype": dtype, "B": B, "T": T, "Hqk": Hqk, "Hv": Hv, "dk": dk, "dv": dv, "N": N,
    }


def make_raw(B, T, Hqk, Hv, dk, dv, dtype, seed, qk_std=1.0):
    """Inputs for a call with in-op preparation: q, k [B, T, Hqk, dk] rows
    ~ N(0, qk_std), not normalised; v [B, T, Hv, dv] ~ N(0, 1); and the raw
    gate values g, beta [B, T, Hv] ~ N(0, 1) fp32 (before logsigmoid and
    sigmoid).  Same dict layout as `make` (no h0, no cu_seqlens)."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    rs = _streams(seed)
    q = _normal_rows(rs["q"], B * T * Hqk, dk, std=qk_std, out_dtype=dtype)
    k = _normal_rows(rs["k"], B * T * Hqk, dk, std=qk_std, out_dtype=dtype)
    v = _normal_rows(rs["v"], B * T * Hv, dv, out_dtype=dtype)
    zg = rs["g"].standard_normal(B * T * Hv, dtype=np.float32)
    zb = rs["beta"].standard_normal(B * T * Hv, dtype=np.float32)
    return {
        "q": q.reshape(B, T, Hqk, dk), "k": k.reshape(B, T, Hqk, dk),
        "v": v.reshape(B, T, Hv, dv), "g": zg.reshape(B, T, Hv), "beta": zb.reshape(B, T, Hv),
        "h0": None, "cu_seqlens": None,
        "dtype": dtype, "B": B, "T": T, "Hqk": Hqk, "Hv": Hv, "dk": dk, "dv": dv, "N": B,
    }


def make_upstream(d, seed, dht_std=0.02):
    """Upstream gradients for the inputs `d` of `make`: do [B, T, Hv, dv] in
    d's dtype (uint16 bf16 bits or fp32) and dht [N, Hv, dk, dv] fp32, drawn
    from their own streams of `seed` (the seed `d` was made with)."""
    rs = _streams(seed)
    B, T, Hv, dv, dk, N = d["B"], d["T"], d["Hv"], d["dv"], d["dk"], d["N"]
    do = _normal_rows(rs["do"], B * T * Hv, dv, out_dtype=d["dtype"]).reshape(B, T, Hv, dv)
    dht = _normal_rows(rs["dht"], N * Hv * dk, dv, std=dht_std).reshape(N, Hv, dk, dv)
    return do, dht


# The workloads: a tiny fp32 case, the 8 x 2K headline, a packed batch with
# grouped value heads, and one long row.  Seeds are 1000 + index.
CONFIGS = {
    "tiny_f32": dict(B=1, T=256, Hqk=2, Hv=2, dk=64, dv=64, dtype="f32", seed=1000),
    "headline_bf16": dict(B=8, T=2048, Hqk=16, Hv=16, dk=128, dv=128, dtype="bf16",
                          seed=1001),
    "packed_gva_bf16": dict(total=16384, mean_len=1024, Hqk=16, Hv=32, dk=128, dv=128,
                            dtype="bf16", seed=1002, h0_std=0.02),
    "long_bf16": dict(B=1, T=1_064_960, Hqk=16, Hv=16, dk=128, dv=128, dtype="bf16",
                      seed=1003),
    # the headline inputs with upstream gradients, for the backward
    "fwd_bwd_bf16": dict(B=8, T=2048, Hqk=16, Hv=16, dk=128, dv=128, dtype="bf16", seed=1004),
    # one decode step: 256 sequences of one token, a 256-slot state cache (h0)
    "decode_bf16": dict(B=256, T=1, Hqk=16, Hv=16, dk=128, dv=128, dtype="bf16", seed=1005,
                        h0_std=0.5),
    # head dim 256: the shape of the B=8, T=2048, H=32, D=256 row of the
    # flash-linear-attention benchmark table (drawn on the device)
    "k256_bf16": dict(B=8, T=2048, Hqk=32, Hv=32, dk=256, dv=256, dtype="bf16", seed=1006),
    # head dimension 64 with upstream gradients, the shape of the B=8, T=1024,
    # H=8, D=64 row of the flash-linear-attention benchmark table
    "fwd_bwd_dk64_bf16": dict(B=8, T=1024, Hqk=8, Hv=8, dk=64, dv=64, dtype="bf16", seed=1008),
    # one long row at head dimension 256 and 8 heads (drawn on the device)
    "long_k256_bf16": dict(B=1, T=65536, Hqk=8, Hv=8, dk=256, dv=256, dtype="bf16", seed=1007),
    # packed documents at few heads: one row of 8 heads, 16,384 tokens in
    # geometric documents of mean length 1024 (about 16 documents)
    "packed_8h_bf16": dict(total=16384, mean_len=1024, Hqk=8, Hv=8, dk=128, dv=128,
                           dtype="bf16", seed=1009, h0_std=0.02),
    # packed documents at few heads with one long document: one row of 8
    # heads, 30,000 tokens, a 20,000-token document among seven short ones
    "packed_long_doc_bf16": dict(lengths=[20000, 2000, 1500, 3000, 900, 1100, 800, 700],
                                 Hqk=8, Hv=8, dk=128, dv=128, dtype="bf16", seed=1010,
                                 h0_std=0.02),
}


def make_device(B, T, Hqk, Hv, dk, dv, seed, device="cuda"):
    """Inputs of the same recipe (bf16 q, k, v; fp32 g, beta; no initial
    state) drawn on the device with torch's Philox generator seeded with
    `seed`, for workloads too large to draw on the host in reasonable time
    (the long row: 6.5e9 normal draws).  Rows are drawn in blocks, so peak
    device memory stays near the size of the returned tensors.  Returns device
    tensors q, k [B, T, Hqk, dk], v [B, T, Hv, dv] (bf16) and g, beta
    [B, T, Hv] (fp32)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def rows(n, width, normalise):
        out = torch.empty((n, width), dtype=torch.bfloat16, device=device)
        step = max(1, (1 << 26) // width)
        for r0 in range(0, n, step):
            r1 = min(n, r0 + step)
            x = torch.randn((r1 - r0, width), generator=gen, device=device, dtype=torch.float32)
            if normalise:
                x /= torch.sqrt(torch.sum(x * x, dim=1, keepdim=True))
            out[r0:r1] = x.to(torch.bfloat16)  # round to nearest even
        return out

    q = rows(B * T * Hqk, dk, True).view(B, T, Hqk, dk)
    k = rows(B * T * Hqk, dk, True).view(B, T, Hqk, dk)
    v = rows(B * T * Hv, dv, False).view(B, T, Hv, dv)
    zg = torch.randn(B * T * Hv, generator=gen, device=device, dtype=torch.float32)
    zb = torch.randn(B * T * Hv, generator=gen, device=device, dtype=torch.float32)
    g = (torch.nn.functional.logsigmoid(zg) / 16.0).view(B, T, Hv)
    beta = torch.sigmoid(zb).view(B, T, Hv)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta,
            "B": B, "T": T, "Hqk": Hqk, "Hv": Hv, "dk": dk, "dv": dv}


def sampled_heads(seed, Hv, n=2):
    """The v-heads a test compares with the oracle, drawn with the seed."""
    rng = np.random.default_rng(seed)
    return sorted(int(j) for j in rng.choice(Hv, size=n, replace=False))


def make_config(name, **override):
    """Inputs of a named workload; keyword overrides change its sizes (tests
    use them to shrink a workload while keeping its recipe)."""
    c = dict(CONFIGS[name])
    c.update(override)
    if "total" in c or "lengths" in c:
        lengths = c.get("lengths") or geometric_lengths(c["total"], c["mean_len"], c["seed"])
        cu = cu_from_lengths(lengths)
        return make(1, int(cu[-1]), c["Hqk"], c["Hv"], c["dk"], c["dv"], c["dtype"],
                    c["seed"], h0_std=c.get("h0_std"), cu_seqlens=cu)
    return make(c["B"], c["T"], c["Hqk"], c["Hv"], c["dk"], c["dv"], c["dtype"], c["seed"],
                h0_std=c.get("h0_std"))
