"""The seeded input generator (shared by both sides; holds no method arithmetic)."""
import numpy as np
import torch

import gdn_inputs as gi


def test_bf16_rounding_is_nearest_even():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100_000).astype(np.float32) * 3
    # exact ties: bf16 value plus half an ulp, in both parities
    base = gi.widen(gi.bf16_bits(x[:1000]))
    ulp_half = (base.view(np.uint32) & 0xFF800000).view(np.float32) * np.float32(2.0 ** -8)
    x = np.concatenate([x, base + ulp_half, -(base + ulp_half)])
    ours = gi.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(gi.widen(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_blocked_draw_equals_whole_draw(monkeypatch):
    whole = gi.make(2, 40, 2, 4, 8, 8, "bf16", 7, h0_std=0.02)
    monkeypatch.setattr(gi, "_BLOCK_ELEMS", 24)  # 3 rows of 8 per block
    blocked = gi.make(2, 40, 2, 4, 8, 8, "bf16", 7, h0_std=0.02)
    for name in ("q", "k", "v", "g", "beta", "h0"):
        assert np.array_equal(whole[name], blocked[name]), name


def test_recipe_properties():
    d = gi.make_config("headline_bf16", B=2, T=128, Hqk=4, Hv=4)
    assert d["q"].shape == (2, 128, 4, 128) and d["q"].dtype == np.uint16
    for name in ("q", "k"):
        n = np.linalg.norm(gi.widen(d[name]).astype(np.float64), axis=-1)
        assert np.all(np.abs(n - 1) < 1e-2)
    assert np.all(d["g"] < 0) and np.all(d["g"] > -2)
    assert np.all(d["beta"] > 0) and np.all(d["beta"] < 1)
    assert d["h0"] is None and d["cu_seqlens"] is None
    again = gi.make_config("headline_bf16", B=2, T=128, Hqk=4, Hv=4)
    assert np.array_equal(d["v"], again["v"])
    t = gi.make_config("tiny_f32")
    assert t["q"].dtype == np.float32 and t["q"].shape == (1, 256, 2, 64)


def test_packed_lengths():
    lengths = gi.geometric_lengths(16384, 1024, 1002)
    assert sum(lengths) == 16384 and min(lengths) >= 1
    d = gi.make_config("packed_gva_bf16", total=4096)
    cu = d["cu_seqlens"]
    assert cu[0] == 0 and cu[-1] == 4096 and np.all(np.diff(cu) >= 1)
    assert d["h0"].shape == (len(cu) - 1, 32, 128, 128)
    assert abs(float(d["h0"].std()) - 0.02) < 1e-3


def test_device_draw_recipe_on_cpu():
    """The device-side generator (used for the long row) keeps the recipe:
    unit q/k rows before the bf16 cast, g <= 0, 0 < beta < 1, seeded."""
    import torch
    a = gi.make_device(1, 300, 2, 4, 64, 32, seed=9, device="cpu")
    b = gi.make_device(1, 300, 2, 4, 64, 32, seed=9, device="cpu")
    assert a["q"].shape == (1, 300, 2, 64) and a["v"].shape == (1, 300, 4, 32)
    assert a["q"].dtype == torch.bfloat16 and a["g"].dtype == torch.float32
    for x in ("q", "k", "v", "g", "beta"):
        assert torch.equal(a[x], b[x])
    norms = a["q"].float().norm(dim=-1)
    assert torch.all((norms - 1).abs() < 1e-2)
    assert torch.all(a["g"] <= 0) and torch.all((a["beta"] > 0) & (a["beta"] < 1))
    assert abs(float(a["v"].float().std()) - 1.0) < 0.05
    heads = gi.sampled_heads(9, 16)
    assert len(set(heads)) == 2 and all(0 <= j < 16 for j in heads)
