"""The test-side bf16 rounding model (tests/bf16_model.py): its algebra is the
oracle's chunk form, and the error it predicts for the kernel's rounding
points stays inside the state tolerance with room to spare under slow decay.
"""
import numpy as np
import pytest

import bf16_model as bm
import gdn_inputs as gi
import oracle
from oracle import chunked


def _rel(x, y):
    return float(np.linalg.norm(x - y) / np.linalg.norm(y))


@pytest.mark.parametrize("dk", [64, 256])
def test_model_without_rounding_is_the_oracle(dk):
    d = gi.make(2, 150, 1, 2, dk, 32, "bf16", 8800 + dk, h0_std=0.1)
    q, k, v = (gi.widen(d[x]) for x in ("q", "k", "v"))
    o, ht = bm.forward(q, k, v, d["g"], d["beta"], h0=d["h0"], scale=0.7, rounding=False)
    ro, rh = oracle.gdn_fwd(q, k, v, d["g"], d["beta"], scale=0.7, h0=d["h0"])
    assert _rel(o, ro) < 1e-12 and _rel(ht, rh) < 1e-12
    co, ch = chunked.fwd(q, k, v, d["g"], d["beta"], bm.chunk_len(dk), scale=0.7, h0=d["h0"])
    assert _rel(o, co) < 1e-13 and _rel(ht, ch) < 1e-13


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -7 + 2.0 ** -9, -3.0])
    want = np.array([1.0, 1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -3.0])
    assert np.array_equal(bm.bf16(x), want)


def _slow_decay_case(dk, div, seed):
    d = gi.make(1, 4096 + 37, 1, 2, dk, 128, "bf16", seed, h0_std=0.1)
    g = (d["g"] / div).astype(np.float32)
    q, k, v = (gi.widen(d[x]) for x in ("q", "k", "v"))
    return q, k, v, g, d["beta"], d["h0"]


def predicted_state_error(dk, div, seed, km0_split=None):
    q, k, v, g, b, h0 = _slow_decay_case(dk, div, seed)
    _, ht = bm.forward(q, k, v, g, b, h0=h0, km0_split=km0_split)
    _, exact = bm.forward(q, k, v, g, b, h0=h0, rounding=False)
    return max(_rel(ht[0, h], exact[0, h]) for h in range(2))


@pytest.mark.parametrize("dk", [64, 128, 256])
@pytest.mark.parametrize("div", [2, 4])
def test_predicted_state_error_has_headroom(dk, div):
    """Log-decays 2 and 4 times slower than the workloads' (mean decay per
    token about 0.975 and 0.987), T = 4133 with an initial state: the
    predicted final-state error is at most half the 1e-3 tolerance."""
    e = predicted_state_error(dk, div, 8900 + dk + div)
    print(f"dk={dk} g/{16 * div}: predicted state rel-L2 {e:.2e}")
    assert e <= 5e-4


def test_hi_only_k_m0_would_lose_the_headroom_at_dk64():
    """Why K M0 takes M0 as hi + lo at dk = 64: with the hi part only, dk = 64
    at g/64 is predicted past half the tolerance, and the split brings it
    down by two orders of magnitude.  At dk = 128 the hi part alone keeps
    more than 2x headroom."""
    hi = predicted_state_error(64, 4, 8968, km0_split=False)
    split = predicted_state_error(64, 4, 8968, km0_split=True)
    assert hi > 5e-4 and split < hi / 100
    assert predicted_state_error(128, 4, 9032, km0_split=False) < 4e-4
