"""The CPU oracle against its pins (closed forms, exact brute force, a hand-worked
example, the independent chunked route, invariants, and for the reverse mode
finite differences and closed forms)."""
import pytest

import oracle
from oracle import prep
from oracle_pins import ALL_PINS, BWD_PINS, PREP_BWD_PINS, PREP_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.gdn_fwd)


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_oracle_bwd_pin(pin):
    pin(oracle.gdn_fwd, oracle.gdn_bwd)


@pytest.mark.parametrize("pin", PREP_PINS, ids=lambda p: p.__name__)
def test_oracle_prep_pin(pin):
    pin(prep, oracle.gdn_fwd)


@pytest.mark.parametrize("pin", PREP_BWD_PINS, ids=lambda p: p.__name__)
def test_oracle_prep_bwd_pin(pin):
    pin(prep, oracle.gdn_fwd)


def test_oracle_rejects_bad_arguments():
    import numpy as np
    q = np.zeros((1, 4, 2, 3), np.float32)
    v = np.zeros((1, 4, 3, 2), np.float32)  # Hv = 3 is not a multiple of Hqk = 2
    gb = np.zeros((1, 4, 3), np.float32)
    with pytest.raises(RuntimeError):
        oracle.gdn_fwd(q, q, v, gb, gb)
    v = np.zeros((1, 4, 2, 2), np.float32)
    gb = np.zeros((1, 4, 2), np.float32)
    with pytest.raises(RuntimeError):  # cu_seqlens not ending at T
        oracle.gdn_fwd(q, q, v, gb, gb, cu_seqlens=[0, 3])
    with pytest.raises(ValueError):  # a value fp32 cannot hold
        oracle.gdn_fwd(q.astype(np.float64) + 1e-12, q, v, gb, gb)
