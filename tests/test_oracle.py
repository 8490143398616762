"""The fp64 oracle against its pins (CPU only).

Every check here comes from outside the oracle: hand-derived closed forms
(tests/golden), invariants of softmax(scale Q K^T) V, scalar brute force and
torch's CPU attention routine. See tests/oracle_pins.py for the citation of
each pin.
"""

import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.sdpa)


def test_chunking_does_not_change_rows():
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((1, 50, 2, 8)) for _ in range(3))
    for causal in (False, True):
        a = oracle.sdpa(q, k, v, scale=0.3, causal=causal, row_chunk=1024)
        b = oracle.sdpa(q, k, v, scale=0.3, causal=causal, row_chunk=3)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_empty_and_errors():
    z = np.zeros((2, 0, 4, 8))
    k = np.zeros((2, 5, 2, 8))
    assert oracle.sdpa(z, k, k, scale=1.0, causal=True).shape == (2, 0, 4, 8)
    with pytest.raises(ValueError):
        oracle.sdpa(np.zeros((1, 3, 3, 8)), np.zeros((1, 3, 2, 8)), np.zeros((1, 3, 2, 8)), scale=1.0, causal=False)
    with pytest.raises(ValueError):
        oracle.sdpa(np.zeros((1, 3, 2, 8)), np.zeros((1, 0, 2, 8)), np.zeros((1, 0, 2, 8)), scale=1.0, causal=False)


def test_sq_ne_skv_top_left():
    """Reading for Sq != Skv (never exercised by the codelab): literal lower
    triangle, key j visible to query i iff j <= i. Row i of a causal call
    equals a non-causal call over keys 0..i only."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 6, 2, 4))
    k = rng.standard_normal((1, 10, 2, 4))
    v = rng.standard_normal((1, 10, 2, 4))
    c = oracle.sdpa(q, k, v, scale=0.5, causal=True)
    for i in range(6):
        f = oracle.sdpa(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1], scale=0.5, causal=False)
        np.testing.assert_allclose(c[:, i:i + 1], f, rtol=0, atol=1e-14)
