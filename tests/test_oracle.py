"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_rejects_bad_arguments(orc):
    q = np.zeros((1, 1, 4, 2), np.uint16)
    with pytest.raises(ValueError):
        orc.attention(q, q[:, :, :3], q, "bf16", 1.0)
    with pytest.raises(ValueError):
        orc.attention(q, q, q, "bf16", 1.0, rows=[1, 1])
    with pytest.raises(RuntimeError):
        orc.attention(q, q, q, "bf16", 1.0, rows=[4])  # out of range


def test_empty_rows(orc):
    q = np.zeros((0, 2, 8, 4), np.uint16)
    o, lse = orc.attention(q, q, q, "fp16", 1.0)
    assert o.shape == (0, 2, 8, 4) and lse.shape == (0, 2, 8)


def test_thread_count_does_not_change_results(orc):
    rng = np.random.default_rng(3)
    q = (rng.integers(0, 2**15, size=(1, 3, 50, 8)) & 0x3FFF).astype(np.uint16)
    k = (rng.integers(0, 2**15, size=(1, 3, 50, 8)) & 0x3FFF).astype(np.uint16)
    v = (rng.integers(0, 2**15, size=(1, 3, 50, 8)) & 0x3FFF).astype(np.uint16)
    a = orc.attention(q, k, v, "fp16", 0.2, nthreads=1)
    b = orc.attention(q, k, v, "fp16", 0.2, nthreads=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
