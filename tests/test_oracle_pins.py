"""The CPU oracle against its pins (no GPU)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
import pins  # noqa: E402


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)


def test_compare_metric():
    ref = np.array([[1.0, -2.0], [0.5, 0.0]])
    dev = ref + np.array([[0.02, 0.0], [0.0, -0.04]])
    emax, emean = oracle.compare(dev, ref)
    assert emax == pytest.approx(0.04 / 2.0)
    assert emean == pytest.approx(0.06 / 4 / 2.0)


def test_bad_segments_rejected():
    x = np.zeros((4, 1, 2))
    with pytest.raises(ValueError):
        oracle.prefill(x, x, x, x, np.ones(2), cu_seqlens=[0, 3])
    with pytest.raises(ValueError):
        oracle.prefill(x, x, x, x, np.ones(2), cu_seqlens=[0, 3, 2, 4])
