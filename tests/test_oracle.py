"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)


def test_golden_matches_pages_doc_example(o):
    # Emily.Fast docs, rms_norm / layer_norm examples: x = [[1, 2, 3, 4]].
    # Closed forms: RMS ms = 7.5; LayerNorm mean 2.5, var 1.25.
    x = np.array([[1, 2, 3, 4]], np.float32)
    eps = float(np.float32(1e-5))
    y = o.rms(x, np.ones(4, np.float32), 1e-5)
    assert abs(y[0, 0] - 1.0 / np.sqrt(7.5 + eps)) < 1e-15
    y = o.layer(x, np.ones(4, np.float32), np.zeros(4, np.float32), 1e-5)
    assert abs(y[0, 3] - 1.5 / np.sqrt(1.25 + eps)) < 1e-15


def test_shapes_and_dtype_checks(o):
    with pytest.raises(TypeError):
        o.rms(np.zeros((2, 4), np.float64), np.ones(4), 1e-6)
    with pytest.raises(ValueError):
        o.rms(np.zeros((2, 4), np.float32), np.ones(5, np.float32), 1e-6)
    y = o.rms(np.zeros((0, 4), np.float32), np.ones(4, np.float32), 1e-6)
    assert y.shape == (0, 4)
