"""The instruction accuracies that the tolerance bounds of tests/helpers.py
assume (hardware sine / cosine in turns, reciprocal square root), measured
exhaustively on the device by tests/c_abi/hw_accuracy (built by build())."""
import os
import subprocess

import pytest

from tests import helpers

pytestmark = pytest.mark.gpu

PROG = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "hw_accuracy")


def test_instruction_accuracy_within_assumed_bounds():
    assert os.path.exists(PROG), "tests/c_abi/hw_accuracy is not built (run build())"
    out = subprocess.run([PROG], capture_output=True, text=True, timeout=60, check=True).stdout
    got = {k: float(v) for k, v in (line.split() for line in out.strip().splitlines())}
    print(got)
    assert got["sin"] <= helpers.HW_TRIG_ABS_ERR, got
    assert got["cos"] <= helpers.HW_TRIG_ABS_ERR, got
    assert got["rsq"] <= helpers.HW_RSQ_REL_ERR, got
    # the bounds take the reciprocal square root's error as under 2 u
    assert helpers.HW_RSQ_REL_ERR < 2 * helpers.U32
