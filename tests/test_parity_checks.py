"""The y acceptance checks themselves (CPU): a correct bf16 output passes, and small
localised mistakes that the global relative L2 alone lets through are caught.

The "correct" output is the oracle's y rounded to bfloat16, i.e. exactly what a
kernel with perfect arithmetic would return; the planted mistakes are those a
tiling or indexing bug produces: one (t, h) row zeroed, a row taken from the
previous token (off by one), one 16 x 16 tile of one head wrong, one element wrong.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import bf16_round, make_forward_inputs
from tests.gpu_util import Y_TOL, assert_close_y, rel_l2


@pytest.fixture(scope="module")
def ref_and_good():
    # 4096 tokens x 16 heads = 65,536 rows of 64 values: one row is 1/256 of the norm
    fi = make_forward_inputs(1, 4096, 16, 64, 32, 1, "bf16", seed=7)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, None)["y"]
    good = bf16_round(ref).astype(np.float64)
    return ref, good


def test_correct_bf16_output_passes(ref_and_good):
    ref, good = ref_and_good
    e = assert_close_y(good, ref, "bf16")
    assert e < 3e-3


def _planted(good, kind):
    bad = good.copy()
    if kind == "zero_row":
        bad[0, 1234, 5, :] = 0.0
    elif kind == "off_by_one_row":
        bad[0, 2047, 9, :] = good[0, 2046, 9, :]
    elif kind == "wrong_tile":
        bad[0, 3008:3024, 11, 16:32] = good[0, 3024:3040, 11, 16:32]
    elif kind == "one_element":
        bad[0, 777, 3, 40] = -good[0, 777, 3, 40] + 0.5
    elif kind == "scaled_row":
        bad[0, 4095, 15, :] *= 1.05
    return bad


@pytest.mark.parametrize("kind", ["zero_row", "off_by_one_row", "wrong_tile", "one_element", "scaled_row"])
def test_local_mistake_is_caught(ref_and_good, kind):
    ref, good = ref_and_good
    bad = _planted(good, kind)
    # the global metric alone would accept it ...
    assert rel_l2(bad, ref) <= Y_TOL["bf16"]
    # ... the row / element checks do not
    with pytest.raises(AssertionError, match="(row|element)"):
        assert_close_y(bad, ref, "bf16")


def test_fp32_bounds():
    fi = make_forward_inputs(1, 300, 2, 16, 16, 1, "f32", seed=8)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, None)["y"]
    good = ref.astype(np.float32).astype(np.float64)
    assert_close_y(good, ref, "f32")
    bad = good.copy()
    bad[0, 100, 1, :] *= 1.001
    with pytest.raises(AssertionError):
        assert_close_y(bad, ref, "f32")
