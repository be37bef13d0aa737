"""The straddle rule (tests/helpers.py) that decides on the GPU's requantised h codes,
checked on the CPU with planted codes: it accepts the oracle's own codes and
mismatches that fp32 accumulation can explain (a value within tol of the block
amax from the other side of a rounding boundary, including several subnormal
steps for an element far below the amax), and rejects a code that is wrong."""

import numpy as np
import pytest

import oracle
from tests.helpers import straddle_check


def _block(seed):
    g = np.random.default_rng(seed)
    h = g.standard_normal((1, 32)) * 3.0
    h[0, 0] = 40.0          # block amax: scaled values span the whole E4M3 range
    h[0, 5] = 40.0 * 3e-5   # far below the amax: E4M3 subnormal territory after scaling
    return h


def test_exact_codes_pass():
    h = _block(1)
    codes, scale = oracle.mx_quantize(h, "e4m3")
    assert straddle_check(codes, scale, h, "e4m3") == (0, 0)


def test_tiny_element_several_subnormal_steps_away_passes():
    h = _block(2)
    codes, scale = oracle.mx_quantize(h, "e4m3")
    planted = codes.copy()
    planted[0, 5] = codes[0, 5] + 2  # two subnormal steps up: far inside 1e-3 of the block amax
    assert straddle_check(planted, scale, h, "e4m3")[0] == 1


def test_large_element_one_step_away_from_any_boundary_fails():
    h = _block(3)
    h[0, 7] = 40.0 * 0.75  # scaled exactly onto a grid value (no boundary near)
    codes, scale = oracle.mx_quantize(h, "e4m3")
    planted = codes.copy()
    planted[0, 7] = codes[0, 7] + 1
    with pytest.raises(AssertionError, match="rounding boundary"):
        straddle_check(planted, scale, h, "e4m3")


def test_e2m1_code_two_steps_away_fails():
    h = _block(4)
    codes, scale = oracle.mx_quantize(h, "e2m1")
    planted = codes.copy()
    # an element at 1.5 x 2^X after scaling: moving it to 3 is two grid steps away
    planted[0, 0] = (codes[0, 0] & 0x8) | 0x5
    with pytest.raises(AssertionError):
        straddle_check(planted, scale, h, "e2m1")
