"""The check that decides on the GPU's requantised h codes (tests/helpers.py),
pinned on the CPU with planted codes and a brute-force check of its error bound.

straddle_check_bound accepts a GPU code when the oracle's exact h, within the
per-element error bound dh, could round to it; h_error_bound derives dh from the
FC1 accumulation bound through silu(g) * u. A planted mistake must fail."""

import numpy as np
import pytest

import oracle
from tests.helpers import MFMA_RESIDUAL, MFMA_WINDOW, h_error_bound, straddle_check_bound


def _block(seed):
    g = np.random.default_rng(seed)
    h = g.standard_normal((1, 32)) * 3.0
    h[0, 0] = 40.0          # block amax: scaled values span the whole E4M3 range
    h[0, 5] = 40.0 * 3e-5   # far below the amax: E4M3 subnormal territory after scaling
    return h


def test_exact_codes_pass():
    h = _block(1)
    codes, scale = oracle.mx_quantize(h, "e4m3")
    assert straddle_check_bound(codes, scale, h, np.zeros_like(h), "e4m3") == (0, 0)


def test_subnormal_steps_pass_only_within_the_bound():
    h = _block(2)
    codes, scale = oracle.mx_quantize(h, "e4m3")
    planted = codes.copy()
    planted[0, 5] = codes[0, 5] + 2  # two subnormal steps up
    step = 2.0 ** -9 * 2.0 ** (int(scale[0, 0]) - 127)  # one subnormal step, unscaled
    dh = np.zeros_like(h)
    dh[0, 5] = 2.0 * step   # the value may be off by two steps: the code is a valid rounding
    assert straddle_check_bound(planted, scale, h, dh, "e4m3")[0] == 1
    dh[0, 5] = 0.5 * step   # half a step: it is not
    with pytest.raises(AssertionError, match="beyond the error bound"):
        straddle_check_bound(planted, scale, h, dh, "e4m3")


def test_large_element_one_step_away_fails():
    h = _block(3)
    h[0, 7] = 40.0 * 0.75  # scaled exactly onto a grid value (no boundary near)
    codes, scale = oracle.mx_quantize(h, "e4m3")
    planted = codes.copy()
    planted[0, 7] = codes[0, 7] + 1
    dh = np.full_like(h, 1e-6 * 40.0)
    with pytest.raises(AssertionError, match="beyond the error bound"):
        straddle_check_bound(planted, scale, h, dh, "e4m3")


def test_midpoint_neighbour_passes():
    h = _block(4)
    codes, scale = oracle.mx_quantize(h, "e2m1")
    X = int(scale[0, 0]) - 127
    h[0, 9] = np.ldexp(2.5 + 1e-9, X)  # just above the 2 | 3 midpoint -> code 3 (0x5)
    codes, scale = oracle.mx_quantize(h, "e2m1")
    assert codes[0, 9] == 0x5
    planted = codes.copy()
    planted[0, 9] = 0x4  # 2.0: the other side of the midpoint
    dh = np.full_like(h, np.ldexp(1e-8, X))
    assert straddle_check_bound(planted, scale, h, dh, "e2m1")[0] == 1
    planted[0, 9] = 0x6  # 4.0: two steps away
    with pytest.raises(AssertionError):
        straddle_check_bound(planted, scale, h, dh, "e2m1")


def test_signed_zero_near_zero():
    h = _block(5)
    codes, scale = oracle.mx_quantize(h, "e2m1")
    h[0, 3] = -1e-30  # rounds to -0
    codes, scale = oracle.mx_quantize(h, "e2m1")
    assert codes[0, 3] == 0x8
    planted = codes.copy()
    planted[0, 3] = 0x0  # +0: a value within 1e-29 of -1e-30 can be positive
    assert straddle_check_bound(planted, scale, h, np.full_like(h, 1e-29), "e2m1")[0] == 1
    planted[0, 3] = 0x1  # +0.5 step: not explained
    with pytest.raises(AssertionError):
        straddle_check_bound(planted, scale, h, np.full_like(h, 1e-29), "e2m1")


def test_scale_byte_mismatch_only_at_a_power_of_two():
    h = _block(6)
    h[0, 0] = 64.0 * (1 - 1e-9)  # amax just below 2^6: byte would be one higher at 2^6
    codes, scale = oracle.mx_quantize(h, "e4m3")
    up = oracle.mx_quantize(np.where(np.arange(32) == 0, 64.0, h), "e4m3")
    gpu_scale = scale + 1
    # the GPU's codes at its own (one higher) byte
    t = np.ldexp(h, -(int(gpu_scale[0, 0]) - 127))
    mag = oracle.round_to_grid(np.abs(t), "e4m3")
    gpu_codes = np.where(np.signbit(h), mag | 0x80, mag).astype(np.uint8)
    assert up[1][0, 0] == gpu_scale[0, 0]
    dh = np.full_like(h, 1e-6)
    assert straddle_check_bound(gpu_codes, gpu_scale, h, dh, "e4m3")[1] == 1
    h2 = h.copy()
    h2[0, 0] = 48.0  # far from a power of two: a different byte is wrong
    c2, s2 = oracle.mx_quantize(h2, "e4m3")
    with pytest.raises(AssertionError, match="power-of-two"):
        straddle_check_bound(c2, s2 + 1, h2, dh, "e4m3")


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_h_error_bound_covers_perturbed_accumulators(fmt):
    """Brute force: perturb gate and up within the accumulation bound (corners and
    random points) and evaluate silu(g') u' in fp64; every change of h must stay
    within h_error_bound (which also budgets the fp32 evaluation of SwiGLU)."""
    g = np.random.default_rng(9)
    I = 64
    G = np.concatenate([g.standard_normal((50, I)) * 8, g.standard_normal((50, I)) * 8], axis=1)
    G[0, :8] = [-40, -10, -1.28, 0.0, 1e-9, 2.4, 12, 35]  # silu's minimum near -1.28, its flat tails
    G_abs = np.abs(G) * 60 + 1.0
    G_gmax = G_abs / 5
    dh = h_error_bound(G, G_abs, I, fmt, G_gmax)
    gg, uu = G[:, :I], G[:, I:]
    h = gg / (1 + np.exp(-gg)) * uu
    d = MFMA_RESIDUAL[fmt] * G_abs + MFMA_WINDOW[fmt] * G_gmax
    dg, du = d[:, :I], d[:, I:]
    for sg, su in [(1, 1), (1, -1), (-1, 1), (-1, -1)] + [tuple(g.uniform(-1, 1, 2)) for _ in range(20)]:
        g2, u2 = gg + sg * dg, uu + su * du
        h2 = g2 / (1 + np.exp(-g2)) * u2
        assert np.all(np.abs(h2 - h) <= dh)
