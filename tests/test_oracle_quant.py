"""Pins for the oracle's MX block quantiser (CPU only).

* hand-worked 32-element blocks (tests/golden/hand_blocks.json);
* the scale exponent against exact rational arithmetic (no frexp);
* element rounding against torch's E4M3 cast (round-to-nearest-even) after
  clamping to +-448, over every finite bf16 magnitude and several shifts;
* element rounding against an exhaustive nearest-code search for E2M1 (torch
  has no FP4 cast), with the tie and saturation rules written independently;
* a half-grid-step error bound for random blocks.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")


def _blocks():
    with open(GOLDEN) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("blk", _blocks(), ids=lambda b: b["name"])
def test_hand_worked_blocks(blk):
    vals = np.zeros((1, 32))
    want = np.zeros(32, dtype=np.uint8)
    for i, (v, code, _why) in enumerate(blk["elements"]):
        vals[0, i] = float(v)
        want[i] = int(code, 16)
    codes, scale = oracle.mx_quantize(vals, blk["fmt"])
    assert int(scale[0, 0]) == blk["scale"]
    assert codes[0].tolist() == want.tolist()


def _floor_log2_exact(x):
    """floor(log2 x) for x > 0 by exact rational comparison."""
    f = Fraction(x)
    e = 0
    while Fraction(2) ** e > f:
        e -= 1
    while Fraction(2) ** (e + 1) <= f:
        e += 1
    return e


def test_scale_byte_vs_exact_rationals():
    g = np.random.default_rng(7)
    samples = list(np.ldexp(g.random(300) + 0.5, g.integers(-150, 130, 300)))
    samples += [2.0 ** e for e in range(-140, 128, 7)]
    samples += [np.nextafter(2.0 ** e, 0) for e in range(-120, 120, 11)]
    samples += [2.0 ** -133, 3 * 2.0 ** -133, 448.0, 6.0]
    for fmt, emax in (("e4m3", 8), ("e2m1", 2)):
        got = oracle.mx_scale_byte(np.array(samples), fmt)
        for a, b in zip(samples, got):
            want = min(max(_floor_log2_exact(a) - emax + 127, 0), 254)
            assert int(b) == want, (fmt, a)
        assert int(oracle.mx_scale_byte(np.array([0.0]), fmt)[0]) == 0


def _all_finite_bf16_magnitudes():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)  # +0 .. largest finite
    return oracle.bf16_bits_to_f64(bits)


@pytest.mark.parametrize("shift", [-20, -12, -8, -3, 0, 5])
def test_e4m3_rounding_vs_torch(shift):
    t = np.ldexp(_all_finite_bf16_magnitudes(), shift)
    t = t[(t < 1e30)]
    got = oracle.round_to_grid(t, "e4m3")
    clamped = torch.from_numpy(np.minimum(t, 448.0).astype(np.float32))
    ref = clamped.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def _brute_e2m1(t_abs):
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    out = np.empty(t_abs.shape, dtype=np.uint8)
    for i, a in enumerate(t_abs):
        if a >= 6.0:
            out[i] = 7
            continue
        d = [abs(a - g) for g in grid]
        best = min(d)
        cands = [c for c in range(8) if d[c] == best]
        out[i] = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return out


@pytest.mark.parametrize("shift", [-14, -6, -2, 0, 2])
def test_e2m1_rounding_vs_brute_force(shift):
    t = np.ldexp(_all_finite_bf16_magnitudes(), shift)
    t = t[t < 64]
    got = oracle.round_to_grid(t, "e2m1")
    assert np.array_equal(got, _brute_e2m1(t))


@pytest.mark.parametrize("fmt,top,spacing_bits", [("e4m3", 448.0, 3), ("e2m1", 6.0, 1)])
def test_quantise_error_bound_and_sign(fmt, top, spacing_bits):
    g = np.random.default_rng(11)
    x = g.standard_normal((64, 256)) * np.ldexp(1.0, g.integers(-30, 30, (64, 1)))
    x[0, :32] = 0.0
    x[1, 5] = -0.0
    codes, scales = oracle.mx_quantize(x, fmt)
    back = oracle.mx_dequantize(codes, scales, fmt)
    blk = x.reshape(64, 8, 32)
    sc = oracle.ue8m0_decode(scales)[..., None]
    t = np.abs(blk) / sc
    # grid spacing at |t|: 2^(floor(log2 max(|t|, min normal)) - mantissa bits)
    minnorm = 2.0 ** -6 if fmt == "e4m3" else 1.0
    step = np.ldexp(1.0, np.floor(np.log2(np.maximum(t, minnorm))).astype(int) - spacing_bits)
    err = np.abs(back.reshape(64, 8, 32) - blk) / sc
    over = t > top
    assert over.any()
    assert np.all(err[~over] <= step[~over] / 2 * (1 + 1e-12))
    # above the largest normal the value saturates to +-top * scale
    b3 = back.reshape(64, 8, 32)
    assert np.all(np.abs(b3[over]) == (top * np.broadcast_to(sc, over.shape))[over])
    # the sign is kept, zeros included
    assert np.array_equal(np.signbit(back), np.signbit(x))
    assert np.all(scales[0, 0] == 0) and np.all(codes[0, :32] == 0)


def test_quantise_is_idempotent_on_representable_blocks():
    # a block whose values are already grid values times its own scale re-encodes to itself
    g = np.random.default_rng(3)
    for fmt, top_code in (("e4m3", 0x7E), ("e2m1", 7)):
        n = 127 if fmt == "e4m3" else 8
        codes = g.integers(0, n, (16, 32)).astype(np.uint8)
        codes[:, 0] = top_code  # pin amax to the largest normal -> scale is recovered exactly
        scales = g.integers(100, 150, (16, 1)).astype(np.uint8)
        if fmt == "e4m3":
            vals = oracle.e4m3_decode(codes)
        else:
            vals = oracle.e2m1_decode(codes)
        x = vals * oracle.ue8m0_decode(scales)
        c2, s2 = oracle.mx_quantize(x, fmt)
        assert np.array_equal(s2, scales)
        assert np.array_equal(c2, codes)
