"""GPU parity: the dense GEMM's in-register activation quantisation (M <= 16 rows).

The weight matrix is one-hot (row n holds E2M1 1.0 at k = n), so C[m, n] is the
decoded activation code a_hat[m, n] times the weight scale: the codes and scale
bytes the kernel derives in registers from the bf16 rows are compared with the
oracle's bit for bit. Rows hit round-to-nearest-even ties at many scales, the
saturation edge of E4M3 (scaled values 446 .. 510), signed zeros, bf16 subnormals
in the same block as large values, all-subnormal blocks and the smallest scale
bytes (where the products are kept normal by a 2^64 weight scale).
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import bf16_dev, host

pytestmark = pytest.mark.gpu


def _one_hot(K, scale_byte):
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = 2  # E2M1 1.0
    return oracle.pack_e2m1(codes), np.full((K, K // 32), scale_byte, np.uint8)


def _check(bits, fmt, scale_byte=127):
    M, K = bits.shape
    assert M <= 16
    w, s = _one_hot(K, scale_byte)
    c = ops.mxfp4_gemm(bf16_dev(bits), torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda(), fmt)
    torch.cuda.synchronize()
    q, qs = oracle.moe.quantize_act(oracle.bf16_bits_to_f64(bits), fmt)
    want = oracle.moe.decode_act(q, qs, fmt) * 2.0 ** (scale_byte - 127)
    got = host(c).astype(np.float64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (fmt, bad[:5], got[tuple(bad[0])], want[tuple(bad[0])])


def _bf16(x):
    return dg.bf16_bits_from_f32(np.asarray(x, np.float32))


def _adversarial(K, seed):
    """16 rows of K bf16 values, every 32-block of a different kind."""
    g = np.random.default_rng(seed)
    blocks = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")) as f:
        for blk in json.load(f)["blocks"]:
            v = np.zeros(32)  # the listed elements, the rest of the block zero
            for i, (val, _c, _w) in enumerate(blk["elements"]):
                v[i] = float(val)
            blocks.append(v)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 1.0625, 1.1875, 1.8125, 2.875,
                     9.0, 11.0, 13.0, 17.0, 19.0, 21.0, 26.0, 30.0, 44.0, 52.0, 88.0, 104.0])
    sat = np.array([446.0, 448.0, 450.0, 462.0, 464.0, 466.0, 496.0, 510.0])  # scaled by 2^k below
    for e in [-30, -8, -1, 0, 3, 11, 60, 100]:
        blocks.append(np.resize(mids, 32) * 2.0 ** e * g.choice([-1.0, 1.0], 32))
        blocks.append(np.resize(sat, 32) * 2.0 ** e * g.choice([-1.0, 1.0], 32))
        # E2M1's saturation edge: block amax exponent 2 + k, scaled values 5 .. 7.75
        blocks.append(np.resize([5.0, 5.5, 6.0, 6.5, 7.0, 7.75, 4.0, 3.0], 32) * 2.0 ** e * g.choice([-1.0, 1.0], 32))
    blocks.append(np.where(g.random(32) < 0.5, -0.0, 0.0))
    sub = (g.integers(1, 128, 32).astype(np.uint32) << 16).view(np.float32)  # bf16 subnormals
    blocks.append(sub.astype(np.float64) * g.choice([-1.0, 1.0], 32))
    # one large value and bf16 subnormals / tiny normals in one block (they encode to +-0)
    mix = np.concatenate([[1.0, -3.0], sub[:15].astype(np.float64), -sub[15:30].astype(np.float64)])
    blocks.append(mix)
    blocks.append(np.concatenate([[2.0 ** 100], -np.ldexp(1.0, g.integers(-133, -20, 31))]))
    for _ in range(6):
        blocks.append(np.ldexp(g.random(32) + 0.5, g.integers(-133, 120, 32)) * g.choice([-1.0, 1.0], 32))
    n = 16 * K // 32
    x = np.concatenate(blocks + [g.standard_normal(32) * (1.0 + 19.0 * (g.random(32) < 0.01))
                                 for _ in range(max(0, n - len(blocks)))])[: 16 * K]
    order = g.permutation(n)  # spread the block kinds over rows and K positions
    return _bf16(x.reshape(n, 32)[order].reshape(16, K))


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("M,K,seed", [(16, 512, 1), (9, 1024, 2), (1, 512, 3), (16, 4096, 4), (7, 1536, 5)])
def test_in_register_codes_bit_exact(fmt, M, K, seed):
    """K = 512 / 1024 / 1536: one launch of four waves (no workspace); K = 4096: a one-hot
    weight matrix of 8 MiB of codes, so two K slices and the fixed-order slice sum."""
    _check(_adversarial(K, seed)[:M], fmt)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_in_register_smallest_scale_bytes(fmt):
    """Blocks whose amax is 2^-133 .. 2^-60 (scale bytes 0 .. 65 for E4M3): grid
    midpoints and their bf16 neighbours; the weight scale 2^64 keeps every product
    a normal fp32 number, so C is exactly 2^64 x a_hat."""
    g = np.random.default_rng(11)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0], np.float64)
    rows = []
    for e in np.linspace(-133, -60, 16 * 16).astype(int):
        v = np.resize(mids, 32) * 2.0 ** e * g.choice([-1.0, 1.0], 32)
        rows.append(v)
    x = np.concatenate(rows).reshape(16, 512)
    bits = _bf16(x)
    bump = g.random(bits.shape) < 0.3  # bf16 neighbours of the midpoints
    bits = np.where(bump, bits + np.where(g.random(bits.shape) < 0.5, 1, -1).astype(bits.dtype), bits)
    q, qs = oracle.moe.quantize_act(oracle.bf16_bits_to_f64(bits), fmt)
    assert qs.min() == 0 and qs.max() < 127
    _check(bits, fmt, scale_byte=191)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_in_register_eight_waves(fmt):
    """One launch by eight waves (at least 8 super-steps, at most 1 MiB of weight codes):
    a one-hot weight row for every 96th k of 24 super-steps (three per wave), so codes
    from every wave's K range come back bit for bit."""
    M, N, K = 11, 128, 12288  # 768 KB of weight codes: one launch
    bits = _adversarial(K, 7)[:M]
    codes = np.zeros((N, K), np.uint8)
    cols = np.arange(N) * (K // N)
    codes[np.arange(N), cols] = 2
    w, s = oracle.pack_e2m1(codes), np.full((N, K // 32), 127, np.uint8)
    c = ops.mxfp4_gemm(bf16_dev(bits), torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda(), fmt)
    torch.cuda.synchronize()
    q, qs = oracle.moe.quantize_act(oracle.bf16_bits_to_f64(bits), fmt)
    want = oracle.moe.decode_act(q, qs, fmt)[:, cols]
    assert np.array_equal(host(c).astype(np.float64), want)
