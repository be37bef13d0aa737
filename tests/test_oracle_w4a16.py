"""Pins for the oracle's FP4-weight x bf16-activation GEMM (MXFP4 and NVFP4 weights)
and the NVFP4 block format, on the CPU, against things other than the oracle itself:
torch's float8_e4m3fn for the UE4M3 scale, the E2M1 value table of the task
statement, closed forms (all-ones codes give row sums; a scale twice as large
doubles the block) and exact-rational brute force on tiny shapes."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg

E2M1_TABLE = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]  # code -> value


def test_ue4m3_decode_matches_torch_float8_e4m3fn():
    b = np.arange(0x7F, dtype=np.uint8)  # every finite byte with the sign bit clear
    want = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(oracle.ue4m3_decode(b), want)
    assert np.isnan(oracle.ue4m3_decode(np.array([0x7F, 0x80, 0xB8], np.uint8))).all()


def test_nvfp4_dequant_elementwise_from_the_tables():
    w, s = dg.nvfp4_weights(3, 5, 64, e_lo=0, e_hi=15)
    s = np.where(s == 0x7F, 0x7E, s).astype(np.uint8)  # keep the NaN byte out
    got = oracle.dequant_nvfp4_weights(w, s)
    sc = torch.from_numpy(s).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    for n in range(5):
        for k in range(64):
            code = (int(w[n, k // 2]) >> (4 * (k % 2))) & 15
            assert got[n, k] == E2M1_TABLE[code] * sc[n, k // 16]


@pytest.mark.parametrize("fmt,one", [("mxfp4", 127), ("nvfp4", 0x38)])
def test_all_ones_codes_give_row_sums(fmt, one):
    M, N, K = 3, 4, 512
    a = dg.activations(5, M, K)
    w = np.full((N, K // 2), 0x22, np.uint8)
    s = np.full((N, K // (16 if fmt == "nvfp4" else 32)), one, np.uint8)
    c = oracle.w4a16_gemm(a, w, s, fmt)
    rows = oracle.bf16_bits_to_f64(a).sum(axis=1)
    assert np.allclose(c, rows[:, None], rtol=1e-14, atol=0)


@pytest.mark.parametrize("fmt,lo,hi", [("mxfp4", 127, 128), ("nvfp4", 0x38, 0x40)])
def test_doubling_one_block_scale_doubles_its_share(fmt, lo, hi):
    M, N, K = 2, 3, 256
    blk = 16 if fmt == "nvfp4" else 32
    a = dg.activations(6, M, K)
    w, _ = dg.dense_weights(6, N, K, 120, 128)
    s = np.full((N, K // blk), lo, np.uint8)
    base = oracle.w4a16_gemm(a, w, s, fmt)
    s2 = s.copy()
    s2[:, 3] = hi  # doubles block 3
    a_only = np.zeros_like(a)
    a_only[:, 3 * blk:4 * blk] = a[:, 3 * blk:4 * blk]
    share = oracle.w4a16_gemm(a_only, w, s, fmt)
    assert np.allclose(oracle.w4a16_gemm(a, w, s2, fmt), base + share, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_tiny_brute_force_exact_rationals(fmt):
    M, N, K = 2, 3, 64
    blk = 16 if fmt == "nvfp4" else 32
    a = dg.activations(7, M, K)
    if fmt == "nvfp4":
        w, s = dg.nvfp4_weights(7, N, K)
        sc = [[Fraction(float(v)) for v in row]
              for row in torch.from_numpy(s).view(torch.float8_e4m3fn).float().numpy()]
    else:
        w, s = dg.dense_weights(7, N, K, 118, 134)
        sc = [[Fraction(2) ** (int(v) - 127) for v in row] for row in s]
    av = [[Fraction(float(x)) for x in row] for row in oracle.bf16_bits_to_f64(a)]
    got = oracle.w4a16_gemm(a, w, s, fmt)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for k in range(K):
                code = (int(w[n, k // 2]) >> (4 * (k % 2))) & 15
                tot += av[m][k] * Fraction(E2M1_TABLE[code]) * sc[n][k // blk]
            assert got[m, n] == float(tot)
