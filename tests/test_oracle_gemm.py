"""Pins for the oracle's MXFP4 GEMM (CPU only).

* all-ones weight codes with unit scales reduce C to a plain dot product (row
  sum of the quantised activations);
* one-hot weights pick single activation columns, times the block scale;
* raising one scale byte by one doubles exactly that block's contribution;
* exact rational brute force on tiny shapes, with the operands decoded through
  torch's float8 dtype (E4M3) and the E2M1 value set, summed with Fractions.
The dense GEMM is the entry the page "DGX Spark 原生 FP4 矩阵指令" (section 二)
calls the dense MXFP4 path.
"""

from fractions import Fraction

import numpy as np
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg


def _act(M, K, seed=0):
    return dg.bf16_bits_from_f32(np.random.default_rng(seed).standard_normal((M, K)).astype(np.float32))


def test_all_ones_weights_is_plain_dot_product():
    M, N, K = 5, 7, 256
    a = _act(M, K)
    w = np.full((N, K // 2), 0x22, dtype=np.uint8)  # code 2 = +1.0 in both nibbles
    s = np.full((N, K // 32), 127, dtype=np.uint8)  # 2^0
    C, q, qs = oracle.dense_gemm(a, w, s)
    a_hat = oracle.mx_dequantize(q, qs, "e4m3")
    rowsum = np.array([sum(float(v) for v in row) for row in a_hat])
    assert np.allclose(C, rowsum[:, None], rtol=0, atol=1e-9 * np.abs(a_hat).sum())
    assert np.all(C == C[:, :1])


def test_one_hot_weights_pick_columns():
    M, N, K = 3, 4, 128
    a = _act(M, K, 1)
    codes = np.zeros((N, K), dtype=np.uint8)
    cols = [0, 33, 64, 127]
    for n, k in enumerate(cols):
        codes[n, k] = 2 if n % 2 == 0 else 10  # +1.0 or -1.0
    w = oracle.pack_e2m1(codes)
    s = np.full((N, K // 32), 127, dtype=np.uint8)
    s[2, 2] = 130  # x8 for block 2 of row 2 (k = 64)
    C, q, qs = oracle.dense_gemm(a, w, s)
    a_hat = oracle.mx_dequantize(q, qs, "e4m3")
    for n, k in enumerate(cols):
        sign = 1.0 if n % 2 == 0 else -1.0
        mult = 8.0 if n == 2 else 1.0
        assert np.array_equal(C[:, n], sign * mult * a_hat[:, k])


def test_scale_increment_doubles_block_contribution():
    M, N, K = 4, 6, 256
    a = _act(M, K, 2)
    w, s = dg.dense_weights(5, N, K, 122, 130)
    C0, q, qs = oracle.dense_gemm(a, w, s)
    s2 = s.copy()
    s2[3, 5] += 1
    C1, _, _ = oracle.dense_gemm(a, w, s2)
    a_hat = oracle.mx_dequantize(q, qs, "e4m3")
    w_hat = oracle.dequant_weights(w, s)
    block = a_hat[:, 160:192] @ w_hat[3, 160:192]
    assert np.allclose(C1[:, 3] - C0[:, 3], block, rtol=1e-12, atol=1e-12 * np.abs(C0).max())
    keep = [n for n in range(N) if n != 3]
    assert np.array_equal(C1[:, keep], C0[:, keep])


def _fraction_e4m3(code):
    v = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
    return Fraction(v)


_E2M1_SET = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
             Fraction(3), Fraction(4), Fraction(6)]


def _fraction_e2m1(code):
    v = _E2M1_SET[code & 7]
    return -v if code & 8 else v


def test_exact_rational_brute_force_tiny():
    for seed, (M, N, K) in enumerate([(1, 1, 32), (2, 3, 64), (3, 2, 128), (4, 4, 96)]):
        a = _act(M, K, 10 + seed)
        w, s = dg.dense_weights(20 + seed, N, K, 118, 134)
        C, q, qs = oracle.dense_gemm(a, w, s)
        for m in range(M):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    byte = int(w[n, k // 2])
                    wc = (byte & 15) if k % 2 == 0 else (byte >> 4)
                    wv = _fraction_e2m1(wc) * Fraction(2) ** (int(s[n, k // 32]) - 127)
                    av = _fraction_e4m3(int(q[m, k])) * Fraction(2) ** (int(qs[m, k // 32]) - 127)
                    acc += av * wv
                assert abs(Fraction(C[m, n]) - acc) <= abs(acc) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 200)


def test_dense_e2m1_activation_variant():
    # the same GEMM with FP4 activations (FP4 x FP4) on a tiny case, exact rationals
    M, N, K = 2, 2, 64
    a = _act(M, K, 40)
    w, s = dg.dense_weights(41, N, K, 124, 130)
    C, q, qs = oracle.dense_gemm(a, w, s, act_fmt="e2m1")
    assert q.shape == (M, K // 2)
    codes = oracle.unpack_e2m1(q)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                byte = int(w[n, k // 2])
                wc = (byte & 15) if k % 2 == 0 else (byte >> 4)
                wv = _fraction_e2m1(wc) * Fraction(2) ** (int(s[n, k // 32]) - 127)
                av = _fraction_e2m1(int(codes[m, k])) * Fraction(2) ** (int(qs[m, k // 32]) - 127)
                acc += av * wv
            assert Fraction(C[m, n]) == acc
