"""Pins for the oracle's lookup-table route (Q8 activations x int8-expanded MXFP4
weights), on the CPU, against hand-worked values, invariants and the MXFP4 decode:

* a hand-worked block 0, 1, .., 31: amax 31, d = fp16(31/127) = 0.244140625 (the
  fp32 quotient 0.2440944.. rounds to 1.953125 x 2^-3 in fp16), q = rint(k x 4.096);
* ties go to even (d = 1: 2.5 -> 2, 3.5 -> 4, -0.5 -> 0);
* invariants on random blocks: the amax element gives +-127 (d is within 2^-11 of
  amax/127), |x - q d| <= d/2, sign(q) = sign(x) or q = 0, a zero block (and a block
  whose d underflows fp16) gives d = 0 and q = 0;
* the 16-entry table is lossless: int8 x 2^(e-128) equals the MXFP4 value exactly;
* the block-wise integer GEMM equals the dequantised product, and exact rationals on
  tiny shapes.
"""

from fractions import Fraction

import numpy as np

import oracle
from mxfp4_block_scaled_amd import datagen as dg

E2M1_TABLE = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]


def _bf16(vals):
    return dg.bf16_bits_from_f32(np.asarray(vals, np.float32))


def test_hand_worked_block():
    x = _bf16(np.arange(32, dtype=np.float32)[None, :])
    q, d = oracle.q8_quantize(x)
    assert float(d[0, 0]) == 0.244140625
    want = [0, 4, 8, 12, 16, 20, 25, 29, 33, 37, 41, 45, 49, 53, 57, 61, 66, 70, 74, 78, 82, 86, 90, 94, 98,
            102, 106, 111, 115, 119, 123, 127]  # rint(k * 4.096)
    assert q[0].tolist() == want


def test_ties_to_even_and_zero_blocks():
    v = np.zeros((3, 32), np.float32)
    v[0, 0] = 127.0  # d = 1 exactly
    v[0, 1:5] = [2.5, 3.5, -0.5, -2.5]
    v[2, :] = 2.0 ** -40  # amax / 127 underflows fp16
    q, d = oracle.q8_quantize(_bf16(v))
    assert float(d[0, 0]) == 1.0
    assert q[0, :5].tolist() == [127, 2, 4, 0, -2]
    assert float(d[1, 0]) == 0.0 and not q[1].any()
    assert float(d[2, 0]) == 0.0 and not q[2].any()


def test_invariants_on_random_blocks():
    x = dg.activations(91, 64, 1024, outliers=True)
    q, d = oracle.q8_quantize(x)
    xv = oracle.bf16_bits_to_f64(x).reshape(64, 32, 32)
    qv = q.astype(np.float64).reshape(64, 32, 32)
    dv = d.astype(np.float64)[..., None]
    assert np.all(np.abs(qv) <= 127)
    am = np.argmax(np.abs(xv), axis=-1)
    assert np.all(np.abs(np.take_along_axis(qv, am[..., None], -1)) == 127)
    assert np.all(np.abs(xv - qv * dv) <= dv / 2 * (1 + 1e-12))
    assert np.all((np.sign(qv) == np.sign(xv)) | (qv == 0))


def test_table_is_lossless():
    w, s = dg.dense_weights(92, 16, 256, 2, 252)
    w8 = oracle.lut_int8_weights(w)
    assert sorted(set(np.abs(w8).ravel().tolist())) <= [0, 1, 2, 3, 4, 6, 8, 12]
    codes = oracle.unpack_e2m1(w)
    assert np.array_equal(w8.astype(np.float64), 2 * np.array(E2M1_TABLE)[codes])
    val = w8.reshape(16, 8, 32) * np.ldexp(1.0, s.astype(np.int64) - 128)[..., None]
    assert np.array_equal(val.reshape(16, 256), oracle.dequant_weights(w, s))


def test_gemm_equals_dequantised_product_and_exact_rationals():
    M, N, K = 5, 7, 256
    x = dg.activations(93, M, K, outliers=True)
    w, s = dg.dense_weights(93, N, K, 118, 134)
    q, d = oracle.q8_quantize(x)
    c = oracle.q8_gemm(q, d, w, s)
    a_hat = (q.astype(np.float64).reshape(M, K // 32, 32) * d.astype(np.float64)[..., None]).reshape(M, K)
    ref = a_hat @ oracle.dequant_weights(w, s).T
    assert np.allclose(c, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    for m in range(2):
        for n in range(2):
            tot = Fraction(0)
            for k in range(K):
                code = (int(w[n, k // 2]) >> (4 * (k % 2))) & 15
                tot += (Fraction(int(q[m, k])) * Fraction(float(d[m, k // 32])) * Fraction(E2M1_TABLE[code])
                        * Fraction(2) ** (int(s[n, k // 32]) - 127))
            assert c[m, n] == float(tot)
