"""Pins for the oracle's element/scale decoders and byte layouts (CPU only).

Each decoder is checked against something other than itself: the E2M1 value
set the formats fix, torch's own float8 dtypes, and the nibble order stated on
the page "【DeepSeek V4】Triton FP4 优化实战" ("第二步：Fused Dequant+Matmul Kernel":
even columns in the low nibble, odd columns in the high nibble).
"""

import numpy as np
import torch

import oracle
from oracle import mx


def test_e2m1_value_set():
    # E2M1 = 1 sign / 2 exponent / 1 mantissa bit ("DGX Spark 原生 FP4 矩阵指令" 一):
    # positive codes 0..7 are {0, 0.5, 1, 1.5, 2, 3, 4, 6}; bit 3 is the sign.
    expected = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = oracle.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == expected
    assert list(got[8:]) == [-v for v in expected]
    assert np.signbit(got[8])  # code 8 is -0


def test_e4m3_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_ue8m0_matches_torch_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.ue8m0_decode(b)
    assert np.isnan(ref[255]) and np.isnan(got[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[128] == 2.0 and got[0] == 2.0 ** -127


def test_nibble_order_even_column_low():
    # page "【DeepSeek V4】Triton FP4 优化实战", 第二步: even column x low nibble
    codes = np.array([[1, 2, 7, 8]], dtype=np.uint8)  # 0.5, 1.0, 6.0, -0.0
    packed = oracle.pack_e2m1(codes)
    assert packed.tolist() == [[0x21, 0x87]]
    assert np.array_equal(oracle.unpack_e2m1(packed), codes)
    vals = oracle.e2m1_decode(oracle.unpack_e2m1(np.array([[0x21]], dtype=np.uint8)))
    assert vals.tolist() == [[0.5, 1.0]]


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_dequant_weights_layout():
    # one row, K = 64: block 0 scale 127 (x1), block 1 scale 129 (x4)
    codes = np.zeros((1, 64), dtype=np.uint8)
    codes[0, 0] = 2    # +1.0 at k = 0
    codes[0, 33] = 11  # -1.5 at k = 33
    w = oracle.pack_e2m1(codes)
    s = np.array([[127, 129]], dtype=np.uint8)
    d = oracle.dequant_weights(w, s)
    expect = np.zeros((1, 64))
    expect[0, 0] = 1.0
    expect[0, 33] = -6.0
    assert np.array_equal(d, expect)
    assert mx.E2M1_EMAX == 2 and mx.E4M3_EMAX == 8
