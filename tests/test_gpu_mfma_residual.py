"""The accumulation error of the GEMM kernels, per output element, at the layer's
K = 7168 (the FC1 contraction): |C_gpu - C_exact| <= c * sum_k |a_k w_k|.

C_exact and sum_k |a_k w_k| are the fp64 oracle's (exact products of the decoded
MX operands). The bound's constants (MFMA_RESIDUAL in tests/helpers.py) are the
ones the requantised-h check derives its per-element tolerance from, so this test
is what pins that tolerance to the hardware:

* E2M1 x E2M1: every product of two E2M1 codes and two power-of-two scales is
  exact, and so is each 32-block's sum; what remains is fp32 accumulation over
  K / 64 (32x32x64) or K / 128 (16x16x128) instruction steps plus the K-slice
  sums, bounded by gamma_n = n 2^-24 of the sum of magnitudes for n roundings:
  2^-17 covers n <= 128.
* E4M3 x E2M1: the products are exact too (4 x 2 significant bits); the test
  shows that the instruction's internal sum adds no error beyond the same
  accumulation bound (measured worst 2^-19.8 of the sum of magnitudes).

Both instruction shapes are covered: M = 64 runs the weight-streaming kernel
(16x16x128), M = 300 with N = 256 the tiled kernels (32x32x64).
"""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import MFMA_RESIDUAL, bf16_dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N", [(64, 512), (300, 256)])
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_accumulation_residual_bound(M, N, fmt):
    K = 7168
    a = dg.activations(41 + M, M, K)
    w, s = dg.dense_weights(42 + M, N, K, 120, 128)
    c = ops.mxfp4_gemm(bf16_dev(a), torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda(), fmt)
    torch.cuda.synchronize()
    got = host(c).astype(np.float64)
    ref, q, qs = oracle.dense_gemm(a, w, s, act_fmt=fmt)
    a_hat = oracle.moe.decode_act(q, qs, fmt)
    S = np.abs(a_hat) @ np.abs(oracle.dequant_weights(w, s)).T
    ratio = np.abs(got - ref) / S
    worst = float(ratio.max())
    print(f"\n[residual] {fmt} M={M} N={N} K={K}: max |C_gpu - C_exact| / sum|a w| = {worst:.3e} "
          f"(2^{np.log2(worst) if worst > 0 else float('-inf'):.2f}); bound {MFMA_RESIDUAL[fmt]:.3e}")
    assert worst <= MFMA_RESIDUAL[fmt], worst
