"""The summation error of the GEMM kernels, per output element, at the layer's
K = 7168 (the FC1 contraction) and K = 2048 (FC2):
    |C_gpu - C_exact| <= MFMA_RESIDUAL * sum_k |a_k w_k| + MFMA_WINDOW * B,
B = oracle.group_max_terms (groups of 8 k). C_exact and the sums of magnitudes are
the fp64 oracle's (exact products of the decoded MX operands). These constants
(tests/helpers.py) are the ones every per-element tolerance of the parity tests is
derived from, so this test is what ties those tolerances to the hardware:

* E2M1 x E2M1: every product is exact and so is each block's sum; what remains is
  fp32 accumulation over K / 64 (32x32x64) or K / 128 (16x16x128) instruction
  steps plus the K-slice sums, bounded by gamma_n = n 2^-24 of the sum of
  magnitudes for n roundings: 2^-17 covers n <= 128.
* E4M3 x E2M1: the products are exact (4 x 2 significant bits), but inside a block
  the instruction aligns each group of 8 products to the group's largest and drops
  the bits below 2^-13 of it (tests/test_gpu_mfma_window.py), so a term of at most
  7 * 2^-13 of each group's largest product joins the accumulation bound. Gaussian
  activations hardly reach the window; heavy-tailed ones (a product of two Gaussians,
  the shape of SwiGLU's output that FC2 consumes) do, and are covered here.

Both instruction shapes are covered: M = 64 runs the weight-streaming kernel
(16x16x128), M = 300 with N = 256 the tiled kernels (32x32x64).
"""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import MFMA_RESIDUAL, bf16_dev, gemm_error_bound, host

pytestmark = pytest.mark.gpu


def _heavy_tailed(seed, M, K):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((M, K)) * 8) * (g.standard_normal((M, K)) * 8)
    return dg.bf16_bits_from_f32(x.astype(np.float32))


@pytest.mark.parametrize("M,N", [(64, 512), (300, 256)])
@pytest.mark.parametrize("fmt,K,data", [("e4m3", 7168, "gauss"), ("e2m1", 7168, "gauss"),
                                        ("e4m3", 2048, "heavy"), ("e2m1", 2048, "heavy")])
def test_accumulation_residual_bound(M, N, fmt, K, data):
    a = dg.activations(41 + M, M, K) if data == "gauss" else _heavy_tailed(43 + M, M, K)
    w, s = dg.dense_weights(42 + M, N, K, 120, 128)
    c = ops.mxfp4_gemm(bf16_dev(a), torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda(), fmt)
    torch.cuda.synchronize()
    got = host(c).astype(np.float64)
    ref, q, qs = oracle.dense_gemm(a, w, s, act_fmt=fmt)
    a_hat = oracle.moe.decode_act(q, qs, fmt)
    w_hat = oracle.dequant_weights(w, s)
    S = np.abs(a_hat) @ np.abs(w_hat).T
    B = oracle.group_max_terms(a_hat, w_hat)
    err = np.abs(got - ref)
    bound = gemm_error_bound(S, B, fmt)
    worst_s = float((err / S).max())
    print(f"\n[residual] {fmt} {data} M={M} N={N} K={K}: max err / sum|a w| = 2^{np.log2(max(worst_s, 1e-300)):.2f}, "
          f"max err / bound = {float((err / bound).max()):.3f}")
    assert np.all(err <= bound)
    if fmt == "e2m1":
        assert worst_s <= MFMA_RESIDUAL[fmt]
