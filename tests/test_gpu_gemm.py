"""GPU parity: dense mxfp4_gemm vs the fp64 oracle (row-normalised error <= 2e-3)."""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import GEMM_TOL, bf16_dev, host

pytestmark = pytest.mark.gpu


def _run(a, w, s, fmt="e4m3"):
    c = ops.mxfp4_gemm(bf16_dev(a), torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda(), fmt)
    torch.cuda.synchronize()
    return host(c).astype(np.float64)


@pytest.mark.parametrize("name", ["dense_m16_n32_k4096", "dense_m64_n4096_k7168"])
def test_dense_workloads(name):
    d = dg.workload_inputs(name)
    got = _run(d["a"], d["w"], d["w_scale"])
    ref, _, _ = oracle.dense_gemm(d["a"], d["w"], d["w_scale"])
    err = oracle.row_normalised_error(got, ref)
    assert err <= GEMM_TOL, err


@pytest.mark.parametrize("M,N,K,fmt", [
    (1, 16, 512, "e4m3"), (5, 48, 1024, "e4m3"), (17, 64, 2048, "e2m1"), (63, 80, 512, "e4m3"),
    (70, 256, 1536, "e4m3"),  # M > 64 with N % 256 == 0 -> LDS-tiled kernel, ragged last tile
    (300, 384, 1024, "e2m1"), (129, 96, 512, "e4m3"),  # M > 64, N % 256 != 0 -> streamed in 64-row chunks
    # E2M1 activations, M > 64, N % 256 == 0 -> 256 x 256 tiles: a 44-row tail unit (runtime
    # stage loop, K = 1536) and an 8-row tail unit whose other row groups skip their MFMAs (K = 2048)
    (300, 512, 1536, "e2m1"), (520, 256, 2048, "e2m1"),
    # M <= 64 with more than 4 super-steps of 512 k: K split into slices summed in a fixed order
    (33, 48, 5120, "e2m1"),   # 3 slices, the last with 2 super-steps (two idle waves)
    (64, 96, 2560, "e4m3"),   # 2 slices, the last with 1 super-step
    # E4M3 activations, M > 64, N % 256 == 0 at the layer's K values (fp32 C: the loop instance)
    (130, 256, 7168, "e4m3"), (100, 512, 2048, "e4m3"),
    (260, 256, 7168, "e2m1"),  # E2M1, 256 x 256 tiles, K = 7168 (fully unrolled stages), 4-row tail unit
    # E4M3 on the 256 x 256 ring of 128-k stages: one full unit with K = 512 (four stages:
    # a three-slot turn and one more), 65 rows (the second row group holds a single row),
    # and 513 rows at K = 2048 (the unrolled 16-stage instance, a 1-row third unit)
    (256, 256, 512, "e4m3"), (65, 512, 1024, "e4m3"), (513, 256, 2048, "e4m3"),
    # at most 16 rows, quantised in registers, one launch by eight waves: 12 super-steps
    # (waves take one or two) and 16 super-steps with a 16-row N
    (3, 48, 6144, "e4m3"), (16, 16, 8192, "e2m1"),
])
def test_dense_ragged_shapes(M, N, K, fmt):
    a = dg.activations(M * 7 + N, M, K, outliers=True)
    w, s = dg.dense_weights(K + N, N, K, 118, 134)
    got = _run(a, w, s, fmt)
    ref, _, _ = oracle.dense_gemm(a, w, s, act_fmt=fmt)
    err = oracle.row_normalised_error(got, ref)
    assert err <= GEMM_TOL, err


def test_dense_identity_all_ones_weights():
    # all-ones codes with unit scales: C[m, n] = sum_k A_hat[m, k] for every n
    M, N, K = 9, 32, 1024
    a = dg.activations(3, M, K)
    w = np.full((N, K // 2), 0x22, np.uint8)
    s = np.full((N, K // 32), 127, np.uint8)
    got = _run(a, w, s)
    ref, q, qs = oracle.dense_gemm(a, w, s)
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())
    assert np.all(got == got[:, :1])


def test_dense_is_deterministic():
    d = dg.workload_inputs("dense_m64_n4096_k7168")
    a, w, s = bf16_dev(d["a"]), torch.from_numpy(d["w"]).cuda(), torch.from_numpy(d["w_scale"]).cuda()
    c1 = ops.mxfp4_gemm(a, w, s)
    c2 = ops.mxfp4_gemm(a, w, s)
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("M,K,fmt", [
    (1, 512, "e4m3"), (16, 4096, "e2m1"), (64, 7168, "e4m3"),  # K slices summed in a second kernel
    (100, 1024, "e2m1"), (130, 2048, "e4m3"),                   # M > 64: tiled kernels (N = K = 1024, 2048)
    (70, 7168, "e4m3"),                                          # the FP8 ring's unrolled 56-stage instance
])
def test_dense_one_hot_weights_return_the_codes(M, K, fmt):
    """Row n of W holds 1.0 at k = n (unit scales), so C[m, n] is the decoded activation
    code a_hat[m, n] itself - one exact product, every other product zero: the codes
    that reach the matrix instruction equal the oracle's, bit for bit, in every K slice."""
    a = dg.activations(300 + M, M, K, outliers=True)
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = 2  # E2M1 1.0
    w, s = oracle.pack_e2m1(codes), np.full((K, K // 32), 127, np.uint8)
    got = _run(a, w, s, fmt)
    q, qs = oracle.moe.quantize_act(oracle.bf16_bits_to_f64(a), fmt)
    assert np.array_equal(got, oracle.moe.decode_act(q, qs, fmt))
