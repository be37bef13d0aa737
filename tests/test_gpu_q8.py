"""GPU parity of the lookup-table route: q8_quantize_act bit-exact against the oracle
(random rows with outliers and adversarial blocks: ties, zeros, scales that underflow
or overflow fp16), and mxfp4_gemm_q8 against the oracle's block-wise integer GEMM -
per element within 2^-16 of the sum of magnitudes (each block's integer sum is exact;
its scaling and the sum over K/32 blocks round in fp32) and row-normalised 2e-3 - at
the pages' accuracy-table shapes and ragged ones."""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import GEMM_TOL, bf16_dev, host

pytestmark = pytest.mark.gpu


def _quant(x):
    q, d = ops.q8_quantize_act(bf16_dev(x))
    torch.cuda.synchronize()
    return q.cpu().numpy(), d.cpu().numpy()


@pytest.mark.parametrize("rows,K", [(1, 4096), (64, 7168), (33, 512)])
def test_quantize_bit_exact_random(rows, K):
    x = dg.activations(100 + rows, rows, K, outliers=True)
    q, d = _quant(x)
    rq, rd = oracle.q8_quantize(x)
    assert np.array_equal(q, rq)
    assert np.array_equal(d.view(np.uint16), rd.view(np.uint16))


def test_quantize_bit_exact_adversarial():
    v = np.random.default_rng(101).standard_normal((8, 256)).astype(np.float32)
    v[0, :32] = 0.0                                       # zero block
    v[1, :32] = 2.0 ** -40                                # d underflows fp16 -> q = 0
    v[2, 0] = 127.0
    v[2, 1:32] = np.arange(31, dtype=np.float32) * 0.5 - 7.25  # ties at d = 1
    v[3, :32] *= 1e7                                      # amax / 127 overflows fp16: d = inf, q = 0
    v[4, :32] = np.float32(2.0 ** -133) * np.arange(32)   # bf16 subnormals
    v[5, 32:64] = -3.0                                    # constant negative block
    q, d = _quant(dg.bf16_bits_from_f32(v))
    rq, rd = oracle.q8_quantize(dg.bf16_bits_from_f32(v))
    assert np.array_equal(q, rq)
    assert np.array_equal(d.view(np.uint16), rd.view(np.uint16))


def _gemm_check(M, N, K, seed):
    x = dg.activations(seed, M, K, outliers=True)
    w, s = dg.dense_weights(seed + 1, N, K, 118, 134)
    qd, dd = ops.q8_quantize_act(bf16_dev(x))
    c = ops.mxfp4_gemm_q8(qd, dd, torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    q, d = qd.cpu().numpy(), dd.cpu().numpy()
    got = host(c).astype(np.float64)
    ref = oracle.q8_gemm(q, d, w, s)
    a_hat = (q.astype(np.float64).reshape(M, K // 32, 32) * d.astype(np.float64)[..., None]).reshape(M, K)
    S = np.abs(a_hat) @ np.abs(oracle.dequant_weights(w, s)).T
    ratio = float((np.abs(got - ref) / np.where(S > 0, S, 1.0)).max())
    err = oracle.row_normalised_error(got, ref)
    assert ratio <= 2.0 ** -16, ratio
    assert err <= GEMM_TOL, err
    return err, ratio


@pytest.mark.parametrize("M,N,K", [(1, 32, 4096), (1, 4096, 7168), (64, 4096, 7168),
                                   (5, 48, 1024), (17, 80, 2048), (70, 64, 512), (33, 48, 5120)])
def test_q8_gemm(M, N, K):
    err, ratio = _gemm_check(M, N, K, 110 + M)
    print(f"\n[q8] {M}x{N}x{K}: row-normalised {err:.2e}, residual/sum|aw| {ratio:.2e}")


def test_q8_route_accuracy_beside_the_mx_paths():
    """Against the exact product of the bf16 activations and the MXFP4 weights (the
    64 x 4096 x 7168 dense workload, 1 % outliers): the Q8 route's error sits between
    the bf16-activation GEMM's (exact weights, no activation rounding) and the MXFP4
    activations' (E2M1, 1 mantissa bit)."""
    d = dg.workload_inputs("dense_m64_n4096_k7168")
    a, w, s = d["a"], d["w"], d["w_scale"]
    exact = oracle.w4a16_gemm(a, w, s, "mxfp4")
    ad, wd, sd = bf16_dev(a), torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda()
    q, dq = ops.q8_quantize_act(ad)
    errs = {"q8": oracle.row_normalised_error(host(ops.mxfp4_gemm_q8(q, dq, wd, sd)), exact),
            "w4a16": oracle.row_normalised_error(host(ops.fp4_gemm_w4a16(ad, wd, sd, "mxfp4")), exact),
            "e4m3": oracle.row_normalised_error(host(ops.mxfp4_gemm(ad, wd, sd, "e4m3")), exact),
            "e2m1": oracle.row_normalised_error(host(ops.mxfp4_gemm(ad, wd, sd, "e2m1")), exact)}
    torch.cuda.synchronize()
    print(f"\n[q8] error against bf16 x MXFP4 exact: {errs}")
    assert errs["w4a16"] < errs["q8"] < errs["e2m1"]


def test_q8_gemm_is_deterministic():
    x = bf16_dev(dg.activations(120, 64, 7168))
    w, s = [torch.from_numpy(t).cuda() for t in dg.dense_weights(120, 4096, 7168, 120, 128)]
    q, d = ops.q8_quantize_act(x)
    assert torch.equal(ops.mxfp4_gemm_q8(q, d, w, s), ops.mxfp4_gemm_q8(q, d, w, s))
