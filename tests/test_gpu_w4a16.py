"""GPU parity of the FP4-weight x bf16-activation GEMMs (mxfp4_gemm_w4a16 with MXFP4
weights, nvfp4_gemm_w4a16 with NVFP4 weights) against the fp64 oracle.

Every weight value (an E2M1 code times its block scale) is exact in bf16 and every
bf16 x bf16 product exact in fp32, so the only error is fp32 accumulation: checked
per element against |C_gpu - C_exact| <= 2^-16 * sum_k |a_k w_k| (gamma_256 covers
K / 32 = 224 instruction steps at K = 7168) and, like every GEMM here, against the
row-normalised 2e-3. Shapes: the accuracy table of "【DeepSeek V4】Triton FP4
优化实战" (第二步: 1 x 32 x 4096, 1 x 4096 x 7168, 64 x 4096 x 7168), ragged shapes
spanning several 64-row weight blocks, 64-row activation chunks and K slices, and
the extreme scale bytes."""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import GEMM_TOL, bf16_dev, host

pytestmark = pytest.mark.gpu

BOUND = 2.0 ** -16


def _weights(fmt, N, K, seed):
    if fmt == "nvfp4":
        return dg.nvfp4_weights(seed, N, K)
    return dg.dense_weights(seed, N, K, 118, 134)


def _check(a, w, s, fmt):
    c = ops.fp4_gemm_w4a16(bf16_dev(a), torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda(), fmt)
    torch.cuda.synchronize()
    got = host(c).astype(np.float64)
    ref = oracle.w4a16_gemm(a, w, s, fmt)
    w_hat = oracle.dequant_nvfp4_weights(w, s) if fmt == "nvfp4" else oracle.dequant_weights(w, s)
    S = np.abs(oracle.bf16_bits_to_f64(a)) @ np.abs(w_hat).T
    ratio = float((np.abs(got - ref) / np.where(S > 0, S, 1.0)).max())
    err = oracle.row_normalised_error(got, ref)
    assert ratio <= BOUND, ratio
    assert err <= GEMM_TOL, err
    return err, ratio


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("M,N,K", [(1, 32, 4096), (1, 4096, 7168), (64, 4096, 7168)])
def test_page_shapes(fmt, M, N, K):
    a = dg.activations(70 + M, M, K, outliers=True)
    w, s = _weights(fmt, N, K, 71)
    err, ratio = _check(a, w, s, fmt)
    print(f"\n[w4a16] {fmt} {M}x{N}x{K}: row-normalised {err:.2e}, residual/sum|aw| {ratio:.2e}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("M,N,K", [
    (5, 48, 1024),     # one partial weight block (48 of 64 rows), 5 token rows
    (17, 80, 2048),    # two weight blocks, the second partial; two token fragments
    (70, 64, 512),     # two 64-row activation chunks (70 = 64 + 6)
    (33, 48, 5120),    # K split into 3 slices of 4 super-steps, the last with idle waves
    (3, 16384, 1024),  # wide N: no K split, 256 weight blocks
])
def test_ragged_shapes(fmt, M, N, K):
    a = dg.activations(M * 3 + N, M, K, outliers=True)
    w, s = _weights(fmt, N, K, K + N)
    _check(a, w, s, fmt)


@pytest.mark.parametrize("choices,shift", [
    ([2, 3, 10], 60),          # weights near the bottom of bf16's normal range (2^-126 ...)
    ([120, 126, 127, 128, 134], 0),
    ([240, 250, 251, 252], -40),  # 6 x 2^125 is the largest weight that stays finite in bf16
])
def test_mxfp4_extreme_scale_bytes(choices, shift):
    """Scale bytes at both ends of the supported range 2 .. 252, with activations scaled
    so that products and sums stay in fp32's normal range."""
    M, N, K = 4, 64, 1024
    x = np.random.default_rng(80 + shift).standard_normal((M, K)).astype(np.float32) * np.float32(2.0 ** shift)
    a = dg.bf16_bits_from_f32(x)
    w, _ = dg.dense_weights(80, N, K, 120, 128)
    ch = np.array(choices, np.uint8)
    s = ch[np.random.default_rng(81 + shift).integers(0, ch.size, (N, K // 32))]
    _check(a, w, s, "mxfp4")


def test_nvfp4_every_scale_code():
    """Every finite UE4M3 scale byte (0x00 .. 0x7E, subnormals included) in one matrix."""
    M, N, K = 3, 128, 2048
    a = dg.activations(81, M, K)
    w, _ = dg.nvfp4_weights(81, N, K)
    s = (np.arange(N * K // 16) % 0x7F).astype(np.uint8).reshape(N, K // 16)
    _check(a, w, s, "nvfp4")


def test_bf16_activations_beat_mx_quantised_activations():
    """The second accuracy point: against the exact product of the bf16 activations and
    the MXFP4 weights, W4A16 is far closer than the MXFP8 (E4M3) path, which is closer
    than the MXFP4 (E2M1) path (both quantise the activations per 32 first)."""
    M, N, K = 64, 4096, 7168
    d = dg.workload_inputs("dense_m64_n4096_k7168")
    a, w, s = d["a"], d["w"], d["w_scale"]
    exact = oracle.w4a16_gemm(a, w, s, "mxfp4")
    errs = {}
    ad, wd, sd = bf16_dev(a), torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda()
    errs["w4a16"] = oracle.row_normalised_error(host(ops.fp4_gemm_w4a16(ad, wd, sd, "mxfp4")), exact)
    for fmt in ("e4m3", "e2m1"):
        errs[fmt] = oracle.row_normalised_error(host(ops.mxfp4_gemm(ad, wd, sd, fmt)), exact)
    torch.cuda.synchronize()
    print(f"\n[w4a16] error against bf16 x MXFP4 exact ({M}x{N}x{K}, 1% outliers): {errs}")
    assert errs["w4a16"] < 1e-5 < errs["e4m3"] < errs["e2m1"]


def test_w4a16_is_deterministic():
    a = bf16_dev(dg.activations(82, 64, 7168))
    w, s = [torch.from_numpy(t).cuda() for t in dg.nvfp4_weights(82, 4096, 7168)]
    c1 = ops.fp4_gemm_w4a16(a, w, s, "nvfp4")
    c2 = ops.fp4_gemm_w4a16(a, w, s, "nvfp4")
    assert torch.equal(c1, c2)
