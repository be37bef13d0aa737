"""mxfp4_gemm_noalloc (its workspace is a fixed device array inside the library)
against mxfp4_gemm with a caller workspace, through the C ABI: the same kernels,
so the results must agree bit for bit - on two calls in a row, the second with a
smaller input than the first (the array keeps the first call's contents), and on
each kernel path (K slices summed through the workspace, 64-row chunks, tiles)."""

import numpy as np
import pytest
import torch

from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import bf16_dev

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, seed):
    a = bf16_dev(dg.activations(seed, M, K, outliers=True))
    w, s = [torch.from_numpy(t).cuda() for t in dg.dense_weights(seed, N, K, 122, 130)]
    return a, w, s


def _both(M, N, K, fmt, seed):
    lib = ops.load()
    st = ops._stream(torch.device("cuda"))
    a, w, s = _inputs(M, N, K, seed)
    f = ops.FMTS[fmt]
    need = lib.mxfp4_gemm_workspace_bytes(M, N, K, f)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    want = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ops._check(lib.mxfp4_gemm(ops._ptr(a), M, N, K, f, ops._ptr(w), ops._ptr(s), ops._ptr(want), ops._ptr(ws),
                              ws.numel(), st), "mxfp4_gemm")
    ops._check(lib.mxfp4_gemm_noalloc(ops._ptr(a), M, N, K, f, ops._ptr(w), ops._ptr(s), ops._ptr(got), st),
               "mxfp4_gemm_noalloc")
    torch.cuda.synchronize()
    return got, want


@pytest.mark.parametrize("first,second", [
    ((64, 4096, 7168, "e4m3"), (16, 32, 4096, "e4m3")),   # the two dense workloads, large then small
    ((300, 512, 1536, "e2m1"), (37, 48, 5120, "e2m1")),   # tiles, then K slices through the scratch
    ((129, 96, 512, "e4m3"), (70, 256, 1536, "e4m3")),    # 64-row chunks, then FP8 tiles
    # at most 16 rows (activations quantised in registers): K-slice partials in the array
    ((16, 4096, 7168, "e4m3"), (5, 2048, 4096, "e2m1")),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for i, (M, N, K, fmt) in enumerate((first, second)):
        got, want = _both(M, N, K, fmt, 60 + i)
        assert torch.isfinite(want).all()
        assert torch.equal(got, want), (M, N, K, fmt)


def test_noalloc_rejects_sizes_beyond_the_array():
    lib = ops.load()
    cap = lib.mxfp4_noalloc_scratch_bytes()
    M, N, K = 8192, 256, 4096  # quantised A alone is 32 MiB
    assert lib.mxfp4_gemm_workspace_bytes(M, N, K, ops.MXF_E4M3) > cap
    a, w, s = _inputs(16, N, K, 3)
    c = torch.empty((16, N), dtype=torch.float32, device="cuda")
    rc = lib.mxfp4_gemm_noalloc(ops._ptr(a), M, N, K, ops.MXF_E4M3, ops._ptr(w), ops._ptr(s), ops._ptr(c),
                                ops._stream(torch.device("cuda")))
    assert rc == 7  # MXF_ERR_WORKSPACE, nothing launched
