"""Canary guards: every output and workspace of every entry point lives inside a
larger device buffer whose bytes before and after it hold a random pattern; after
the calls (and a synchronisation) the pattern must be unchanged. The tiled
kernels load through range-checked buffer resources, which read zeros instead of
faulting, so an offset mistake there shows up only in the results or as a stray
store: this test catches the stores. Shapes end in partial tiles and partial
row units on purpose."""

import numpy as np
import pytest
import torch

from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import bf16_dev

pytestmark = pytest.mark.gpu

GUARD = 8192  # bytes of pattern on each side (a multiple of 256: the payload stays aligned)


class Guarded:
    def __init__(self, shape, dtype, seed):
        nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.nbytes = nbytes
        pad = (-nbytes) % 256
        g = torch.Generator(device="cuda").manual_seed(seed)
        self.raw = torch.randint(0, 256, (2 * GUARD + nbytes + pad,), dtype=torch.uint8, device="cuda", generator=g)
        self.before = self.raw[:GUARD].clone()
        self.after = self.raw[GUARD + nbytes:].clone()
        self.t = self.raw[GUARD:GUARD + nbytes].view(dtype).view(shape) if nbytes else self.raw[GUARD:GUARD]

    def check(self, name):
        assert torch.equal(self.raw[:GUARD], self.before), f"{name}: bytes before the buffer changed"
        assert torch.equal(self.raw[GUARD + self.nbytes:], self.after), f"{name}: bytes after the buffer changed"


def _p(t):
    return ops._ptr(t)


@pytest.mark.parametrize("T,H,I,E,k,fmt,routing,y_dtype", [
    (8, 1024, 512, 16, 6, "e4m3", "normal", torch.bfloat16),    # decode: streaming kernels
    (13, 1024, 2048, 16, 6, "e2m1", "normal", torch.float32),   # decode FP4, fp32 y, FC2 two row blocks
    (301, 1024, 512, 8, 6, "e4m3", "normal", torch.bfloat16),   # FP8 256-row ring tiles, ragged
    (333, 1024, 1024, 32, 4, "e2m1", "normal", torch.float32),  # FP4 256-row tiles, fp32 y
    (700, 2048, 2048, 4, 2, "e2m1", "normal", torch.bfloat16),  # FP4, K = 2048 chained n-tiles
    (241, 1024, 1024, 64, 2, "e4m3", "zipf", torch.bfloat16),   # split: streamed small experts + tiles
])
def test_layer_outputs_stay_inside_their_buffers(T, H, I, E, k, fmt, routing, y_dtype):
    lib = ops.load()
    st = ops._stream(torch.device("cuda"))
    x = bf16_dev(dg.activations(51, T, H))
    logits = torch.from_numpy(dg.logits(51, T, E, routing)).cuda()
    w1, s1, w2, s2 = [torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in dg.moe_weights(51, E, H, I, 120, 128)]
    fp4 = fmt == "e2m1"
    f = ops.FMTS[fmt]
    R = T * k
    bufs = {
        "q": Guarded((T, H // 2 if fp4 else H), torch.uint8, 1), "q_scale": Guarded((T, H // 32), torch.uint8, 2),
        "ids": Guarded((T, k), torch.int32, 3), "gates": Guarded((T, k), torch.float32, 4),
        "offs": Guarded((E + 1,), torch.int32, 5), "sp": Guarded((R,), torch.int32, 6),
        "pr": Guarded((R,), torch.int32, 7), "h": Guarded((R, I // 2 if fp4 else I), torch.uint8, 8),
        "hs": Guarded((R, I // 32), torch.uint8, 9), "y": Guarded((R, H), y_dtype, 10),
        "out": Guarded((T, H), torch.bfloat16, 11),
    }
    b = {n: v.t for n, v in bufs.items()}
    ops._check(lib.mxfp4_quantize_act(_p(x), ops.MXF_BF16, T, H, f, _p(b["q"]), _p(b["q_scale"]), st), "quantize")
    ops._check(lib.moe_route_permute(_p(logits), T, E, k, _p(b["ids"]), _p(b["gates"]), _p(b["offs"]), _p(b["sp"]),
                                     _p(b["pr"]), st), "route")
    ops._check(lib.moe_grouped_mxfp4_gemm(_p(b["q"]), _p(b["q_scale"]), f, T, k, H, I, E, _p(b["offs"]), _p(b["sp"]),
                                          _p(w1), _p(s1), _p(w2), _p(s2), _p(b["h"]), _p(b["hs"]), _p(b["y"]),
                                          ops.DTYPES[y_dtype], st), "grouped")
    ops._check(lib.moe_unpermute_combine(_p(b["y"]), ops.DTYPES[y_dtype], _p(b["gates"]), _p(b["pr"]), T, k, H,
                                         _p(b["out"]), ops.MXF_BF16, st), "combine")
    torch.cuda.synchronize()
    for name, v in bufs.items():
        v.check(name)
    # the payloads were written (not just left alone): the last row of out is finite
    assert torch.isfinite(b["out"][-1].float()).all()


@pytest.mark.parametrize("T,H,I,E,k,fmt,out_dtype", [
    (8, 1024, 512, 16, 6, "e4m3", torch.bfloat16),   # decode-shaped
    (61, 1024, 1536, 4, 2, "e2m1", torch.float32),   # ~30 rows per expert, 3 super-steps
    (64, 512, 512, 300, 8, "e4m3", torch.float32),   # T * topk = 512, more than 256 experts
])
def test_fused_fc2_combine_outputs_stay_inside_their_buffers(T, H, I, E, k, fmt, out_dtype):
    lib = ops.load()
    st = ops._stream(torch.device("cuda"))
    x = bf16_dev(dg.activations(53, T, H))
    logits = torch.from_numpy(dg.logits(53, T, E, "normal")).cuda()
    w1, s1, w2, s2 = [torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in dg.moe_weights(53, E, H, I, 120, 128)]
    fp4 = fmt == "e2m1"
    f = ops.FMTS[fmt]
    R = T * k
    bufs = {
        "q": Guarded((T, H // 2 if fp4 else H), torch.uint8, 31), "q_scale": Guarded((T, H // 32), torch.uint8, 32),
        "ids": Guarded((T, k), torch.int32, 33), "gates": Guarded((T, k), torch.float32, 34),
        "offs": Guarded((E + 1,), torch.int32, 35), "sp": Guarded((R,), torch.int32, 36),
        "pr": Guarded((R,), torch.int32, 37), "h": Guarded((R, I // 2 if fp4 else I), torch.uint8, 38),
        "hs": Guarded((R, I // 32), torch.uint8, 39), "out": Guarded((T, H), out_dtype, 40),
    }
    b = {n: v.t for n, v in bufs.items()}
    ops._check(lib.mxfp4_quantize_act(_p(x), ops.MXF_BF16, T, H, f, _p(b["q"]), _p(b["q_scale"]), st), "quantize")
    ops._check(lib.moe_route_permute(_p(logits), T, E, k, _p(b["ids"]), _p(b["gates"]), _p(b["offs"]), _p(b["sp"]),
                                     _p(b["pr"]), st), "route")
    ops._check(lib.moe_grouped_mxfp4_gemm_combine(
        _p(b["q"]), _p(b["q_scale"]), f, T, k, H, I, E, _p(b["offs"]), _p(b["sp"]), _p(b["ids"]), _p(b["pr"]),
        _p(b["gates"]), _p(w1), _p(s1),
        _p(w2), _p(s2), _p(b["h"]), _p(b["hs"]), _p(b["out"]), ops.DTYPES[out_dtype], st), "grouped+combine")
    torch.cuda.synchronize()
    for name, v in bufs.items():
        v.check(name)
    assert torch.isfinite(b["out"].float()).all()


@pytest.mark.parametrize("M,N,K,fmt", [
    (37, 48, 5120, "e2m1"),   # M <= 64: K slices summed through the workspace
    (64, 4096, 7168, "e4m3"),  # the dense 64 x 4096 x 7168 shape
    (70, 256, 1536, "e4m3"),   # FP8 256-row ring tiles, ragged
    (300, 512, 1536, "e2m1"),  # FP4 256-row tiles, ragged
    (129, 96, 512, "e4m3"),    # N % 256 != 0: streamed in 64-row chunks
])
def test_dense_outputs_stay_inside_their_buffers(M, N, K, fmt):
    lib = ops.load()
    st = ops._stream(torch.device("cuda"))
    a = bf16_dev(dg.activations(52, M, K, outliers=True))
    w, s = [torch.from_numpy(t).cuda() for t in dg.dense_weights(52, N, K, 122, 130)]
    f = ops.FMTS[fmt]
    need = lib.mxfp4_gemm_workspace_bytes(M, N, K, f)
    c = Guarded((M, N), torch.float32, 21)
    ws = Guarded((need,), torch.uint8, 22)
    ops._check(lib.mxfp4_gemm(_p(a), M, N, K, f, _p(w), _p(s), _p(c.t), _p(ws.t), need, st), "mxfp4_gemm")
    torch.cuda.synchronize()
    c.check("c")
    ws.check("workspace")
    assert torch.isfinite(c.t).all()
