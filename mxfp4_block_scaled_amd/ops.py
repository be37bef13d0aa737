"""Python binding of the C ABI in include/mxfp4_moe.h (argument marshalling only).

torch supplies device memory and the current HIP stream; every step of the
computation runs in the HIP kernels of libmxfp4moe.so. There is no fallback:
if the library is missing, or a call returns a non-zero status, a
RuntimeError is raised.
"""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp4moe.so")
_lib = None

MXF_E4M3, MXF_E2M1 = 0, 1
MXF_F32, MXF_BF16 = 0, 1
FMTS = {"e4m3": MXF_E4M3, "e2m1": MXF_E2M1}
DTYPES = {torch.float32: MXF_F32, torch.bfloat16: MXF_BF16}

_c_i64, _c_i32, _c_int, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t

SIGNATURES = {
    "mxf_status_str": (ctypes.c_char_p, [_c_int]),
    "mxf_abi_version": (_c_int, []),
    "mxfp4_quantize_act": (_c_int, [_p, _c_int, _c_i64, _c_i64, _c_int, _p, _p, _p]),
    "mxfp4_gemm_workspace_bytes": (_sz, [_c_i64, _c_i64, _c_i64, _c_int]),
    "mxfp4_gemm": (_c_int, [_p, _c_i64, _c_i64, _c_i64, _c_int, _p, _p, _p, _p, _sz, _p]),
    "moe_route_permute": (_c_int, [_p, _c_i64, _c_i32, _c_i32, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_mxfp4_gemm": (_c_int, [_p, _p, _c_int, _c_i64, _c_i32, _c_i64, _c_i64, _c_i32,
                                        _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_int, _p]),
    "moe_unpermute_combine": (_c_int, [_p, _c_int, _p, _p, _c_i64, _c_i32, _c_i64, _p, _c_int, _p]),
    # include/mxf_ceilings.h: achievable-rate probes (measurement helpers)
    "mxf_ceiling_mfma_flops": (_c_i64, [_c_int]),
    "mxf_ceiling_mfma": (_c_int, [_c_int, _p, _c_i64, _c_int, _c_int, _p, _p]),
    "mxf_ceiling_read": (_c_int, [_p, _c_i64, _p, _p]),
}

CEILING_MFMA_GROUPS = 512
CEILING_MFMA_WORDS = 64 * 6 * 64 * 8


def lib_path():
    return _LIB_PATH


def load():
    """Load libmxfp4moe.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built: run mxfp4_block_scaled_amd/build.py "
                               "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc, what):
    if rc != 0:
        msg = load().mxf_status_str(rc).decode()
        raise RuntimeError(f"{what} failed with status {rc}: {msg}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t):
    if not t.is_cuda:
        raise RuntimeError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise RuntimeError("tensors must be contiguous")
    return t.device


def mxfp4_quantize_act(x, fmt="e4m3"):
    """x [rows][K] bf16/fp32 -> (q [rows][K] or [rows][K/2] uint8, q_scale [rows][K/32] uint8)."""
    dev = _dev(x)
    rows, K = x.shape
    f = FMTS[fmt]
    q = torch.empty((rows, K // 2 if f == MXF_E2M1 else K), dtype=torch.uint8, device=dev)
    qs = torch.empty((rows, K // 32), dtype=torch.uint8, device=dev)
    _check(load().mxfp4_quantize_act(_ptr(x), DTYPES[x.dtype], rows, K, f, _ptr(q), _ptr(qs), _stream(dev)),
           "mxfp4_quantize_act")
    return q, qs


def mxfp4_gemm(a, w, w_scale, act_fmt="e4m3", out=None, workspace=None):
    """a [M][K] bf16, w [N][K/2] uint8, w_scale [N][K/32] uint8 -> c [M][N] fp32."""
    dev = _dev(a)
    _dev(w), _dev(w_scale)
    M, K = a.shape
    N = w.shape[0]
    f = FMTS[act_fmt]
    lib = load()
    need = lib.mxfp4_gemm_workspace_bytes(M, N, K, f)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    _check(lib.mxfp4_gemm(_ptr(a), M, N, K, f, _ptr(w), _ptr(w_scale), _ptr(c), _ptr(workspace),
                          workspace.numel(), _stream(dev)), "mxfp4_gemm")
    return c


def moe_route_permute(logits, topk):
    """logits [T][E] fp32 -> (topk_ids, gates, expert_offsets, sorted_pair, pair_row)."""
    dev = _dev(logits)
    T, E = logits.shape
    ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    gates = torch.empty((T, topk), dtype=torch.float32, device=dev)
    offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    sp = torch.empty((max(T * topk, 1),), dtype=torch.int32, device=dev)
    pr = torch.empty((max(T * topk, 1),), dtype=torch.int32, device=dev)
    _check(load().moe_route_permute(_ptr(logits), T, E, topk, _ptr(ids), _ptr(gates), _ptr(offs), _ptr(sp),
                                    _ptr(pr), _stream(dev)), "moe_route_permute")
    return ids, gates, offs, sp[:T * topk], pr[:T * topk]


def moe_grouped_mxfp4_gemm(q, q_scale, act_fmt, T, topk, expert_offsets, sorted_pair, w1, w1_scale, w2,
                           w2_scale, y_dtype=torch.bfloat16, h=None, h_scale=None, y=None):
    """Both expert FCs. Returns (h, h_scale, y) with y [T*topk][H] in permuted row order."""
    dev = _dev(q)
    E, twoI, Hh = w1.shape
    I = twoI // 2
    H = Hh * 2
    f = FMTS[act_fmt]
    R = T * topk
    if h is None:
        h = torch.empty((max(R, 1), I // 2 if f == MXF_E2M1 else I), dtype=torch.uint8, device=dev)
    if h_scale is None:
        h_scale = torch.empty((max(R, 1), I // 32), dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((max(R, 1), H), dtype=y_dtype, device=dev)
    _check(load().moe_grouped_mxfp4_gemm(
        _ptr(q), _ptr(q_scale), f, T, topk, H, I, E, _ptr(expert_offsets), _ptr(sorted_pair), _ptr(w1),
        _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(h), _ptr(h_scale), _ptr(y), DTYPES[y.dtype],
        _stream(dev)), "moe_grouped_mxfp4_gemm")
    return h[:R], h_scale[:R], y[:R]


def moe_unpermute_combine(y, gates, pair_row, T, topk, out_dtype=torch.bfloat16, out=None):
    """out [T][H] = sum_j gates[t, j] * y[pair_row[t*topk + j]]."""
    dev = _dev(y)
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    _check(load().moe_unpermute_combine(_ptr(y), DTYPES[y.dtype], _ptr(gates), _ptr(pair_row), T, topk, H,
                                        _ptr(out), DTYPES[out.dtype], _stream(dev)), "moe_unpermute_combine")
    return out


def moe_layer(x, logits, w1, w1_scale, w2, w2_scale, topk, act_fmt="e4m3", y_dtype=torch.bfloat16,
              out_dtype=torch.bfloat16):
    """The whole expert layer through the four C-ABI calls (one stream, no host sync)."""
    T = x.shape[0]
    q, qs = mxfp4_quantize_act(x, act_fmt)
    ids, gates, offs, sp, pr = moe_route_permute(logits, topk)
    h, hs, y = moe_grouped_mxfp4_gemm(q, qs, act_fmt, T, topk, offs, sp, w1, w1_scale, w2, w2_scale, y_dtype)
    out = moe_unpermute_combine(y, gates, pr, T, topk, out_dtype)
    return dict(q=q, q_scale=qs, topk_ids=ids, gates=gates, expert_offsets=offs, sorted_pair=sp, pair_row=pr,
                h=h, h_scale=hs, y=y, out=out)


def ceiling_mfma(operands, act_fmt="e2m1", scale=127, iters=2000, sink=None):
    """Register-only scaled-MFMA loop (include/mxf_ceilings.h); returns (sink, flops).
    operands: int32 device tensor of >= CEILING_MFMA_WORDS words."""
    dev = _dev(operands)
    if operands.dtype != torch.int32:
        raise RuntimeError("operands must be int32")
    if sink is None:
        sink = torch.empty(CEILING_MFMA_GROUPS, dtype=torch.float32, device=dev)
    lib = load()
    _check(lib.mxf_ceiling_mfma(FMTS[act_fmt], _ptr(operands), operands.numel(), scale, iters, _ptr(sink),
                                _stream(dev)), "mxf_ceiling_mfma")
    return sink, lib.mxf_ceiling_mfma_flops(iters)


def ceiling_read(buf, xor_out=None):
    """Streaming non-temporal read of a device buffer; returns the int32 tensor holding
    the XOR of all its 32-bit words (accumulated into xor_out when given)."""
    dev = _dev(buf)
    if xor_out is None:
        xor_out = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * buf.element_size()
    _check(load().mxf_ceiling_read(_ptr(buf), nbytes, _ptr(xor_out), _stream(dev)), "mxf_ceiling_read")
    return xor_out
