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
    "mxfp4_noalloc_scratch_bytes": (_sz, []),
    "mxfp4_gemm_noalloc": (_c_int, [_p, _c_i64, _c_i64, _c_i64, _c_int, _p, _p, _p, _p]),
    "fp4_w4a16_workspace_bytes": (_sz, [_c_i64, _c_i64, _c_i64]),
    "mxfp4_gemm_w4a16": (_c_int, [_p, _c_i64, _c_i64, _c_i64, _p, _p, _p, _p, _sz, _p]),
    "nvfp4_gemm_w4a16": (_c_int, [_p, _c_i64, _c_i64, _c_i64, _p, _p, _p, _p, _sz, _p]),
    "q8_quantize_act": (_c_int, [_p, _c_i64, _c_i64, _p, _p, _p]),
    "mxfp4_gemm_q8_workspace_bytes": (_sz, [_c_i64, _c_i64, _c_i64]),
    "mxfp4_gemm_q8": (_c_int, [_p, _p, _c_i64, _c_i64, _c_i64, _p, _p, _p, _p, _sz, _p]),
    "moe_route_permute": (_c_int, [_p, _c_i64, _c_i32, _c_i32, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_mxfp4_gemm": (_c_int, [_p, _p, _c_int, _c_i64, _c_i32, _c_i64, _c_i64, _c_i32,
                                        _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_int, _p]),
    "moe_unpermute_combine": (_c_int, [_p, _c_int, _p, _p, _c_i64, _c_i32, _c_i64, _p, _c_int, _p]),
    "moe_quantize_route": (_c_int, [_p, _c_int, _p, _c_i64, _c_i64, _c_i32, _c_i32, _c_int, _p, _p, _p, _p, _p, _p,
                                    _p, _p]),
    "moe_grouped_mxfp4_gemm_combine": (_c_int, [_p, _p, _c_int, _c_i64, _c_i32, _c_i64, _c_i64, _c_i32, _p, _p,
                                                _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_int, _p]),
    # include/mxf_ceilings.h: achievable-rate probes (measurement helpers)
    "mxf_ceiling_mfma_flops": (_c_i64, [_c_int]),
    "mxf_ceiling_mfma": (_c_int, [_c_int, _p, _c_i64, _c_int, _c_int, _p, _p]),
    "mxf_ceiling_read": (_c_int, [_p, _c_i64, _p, _p]),
    "mxf_ceiling_lds_copy_bytes": (_c_i64, [_c_int, _c_int]),
    "mxf_ceiling_lds_copy": (_c_int, [_p, _c_i64, _c_int, _c_int, _p, _p]),
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


def _need(t, name, dtypes, shape):
    """Raise unless t has one of `dtypes` and the given shape; a shape entry given
    as (">=", n) only bounds that dimension from below."""
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise RuntimeError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if t.dim() != len(shape):
        raise RuntimeError(f"{name}: {t.dim()}-d, expected {len(shape)}-d {shape}")
    for i, (got, want) in enumerate(zip(t.shape, shape)):
        ok = got >= want[1] if isinstance(want, tuple) else got == want
        if not ok:
            raise RuntimeError(f"{name}: shape {tuple(t.shape)}, expected {shape} (dimension {i})")


def mxfp4_quantize_act(x, fmt="e4m3"):
    """x [rows][K] bf16/fp32 -> (q [rows][K] or [rows][K/2] uint8, q_scale [rows][K/32] uint8)."""
    dev = _dev(x)
    if x.dim() != 2:
        raise RuntimeError("x must be 2-d [rows][K]")
    rows, K = x.shape
    _need(x, "x", (torch.bfloat16, torch.float32), (rows, K))
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
    if a.dim() != 2 or w.dim() != 2:
        raise RuntimeError("a must be [M][K] and w [N][K/2]")
    M, K = a.shape
    N = w.shape[0]
    _need(a, "a", torch.bfloat16, (M, K))
    _need(w, "w", torch.uint8, (N, K // 2))
    _need(w_scale, "w_scale", torch.uint8, (N, K // 32))
    f = FMTS[act_fmt]
    lib = load()
    need = lib.mxfp4_gemm_workspace_bytes(M, N, K, f)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace)
    _need(workspace, "workspace", torch.uint8, ((">=", need),))
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    _dev(c)
    _need(c, "out", torch.float32, (M, N))
    _check(lib.mxfp4_gemm(_ptr(a), M, N, K, f, _ptr(w), _ptr(w_scale), _ptr(c), _ptr(workspace),
                          workspace.numel(), _stream(dev)), "mxfp4_gemm")
    return c


def mxfp4_gemm_noalloc(a, w, w_scale, out, act_fmt="e4m3"):
    """mxfp4_gemm with the library's own fixed workspace (no allocation in the call):
    a [M][K] bf16, w [N][K/2] uint8, w_scale [N][K/32] uint8 -> out [M][N] fp32."""
    dev = _dev(a)
    _dev(w), _dev(w_scale), _dev(out)
    if a.dim() != 2 or w.dim() != 2:
        raise RuntimeError("a must be [M][K] and w [N][K/2]")
    M, K = a.shape
    N = w.shape[0]
    _need(a, "a", torch.bfloat16, (M, K))
    _need(w, "w", torch.uint8, (N, K // 2))
    _need(w_scale, "w_scale", torch.uint8, (N, K // 32))
    _need(out, "out", torch.float32, (M, N))
    _check(load().mxfp4_gemm_noalloc(_ptr(a), M, N, K, FMTS[act_fmt], _ptr(w), _ptr(w_scale), _ptr(out),
                                     _stream(dev)), "mxfp4_gemm_noalloc")
    return out


def fp4_gemm_w4a16(a, w, w_scale, fmt="mxfp4", out=None, workspace=None):
    """FP4 weights x bf16 activations: a [M][K] bf16, w [N][K/2] uint8, w_scale [N][K/32]
    (fmt "mxfp4", UE8M0) or [N][K/16] (fmt "nvfp4", UE4M3) uint8 -> c [M][N] fp32."""
    dev = _dev(a)
    _dev(w), _dev(w_scale)
    if a.dim() != 2 or w.dim() != 2:
        raise RuntimeError("a must be [M][K] and w [N][K/2]")
    M, K = a.shape
    N = w.shape[0]
    if fmt not in ("mxfp4", "nvfp4"):
        raise RuntimeError(f"unknown weight format {fmt!r}")
    _need(a, "a", torch.bfloat16, (M, K))
    _need(w, "w", torch.uint8, (N, K // 2))
    _need(w_scale, "w_scale", torch.uint8, (N, K // (16 if fmt == "nvfp4" else 32)))
    lib = load()
    need = lib.fp4_w4a16_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace)
    _need(workspace, "workspace", torch.uint8, ((">=", need),))
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    _dev(c)
    _need(c, "out", torch.float32, (M, N))
    fn = lib.nvfp4_gemm_w4a16 if fmt == "nvfp4" else lib.mxfp4_gemm_w4a16
    _check(fn(_ptr(a), M, N, K, _ptr(w), _ptr(w_scale), _ptr(c), _ptr(workspace), workspace.numel(), _stream(dev)),
           f"{fmt}_gemm_w4a16")
    return c


def q8_quantize_act(x):
    """x [rows][K] bf16 -> (q [rows][K] int8, d [rows][K/32] fp16): Q8 blocks of 32."""
    dev = _dev(x)
    if x.dim() != 2:
        raise RuntimeError("x must be [rows][K]")
    rows, K = x.shape
    _need(x, "x", torch.bfloat16, (rows, K))
    q = torch.empty((rows, K), dtype=torch.int8, device=dev)
    d = torch.empty((rows, K // 32), dtype=torch.float16, device=dev)
    _check(load().q8_quantize_act(_ptr(x), rows, K, _ptr(q), _ptr(d), _stream(dev)), "q8_quantize_act")
    return q, d


def mxfp4_gemm_q8(q, d, w, w_scale, out=None, workspace=None):
    """The lookup-table route: q [M][K] int8, d [M][K/32] fp16 (from q8_quantize_act),
    w [N][K/2] uint8, w_scale [N][K/32] uint8 -> c [M][N] fp32."""
    dev = _dev(q)
    for t in (d, w, w_scale):
        _dev(t)
    if q.dim() != 2 or w.dim() != 2:
        raise RuntimeError("q must be [M][K] and w [N][K/2]")
    M, K = q.shape
    N = w.shape[0]
    _need(q, "q", torch.int8, (M, K))
    _need(d, "d", torch.float16, (M, K // 32))
    _need(w, "w", torch.uint8, (N, K // 2))
    _need(w_scale, "w_scale", torch.uint8, (N, K // 32))
    lib = load()
    need = lib.mxfp4_gemm_q8_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace)
    _need(workspace, "workspace", torch.uint8, ((">=", need),))
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    _dev(c)
    _need(c, "out", torch.float32, (M, N))
    _check(lib.mxfp4_gemm_q8(_ptr(q), _ptr(d), M, N, K, _ptr(w), _ptr(w_scale), _ptr(c), _ptr(workspace),
                             workspace.numel(), _stream(dev)), "mxfp4_gemm_q8")
    return c


def moe_route_permute(logits, topk):
    """logits [T][E] fp32 -> (topk_ids, gates, expert_offsets, sorted_pair, pair_row)."""
    dev = _dev(logits)
    if logits.dim() != 2:
        raise RuntimeError("logits must be [T][E]")
    T, E = logits.shape
    _need(logits, "logits", torch.float32, (T, E))
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
    for t in (q_scale, expert_offsets, sorted_pair, w1, w1_scale, w2, w2_scale):
        _dev(t)
    if w1.dim() != 3:
        raise RuntimeError("w1 must be [E][2I][H/2]")
    E, twoI, Hh = w1.shape
    I = twoI // 2
    H = Hh * 2
    f = FMTS[act_fmt]
    R = T * topk
    fp4 = f == MXF_E2M1
    _need(q, "q", torch.uint8, (T, H // 2 if fp4 else H))
    _need(q_scale, "q_scale", torch.uint8, (T, H // 32))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    _need(sorted_pair, "sorted_pair", torch.int32, ((">=", R),))
    _need(w1, "w1", torch.uint8, (E, 2 * I, H // 2))
    _need(w1_scale, "w1_scale", torch.uint8, (E, 2 * I, H // 32))
    _need(w2, "w2", torch.uint8, (E, H, I // 2))
    _need(w2_scale, "w2_scale", torch.uint8, (E, H, I // 32))
    if h is None:
        h = torch.empty((max(R, 1), I // 2 if fp4 else I), dtype=torch.uint8, device=dev)
    if h_scale is None:
        h_scale = torch.empty((max(R, 1), I // 32), dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((max(R, 1), H), dtype=y_dtype, device=dev)
    for t in (h, h_scale, y):
        _dev(t)
    _need(h, "h", torch.uint8, ((">=", R), I // 2 if fp4 else I))
    _need(h_scale, "h_scale", torch.uint8, ((">=", R), I // 32))
    _need(y, "y", (torch.float32, torch.bfloat16), ((">=", R), H))
    _check(load().moe_grouped_mxfp4_gemm(
        _ptr(q), _ptr(q_scale), f, T, topk, H, I, E, _ptr(expert_offsets), _ptr(sorted_pair), _ptr(w1),
        _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(h), _ptr(h_scale), _ptr(y), DTYPES[y.dtype],
        _stream(dev)), "moe_grouped_mxfp4_gemm")
    return h[:R], h_scale[:R], y[:R]


def moe_unpermute_combine(y, gates, pair_row, T, topk, out_dtype=torch.bfloat16, out=None):
    """out [T][H] = sum_j gates[t, j] * y[pair_row[t*topk + j]]."""
    dev = _dev(y)
    _dev(gates), _dev(pair_row)
    if y.dim() != 2:
        raise RuntimeError("y must be [T*topk][H]")
    H = y.shape[1]
    _need(y, "y", (torch.float32, torch.bfloat16), ((">=", T * topk), H))
    _need(gates, "gates", torch.float32, (T, topk))
    _need(pair_row, "pair_row", torch.int32, ((">=", T * topk),))
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    _dev(out)
    _need(out, "out", (torch.float32, torch.bfloat16), (T, H))
    _check(load().moe_unpermute_combine(_ptr(y), DTYPES[y.dtype], _ptr(gates), _ptr(pair_row), T, topk, H,
                                        _ptr(out), DTYPES[out.dtype], _stream(dev)), "moe_unpermute_combine")
    return out


def moe_quantize_route(x, logits, topk, act_fmt="e4m3"):
    """mxfp4_quantize_act(x) and moe_route_permute(logits) in one launch (T <= 64,
    E <= 256). Returns (q, q_scale, topk_ids, gates, expert_offsets, sorted_pair, pair_row)."""
    dev = _dev(x)
    _dev(logits)
    if x.dim() != 2 or logits.dim() != 2:
        raise RuntimeError("x must be [T][H] and logits [T][E]")
    T, H = x.shape
    E = logits.shape[1]
    _need(x, "x", (torch.bfloat16, torch.float32), (T, H))
    _need(logits, "logits", torch.float32, (T, E))
    f = FMTS[act_fmt]
    fp4 = f == MXF_E2M1
    R = T * topk
    q = torch.empty((T, H // 2 if fp4 else H), dtype=torch.uint8, device=dev)
    qs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    gates = torch.empty((T, topk), dtype=torch.float32, device=dev)
    offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    sp = torch.empty((max(R, 1),), dtype=torch.int32, device=dev)
    pr = torch.empty((max(R, 1),), dtype=torch.int32, device=dev)
    _check(load().moe_quantize_route(_ptr(x), DTYPES[x.dtype], _ptr(logits), T, H, E, topk, f, _ptr(q), _ptr(qs),
                                     _ptr(ids), _ptr(gates), _ptr(offs), _ptr(sp), _ptr(pr), _stream(dev)),
           "moe_quantize_route")
    return q, qs, ids, gates, offs, sp[:R], pr[:R]


def moe_grouped_mxfp4_gemm_combine(q, q_scale, act_fmt, T, topk, expert_offsets, sorted_pair, topk_ids, pair_row,
                                   gates, w1, w1_scale, w2, w2_scale, out_dtype=torch.bfloat16, h=None,
                                   h_scale=None, out=None):
    """Both expert FCs with FC2 fused into the gate-weighted combine (T <= 64).
    Returns (h, h_scale, out) with out [T][H]."""
    dev = _dev(q)
    for t in (q_scale, expert_offsets, sorted_pair, topk_ids, pair_row, gates, w1, w1_scale, w2, w2_scale):
        _dev(t)
    if w1.dim() != 3:
        raise RuntimeError("w1 must be [E][2I][H/2]")
    E, twoI, Hh = w1.shape
    I = twoI // 2
    H = Hh * 2
    f = FMTS[act_fmt]
    R = T * topk
    fp4 = f == MXF_E2M1
    _need(q, "q", torch.uint8, (T, H // 2 if fp4 else H))
    _need(q_scale, "q_scale", torch.uint8, (T, H // 32))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    _need(sorted_pair, "sorted_pair", torch.int32, ((">=", R),))
    _need(topk_ids, "topk_ids", torch.int32, (T, topk))
    _need(pair_row, "pair_row", torch.int32, ((">=", R),))
    _need(gates, "gates", torch.float32, (T, topk))
    _need(w1, "w1", torch.uint8, (E, 2 * I, H // 2))
    _need(w1_scale, "w1_scale", torch.uint8, (E, 2 * I, H // 32))
    _need(w2, "w2", torch.uint8, (E, H, I // 2))
    _need(w2_scale, "w2_scale", torch.uint8, (E, H, I // 32))
    if h is None:
        h = torch.empty((max(R, 1), I // 2 if fp4 else I), dtype=torch.uint8, device=dev)
    if h_scale is None:
        h_scale = torch.empty((max(R, 1), I // 32), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((max(T, 1), H), dtype=out_dtype, device=dev)
    for t in (h, h_scale, out):
        _dev(t)
    _need(h, "h", torch.uint8, ((">=", R), I // 2 if fp4 else I))
    _need(h_scale, "h_scale", torch.uint8, ((">=", R), I // 32))
    _need(out, "out", (torch.float32, torch.bfloat16), ((">=", T), H))
    _check(load().moe_grouped_mxfp4_gemm_combine(
        _ptr(q), _ptr(q_scale), f, T, topk, H, I, E, _ptr(expert_offsets), _ptr(sorted_pair), _ptr(topk_ids),
        _ptr(pair_row), _ptr(gates), _ptr(w1), _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(h), _ptr(h_scale), _ptr(out),
        DTYPES[out.dtype], _stream(dev)), "moe_grouped_mxfp4_gemm_combine")
    return h[:R], h_scale[:R], out[:T]


def moe_layer(x, logits, w1, w1_scale, w2, w2_scale, topk, act_fmt="e4m3", y_dtype=torch.bfloat16,
              out_dtype=torch.bfloat16, fused=False):
    """The whole expert layer through the C-ABI calls (one stream, no host sync).
    fused=True (T <= 64): quantisation and routing in one launch (E <= 256), FC2 and
    the combine in one kernel; y is not formed (None)."""
    T = x.shape[0]
    if fused and logits.shape[1] <= 256:
        q, qs, ids, gates, offs, sp, pr = moe_quantize_route(x, logits, topk, act_fmt)
    else:
        q, qs = mxfp4_quantize_act(x, act_fmt)
        ids, gates, offs, sp, pr = moe_route_permute(logits, topk)
    if fused:
        h, hs, out = moe_grouped_mxfp4_gemm_combine(q, qs, act_fmt, T, topk, offs, sp, ids, pr, gates, w1, w1_scale,
                                                    w2, w2_scale, out_dtype)
        y = None
    else:
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


CEILING_COPY_STAGES = 28
CEILING_COPY_REGION = CEILING_COPY_STAGES * 32768


def ceiling_lds_copy(buf, pattern, groups, sum_out=None):
    """HBM -> LDS copy-path probe (include/mxf_ceilings.h): `groups` workgroups each fill
    28 stages of 64 KB from their two regions of buf (pattern 0: their own; pattern 1:
    shared as in the grouped FC1 launch). Returns the int32 tensor holding the sum, mod
    2^32, of every 32-bit word read (accumulated into sum_out when given)."""
    dev = _dev(buf)
    if sum_out is None:
        sum_out = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * buf.element_size()
    _check(load().mxf_ceiling_lds_copy(_ptr(buf), nbytes, pattern, groups, _ptr(sum_out), _stream(dev)),
           "mxf_ceiling_lds_copy")
    return sum_out
