"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments with the documented status before any HIP
call (so these run without a GPU; no compute call is made)."""

import ctypes
import os
import re

import pytest

from mxfp4_block_scaled_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4_moe.h")

OK, NULL, SHAPE, ALIGN, FORMAT, UNSUPPORTED, LAUNCH, WORKSPACE = range(8)
P = ctypes.c_void_p


def _lib():
    if not os.path.exists(ops.lib_path()):
        pytest.skip("library not built (run __graft_entry__.build())")
    return ops.load()


def _declared(headers=(HEADER,)):
    text = "".join(open(h).read() for h in headers)
    return re.findall(r"^\s*(?:int|int64_t|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def _all_headers():
    inc = os.path.join(ROOT, "include")
    return [os.path.join(inc, f) for f in sorted(os.listdir(inc)) if f.endswith(".h")]


def test_header_declares_the_five_entry_points():
    names = set(_declared())
    for n in ["mxfp4_quantize_act", "mxfp4_gemm", "moe_route_permute", "moe_grouped_mxfp4_gemm",
              "moe_unpermute_combine"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    names = _declared(_all_headers())
    assert "mxf_ceiling_mfma" in names and "mxf_ceiling_read" in names
    for name in names:
        assert hasattr(lib, name), name
    assert lib.mxf_abi_version() == 2
    for s in range(8):
        assert lib.mxf_status_str(s)


A = P(4096)      # a fake, aligned, non-null device address (never dereferenced: validation fails first)
U = P(4096 + 4)  # misaligned


def test_quantize_errors():
    lib = _lib()
    assert lib.mxfp4_quantize_act(A, 1, 4, 48, 0, A, A, None) == SHAPE        # K % 32
    assert lib.mxfp4_quantize_act(A, 1, -1, 64, 0, A, A, None) == SHAPE
    assert lib.mxfp4_quantize_act(A, 7, 4, 64, 0, A, A, None) == FORMAT       # dtype
    assert lib.mxfp4_quantize_act(A, 1, 4, 64, 3, A, A, None) == FORMAT       # element format
    assert lib.mxfp4_quantize_act(None, 1, 4, 64, 0, A, A, None) == NULL
    assert lib.mxfp4_quantize_act(U, 1, 4, 64, 0, A, A, None) == ALIGN
    assert lib.mxfp4_quantize_act(None, 1, 0, 64, 0, None, None, None) == OK  # empty: nothing to do


def test_gemm_errors():
    lib = _lib()
    need = lib.mxfp4_gemm_workspace_bytes(32, 32, 4096, 0)
    # 17..64 rows: E4M3 codes + scale bytes + fp32 partial sums of the 2 K slices (8 super-steps of 512)
    assert need >= 32 * 4096 + 32 * 128 + 2 * 32 * 32 * 4
    assert lib.mxfp4_gemm_workspace_bytes(32, 32, 4096, 1) < need
    # no K split above 64 rows, nor when K fits one slice of 4 super-steps
    assert lib.mxfp4_gemm_workspace_bytes(100, 32, 4096, 0) < 100 * 4096 + 100 * 128 + 512
    assert lib.mxfp4_gemm_workspace_bytes(32, 32, 2048, 0) < 32 * 2048 + 32 * 64 + 512
    assert lib.mxfp4_gemm_workspace_bytes(0, 32, 4096, 0) == 0
    # at most 16 rows: quantised in registers, so no codes; a weight matrix of at most
    # 1 MiB of codes runs in one launch (no workspace), a larger one in 4-super-step
    # K slices (fp32 partial sums only)
    assert lib.mxfp4_gemm_workspace_bytes(16, 32, 4096, 0) == 0
    assert lib.mxfp4_gemm_workspace_bytes(1, 512, 4096, 1) == 0
    assert lib.mxfp4_gemm_workspace_bytes(16, 4096, 7168, 0) == 4 * 16 * 4096 * 4
    assert lib.mxfp4_gemm_workspace_bytes(5, 4096, 7168, 1) == (4 * 5 * 4096 * 4 + 255) // 256 * 256
    assert lib.mxfp4_gemm(A, 32, 32, 4096 + 64, 0, A, A, A, A, need, None) == SHAPE  # K % 512
    assert lib.mxfp4_gemm(A, 32, 40, 4096, 0, A, A, A, A, need, None) == SHAPE       # N % 16
    assert lib.mxfp4_gemm(A, 32, 32, 4096, 2, A, A, A, A, need, None) == FORMAT
    assert lib.mxfp4_gemm(A, 32, 32, 4096, 0, None, A, A, A, need, None) == NULL
    assert lib.mxfp4_gemm(A, 32, 32, 4096, 0, A, A, A, A, need - 1, None) == WORKSPACE
    assert lib.mxfp4_gemm(A, 32, 32, 4096, 0, A, A, A, None, need, None) == WORKSPACE
    assert lib.mxfp4_gemm(A, 32, 32, 4096, 0, A, U, A, A, need, None) == ALIGN
    need16 = lib.mxfp4_gemm_workspace_bytes(16, 4096, 7168, 0)
    assert lib.mxfp4_gemm(A, 16, 4096, 7168, 0, A, A, A, None, need16, None) == WORKSPACE
    assert lib.mxfp4_gemm(A, 16, 4096, 7168, 0, A, A, A, A, need16 - 1, None) == WORKSPACE
    assert lib.mxfp4_gemm(A, 16, 4096, 7168, 0, A, A, A, U, need16, None) == ALIGN
    assert lib.mxfp4_gemm(None, 0, 32, 4096, 0, None, None, None, None, 0, None) == OK
    # M > 64 with N % 256 == 0 runs the tiled kernels: operands below 4 GiB (32-bit offsets)
    assert lib.mxfp4_gemm(A, 1 << 20, 256, 8192, 0, A, A, A, A, 1 << 40, None) == UNSUPPORTED
    assert lib.mxfp4_gemm(A, 1 << 20, 272, 8192, 0, A, A, A, A, need, None) == WORKSPACE  # streamed path
    # the streamed path addresses 64 weight rows (64 x K/2 bytes) with 32-bit offsets
    assert lib.mxfp4_gemm(A, 16, 32, 1 << 27, 0, A, A, A, A, 1 << 40, None) == UNSUPPORTED
    assert lib.mxfp4_gemm(A, 16, 32, (1 << 27) - 512, 0, A, A, A, A, 0, None) == WORKSPACE


def test_route_errors():
    lib = _lib()
    args = [A, A, A, A, A, None]
    assert lib.moe_route_permute(A, 8, 256, 9, *args) == SHAPE         # topk > 8
    assert lib.moe_route_permute(A, 8, 4, 6, *args) == SHAPE           # topk > E
    assert lib.moe_route_permute(A, 8, 256, 0, *args) == SHAPE
    assert lib.moe_route_permute(A, 8, 2048, 6, *args) == UNSUPPORTED  # E > 1024
    assert lib.moe_route_permute(A, 2 ** 30, 256, 6, *args) == UNSUPPORTED  # T*topk >= 2^31
    assert lib.moe_route_permute(A, 100000, 1024, 1, *args) == UNSUPPORTED  # no room for block counts
    assert lib.moe_route_permute(None, 8, 256, 6, *args) == NULL
    assert lib.moe_route_permute(A, 8, 256, 6, U, A, A, A, A, None) == ALIGN


def test_grouped_gemm_errors():
    lib = _lib()

    def call(**kw):
        a = dict(q=A, qs=A, fmt=0, T=8, k=6, H=7168, I=2048, E=256, off=A, sp=A, w1=A, s1=A, w2=A, s2=A,
                 h=A, hs=A, y=A, yd=1)
        a.update(kw)
        return lib.moe_grouped_mxfp4_gemm(a["q"], a["qs"], a["fmt"], a["T"], a["k"], a["H"], a["I"], a["E"],
                                          a["off"], a["sp"], a["w1"], a["s1"], a["w2"], a["s2"], a["h"],
                                          a["hs"], a["y"], a["yd"], None)

    assert call(H=7168 + 128) == SHAPE
    assert call(I=2048 + 32) == SHAPE
    assert call(k=9) == SHAPE
    assert call(fmt=5) == FORMAT
    assert call(yd=3) == FORMAT
    assert call(w2=None) == NULL
    assert call(h=U) == ALIGN
    assert call(E=4096) == UNSUPPORTED
    # tiled path (T > 64): q, h and one expert's weights must stay below 4 GiB (32-bit offsets)
    assert call(T=600_000) == UNSUPPORTED            # q = 600000 x 7168 bytes (E4M3)
    assert call(T=1_000_000, fmt=1) == UNSUPPORTED   # h = 6e6 x 1024 bytes (E2M1)
    assert call(T=600_000, fmt=1, k=1, w2=None) == NULL  # fits: checked up to the NULL test, nothing runs
    assert call(H=1 << 20, I=4096, T=100) == UNSUPPORTED  # w1 = 8192 x 2^19 bytes per expert
    assert call(H=1 << 20, I=4096, T=8) == UNSUPPORTED    # the streaming kernel too
    assert call(H=1 << 20, I=2048, T=8, w2=None) == NULL  # 4096 x 2^19 bytes: fits
    assert call(T=0, q=None) == OK


def test_quantize_route_errors():
    lib = _lib()

    def call(**kw):
        a = dict(x=A, xd=1, lg=A, T=8, H=7168, E=256, k=6, fmt=0, q=A, qs=A, ids=A, g=A, off=A, sp=A, pr=A)
        a.update(kw)
        return lib.moe_quantize_route(a["x"], a["xd"], a["lg"], a["T"], a["H"], a["E"], a["k"], a["fmt"], a["q"],
                                      a["qs"], a["ids"], a["g"], a["off"], a["sp"], a["pr"], None)

    assert call(T=65) == UNSUPPORTED  # decode-sized batches only
    assert call(E=257) == UNSUPPORTED
    assert call(H=7168 + 16) == SHAPE
    assert call(k=9) == SHAPE
    assert call(k=7, E=6) == SHAPE
    assert call(xd=3) == FORMAT
    assert call(fmt=2) == FORMAT
    assert call(lg=None) == NULL
    assert call(off=None, T=0) == NULL  # the offsets are written even for no tokens
    assert call(pr=U) == ALIGN
    assert call(x=U) == ALIGN


def test_fused_fc2_combine_errors():
    lib = _lib()

    def call(**kw):
        a = dict(q=A, qs=A, fmt=1, T=8, k=6, H=7168, I=2048, E=256, off=A, sp=A, ids=A, pr=A, g=A, w1=A, s1=A,
                 w2=A, s2=A, h=A, hs=A, out=A, od=1)
        a.update(kw)
        return lib.moe_grouped_mxfp4_gemm_combine(
            a["q"], a["qs"], a["fmt"], a["T"], a["k"], a["H"], a["I"], a["E"], a["off"], a["sp"], a["ids"],
            a["pr"], a["g"], a["w1"], a["s1"], a["w2"], a["s2"], a["h"], a["hs"], a["out"], a["od"], None)

    assert call(T=65) == UNSUPPORTED  # decode-sized batches only
    assert call(H=7168 + 128) == SHAPE
    assert call(I=2048 + 32) == SHAPE
    assert call(k=9) == SHAPE
    assert call(k=7, E=6) == SHAPE
    assert call(fmt=5) == FORMAT
    assert call(od=3) == FORMAT
    assert call(E=4096) == UNSUPPORTED
    assert call(H=1 << 20, I=4096) == UNSUPPORTED  # one expert's w1 above 4 GiB
    assert call(g=None) == NULL
    assert call(ids=None) == NULL
    assert call(pr=U) == ALIGN
    assert call(out=None) == NULL
    assert call(g=U) == ALIGN
    assert call(out=U) == ALIGN
    assert call(T=0, q=None, g=None) == OK


def test_combine_errors():
    lib = _lib()
    assert lib.moe_unpermute_combine(A, 1, A, A, 8, 6, 7164, A, 1, None) == SHAPE  # H % 8
    assert lib.moe_unpermute_combine(A, 2, A, A, 8, 6, 7168, A, 1, None) == FORMAT
    assert lib.moe_unpermute_combine(A, 1, None, A, 8, 6, 7168, A, 1, None) == NULL
    assert lib.moe_unpermute_combine(A, 1, A, A, 8, 6, 7168, U, 1, None) == ALIGN
    assert lib.moe_unpermute_combine(None, 1, None, None, 0, 6, 7168, None, 1, None) == OK


def test_ceiling_probe_errors():
    lib = _lib()
    W = ops.CEILING_MFMA_WORDS
    assert lib.mxf_ceiling_mfma_flops(10) == 512 * 4 * 10 * 8 * 131072
    assert lib.mxf_ceiling_mfma_flops(0) == 0
    assert lib.mxf_ceiling_mfma(2, A, W, 127, 10, A, None) == FORMAT
    assert lib.mxf_ceiling_mfma(1, A, W - 1, 127, 10, A, None) == SHAPE
    assert lib.mxf_ceiling_mfma(1, A, W, 127, 0, A, None) == SHAPE
    assert lib.mxf_ceiling_mfma(1, A, W, 255, 10, A, None) == SHAPE
    assert lib.mxf_ceiling_mfma(1, None, W, 127, 10, A, None) == NULL
    assert lib.mxf_ceiling_mfma(1, U, W, 127, 10, A, None) == ALIGN
    assert lib.mxf_ceiling_read(A, 40, A, None) == SHAPE
    assert lib.mxf_ceiling_read(None, 64, A, None) == NULL
    assert lib.mxf_ceiling_read(U, 64, A, None) == ALIGN
    assert lib.mxf_ceiling_read(None, 0, None, None) == OK
    R = ops.CEILING_COPY_REGION
    assert R == 28 * 32768
    assert lib.mxf_ceiling_lds_copy_bytes(0, 1024) == 2 * 1024 * R
    assert lib.mxf_ceiling_lds_copy_bytes(1, 2048) == (128 + 1024) * R
    assert lib.mxf_ceiling_lds_copy_bytes(1, 100) == 0 and lib.mxf_ceiling_lds_copy_bytes(2, 256) == 0
    assert lib.mxf_ceiling_lds_copy_bytes(0, 65536 + 256) == 0
    assert lib.mxf_ceiling_lds_copy(A, 2 * 256 * R - 16, 0, 256, A, None) == SHAPE
    assert lib.mxf_ceiling_lds_copy(A, 1 << 40, 1, 255, A, None) == SHAPE
    assert lib.mxf_ceiling_lds_copy(A, 1 << 40, 3, 256, A, None) == SHAPE
    assert lib.mxf_ceiling_lds_copy(None, 1 << 40, 0, 256, A, None) == NULL
    assert lib.mxf_ceiling_lds_copy(A, 1 << 40, 0, 256, None, None) == NULL
    assert lib.mxf_ceiling_lds_copy(U, 1 << 40, 0, 256, A, None) == ALIGN


def test_noalloc_gemm_rejects_before_touching_the_device():
    """Validation and the size limit come before any HIP call."""
    lib = _lib()
    cap = lib.mxfp4_noalloc_scratch_bytes()
    assert cap == 16 << 20
    assert lib.mxfp4_gemm_noalloc(A, 8192, 256, 4096, 0, A, A, A, None) == WORKSPACE   # 32 MiB of quantised A
    assert lib.mxfp4_gemm_noalloc(A, 16, 256, 4000, 0, A, A, A, None) == SHAPE         # K % 512
    assert lib.mxfp4_gemm_noalloc(A, 16, 24, 4096, 0, A, A, A, None) == SHAPE          # N % 16
    assert lib.mxfp4_gemm_noalloc(A, 16, 256, 4096, 9, A, A, A, None) == FORMAT
    assert lib.mxfp4_gemm_noalloc(None, 16, 256, 4096, 0, A, A, A, None) == NULL
    assert lib.mxfp4_gemm_noalloc(A, 0, 256, 4096, 0, A, A, A, None) == OK             # M == 0: no-op


def test_w4a16_errors_before_any_device_call():
    lib = _lib()
    for fn in (lib.mxfp4_gemm_w4a16, lib.nvfp4_gemm_w4a16):
        assert fn(A, 4, 64, 1000, A, A, A, A, 1 << 20, None) == SHAPE      # K % 512
        assert fn(A, 4, 40, 1024, A, A, A, A, 1 << 20, None) == SHAPE      # N % 16
        assert fn(A, -1, 64, 1024, A, A, A, A, 1 << 20, None) == SHAPE
        assert fn(A, 0, 64, 1024, A, A, A, A, 0, None) == OK               # M == 0: no-op
        assert fn(None, 4, 64, 1024, A, A, A, A, 1 << 20, None) == NULL
        assert fn(U, 4, 64, 1024, A, A, A, A, 1 << 20, None) == ALIGN
        need = lib.fp4_w4a16_workspace_bytes(4, 64, 4096)                   # narrow N: K slices
        assert need > 0
        assert fn(A, 4, 64, 4096, A, A, A, A, need - 1, None) == WORKSPACE
        assert fn(A, 4, 64, 4096, A, A, A, None, need, None) == WORKSPACE
    assert lib.fp4_w4a16_workspace_bytes(4, 16384, 4096) == 0            # wide N: no K split


def test_q8_errors_before_any_device_call():
    lib = _lib()
    assert lib.q8_quantize_act(A, 4, 48, A, A, None) == SHAPE          # K % 32
    assert lib.q8_quantize_act(A, 0, 64, A, A, None) == OK             # rows == 0
    assert lib.q8_quantize_act(None, 4, 64, A, A, None) == NULL
    assert lib.q8_quantize_act(A, 4, 64, A, P(4096 + 1), None) == ALIGN  # fp16 scales: 2-byte aligned
    assert lib.mxfp4_gemm_q8(A, A, 4, 64, 1000, A, A, A, A, 1 << 20, None) == SHAPE
    assert lib.mxfp4_gemm_q8(A, A, 0, 64, 1024, A, A, A, None, 0, None) == OK
    assert lib.mxfp4_gemm_q8(A, None, 4, 64, 1024, A, A, A, A, 1 << 20, None) == NULL
    need = lib.mxfp4_gemm_q8_workspace_bytes(4, 64, 4096)
    assert need > 0 and lib.mxfp4_gemm_q8(A, A, 4, 64, 4096, A, A, A, A, need - 1, None) == WORKSPACE
