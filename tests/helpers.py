"""Shared helpers for the GPU parity tests (not a test module)."""

import numpy as np
import torch

import oracle

GEMM_TOL = 2e-3  # max over rows of max |gpu - ref| / ||ref_row||_2


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    return t.numpy()


def straddle_check(gpu_codes, gpu_scale, h_pre, fmt, tol=1e-3):
    """Requantised h: every GPU-vs-oracle difference must be explained by the
    GPU's pre-quantisation value being on the other side of a rounding boundary
    within `tol` (relative to the block amax), or by a block whose amax sits
    within `tol` of a power of two (scale-byte boundary).

    gpu_codes: [R][I] unpacked codes; gpu_scale: [R][I/32]; h_pre: fp64 oracle
    values [R][I]. Returns (n_code_mismatch, n_block_scale_mismatch)."""
    ref_codes, ref_scale = oracle.mx_quantize(h_pre, fmt)
    R, I = h_pre.shape
    nb = I // 32
    blk = h_pre.reshape(R, nb, 32)
    amax = np.abs(blk).max(-1)
    sc_bad = gpu_scale != ref_scale
    if sc_bad.any():
        a = amax[sc_bad]
        near = np.abs(a / np.exp2(np.round(np.log2(np.maximum(a, 1e-300)))) - 1.0) <= tol
        assert near.all(), f"scale byte differs away from a power-of-two amax: {a[~near][:5]}"
    bad = (gpu_codes != ref_codes).reshape(R, nb, 32)
    bad &= ~sc_bad[..., None]
    n_code = int(bad.sum())
    if n_code:
        rr, bb, kk = np.nonzero(bad)
        xp = ref_scale[rr, bb].astype(np.int64) - 127
        t = np.abs(np.ldexp(blk[rr, bb, kk], -xp))
        tmax = np.ldexp(amax[rr, bb], -xp)
        dec = oracle.e4m3_decode if fmt == "e4m3" else oracle.e2m1_decode
        g = np.abs(dec(gpu_codes.reshape(R, nb, 32)[rr, bb, kk]))
        r = np.abs(dec(ref_codes.reshape(R, nb, 32)[rr, bb, kk]))
        # the oracle's scaled value must lie within tol * tmax of the rounding interval of
        # the GPU's code (for neighbouring codes: of the midpoint between them). Far below
        # the block amax the grid is finer than that tolerance (E4M3 subnormals), so
        # codes there may legitimately be more than one grid step apart.
        grid = np.unique(np.abs(dec(np.arange(256 if fmt == "e4m3" else 16, dtype=np.uint8))))
        grid = grid[np.isfinite(grid)]
        i = np.searchsorted(grid, g)
        assert np.all(grid[np.minimum(i, grid.size - 1)] == g), "GPU code off the grid"
        lo_b = np.where(i > 0, (grid[np.maximum(i - 1, 0)] + g) / 2, 0.0)
        hi_b = np.where(i + 1 < grid.size, (g + grid[np.minimum(i + 1, grid.size - 1)]) / 2, np.inf)
        dist = np.maximum(np.maximum(lo_b - t, t - hi_b), 0.0)
        assert np.all(dist <= tol * tmax), "code differs away from a rounding boundary"
    return n_code, int(sc_bad.sum())


def unpack_codes(h, fmt):
    return oracle.unpack_e2m1(h) if fmt == "e2m1" else h
