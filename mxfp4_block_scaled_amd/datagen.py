"""Seeded synthetic inputs for the MXFP4 expert path.

This module draws random inputs and nothing else: it holds none of the
method's arithmetic (no quantisation, routing, GEMM or combine). Both the HIP
path and the CPU oracle consume exactly these arrays.

Sub-streams: ``rng(seed, tag, *idx)`` is numpy's PCG64 seeded with the tuple
(seed, tag, *idx), so every tensor - and every expert's weights - has its own
stream and its bytes do not depend on draw order or on which experts are
touched.

Tags: 1 activations (standard normal fp32), 2 outlier mask (p = 0.01),
3 routing logits (standard normal fp32), 4 / 5 dense weight codes / scale
exponents, 6 / 7 FC1 codes / scale exponents per expert, 8 / 9 FC2 codes /
scale exponents per expert, 10 / 11 NVFP4 weight codes / UE4M3 scale fields.

Workloads (shapes of the pages' DeepSeek-V4-Flash expert layer: 256 experts,
top-6, expert FC1 4096 x 7168 (gate||up) and FC2 7168 x 2048; and the dense
(M, N, K) shapes of the pages' accuracy table):
"""

import numpy as np

TAG_ACT, TAG_OUTLIER, TAG_LOGITS = 1, 2, 3
TAG_DENSE_W, TAG_DENSE_S = 4, 5
TAG_W1, TAG_S1, TAG_W2, TAG_S2 = 6, 7, 8, 9
TAG_NV_W, TAG_NV_S = 10, 11

WORKLOADS = {
    # dense MXFP4 GEMM, bf16 activations quantised inside the call to E4M3
    "dense_m16_n32_k4096": dict(kind="dense", M=16, N=32, K=4096, seed=0,
                                exp_lo=122, exp_hi=130, outliers=False, act_fmt="e4m3"),
    "dense_m64_n4096_k7168": dict(kind="dense", M=64, N=4096, K=7168, seed=1,
                                  exp_lo=122, exp_hi=130, outliers=True, act_fmt="e4m3"),
    # MoE expert layer: hidden 7168, intermediate 2048, 256 experts, top-6
    "moe_decode_t8": dict(kind="moe", T=8, H=7168, I=2048, E=256, k=6, seed=2,
                          exp_lo=120, exp_hi=128, routing="normal", act_fmt="e4m3"),
    "moe_prefill_t2048_zipf": dict(kind="moe", T=2048, H=7168, I=2048, E=256, k=6, seed=3,
                                   exp_lo=120, exp_hi=128, routing="zipf", act_fmt="e4m3"),
    "moe_prefill_t16384_fp4": dict(kind="moe", T=16384, H=7168, I=2048, E=256, k=6, seed=4,
                                   exp_lo=120, exp_hi=128, routing="uniform", act_fmt="e2m1"),
}


def rng(seed, tag, *idx):
    return np.random.default_rng([int(seed), int(tag)] + [int(i) for i in idx])


def bf16_bits_from_f32(x):
    """fp32 -> bfloat16 bit patterns, round-to-nearest-even (input synthesis)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def activations(seed, T, H, outliers=False):
    """bf16 N(0,1) activations [T][H]; with outliers, 1% of entries x20 (fp32)."""
    x = rng(seed, TAG_ACT).standard_normal((T, H), dtype=np.float32)
    if outliers:
        mask = rng(seed, TAG_OUTLIER).random((T, H)) < 0.01
        x = np.where(mask, x * np.float32(20.0), x).astype(np.float32)
    return bf16_bits_from_f32(x)


def logits(seed, T, E, routing="normal"):
    """fp32 routing logits [T][E]: N(0,1), plus a Zipf(s=1.1) expert bias
    -1.1 * ln(e + 1) for the skewed workload (expert 0 hottest)."""
    z = rng(seed, TAG_LOGITS).standard_normal((T, E), dtype=np.float32)
    if routing == "zipf":
        bias = np.float32(-1.1) * np.log(np.arange(1, E + 1, dtype=np.float32))
        z = (z + bias.astype(np.float32)[None, :]).astype(np.float32)
    elif routing not in ("normal", "uniform"):
        raise ValueError(routing)
    return z


def _random_bytes(g, shape):
    n = int(np.prod(shape))
    return np.frombuffer(bytearray(g.bytes(n)), dtype=np.uint8).reshape(shape)


def _scale_bytes(g, shape, lo, hi):
    return g.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def dense_weights(seed, N, K, exp_lo, exp_hi):
    """Packed E2M1 codes [N][K/2] (uniform over all 16 codes per nibble) and
    UE8M0 scale bytes [N][K/32] uniform in [exp_lo, exp_hi]."""
    w = _random_bytes(rng(seed, TAG_DENSE_W), (N, K // 2))
    s = _scale_bytes(rng(seed, TAG_DENSE_S), (N, K // 32), exp_lo, exp_hi)
    return w, s


def nvfp4_weights(seed, N, K, e_lo=4, e_hi=10):
    """NVFP4 weights: packed E2M1 codes [N][K/2] (uniform over all 16 codes per nibble)
    and one UE4M3 scale byte per 16 elements [N][K/16]: exponent field uniform in
    [e_lo, e_hi], mantissa field uniform in 0..7, sign bit clear."""
    w = _random_bytes(rng(seed, TAG_NV_W), (N, K // 2))
    g = rng(seed, TAG_NV_S)
    e = g.integers(e_lo, e_hi + 1, size=(N, K // 16), dtype=np.uint8)
    m = g.integers(0, 8, size=(N, K // 16), dtype=np.uint8)
    return w, ((e << 3) | m).astype(np.uint8)


def expert_weights(seed, e, H, I, exp_lo, exp_hi, out=None):
    """One expert's (w1 [2I][H/2], s1 [2I][H/32], w2 [H][I/2], s2 [H][I/32]).

    If ``out`` is a 4-tuple of writable uint8 arrays of those shapes the
    values are written there (lets callers fill pinned or stacked buffers)."""
    parts = (
        _random_bytes(rng(seed, TAG_W1, e), (2 * I, H // 2)),
        _scale_bytes(rng(seed, TAG_S1, e), (2 * I, H // 32), exp_lo, exp_hi),
        _random_bytes(rng(seed, TAG_W2, e), (H, I // 2)),
        _scale_bytes(rng(seed, TAG_S2, e), (H, I // 32), exp_lo, exp_hi),
    )
    if out is None:
        return parts
    for dst, src in zip(out, parts):
        dst[...] = src
    return out


def moe_weights(seed, E, H, I, exp_lo, exp_hi):
    """All experts stacked: w1 [E][2I][H/2], s1 [E][2I][H/32], w2 [E][H][I/2], s2 [E][H][I/32]."""
    w1 = np.empty((E, 2 * I, H // 2), np.uint8)
    s1 = np.empty((E, 2 * I, H // 32), np.uint8)
    w2 = np.empty((E, H, I // 2), np.uint8)
    s2 = np.empty((E, H, I // 32), np.uint8)
    for e in range(E):
        expert_weights(seed, e, H, I, exp_lo, exp_hi, out=(w1[e], s1[e], w2[e], s2[e]))
    return w1, s1, w2, s2


def workload_inputs(name, weights=True, **override):
    """Inputs of a named workload (optionally with shapes overridden, for
    scaled-down parity cases). Returns a dict of numpy arrays + parameters."""
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    out = dict(cfg=cfg)
    if cfg["kind"] == "dense":
        out["a"] = activations(cfg["seed"], cfg["M"], cfg["K"], cfg["outliers"])
        if weights:
            out["w"], out["w_scale"] = dense_weights(cfg["seed"], cfg["N"], cfg["K"],
                                                     cfg["exp_lo"], cfg["exp_hi"])
    else:
        out["x"] = activations(cfg["seed"], cfg["T"], cfg["H"], False)
        out["logits"] = logits(cfg["seed"], cfg["T"], cfg["E"], cfg["routing"])
        if weights:
            out["w1"], out["s1"], out["w2"], out["s2"] = moe_weights(
                cfg["seed"], cfg["E"], cfg["H"], cfg["I"], cfg["exp_lo"], cfg["exp_hi"])
    return out
