"""GPU parity of the MoE expert path: grouped FC1 (+ fused SwiGLU/requantise),
FC2, combine, stage by stage and end to end, against the fp64 oracle.

* h (requantised SwiGLU output): every code must be a correct rounding of a value
  within the per-element error bound of the oracle's exact h (tests/helpers.py:
  the bound follows from the measured FC1 accumulation residual);
* y (FC2): stage-isolated - the oracle's FC2 is fed the GPU's own h;
* out (combine): stage-isolated on the GPU's y, and end to end against the
  fully independent oracle chain; both within 2e-3 row-normalised.
"""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import GEMM_TOL, bf16_dev, h_error_bound, host, straddle_check_bound, unpack_codes

pytestmark = pytest.mark.gpu


def _dev_weights(w1, s1, w2, s2):
    return [torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in (w1, s1, w2, s2)]


def _layer(x, logits, w, k, fmt, y_dtype=torch.bfloat16):
    r = ops.moe_layer(bf16_dev(x), torch.from_numpy(logits).cuda(), *w, topk=k, act_fmt=fmt, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return {name: host(t) for name, t in r.items()}


def _compare(g, ref, x, logits, w1, s1, w2, s2, k, fmt, rows=None, tokens=None):
    T = x.shape[0]
    for key in ("q", "q_scale", "topk_ids", "expert_offsets", "sorted_pair", "pair_row"):
        assert np.array_equal(g[key], ref[key]), key
    rows = np.arange(T * k) if rows is None else np.asarray(rows)
    # h: the GPU's codes against the oracle's exact values within the error bound
    I = ref["h_pre"].shape[1]
    dh = h_error_bound(ref["G"][rows], ref["G_abs"][rows], I, fmt, ref["G_gmax"][rows])
    straddle_check_bound(unpack_codes(g["h"][rows], fmt), g["h_scale"][rows], ref["h_pre"][rows], dh, fmt)
    # y: stage-isolated (oracle FC2 on the GPU's own h)
    e_of_row = np.searchsorted(ref["expert_offsets"], rows, side="right") - 1
    y_ref = np.zeros((rows.size, g["y"].shape[1]))
    for e in np.unique(e_of_row):
        sel = e_of_row == e
        y_ref[sel] = oracle.fc2_rows(g["h"][rows[sel]], g["h_scale"][rows[sel]], fmt, w2[e], s2[e])
    err_y = oracle.row_normalised_error(g["y"][rows], y_ref)
    assert err_y <= GEMM_TOL, f"y error {err_y}"
    # out: stage-isolated combine and end to end
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    gates = g["gates"].astype(np.float64)
    y_full = np.zeros((T * k, g["y"].shape[1]))
    y_full[rows] = g["y"][rows]
    comb = oracle.combine(y_full, gates, g["pair_row"], T, k)
    err_c = oracle.row_normalised_error(g["out"][tok], comb[tok])
    assert err_c <= GEMM_TOL, f"combine error {err_c}"
    err_e = oracle.row_normalised_error(g["out"][tok], ref["out"][tok])
    assert err_e <= GEMM_TOL, f"end-to-end error {err_e}"
    return err_y, err_c, err_e


@pytest.mark.parametrize("T,H,I,E,k,fmt,seed", [
    (8, 1024, 512, 16, 6, "e4m3", 0),      # decode-shaped: weight-streaming kernel
    (40, 1536, 1024, 8, 3, "e2m1", 1),     # 40 tokens: streaming kernel, several rows per expert
    (300, 1024, 512, 8, 6, "e4m3", 2),     # LDS-ring kernels, several 256-row units, ragged tails
    (333, 1024, 1024, 32, 4, "e2m1", 3),   # FP4 x FP4 tiles, some experts empty
    (65, 512, 512, 4, 2, "e4m3", 4),       # just past the streaming threshold
    (700, 2048, 512, 4, 2, "e2m1", 5),     # FP4 x FP4, ~350 rows per expert: full and partial 256-row units
    (300, 1024, 2048, 8, 2, "e2m1", 6),    # FP4 FC2 with K = 2048: four n-tiles per workgroup
    (12, 1024, 2048, 16, 6, "e2m1", 7),    # FP4 decode: one-fragment kernels, FC2 two row blocks per workgroup
])
def test_layer_small_shapes_full_oracle(T, H, I, E, k, fmt, seed):
    x = dg.activations(seed, T, H)
    logits = dg.logits(seed, T, E, "normal")
    w1, s1, w2, s2 = dg.moe_weights(seed, E, H, I, 120, 128)
    g = _layer(x, logits, _dev_weights(w1, s1, w2, s2), k, fmt)
    ref = oracle.moe_layer(x, logits, w1, s1, w2, s2, k, fmt, abs_terms=True)
    _compare(g, ref, x, logits, w1, s1, w2, s2, k, fmt)


def test_layer_skewed_routing_one_expert_takes_all():
    T, H, I, E, k = 200, 512, 512, 8, 2
    x = dg.activations(11, T, H)
    logits = dg.logits(11, T, E, "normal")
    logits[:, 5] += 50.0  # every token's first choice is expert 5 (two full tiles + a tail)
    w1, s1, w2, s2 = dg.moe_weights(11, E, H, I, 120, 128)
    g = _layer(x, logits, _dev_weights(w1, s1, w2, s2), k, "e4m3")
    ref = oracle.moe_layer(x, logits, w1, s1, w2, s2, k, "e4m3", abs_terms=True)
    _compare(g, ref, x, logits, w1, s1, w2, s2, k, "e4m3")


@pytest.mark.parametrize("fmt,y_dtype", [("e4m3", torch.bfloat16), ("e2m1", torch.bfloat16),
                                         ("e4m3", torch.float32)])
def test_layer_split_small_experts_stream(fmt, y_dtype):
    """Past 64 tokens with fewer than 64 rows per expert, experts of at most 16 rows
    run in the streaming kernel and the others in the tiled kernels: expert loads of
    16 | 17 | 1 | 0 | 2 x 128 + 5 | 40 | 16 | 15 rows straddle both boundaries."""
    counts = [16, 17, 1, 0, 261, 40, 16, 15]
    T, H, I, E, k = sum(counts), 1024, 512, len(counts), 1
    x = dg.activations(15, T, H)
    logits = dg.logits(15, T, E, "normal")
    owner = np.repeat(np.arange(E), counts)
    np.random.default_rng(15).shuffle(owner)
    logits[np.arange(T), owner] += 50.0
    w1, s1, w2, s2 = dg.moe_weights(15, E, H, I, 120, 128)
    g = _layer(x, logits, _dev_weights(w1, s1, w2, s2), k, fmt, y_dtype=y_dtype)
    assert np.array_equal(np.diff(g["expert_offsets"]), counts)
    ref = oracle.moe_layer(x, logits, w1, s1, w2, s2, k, fmt, abs_terms=True)
    _compare(g, ref, x, logits, w1, s1, w2, s2, k, fmt)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_layer_split_zipf_routing(fmt):
    # skewed routing over 64 experts: a few hot experts in tiles, a long tail streamed
    T, H, I, E, k = 240, 1024, 1024, 64, 2
    x = dg.activations(16, T, H)
    logits = dg.logits(16, T, E, "zipf")
    w1, s1, w2, s2 = dg.moe_weights(16, E, H, I, 120, 128)
    g = _layer(x, logits, _dev_weights(w1, s1, w2, s2), k, fmt)
    c = np.diff(g["expert_offsets"])
    assert (c > 16).any() and ((c > 0) & (c <= 16)).any()
    ref = oracle.moe_layer(x, logits, w1, s1, w2, s2, k, fmt, abs_terms=True)
    _compare(g, ref, x, logits, w1, s1, w2, s2, k, fmt)


@pytest.mark.parametrize("T", [24, 10])  # two 16-row fragments / one (FC2 with two row blocks)
def test_layer_fp32_y(T):
    H, I, E, k = 512, 512, 8, 3
    x = dg.activations(12, T, H)
    logits = dg.logits(12, T, E, "normal")
    w1, s1, w2, s2 = dg.moe_weights(12, E, H, I, 120, 128)
    g = _layer(x, logits, _dev_weights(w1, s1, w2, s2), k, "e4m3", y_dtype=torch.float32)
    ref = oracle.moe_layer(x, logits, w1, s1, w2, s2, k, "e4m3", abs_terms=True)
    _compare(g, ref, x, logits, w1, s1, w2, s2, k, "e4m3")


def test_layer_fp32_y_fp8_tiles():
    # FP8 activations past 64 tokens: the 256 x 256 FP8 ring, FC2 with fp32 y and K = I = 2048
    T, H, I, E, k = 200, 1024, 2048, 8, 3
    x = dg.activations(14, T, H)
    logits = dg.logits(14, T, E, "normal")
    w1, s1, w2, s2 = dg.moe_weights(14, E, H, I, 120, 128)
    g = _layer(x, logits, _dev_weights(w1, s1, w2, s2), k, "e4m3", y_dtype=torch.float32)
    ref = oracle.moe_layer(x, logits, w1, s1, w2, s2, k, "e4m3", abs_terms=True)
    _compare(g, ref, x, logits, w1, s1, w2, s2, k, "e4m3")


@pytest.mark.parametrize("I", [512, 2048])  # FC2 stage loop / four chained n-tiles (K = 2048)
def test_layer_fp32_y_fp4_tiles(I):
    T, H, E, k = 300, 1024, 8, 4
    x = dg.activations(13, T, H)
    logits = dg.logits(13, T, E, "normal")
    w1, s1, w2, s2 = dg.moe_weights(13, E, H, I, 120, 128)
    g = _layer(x, logits, _dev_weights(w1, s1, w2, s2), k, "e2m1", y_dtype=torch.float32)
    ref = oracle.moe_layer(x, logits, w1, s1, w2, s2, k, "e2m1", abs_terms=True)
    _compare(g, ref, x, logits, w1, s1, w2, s2, k, "e2m1")


def test_decode_workload_every_row():
    """The full-size 8-token decode layer; the oracle computes every row."""
    d = dg.workload_inputs("moe_decode_t8")
    cfg = d["cfg"]
    k, fmt = cfg["k"], cfg["act_fmt"]
    w = (d["w1"], d["s1"], d["w2"], d["s2"])
    g = _layer(d["x"], d["logits"], _dev_weights(*w), k, fmt)
    ref = oracle.moe_layer(d["x"], d["logits"], *w, k, fmt, workers=8, abs_terms=True)
    _compare(g, ref, d["x"], d["logits"], *w, k, fmt)


def test_layer_is_deterministic():
    T, H, I, E, k = 300, 1024, 512, 8, 6
    x = bf16_dev(dg.activations(21, T, H))
    logits = torch.from_numpy(dg.logits(21, T, E, "normal")).cuda()
    w = _dev_weights(*dg.moe_weights(21, E, H, I, 120, 128))
    a = ops.moe_layer(x, logits, *w, topk=k, act_fmt="e4m3")
    b = ops.moe_layer(x, logits, *w, topk=k, act_fmt="e4m3")
    for key in a:
        assert torch.equal(a[key], b[key]), key
