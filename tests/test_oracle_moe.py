"""Pins for the oracle's routing, permutation, SwiGLU, combine and the whole
expert chain (CPU only).

The layer follows "【DeepSeek V4】Triton FP4 优化实战" ("FP4 MoE GEMM 是什么？":
256 experts, 6 active per token, 2 FC per expert) and "Domestic GPUs are
awesome! Moore thread full-link adaptation DeepSeek-V4" (routing / Top-k,
"SwiGLU + FP8 quant", dispatch/combine).
"""

import math

import numpy as np
import pytest
import scipy.special

import oracle
from mxfp4_block_scaled_amd import datagen as dg


def _brute_topk(logits, k):
    """Rank of an expert = number of experts that beat it (higher logit, or an
    equal logit with a lower index). The chosen ones have rank < k, slot = rank."""
    T, E = logits.shape
    ids = np.full((T, k), -1)
    for t in range(T):
        for e in range(E):
            rank = sum(1 for f in range(E)
                       if logits[t, f] > logits[t, e] or (logits[t, f] == logits[t, e] and f < e))
            if rank < k:
                ids[t, rank] = e
    return ids


@pytest.mark.parametrize("T,E,k", [(5, 8, 3), (7, 16, 6), (3, 6, 6)])
def test_route_vs_brute_force_with_ties(T, E, k):
    g = np.random.default_rng(T * 100 + E)
    logits = g.integers(-3, 3, (T, E)).astype(np.float32)  # many exact ties
    ids, gates = oracle.route_topk(logits, k)
    assert np.array_equal(ids, _brute_topk(logits, k))
    for t in range(T):
        l0 = float(logits[t, ids[t, 0]])
        z = [math.exp(float(logits[t, e]) - l0) for e in ids[t]]
        assert np.allclose(gates[t], np.array(z) / sum(z), rtol=1e-15, atol=0)


def test_route_real_shapes_invariants():
    L = dg.logits(2, 64, 256, "normal")
    ids, gates = oracle.route_topk(L, 6)
    assert ids.shape == (64, 6)
    for t in range(64):
        assert len(set(ids[t].tolist())) == 6
        vals = L[t, ids[t]]
        assert np.all(np.diff(vals) <= 0)
        assert vals[-1] >= np.sort(L[t])[-6]
    assert np.allclose(gates.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(gates, axis=1) <= 0)


def test_equal_logits_give_equal_gates_and_lowest_indices():
    L = np.zeros((2, 256), np.float32)
    ids, gates = oracle.route_topk(L, 6)
    assert ids.tolist() == [[0, 1, 2, 3, 4, 5]] * 2
    assert np.allclose(gates, 1 / 6, rtol=0, atol=1e-16)


@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (9, 8, 3), (50, 256, 6)])
def test_permute_vs_brute_force(T, E, k):
    g = np.random.default_rng(T + E)
    L = g.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route_topk(L, k)
    off, sp, pr = oracle.permute(ids, E)
    flat = ids.reshape(-1)
    counts = [int((flat == e).sum()) for e in range(E)]
    assert off.tolist() == [0] + list(np.cumsum(counts))
    for p in range(T * k):
        e = flat[p]
        pos = off[e] + sum(1 for q in range(p) if flat[q] == e)
        assert pr[p] == pos and sp[pos] == p
    assert sorted(sp.tolist()) == list(range(T * k))


def test_swiglu_closed_forms():
    g = np.random.default_rng(5)
    G = g.standard_normal((4, 64)) * 8
    h = oracle.swiglu(G, 32)
    ref = G[:, :32] * scipy.special.expit(G[:, :32]) * G[:, 32:]
    assert np.allclose(h, ref, rtol=1e-14, atol=1e-300)
    Z = np.zeros((1, 4))
    Z[0, 2:] = 5.0
    assert np.all(oracle.swiglu(Z, 2) == 0.0)  # silu(0) = 0
    big = np.array([[800.0, -800.0, 2.0, 3.0]])
    assert np.allclose(oracle.swiglu(big, 2), [[1600.0, -0.0]])


def test_combine_one_hot_gates_is_a_copy_and_linear():
    T, k, H = 4, 3, 16
    g = np.random.default_rng(9)
    y = g.standard_normal((T * k, H))
    pr = g.permutation(T * k).astype(np.int32)
    gates = np.zeros((T, k))
    gates[np.arange(T), np.arange(T) % k] = 1.0
    out = oracle.combine(y, gates, pr, T, k)
    for t in range(T):
        assert np.array_equal(out[t], y[pr[t * k + t % k]])
    gates2 = g.random((T, k))
    out2 = oracle.combine(y, gates2, pr, T, k)
    for t in range(T):
        ref = sum(gates2[t, j] * y[pr[t * k + j]] for j in range(k))
        assert np.allclose(out2[t], ref, rtol=1e-15, atol=1e-15)


def _tiny_layer_inputs(T=6, H=128, I=64, E=8, seed=0):
    x = dg.activations(seed, T, H)
    L = dg.logits(seed, T, E)
    w1, s1, w2, s2 = dg.moe_weights(seed, E, H, I, 124, 130)
    return x, L, w1, s1, w2, s2


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_layer_closed_form_all_ones_weights(fmt):
    # With every weight +1 and unit scales: G[r, :] = S_t (the row sum of the
    # token's quantised activations), h = silu(S_t) * S_t in every column,
    # y[r, :] = I * Q(h) and out[t] = sum_j gate_j * I * Q(h) = I * Q(h).
    T, H, I, E, k = 5, 128, 64, 8, 3
    x, L, w1, s1, w2, s2 = _tiny_layer_inputs(T, H, I, E)
    w1[:] = 0x22
    s1[:] = 127
    w2[:] = 0x22
    s2[:] = 127
    r = oracle.moe_layer(x, L, w1, s1, w2, s2, k, fmt)
    q_hat = oracle.moe.decode_act(r["q"], r["q_scale"], fmt)
    S = q_hat.sum(1)
    hval = S * scipy.special.expit(S) * S
    half_ulp = 2.0 ** -4 if fmt == "e4m3" else 2.0 ** -2
    for t in range(T):
        assert np.all(r["out"][t] == r["out"][t, 0])
        assert abs(r["out"][t, 0] - I * hval[t]) <= I * abs(hval[t]) * half_ulp * (1 + 1e-9)
        for j in range(k):
            row = r["pair_row"][t * k + j]
            assert np.allclose(r["G"][row], S[t], rtol=1e-12)


def test_layer_fc1_gathers_the_right_token():
    # FC1 weight row n = one-hot at column n (n < H) -> G[r, n] = q_hat[t(r), n]
    T, H, I, E, k = 7, 128, 64, 4, 2
    x, L, w1, s1, w2, s2 = _tiny_layer_inputs(T, H, I, E, seed=3)
    codes = np.zeros((E, 2 * I, H), np.uint8)
    for n in range(2 * I):
        codes[:, n, n] = 2
    w1 = oracle.pack_e2m1(codes)
    s1[:] = 127
    r = oracle.moe_layer(x, L, w1, s1, w2, s2, k, "e4m3")
    q_hat = oracle.moe.decode_act(r["q"], r["q_scale"], "e4m3")
    for row in range(T * k):
        t = r["sorted_pair"][row] // k
        assert np.array_equal(r["G"][row], q_hat[t, :2 * I])
        e = r["topk_ids"].reshape(-1)[r["sorted_pair"][row]]
        assert r["expert_offsets"][e] <= row < r["expert_offsets"][e + 1]


def test_layer_sampled_rows_match_full():
    x, L, w1, s1, w2, s2 = _tiny_layer_inputs(T=8, H=128, I=64, E=8, seed=4)
    full = oracle.moe_layer(x, L, w1, s1, w2, s2, 3, "e4m3")
    tok = [1, 6]
    rows = [full["pair_row"][t * 3 + j] for t in tok for j in range(3)]
    part = oracle.moe_layer(x, L, w1, s1, w2, s2, 3, "e4m3", rows=rows)
    assert np.array_equal(part["out"][tok], full["out"][tok])
    assert np.array_equal(part["y"][rows], full["y"][rows])
    assert np.isnan(part["out"][0]).all()


def test_row_normalised_error():
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    got = np.array([[3.0, 4.5], [0.0, 0.1]])
    assert oracle.row_normalised_error(got, ref) == pytest.approx(0.1)
    assert oracle.row_normalised_error(got[:1], ref[:1]) == pytest.approx(0.1)


def test_threaded_layer_equals_serial_and_abs_terms_brute_force():
    """workers > 1 runs the same per-expert arithmetic on threads: bit-identical
    results. G_abs = sum_k |a_k w_k| against a plain loop over k, and the triangle
    inequality |G| <= G_abs with equality when every product is non-negative."""
    T, H, I, E, k = 6, 64, 32, 4, 2
    x = dg.activations(3, T, H)
    L = dg.logits(3, T, E, "normal")
    w1, s1, w2, s2 = dg.moe_weights(3, E, H, I, 124, 130)
    a = oracle.moe_layer(x, L, w1, s1, w2, s2, k, "e4m3", abs_terms=True)
    b = oracle.moe_layer(x, L, w1, s1, w2, s2, k, "e4m3", workers=3, abs_terms=True)
    for key in ("G", "G_abs", "h_pre", "h", "h_scale", "y", "out"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key
    q_hat = oracle.moe.decode_act(a["q"], a["q_scale"], "e4m3")
    for r in range(T * k):
        t = int(a["sorted_pair"][r]) // k
        e = int(np.searchsorted(a["expert_offsets"], r, side="right") - 1)
        W = oracle.dequant_weights(w1[e], s1[e])
        for n in (0, 5, 2 * I - 1):
            s = 0.0
            for kk in range(H):
                s += abs(q_hat[t, kk] * W[n, kk])
            assert math.isclose(a["G_abs"][r, n], s, rel_tol=1e-12)
    assert np.all(np.abs(a["G"]) <= a["G_abs"] * (1 + 1e-12))
    pos = oracle.fc1_abs_terms(np.abs(q_hat[:2]), np.full((3, H // 2), 0x22, np.uint8),
                               np.full((3, H // 32), 127, np.uint8))
    assert np.allclose(pos, np.abs(q_hat[:2]).sum(1)[:, None], rtol=1e-15)


def test_group_max_terms_against_loops():
    """group_max_terms against plain loops over rows, columns and groups, and the
    property it exists for: it bounds the sum over groups of the largest |a_k w_k|."""
    rng = np.random.default_rng(31)
    a = rng.standard_normal((3, 48)) * np.exp2(rng.integers(-8, 8, (3, 48)))
    w = rng.standard_normal((5, 48))
    B = oracle.group_max_terms(a, w)
    for r in range(3):
        for n in range(5):
            want = sum(max(abs(a[r, k]) for k in range(g, g + 8)) * max(abs(w[n, k]) for k in range(g, g + 8))
                       for g in range(0, 48, 8))
            assert math.isclose(B[r, n], want, rel_tol=1e-12)
            top = sum(max(abs(a[r, k] * w[n, k]) for k in range(g, g + 8)) for g in range(0, 48, 8))
            assert top <= B[r, n] * (1 + 1e-12)
    assert np.array_equal(oracle.group_max_terms(a, w, group=48), np.abs(a).max(1)[:, None] * np.abs(w).max(1)[None])
