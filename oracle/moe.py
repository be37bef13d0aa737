"""fp64 MoE expert-layer oracle (TEST INFRASTRUCTURE ONLY - see package docstring).

What the layer computes, in the pages' order:

* route: each token picks the top-6 of 256 experts [TRITON-FP4, "FP4 MoE GEMM
  是什么？"; MTT-DSV4: routing / Top-k]. Readings: higher logit first, equal
  logits broken by the lower expert index; the slot order j = 0..5 is that
  order; the gates are the softmax over the 6 selected logits.
* permute (dispatch on one GPU) [MTT-DSV4: dispatch/combine]: the pairs
  p = t*k + j are grouped by expert; reading: expert-major, ascending p inside
  an expert (a stable sort), offsets not padded.
* FC1 (gate||up, 2I x H per expert, [TRITON-FP4] gives 4096 x 7168), then
  SwiGLU h = silu(gate) * up (reading: no clamp), then the fused requantisation
  of h to the layer's activation element format per 32 along I [MTT-DSV4:
  "SwiGLU + FP8 quant"], then FC2 (H x I per expert). Both FCs take
  MX-quantised activations times MXFP4 weights with no dequantisation to a
  16-bit type before the product [DS4-FP4 section 一/二]; here both operands are
  decoded exactly to fp64 and multiplied in fp64.
* combine: out[t] = sum_j gate[t, j] * y[row of pair (t, j)], in fp64 here
  (the oracle does not round to bf16).
"""

import numpy as np

from .mx import (
    FMT_E2M1,
    dequant_nvfp4_weights,
    e2m1_decode,
    FMT_E4M3,
    bf16_bits_to_f64,
    dequant_weights,
    mx_dequantize,
    mx_quantize,
    pack_e2m1,
    unpack_e2m1,
)


def decode_act(q, q_scale, fmt):
    """Boundary-layout activations (E4M3 bytes, or packed E2M1) -> fp64."""
    codes = unpack_e2m1(q) if fmt == FMT_E2M1 else np.asarray(q, dtype=np.uint8)
    return mx_dequantize(codes, q_scale, fmt)


def quantize_act(x, fmt):
    """fp64 rows -> (q in boundary layout, q_scale). E2M1 is packed two per byte."""
    codes, scales = mx_quantize(x, fmt)
    return (pack_e2m1(codes) if fmt == FMT_E2M1 else codes), scales


def dense_gemm(a_bf16, w, w_scale, act_fmt=FMT_E4M3):
    """C = A_hat @ W_hat^T in fp64 [DS4-FP4 section 二, dense MXFP4 entry].

    a_bf16: [M][K] bf16 bit patterns, quantised per 32-block to act_fmt first.
    w: [N][K/2] packed E2M1, w_scale: [N][K/32] UE8M0.
    Returns (C fp64 [M][N], q, q_scale) with q in the boundary layout.
    """
    a = bf16_bits_to_f64(a_bf16)
    q, qs = quantize_act(a, act_fmt)
    a_hat = decode_act(q, qs, act_fmt)
    w_hat = dequant_weights(w, w_scale)
    return a_hat @ w_hat.T, q, qs


def w4a16_gemm(a_bf16, w, w_scale, fmt="mxfp4"):
    """C = A @ W_hat^T in fp64 with the activations as given (bf16, not quantised) and
    FP4 weights dequantised exactly [TRITON-FP4, "第二步": the fused dequantise + matmul;
    DS4-FP4 section 一 for the NVFP4 block format]. fmt "mxfp4": w_scale [N][K/32]
    UE8M0; "nvfp4": w_scale [N][K/16] UE4M3."""
    a = bf16_bits_to_f64(a_bf16)
    w_hat = dequant_nvfp4_weights(w, w_scale) if fmt == "nvfp4" else dequant_weights(w, w_scale)
    return a @ w_hat.T


def q8_quantize(x_bf16):
    """Q8 activation blocks [DS4-FP4 sections 二/三: Q8_1-style activations on the
    generic path; FP8-GGUF section 四: a Q8_0 block is 32 int8 plus an fp16 scale].
    Readings (the pages give the block layout only): per 32-block d = fp16(amax / 127)
    with the quotient in fp32 and rounded to nearest even, q = x / d in fp32 rounded to
    nearest even and clamped to [-127, 127], q = 0 where d = 0. The integers are
    decided in fp32, as the kernel decides them. Returns (q int8 [rows][K],
    d float16 [rows][K/32])."""
    x = bf16_bits_to_f64(x_bf16).astype(np.float32)  # exact
    rows, K = x.shape
    blk = x.reshape(rows, K // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(over="ignore"):  # amax / 127 beyond fp16's range gives d = inf (then q = 0)
        d = (amax / np.float32(127.0)).astype(np.float16)
    d32 = d.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(d32 > 0, np.rint(blk / np.where(d32 > 0, d32, np.float32(1))), np.float32(0))
    q = np.clip(t, -127, 127).astype(np.int8)
    return q.reshape(rows, K), d


def lut_int8_weights(w):
    """The 16-entry table [DS4-FP4 section 二; FP8-GGUF section 五: FP4 codes map onto a
    4-bit lookup-table type]: code -> 2 * e2m1(code), an int8 in {0, +-1, .., +-12};
    returns int8 [N][K]."""
    return (2.0 * e2m1_decode(unpack_e2m1(w))).astype(np.int8)


def q8_gemm(q, d, w, w_scale):
    """The lookup-table route in fp64: C[m][n] = sum over blocks b of
    (sum_k q[m][k] w8[n][k]) * d[m][b] * 2^(e[n][b] - 128), w8 = lut_int8_weights(w)."""
    q = np.asarray(q, dtype=np.int64)
    M, K = q.shape
    w8 = lut_int8_weights(w).astype(np.int64)
    N = w8.shape[0]
    da = np.asarray(d, dtype=np.float16).astype(np.float64)
    dw = np.ldexp(1.0, np.asarray(w_scale, dtype=np.int64) - 128)
    out = np.zeros((M, N))
    for b in range(K // 32):
        ib = q[:, 32 * b:32 * b + 32] @ w8[:, 32 * b:32 * b + 32].T  # exact integers
        out += ib * da[:, b:b + 1] * dw[None, :, b]
    return out


def route_topk(logits, k):
    """Top-k experts per token and softmax gates over them (fp64 gates)."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -logits), axis=-1)  # primary key -logit, then index
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    gates = z / z.sum(axis=1, keepdims=True)
    return ids, gates


def permute(topk_ids, E):
    """Group pairs p = t*k + j by expert, stable in p.

    Returns (expert_offsets int32 [E+1], sorted_pair int32 [T*k],
             pair_row int32 [T*k]) with sorted_pair[pair_row[p]] == p.
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    sorted_pair = np.argsort(flat, kind="stable").astype(np.int32)
    pair_row = np.empty_like(sorted_pair)
    pair_row[sorted_pair] = np.arange(flat.size, dtype=np.int32)
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return offsets, sorted_pair, pair_row


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def swiglu(G, I):
    """h = silu(G[:, :I]) * G[:, I:2I], silu(x) = x * sigmoid(x)."""
    g = G[:, :I]
    return g * _sigmoid(g) * G[:, I:2 * I]


def fc1_swiglu_rows(a_hat_rows, w1, w1_scale, I):
    """FC1 on already-decoded activation rows, then SwiGLU. Returns (G, h_pre)."""
    G = a_hat_rows @ dequant_weights(w1, w1_scale).T
    return G, swiglu(G, I)


def fc2_rows(h, h_scale, act_fmt, w2, w2_scale):
    """FC2 on boundary-layout h rows (codes + scales) -> y fp64."""
    return decode_act(h, h_scale, act_fmt) @ dequant_weights(w2, w2_scale).T


def combine(y, gates, pair_row, T, k):
    """out[t] = sum_j gates[t, j] * y[pair_row[t*k + j]] in fp64."""
    y = np.asarray(y, dtype=np.float64)
    rows = np.asarray(pair_row, dtype=np.int64).reshape(T, k)
    g = np.asarray(gates, dtype=np.float64)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += g[:, j:j + 1] * y[rows[:, j]]
    return out


def fc1_abs_terms(a_hat_rows, w1, w1_scale):
    """S[r, n] = sum_k |a_hat[r, k]| * |W1_hat[n, k]|: the sum of the magnitudes of
    the products that FC1 adds up (not part of the layer's result; it scales the
    rounding error of any finite-precision summation of those products)."""
    return np.abs(a_hat_rows) @ np.abs(dequant_weights(w1, w1_scale)).T


def group_max_terms(a_hat_rows, w_hat, group=8):
    """B[r, n] = sum over the K / group groups of `group` consecutive k of
    (max over the group of |a_hat[r, k]|) * (max over the group of |w_hat[n, k]|).

    Not part of the layer's result. It bounds from above the sum over groups of the
    largest |a_k w_k| in each group, which scales the error of a summation that
    aligns every group's products to the group's largest one before adding them."""
    a = np.abs(np.asarray(a_hat_rows, dtype=np.float64))
    w = np.abs(np.asarray(w_hat, dtype=np.float64))
    K = a.shape[1]
    am = a.reshape(a.shape[0], K // group, group).max(axis=2)
    wm = w.reshape(w.shape[0], K // group, group).max(axis=2)
    return am @ wm.T


def moe_layer(x_bf16, logits, w1, s1, w2, s2, k, act_fmt, rows=None, workers=1, abs_terms=False):
    """The whole expert layer, expert by expert, in fp64.

    x_bf16 [T][H] bf16 bits; logits [T][E] fp32; w1 [E][2I][H/2], s1 [E][2I][H/32],
    w2 [E][H][I/2], s2 [E][H][I/32] (packed E2M1 + UE8M0).
    rows: optional iterable of permuted row indices to compute (a sample);
    None computes every row. Returns a dict of every intermediate; y / h / G
    entries are only filled for the computed rows, and 'out' only for tokens
    all of whose k rows were computed (others are NaN).
    workers: experts are independent; with workers > 1 they are computed on that
    many threads (the same per-expert arithmetic, only run concurrently).
    abs_terms: also return 'G_abs' = fc1_abs_terms and 'G_gmax' = group_max_terms
    (groups of 8 along H) of FC1 for the computed rows.
    """
    x_bf16 = np.asarray(x_bf16)
    T, H = x_bf16.shape
    E = w1.shape[0]
    I = w1.shape[1] // 2
    q, q_scale = quantize_act(bf16_bits_to_f64(x_bf16), act_fmt)
    topk_ids, gates = route_topk(logits, k)
    offsets, sorted_pair, pair_row = permute(topk_ids, E)
    R = T * k
    want = np.zeros(R, dtype=bool)
    if rows is None:
        want[:] = True
    else:
        want[np.asarray(list(rows), dtype=np.int64)] = True
    G = np.full((R, 2 * I), np.nan)
    h_pre = np.full((R, I), np.nan)
    h_codes = np.zeros((R, I // 2 if act_fmt == FMT_E2M1 else I), dtype=np.uint8)
    h_scale = np.zeros((R, I // 32), dtype=np.uint8)
    y = np.full((R, H), np.nan)
    G_abs = np.full((R, 2 * I), np.nan) if abs_terms else None
    G_gmax = np.full((R, 2 * I), np.nan) if abs_terms else None

    def one_expert(e):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        r = np.arange(lo, hi)
        r = r[want[lo:hi]]
        if r.size == 0:
            return
        tok = sorted_pair[r] // k
        a_hat = decode_act(q[tok], q_scale[tok], act_fmt)
        Ge, he = fc1_swiglu_rows(a_hat, w1[e], s1[e], I)
        hq, hs = quantize_act(he, act_fmt)
        G[r], h_pre[r], h_codes[r], h_scale[r] = Ge, he, hq, hs
        y[r] = fc2_rows(hq, hs, act_fmt, w2[e], s2[e])
        if abs_terms:
            G_abs[r] = fc1_abs_terms(a_hat, w1[e], s1[e])
            G_gmax[r] = group_max_terms(a_hat, dequant_weights(w1[e], s1[e]))

    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_expert, range(E)))
    else:
        for e in range(E):
            one_expert(e)
    out = np.full((T, H), np.nan)
    done = want[pair_row.reshape(T, k)].all(axis=1)
    if done.any():
        tk = np.nonzero(done)[0]
        rws = pair_row.reshape(T, k)[tk]
        acc = np.zeros((tk.size, H))
        for j in range(k):
            acc += gates[tk, j:j + 1] * y[rws[:, j]]
        out[tk] = acc
    return dict(q=q, q_scale=q_scale, topk_ids=topk_ids, gates=gates,
                expert_offsets=offsets, sorted_pair=sorted_pair, pair_row=pair_row,
                G=G, G_abs=G_abs, G_gmax=G_gmax, h_pre=h_pre, h=h_codes, h_scale=h_scale, y=y, out=out,
                computed_rows=want, computed_tokens=done)


def row_normalised_error(got, ref):
    """max over rows of max_n |got - ref| / ||ref_row||_2 (rows with zero norm use 1)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    norm = np.linalg.norm(ref, axis=-1)
    norm = np.where(norm > 0, norm, 1.0)
    return float(np.max(np.max(np.abs(got - ref), axis=-1) / norm)) if ref.size else 0.0
