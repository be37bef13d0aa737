"""GPU parity of moe_grouped_mxfp4_gemm_combine: FC2 fused with the gate-weighted
combine for batches of at most 64 tokens.

* h: as for the unfused path, every code a correct rounding of a value within the
  per-element error bound of the oracle's exact h;
* out, stage-isolated: against the exact (fp64) combine of the exact FC2 of the
  GPU's own h, with the GPU's own gates, element by element within
      sum_j |g_j| * dy_j  +  k * 2^-24 * sum_j |g_j y_j|  (+ bf16 rounding),
  dy_j the matrix instructions' error bound for y_j (fp32 accumulation plus the
  in-group alignment loss of E4M3 x E2M1 sums, tests/helpers.py), then one
  rounding per fused multiply-add of the slot-order chain;
* out, end to end: within 2e-3 row-normalised of the fully independent oracle;
* against the unfused path with fp32 y (same products, other summation order).
Shapes cover empty experts, several 16-row fragments per expert (up to 64 rows),
more than 256 experts, the largest T * topk (512), K = I of 1 and 3 super-steps
(partly idle load chunks) and both activation formats and output types."""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import (GEMM_TOL, bf16_dev, gemm_error_bound, h_error_bound, host, straddle_check_bound,
                           unpack_codes)

pytestmark = pytest.mark.gpu


def _dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in arrs]


def _fused(x, logits, w, k, fmt, out_dtype):
    r = ops.moe_layer(bf16_dev(x), torch.from_numpy(logits).cuda(), *w, topk=k, act_fmt=fmt, out_dtype=out_dtype,
                      fused=True)
    torch.cuda.synchronize()
    return {n: host(t) for n, t in r.items() if t is not None}


def _check_out_stage(g, w2, s2, k, fmt, bf16_out, tokens=None):
    """out against the exact combine of the exact FC2 of the GPU's own h and gates."""
    T = g["gates"].shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    pr = g["pair_row"].reshape(T, k)
    offs = g["expert_offsets"]
    gates = g["gates"].astype(np.float64)
    H = g["out"].shape[1]
    rows = np.unique(pr[tok].ravel())
    e_of_row = np.searchsorted(offs, rows, side="right") - 1
    y = np.zeros((T * k, H))
    dy = np.zeros((T * k, H))
    for e in np.unique(e_of_row):
        r = rows[e_of_row == e]
        a = oracle.mx_dequantize(unpack_codes(g["h"][r], fmt), g["h_scale"][r], fmt)
        wd = oracle.dequant_weights(w2[e], s2[e])
        y[r] = a @ wd.T
        dy[r] = gemm_error_bound(np.abs(a) @ np.abs(wd).T, oracle.group_max_terms(a, wd), fmt)
    exact = np.zeros((tok.size, H))
    bound = np.zeros((tok.size, H))
    for j in range(k):
        r = pr[tok, j]
        gj = gates[tok, j:j + 1]
        exact += gj * y[r]
        bound += np.abs(gj) * (dy[r] + k * 2.0 ** -24 * np.abs(y[r]))
    got = g["out"][tok]
    if bf16_out:
        # round to nearest into 8 significant bits: |x - bf16(x)| <= 2^-8 |x| <= 2^-8 / (1 - 2^-8) |bf16(x)|
        bound += 2.0 ** -8 / (1 - 2.0 ** -8) * np.abs(got)
    excess = np.abs(got - exact) - bound
    assert (excess <= 0).all(), f"out outside its bound by up to {excess.max():.3e}"
    return exact


@pytest.mark.parametrize("T,H,I,E,k,fmt,out_dtype,seed", [
    (8, 1024, 512, 16, 6, "e2m1", torch.bfloat16, 0),    # one super-step: three idle chunk slots (FP4 loads 4)
    (8, 1024, 512, 16, 6, "e4m3", torch.float32, 1),     # FP8 activations, loads 2 super-steps at a time
    (40, 1536, 1536, 8, 3, "e2m1", torch.bfloat16, 2),   # 3 super-steps, experts of 15 +- rows: 1-2 fragments
    (64, 512, 1024, 4, 2, "e4m3", torch.bfloat16, 3),    # 64 tokens, ~32 rows per expert
    (64, 512, 512, 2, 2, "e2m1", torch.float32, 4),      # every token in both experts: 4 full fragments each
    (12, 1024, 2048, 300, 8, "e2m1", torch.bfloat16, 5),  # more than 256 experts, topk 8
    (64, 512, 512, 1024, 8, "e4m3", torch.float32, 6),   # E = 1024, T * topk = 512 (the LDS table's size)
    (1, 512, 512, 8, 1, "e2m1", torch.bfloat16, 7),      # one token, one slot
])
def test_fused_small_shapes(T, H, I, E, k, fmt, out_dtype, seed):
    x = dg.activations(100 + seed, T, H)
    logits = dg.logits(100 + seed, T, E, "normal")
    w1, s1, w2, s2 = dg.moe_weights(100 + seed, E, H, I, 120, 128)
    wd = _dev(w1, s1, w2, s2)
    g = _fused(x, logits, wd, k, fmt, out_dtype)
    ref = oracle.moe_layer(x, logits, w1, s1, w2, s2, k, fmt, abs_terms=True)
    for key in ("q", "q_scale", "topk_ids", "expert_offsets", "sorted_pair", "pair_row"):
        assert np.array_equal(g[key], ref[key]), key
    dh = h_error_bound(ref["G"], ref["G_abs"], I, fmt, ref["G_gmax"])
    straddle_check_bound(unpack_codes(g["h"], fmt), g["h_scale"], ref["h_pre"], dh, fmt)
    _check_out_stage(g, w2, s2, k, fmt, out_dtype == torch.bfloat16)
    err = oracle.row_normalised_error(g["out"], ref["out"])
    assert err <= GEMM_TOL, err
    # the unfused path with fp32 y: the same products, summed in another order
    u = ops.moe_layer(bf16_dev(x), torch.from_numpy(logits).cuda(), *wd, topk=k, act_fmt=fmt,
                      y_dtype=torch.float32, out_dtype=out_dtype)
    diff = oracle.row_normalised_error(g["out"], host(u["out"]))
    # fp32 out: a few fp32 roundings apart; bf16 out: at most one bf16 ulp (2^-7 of the element) apart
    assert diff <= (1e-5 if out_dtype == torch.float32 else 2.0 ** -7 + 1e-5), diff


def test_fused_decode_workload_every_token():
    """The full-size 8-token decode layer (H 7168, I 2048, 256 experts, top-6, E4M3
    activations) in the launch configuration the benchmark times; every token."""
    d = dg.workload_inputs("moe_decode_t8")
    cfg = d["cfg"]
    k, fmt = cfg["k"], cfg["act_fmt"]
    w = (d["w1"], d["s1"], d["w2"], d["s2"])
    g = _fused(d["x"], d["logits"], _dev(*w), k, fmt, torch.bfloat16)
    ref = oracle.moe_layer(d["x"], d["logits"], *w, k, fmt, workers=8, abs_terms=True)
    I = cfg["I"]
    dh = h_error_bound(ref["G"], ref["G_abs"], I, fmt, ref["G_gmax"])
    straddle_check_bound(unpack_codes(g["h"], fmt), g["h_scale"], ref["h_pre"], dh, fmt)
    _check_out_stage(g, d["w2"], d["s2"], k, fmt, True)
    err = oracle.row_normalised_error(g["out"], ref["out"])
    print(f"\n[fused fc2+combine] decode t8 end-to-end row-normalised error {err:.2e}")
    assert err <= GEMM_TOL, err


def test_fused_is_deterministic_and_rejects_prefill():
    T, H, I, E, k = 48, 1024, 1024, 32, 6
    x = bf16_dev(dg.activations(120, T, H))
    logits = torch.from_numpy(dg.logits(120, T, E, "normal")).cuda()
    w = _dev(*dg.moe_weights(120, E, H, I, 120, 128))
    a = ops.moe_layer(x, logits, *w, topk=k, act_fmt="e2m1", fused=True)
    b = ops.moe_layer(x, logits, *w, topk=k, act_fmt="e2m1", fused=True)
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["h"], b["h"])
    x65 = bf16_dev(dg.activations(121, 65, H))
    l65 = torch.from_numpy(dg.logits(121, 65, E, "normal")).cuda()
    with pytest.raises(RuntimeError, match="UNSUPPORTED|unsupported"):
        ops.moe_layer(x65, l65, *w, topk=k, act_fmt="e2m1", fused=True)
