"""The seeded input generator: determinism and stream independence (CPU only)."""

import numpy as np
import torch

from mxfp4_block_scaled_amd import datagen as dg


def test_same_seed_same_bytes():
    a = dg.workload_inputs("moe_decode_t8", weights=False)
    b = dg.workload_inputs("moe_decode_t8", weights=False)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["logits"], b["logits"])
    w1, s1, w2, s2 = dg.expert_weights(2, 17, 256, 64, 120, 128)
    v1, t1, v2, t2 = dg.expert_weights(2, 17, 256, 64, 120, 128)
    assert all(np.array_equal(p, q) for p, q in [(w1, v1), (s1, t1), (w2, v2), (s2, t2)])


def test_expert_streams_do_not_depend_on_which_experts_are_drawn():
    stacked = dg.moe_weights(9, 4, 256, 64, 120, 128)
    alone = dg.expert_weights(9, 2, 256, 64, 120, 128)
    for s, a in zip(stacked, alone):
        assert np.array_equal(s[2], a)
    assert not np.array_equal(stacked[0][1], stacked[0][2])


def test_value_ranges():
    w, s = dg.dense_weights(0, 64, 4096, 122, 130)
    assert s.min() >= 122 and s.max() <= 130
    nib = np.concatenate([w & 15, w >> 4]).ravel()
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * nib.size / 16  # all 16 codes, roughly uniform
    a = dg.activations(1, 64, 7168, outliers=True)
    f = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert 0.005 < np.mean(np.abs(f) > 6) < 0.02  # ~1% outliers (x20)


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 1e3
    x[:4] = [1.00390625, 1.01171875, -2.0 ** -130, 3.0e38]  # ties and extremes
    ours = dg.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_zipf_bias_skews_expert_zero():
    L = dg.logits(3, 2048, 256, "zipf")
    top1 = np.argmax(L, axis=1)
    assert np.mean(top1 == 0) > 0.3
