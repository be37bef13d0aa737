"""GPU parity: moe_route_permute - integer outputs bit-exact, gates within 1e-6."""

import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_amd import datagen as dg
from mxfp4_block_scaled_amd import ops
from tests.helpers import host

pytestmark = pytest.mark.gpu


def _check(logits, k):
    T, E = logits.shape
    ids, gates, offs, sp, pr = ops.moe_route_permute(torch.from_numpy(logits).cuda(), k)
    ref_ids, ref_g = oracle.route_topk(logits, k)
    ref_off, ref_sp, ref_pr = oracle.permute(ref_ids, E)
    assert np.array_equal(host(ids), ref_ids)
    assert np.array_equal(host(offs), ref_off)
    assert np.array_equal(host(sp), ref_sp)
    assert np.array_equal(host(pr), ref_pr)
    if T:
        # 1e-6 relative; below fp32's normal range (gates of e^-100) only fp32's own
        # subnormal spacing 2^-149 is attainable, so allow a few of those
        err = np.abs(host(gates).astype(np.float64) - ref_g)
        assert np.all(err <= 1e-6 * ref_g + 4 * 2.0 ** -149)


@pytest.mark.parametrize("name", ["moe_decode_t8", "moe_prefill_t2048_zipf", "moe_prefill_t16384_fp4"])
def test_route_workloads(name):
    d = dg.workload_inputs(name, weights=False)
    _check(d["logits"], d["cfg"]["k"])


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 255, 256, 257, 300, 1000, 4097])
def test_route_sizes_across_the_small_and_multi_block_paths(T):
    _check(dg.logits(100 + T, T, 256, "normal"), 6)


@pytest.mark.parametrize("T,E,k", [(50, 8, 3), (700, 16, 8), (300, 64, 1), (5, 6, 6), (900, 1024, 8),
                                   (40, 512, 8),   # T <= 64 with E > 256: the general small-T kernel
                                   (64, 256, 8),   # the 4-wave kernel at its largest T and E
                                   (33, 300, 6)])  # E not a multiple of 16 lanes
def test_route_ties_and_other_shapes(T, E, k):
    g = np.random.default_rng(T + E + k)
    logits = g.integers(-2, 3, (T, E)).astype(np.float32)  # many exact ties
    _check(logits, k)


def test_route_single_hot_expert():
    # every token's top expert is expert 7 (one very large segment)
    logits = dg.logits(3, 3000, 256, "normal")
    logits[:, 7] += 100.0
    _check(logits, 6)


def test_route_is_deterministic():
    logits = torch.from_numpy(dg.logits(4, 5000, 256, "uniform")).cuda()
    a = ops.moe_route_permute(logits, 6)
    b = ops.moe_route_permute(logits, 6)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
