"""The achievable-rate probes (include/mxf_ceilings.h) compute what they claim:
the streaming read visits every byte (its XOR of all 32-bit words equals the
host's), the MFMA loop with all operands 1.0 and scale 2^0 accumulates 64 per
element per instruction exactly, and the LDS-fill probe lands every byte of every
region it copies, as often as its sharing pattern says (its wrapping sum of the
words it read equals the one torch computes from the regions)."""

import numpy as np
import pytest
import torch

from mxfp4_block_scaled_amd import ops

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [4, 4 * 1_000_003, 64 << 20])
def test_read_probe_visits_every_word(words):
    h = np.random.default_rng(words).integers(-2**31, 2**31, size=words, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(h).cuda()
    got = ops.ceiling_read(buf)
    torch.cuda.synchronize()
    assert int(got.item()) == int(np.bitwise_xor.reduce(h))


def _operands(a_word, b_word):
    ops_ = np.empty((64, 6, 64, 8), dtype=np.uint32)
    ops_[:, :2] = a_word
    ops_[:, 2:] = b_word
    return torch.from_numpy(ops_.view(np.int32).reshape(-1)).cuda()


@pytest.mark.parametrize("fmt,a_word", [("e2m1", 0x22222222), ("e4m3", 0x38383838)])
def test_mfma_probe_ones_accumulate_exactly(fmt, a_word):
    iters = 2000
    sink, flops = ops.ceiling_mfma(_operands(a_word, 0x22222222), fmt, 127, iters)
    torch.cuda.synchronize()
    assert flops == 512 * 4 * iters * 8 * 131072
    assert torch.all(sink == 8192.0 * iters), sink[:4]


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_mfma_probe_random_operands_run(fmt):
    g = torch.Generator(device="cuda").manual_seed(5)
    words = torch.randint(-2**31, 2**31 - 1, (ops.CEILING_MFMA_WORDS,), dtype=torch.int32, device="cuda",
                          generator=g)
    sink, _ = ops.ceiling_mfma(words, fmt, 124, 100)
    torch.cuda.synchronize()
    assert sink.shape == (512,)


@pytest.mark.parametrize("pattern,groups", [(0, 256), (1, 256), (1, 512)])
def test_lds_copy_probe_lands_every_region(pattern, groups):
    lib = ops.load()
    nbytes = lib.mxf_ceiling_lds_copy_bytes(pattern, groups)
    R = ops.CEILING_COPY_REGION
    g = torch.Generator(device="cuda").manual_seed(groups + pattern)
    words = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
    got = ops.ceiling_lds_copy(words, pattern, groups)
    torch.cuda.synchronize()
    region_sums = words.view(-1, R // 4).to(torch.int64).sum(dim=1)   # one per region
    if pattern == 0:
        want = int(region_sums.sum().item())
    else:
        na = groups // 16
        want = 16 * int(region_sums[:na].sum().item()) + 2 * int(region_sums[na:].sum().item())
    assert (int(got.item()) & 0xFFFFFFFF) == (want & 0xFFFFFFFF)

