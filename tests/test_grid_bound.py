"""Host-side check of the tiled GEMMs' grid size (tile256_grid in csrc/tile256.hpp)
against the work split of grouped_work_item (csrc/gemm_common.hpp).

The host sizes the grouped launch without the per-expert row counts: m_units =
cdiv(rows, 256) + E bounds the 256-row units, and each of the 8 XCDs gets
ceil(m_units * ntiles / ntg / 8) blocks. On the device the T = units * ntiles / ntg
items are split into 8 contiguous ranges [x T / 8, (x + 1) T / 8); block j of XCD x
takes item x T / 8 + j. Every item must have a block, and no block may get two.
"""

import numpy as np
import pytest


def cdiv(a, b):
    return -(-a // b)


def grid_per_xcd(m_units, ntiles, ntg):
    return cdiv(m_units * (ntiles // ntg), 8)


def device_items(counts, ntiles, ntg, per_xcd, bm=256, split=0):
    units = sum(0 if (split and c <= split) else cdiv(c, bm) for c in counts)
    total = units * (ntiles // ntg)
    seen = []
    for x in range(8):
        lo, hi = x * total // 8, (x + 1) * total // 8
        for j in range(per_xcd):
            w = lo + j
            if w < hi:
                seen.append(w)
        assert hi - lo <= per_xcd, "an XCD has more items than blocks"
    assert sorted(seen) == list(range(total)), "items missed or taken twice"
    return total


@pytest.mark.parametrize("seed", range(40))
def test_grid_covers_every_item(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.choice([1, 8, 64, 256]))
    T = int(rng.integers(1, 20000))
    topk = int(min(E, rng.choice([1, 2, 6, 8])))
    rows = T * topk
    # uniform, skewed and adversarial (every expert just past a unit boundary) loads
    kind = seed % 3
    if kind == 0:
        counts = np.bincount(rng.integers(0, E, rows), minlength=E)
    elif kind == 1:
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        counts = np.bincount(rng.choice(E, rows, p=p / p.sum()), minlength=E)
    else:
        # as many experts as possible one row past a 256-row unit (the most units per row)
        counts = np.zeros(E, dtype=np.int64)
        n = min(E, rows // 257)
        counts[:n] = 257
        counts[0] += rows - counts.sum()
    assert counts.sum() == rows
    m_units = cdiv(rows, 256) + E   # the host's bound (experts that may hold a partial unit: E)
    for ntiles, ntg in ((16, 1), (28, 4), (28, 1), (8, 2), (4, 4)):
        per_xcd = grid_per_xcd(m_units, ntiles, ntg)
        device_items([int(c) for c in counts], ntiles, ntg, per_xcd)


def test_grid_bound_is_tight_enough():
    # the 16384-token layer: 98,304 rows over 256 experts; FC2 chains 4 of its 28 n-tiles
    m_units = cdiv(98304, 256) + 256
    assert 8 * grid_per_xcd(m_units, 28, 4) == 4480   # 3,584 real items at 335-429 rows per expert
    assert 8 * grid_per_xcd(m_units, 16, 1) == 10240
