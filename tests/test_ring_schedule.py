"""Host-side replay of the FP8-activation LDS-ring kernel's issue schedule
(csrc/gemm_f8ring.hip), run on the CPU before the kernel ever runs on a GPU.

The model restates the kernel's index arithmetic - per-lane copy sources, LDS
destinations, ring slots, wait counts and fragment read addresses - and checks:
  * every copy source lies inside its operand (activation codes / scales of the
    gathered rows, one expert's weight codes / scales);
  * each stage's copies cover every byte of their slot exactly once;
  * every fragment read, at every step of every stage, returns the bytes the MFMA
    lane layout asks for (row, K block, half) under the kernel's K order - for the
    E4M3 activations, the E2M1 weights and both scale operands alike, so the two
    operands and their scales pair up the same K;
  * a slot is refilled only after the stage that read it has passed a barrier, and
    the wait before each barrier leaves in flight only copies issued later.
No kernel code is executed: a mistake in this arithmetic on the device side would
show here as a mismatch before the first GPU run of a changed geometry.
"""

import numpy as np
import pytest

BM = BN = 256
KS = 128
S = KS // 64
RA, RB = KS, KS // 2          # bytes per row per stage: E4M3 activations, E2M1 weights
CA, CB = RA // 16, RB // 16   # 16-byte chunks per row per stage
IA = BM * CA // 64 // 8
IB = BN * CB // 64 // 8
D = IA + IB + 1
NSLOT = 3
SLOT_A, SLOT_B = BM * RA, BN * RB
SLOT_AS, SLOT_BS = BM * 4, BN * 4


def swz_a(r):
    return (r & 7) ^ ((r >> 3) & 1)


def swz_b(r):
    return (r >> 2) & 3


def copies(wave, lane, a_src_row, b_row, K):
    """The kernel's per-lane copy descriptors of stage 0 (offsets grow by a scalar per stage)."""
    arow, wrow, srow = K, K // 2, K // 32
    out = []
    for q in range(IB):
        chunk = (wave * IB + q) * 64 + lane
        r, pc = divmod(chunk, CB)
        out.append(("B", (wave * IB + q) * 1024 + 16 * lane, 16, b_row(r) * wrow + 16 * (pc ^ swz_b(r)), RB))
    for q in range(IA):
        chunk = (wave * IA + q) * 64 + lane
        r, pc = divmod(chunk, CA)
        out.append(("A", (wave * IA + q) * 1024 + 16 * lane, 16, a_src_row(r) * arow + 16 * (pc ^ swz_a(r)), RA))
    sc_row = 64 * (wave & 3) + lane
    if wave < 4:
        out.append(("As", (wave & 3) * 256 + 4 * lane, 4, a_src_row(sc_row) * srow, 4))
    else:
        out.append(("Bs", (wave & 3) * 256 + 4 * lane, 4, b_row(sc_row) * srow, 4))
    return out


def replay(mode, K, N, I, m, act_rows, gather, n_tile):
    """Replay one work item; gather(r) is the activation row of tile row r < m."""
    nst = K // KS
    arow, wrow, srow = K, K // 2, K // 32

    def a_src_row(r):
        return gather(0 if r >= m else r)

    def b_row(r):
        if mode == "fc1":
            return (0 if r < BN // 2 else I - BN // 2) + n_tile * (BN // 2) + r
        return n_tile * BN + r

    ext = {"A": act_rows * arow, "As": act_rows * srow, "B": N * wrow, "Bs": N * srow}
    size = {"A": SLOT_A, "B": SLOT_B, "As": SLOT_AS, "Bs": SLOT_BS}
    # symbolic LDS: per slot and member, the global byte offset each LDS byte came from
    lds = [{k: np.full(v, -1, dtype=np.int64) for k, v in size.items()} for _ in range(NSLOT)]
    desc = {(w, l): copies(w, l, a_src_row, b_row, K) for w in range(8) for l in range(64)}
    assert all(len(v) == D for v in desc.values())

    issued = {}   # stage -> slot
    in_flight = {w: [] for w in range(8)}   # per wave: stages whose copies are outstanding, in order

    def issue(st):
        slot = st % NSLOT
        for k in size:
            lds[slot][k][:] = -1
        for (w, l), ds in desc.items():
            for member, dst, nbytes, src0, step in ds:
                src = src0 + st * step
                assert 0 <= src and src + nbytes <= ext[member], (member, w, l, st, src)
                seg = lds[slot][member][dst:dst + nbytes]
                assert seg.size == nbytes and np.all(seg == -1), (member, w, l, st, dst)
                lds[slot][member][dst:dst + nbytes] = src + np.arange(nbytes)
        for k in size:
            assert np.all(lds[slot][k] >= 0), f"stage {st}: slot member {k} not fully covered"
        issued[st] = slot
        for w in range(8):
            in_flight[w].append(st)

    def wait(allowed):   # s_waitcnt vmcnt(allowed) on every wave: copies complete in issue order
        for w in range(8):
            while len(in_flight[w]) * D > allowed:
                in_flight[w].pop(0)

    issue(0)
    if nst > 1:
        issue(1)
    read_by = {}
    for st in range(nst):
        wait(D if st + 1 < nst else 0)
        for w in range(8):
            assert st not in in_flight[w], f"stage {st} read before its copies completed"
        # barrier: every stage < st is done; refill the slot of st - 1
        if st + 2 < nst:
            slot = (st + 2) % NSLOT
            assert read_by.get(slot, -1) < st, "slot refilled while a later stage reads it"
            issue(st + 2)
        slot = issued[st]
        read_by[slot] = st
        for w in range(8):
            wm, wn = w >> 1, w & 1
            if 64 * wm >= m:
                continue   # inactive row group: no reads
            for l in range(64):
                g, r32 = l >> 5, l & 31
                arows = [64 * wm + 32 * f + r32 for f in range(2)]
                if mode == "fc1":
                    brows = [(0 if f < 2 else BN // 2) + 64 * wn + 32 * (f & 1) + r32 for f in range(4)]
                else:
                    brows = [128 * wn + 32 * f + r32 for f in range(4)]
                aoff = [r * RA + 16 * (g ^ swz_a(r)) for r in arows]
                boff = [r * RB + 16 * (g ^ swz_b(r)) for r in brows]
                for s in range(S):
                    for f, r in enumerate(arows):
                        gr = a_src_row(r)
                        for half, o in ((0, aoff[f] ^ (64 * s)), (1, aoff[f] ^ (64 * s + 32))):
                            # hardware block `half`, k [16 g, 16 g + 16) of it, from memory block 2 s + half
                            k0 = st * KS + 32 * (2 * s + half) + 16 * g
                            want = gr * arow + k0 + np.arange(16)
                            assert np.array_equal(lds[slot]["A"][o:o + 16], want), ("A", st, w, l, s, f, half)
                    for f, r in enumerate(brows):
                        gr = b_row(r)
                        o = boff[f] ^ (32 * s)
                        k0 = st * KS + 32 * (2 * s + g)       # hardware block g <- memory block 2 s + g
                        want = gr * wrow + k0 // 2 + np.arange(16)
                        assert np.array_equal(lds[slot]["B"][o:o + 16], want), ("B", st, w, l, s, f)
                    # scales: the lane's dword shifted right by 8 g; op_sel 2 s picks block 2 s + g
                    for member, rows, rowf in (("As", arows, a_src_row), ("Bs", brows, b_row)):
                        for r in rows:
                            dword = lds[slot][member][4 * r:4 * r + 4]
                            shifted = dword[g:]
                            byte = shifted[2 * s]
                            want = rowf(r) * srow + st * (KS // 32) + 2 * s + g
                            assert byte == want, (member, st, w, l, s, r)
    for w in range(8):
        assert not in_flight[w], "copies still in flight at the end of the workgroup"


@pytest.mark.parametrize("mode,K,N,I,m", [
    ("fc1", 7168, 4096, 2048, 256),   # a full unit of the 2048-token FP8 layer's FC1
    ("fc1", 7168, 4096, 2048, 77),    # a partial unit (rows past m read row 0)
    ("fc2", 2048, 7168, 2048, 200),
    ("dense", 1024, 512, 0, 129),
    ("dense", 512, 256, 0, 256),
])
def test_f8ring_schedule(mode, K, N, I, m):
    rng = np.random.default_rng(7)
    if mode == "fc1":
        T, topk = 3000, 6
        pairs = rng.choice(T * topk, size=m, replace=False)
        act_rows = T
        gather = lambda r: int(pairs[r]) // topk   # noqa: E731 (sorted_pair[row0 + r] / topk)
        n_tile = (2 * I) // BN - 1                   # the last gate/up tile
    else:
        act_rows = 1000 + m
        row0 = 1000
        gather = lambda r: row0 + r                  # noqa: E731
        n_tile = N // BN - 1
    replay(mode, K, N, I, m, act_rows, gather, n_tile)


def test_f8ring_slot_fits_lds():
    assert NSLOT * (SLOT_A + SLOT_B + SLOT_AS + SLOT_BS) <= 160 * 1024
    assert 8 * 8192 <= NSLOT * (SLOT_A + SLOT_B + SLOT_AS + SLOT_BS)   # the epilogue's staging
