"""Host model of the sliding-window band kernel's LDS ring schedule.

The band kernel (prefill.hip, prefill_band_kernel) keeps the 32-key K/V tiles of a
query block's window in a 7-slot LDS ring and runs its odd waves one iteration
behind the even ones: in iteration n the late waves take block n - 1 whole, the
early waves finish block n - 1 (tiles from mid(n - 1) on) and start block n
(tiles tlo(n) .. mid(n) - 1), and every thread stages tile thi(n) when it is new.
This model replays that schedule over many shapes and checks what the kernel's
correctness rests on: every tile read in an iteration was published at an earlier
barrier and still sits in its slot, the slot written in an iteration is read by
no wave in it, and each wave visits every tile of each of its blocks exactly once.
The window (a query at key index i sees keys i - W + 1 .. i, W = 128 counting
the query itself) is the convention of "Notable quirks" on the miles recipe page.
"""
import pytest

NK = QW = 32
SLOTS = 7


def tile_range(Tq, Tk, W):
    off = Tk - Tq

    def tlo(qb):
        j = qb * QW + off - W + 1
        return j // NK if j > 0 else 0

    def thi(qb):
        return (min(qb * QW + QW - 1, Tq - 1) + off) // NK

    return tlo, thi


def replay(Tq, Tk, W, runs):
    tlo, thi = tile_range(Tq, Tk, W)
    nqb = (Tq + QW - 1) // QW
    per = (nqb + runs - 1) // runs

    def mid(qb):
        return min(tlo(qb) + 1, thi(qb))

    for r in range(runs):
        qb0, qb1 = r * per, min(nqb, r * per + per)
        if qb0 >= qb1:
            continue
        slot = {}
        t0, tp = tlo(qb0), thi(qb0) - 1
        for jt in range(t0, tp + 1):            # prologue
            slot[jt % SLOTS] = jt
        staged = max(tp, t0 - 1)
        seen = {}
        for n in range(qb0, qb1 + 1):
            write = None
            if n < qb1 and thi(n) > staged:
                assert thi(n) == staged + 1       # one new tile per block at most
                write = staged = thi(n)
            reads = []
            if n > qb0:                           # early: rest of block n - 1
                reads += [("E", n - 1, jt) for jt in range(mid(n - 1), thi(n - 1) + 1)]
            if n < qb1:                           # early: start of block n
                reads += [("E", n, jt) for jt in range(tlo(n), mid(n))]
            if n > qb0:                           # late: block n - 1 whole
                reads += [("L", n - 1, jt) for jt in range(tlo(n - 1), thi(n - 1) + 1)]
            for grp, qb, jt in reads:
                assert slot.get(jt % SLOTS) == jt, (Tq, Tk, W, runs, n, jt)
                if write is not None:
                    assert jt % SLOTS != write % SLOTS, (Tq, Tk, W, runs, n, jt, write)
                seen.setdefault((grp, qb), []).append(jt)
            if write is not None:
                slot[write % SLOTS] = write
        for qb in range(qb0, qb1):
            want = list(range(tlo(qb), thi(qb) + 1))
            assert sorted(seen[("E", qb)]) == want
            assert sorted(seen[("L", qb)]) == want


@pytest.mark.parametrize("W", [1, 2, 31, 32, 33, 64, 100, 127, 128])
def test_band_ring_schedule(W):
    for Tq in [1, 2, 31, 32, 33, 65, 77, 100, 150, 200, 300, 512, 1000, 8192]:
        for extra in [0, 1, 5, 31, 32, 127, 200]:
            for runs in [1, 3, 8, 64]:
                replay(Tq, Tq + extra, W, runs)


def test_band_ring_needs_seven_slots():
    # the widest iteration (128-key window, keys not tile-aligned) reads 6 tiles
    # while it writes a 7th: a 6-slot ring would overwrite a tile still in use
    tlo, thi = tile_range(8192, 8192 + 5, 128)
    n = 100
    reads = set(range(tlo(n - 1), thi(n - 1) + 1)) | set(range(tlo(n), min(tlo(n) + 1, thi(n))))
    assert len(reads | {thi(n)}) == SLOTS
