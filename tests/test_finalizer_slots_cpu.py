"""The tile finalizer's processing-order slots (CPU replay of the kernel's rules).

The binning's tile finalizer (one workgroup, `tile_finalize` in csrc/bin.hip) orders the tiles for
the raster calls. Workgroup b of a raster launch runs on XCD b mod 8, so each tile has an XCD
(plan_xcd: 2x1 blocks of tiles round the 8 XCDs, each row of tiles shifted by three), and each
XCD a list of its tiles by count class (the bit length of a tile's pair count, 0 for an empty
tile), heaviest class first. A first sweep counts the tiles of each (XCD, class); each list's
class cursors start at the prefix of its counts from class 32 down to class 0; the second sweep
gives each tile the next place of its (XCD, class), a wave at a time (the lanes of one key share
one atomic on the cursor and take consecutive places in lane order). Place p of XCD x's list goes
to slot 8 p + x while p is below the shortest list's length m; the lists' rest take the slots
from 8 m on, a wave's such lanes in lane order. The slots must be a permutation of [0, ntiles):
a slot at or past ntiles would write past the plan's order. This test replays those rules on grids
of 141 x 92 (12,972) and 263 x 263 (69,169) tiles and on small odd grids, including the overflow
case, where every tile counts as empty, and checks the finalizer's LDS
layout (steps of tiles, then the auxiliary words) against the constants in the source.
"""
import os
import re

import numpy as np
import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "gaussian_splatting_tile_gs_amd", "csrc", "bin.hip")


def _const(name):
    m = re.search(r"constexpr (?:int|uint32_t) " + name + r" = ([^;]+);", open(SRC).read())
    assert m, name
    return m.group(1)


def _layout():
    return int(_const("kSortThreads")), int(_const("kRadix")), int(_const("kFinRows"))


def test_finalizer_lds_layout_fits():
    threads, radix, rows = _layout()
    src = open(SRC).read()
    step = threads * rows                 # kFinStep: the tiles of one step
    aux = 8 * radix                       # kFinAuxWords
    lds = 12288                           # the finalizer pass's s_mem words (2 x 4096 keys < 12288)
    assert "kFinAuxWords = 8 * kRadix" in src
    assert step + aux <= lds, "steps of tiles overlap the auxiliary words"
    # the auxiliary words: three histogram rows, then the (XCD, class) counts and cursors, the
    # counters, the scan partials (rows x 16) and the row sums (rows); the zeroing covers the
    # counts, cursors and counters in one pass of the workgroup's threads
    keys = 8 * int(_const("kFinClasses"))
    misc = int(_const("kFinMisc"))
    assert "kFinKeys = kXcds * kFinClasses" in src and int(_const("kFinClasses")) == 33
    assert 3 * radix + 2 * keys + misc + 17 * rows <= aux
    assert "if (tid < (int)(2 * kFinKeys + kFinMisc)) s_cls[tid] = 0;" in src and 2 * keys + misc <= threads
    # the counters: [0..3] and the eight list lengths at [8 + x]
    assert "s_misc[8 + tid] = place;" in src and 8 + 8 <= misc


def _count_class(c):
    return np.where(c > 0, np.floor(np.log2(np.maximum(c, 1))).astype(np.int64) + 1, 0)


def _xcd(t, tiles_x):
    return ((t % tiles_x) // 2 + 3 * (t // tiles_x)) % 8


def _replay_slots(counts, fits, tiles_x, threads, rows):
    ntiles = counts.size
    c = counts.astype(np.int64) if fits else np.zeros_like(counts, dtype=np.int64)
    cls = _count_class(c)
    assert cls.max() <= 32
    xcd = _xcd(np.arange(ntiles), tiles_x)
    key = xcd * 33 + cls
    # per XCD list: cursors heaviest class first, empty tiles last (on overflow all tiles class 0)
    per = np.bincount(key, minlength=8 * 33).reshape(8, 33)
    cur = np.zeros((8, 33), np.int64)
    lens = per.sum(axis=1)
    for x in range(8):
        place = 0
        for k in range(32, -1, -1):
            cur[x, k] = place
            place += per[x, k]
    m = int(lens.min())
    cur = cur.ravel()
    tail = 0
    slots = np.full(ntiles, -1, np.int64)
    places = np.full(ntiles, -1, np.int64)
    step = threads * rows
    for cb in range(0, ntiles, step):
        mm = min(step, ntiles - cb)
        for q in range(-(-mm // threads)):
            for w in range(threads // 64):  # a wave: 64 consecutive tiles of the row
                i0 = q * threads + w * 64
                idx = np.arange(i0, i0 + 64)
                valid = idx < mm
                t = cb + idx[valid]
                kc = key[t]
                pl = np.empty(t.size, np.int64)
                for k in np.unique(kc):  # lanes of one key: one cursor add, places in lane order
                    sel = kc == k
                    pl[sel] = cur[k] + np.arange(sel.sum())
                    cur[k] += sel.sum()
                places[t] = pl
                rest = pl >= m
                slots[t[~rest]] = 8 * pl[~rest] + xcd[t[~rest]]
                slots[t[rest]] = 8 * m + tail + np.arange(rest.sum())  # the wave's rest in lane order
                tail += int(rest.sum())
    return slots, places, cls, xcd, m


@pytest.mark.parametrize("grid", [(141, 92), (263, 263), (7, 3), (1, 5), (3, 1)])
@pytest.mark.parametrize("kind", ["random", "empty", "equal", "huge", "overflow"])
def test_order_slots_are_a_permutation(grid, kind):
    threads, _, rows = _layout()
    tiles_x, tiles_y = grid
    ntiles = tiles_x * tiles_y
    rng = np.random.default_rng(ntiles)
    if kind == "random":
        counts = rng.integers(0, 5000, ntiles) * (rng.random(ntiles) < 0.7)
    elif kind == "empty":
        counts = np.zeros(ntiles, np.int64)
    elif kind == "equal":
        counts = np.full(ntiles, 257, np.int64)
    elif kind == "huge":  # every class, up to 32 bits (a count of 2^32 - 1)
        counts = (rng.integers(0, 2**32 - 1, ntiles, dtype=np.int64) >> rng.integers(0, 32, ntiles)).astype(np.int64)
        counts[:min(3, ntiles)] = [2**32 - 1, 2**31, 1][:min(3, ntiles)]
    else:
        counts = rng.integers(1, 10**6, ntiles)
    slots, places, cls, xcd, m = _replay_slots(counts, kind != "overflow", tiles_x, threads, rows)
    assert slots.min() >= 0 and slots.max() < ntiles
    assert np.array_equal(np.sort(slots), np.arange(ntiles)), "slots are not a permutation"
    head = slots < 8 * m
    assert np.all(slots[head] % 8 == xcd[head]), "a slot below 8 m is not on its tile's XCD"
    if kind != "overflow":
        for x in range(8):  # each XCD's list heaviest class first, places 0 .. len - 1
            t = np.nonzero(xcd == x)[0]
            o = t[np.argsort(places[t])]
            assert np.array_equal(np.sort(places[t]), np.arange(t.size))
            assert np.all(np.diff(cls[o]) <= 0), "a list is not heaviest class first"


def test_xcd_lists_are_balanced():
    """The XCD lists of the workloads' tile grids differ in length by a few tiles, so the slots
    from 8 m on (the lists' rest, not on their XCDs) are few."""
    for tiles_x, tiles_y in [(80, 45), (62, 35), (120, 68), (123, 69), (8, 8), (141, 92), (263, 263)]:
        n = tiles_x * tiles_y
        lens = np.bincount(_xcd(np.arange(n), tiles_x), minlength=8)
        assert n - 8 * lens.min() <= 32, (tiles_x, tiles_y, lens)
