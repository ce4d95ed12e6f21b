"""The tile finalizer's processing-order slots (CPU replay of the kernel's rules).

The binning's tile finalizer (one workgroup, `tile_finalize` in csrc/bin.hip) orders the tiles for
the raster calls by count class (the bit length of a tile's pair count, 0 for an empty tile),
heaviest class first: a first sweep counts the tiles of each class, the class cursors start at the
prefix of the counts from class 32 down to class 0, and the second sweep gives each tile the next
slot of its class, a wave at a time (the lanes of one class share one atomic on the cursor and
take consecutive slots in lane order). The slots must be a permutation of [0, ntiles): a slot at
or past ntiles would write past the plan's order. This test replays those rules for the tile
counts of the large frames (12,972 and 69,169 tiles), including the overflow case, where every
tile counts as empty, and checks the finalizer's LDS layout (steps of tiles, then the auxiliary
words) against the constants in the source.
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
    step = threads * rows                 # kFinStep: the tiles of one step
    aux = 8 * radix                       # kFinAuxWords
    lds = 12288                           # the finalizer pass's s_mem words (2 x 4096 keys < 12288)
    assert "kFinAuxWords = 8 * kRadix" in open(SRC).read()
    assert step + aux <= lds, "steps of tiles overlap the auxiliary words"
    # the auxiliary words: three histogram rows, then classes (33), cursors (33) and three
    # counters in the fourth row, scan partials (rows x 16) in the fifth, row sums (rows) in the
    # sixth; the zeroing covers the classes, cursors and counters
    cls, cur, misc = 3 * radix, 3 * radix + 64, 3 * radix + 128
    assert cls + 33 <= cur and cur + 33 <= misc and misc + 3 <= 4 * radix
    assert "if (tid < 131) s_cls[tid] = 0;" in open(SRC).read()
    assert 4 * radix + rows * 16 <= 5 * radix and 5 * radix + rows <= aux


def _count_class(c):
    return np.where(c > 0, np.floor(np.log2(np.maximum(c, 1))).astype(np.int64) + 1, 0)


def _replay_slots(counts, fits, threads, rows):
    ntiles = counts.size
    c = counts.astype(np.int64) if fits else np.zeros_like(counts, dtype=np.int64)
    cls = _count_class(c)
    assert cls.max() <= 32
    # cursors: heaviest class first, empty tiles last (on overflow all tiles are class 0)
    per = np.bincount(cls, minlength=33)
    cur = np.zeros(33, np.int64)
    slot = 0
    for k in range(32, -1, -1):
        cur[k] = slot
        slot += per[k]
    slots = np.full(ntiles, -1, np.int64)
    step = threads * rows
    for cb in range(0, ntiles, step):
        m = min(step, ntiles - cb)
        for q in range(-(-m // threads)):
            for w in range(threads // 64):  # a wave: 64 consecutive tiles of the row
                i0 = q * threads + w * 64
                idx = np.arange(i0, i0 + 64)
                valid = idx < m
                t = cb + idx[valid]
                kc = cls[t]
                for k in np.unique(kc):  # lanes of one class: one cursor add, slots in lane order
                    lanes = t[kc == k]
                    slots[lanes] = cur[k] + np.arange(lanes.size)
                    cur[k] += lanes.size
    return slots, cls


@pytest.mark.parametrize("ntiles", [12972, 69169])
@pytest.mark.parametrize("kind", ["random", "empty", "equal", "huge", "overflow"])
def test_order_slots_are_a_permutation(ntiles, kind):
    threads, _, rows = _layout()
    rng = np.random.default_rng(ntiles)
    if kind == "random":
        counts = rng.integers(0, 5000, ntiles) * (rng.random(ntiles) < 0.7)
    elif kind == "empty":
        counts = np.zeros(ntiles, np.int64)
    elif kind == "equal":
        counts = np.full(ntiles, 257, np.int64)
    elif kind == "huge":  # every class, up to 32 bits (a count of 2^32 - 1)
        counts = (rng.integers(0, 2**32 - 1, ntiles, dtype=np.int64) >> rng.integers(0, 32, ntiles)).astype(np.int64)
        counts[:3] = [2**32 - 1, 2**31, 1]
    else:
        counts = rng.integers(1, 10**6, ntiles)
    slots, cls = _replay_slots(counts, kind != "overflow", threads, rows)
    assert slots.min() >= 0 and slots.max() < ntiles
    assert np.array_equal(np.sort(slots), np.arange(ntiles)), "slots are not a permutation"
    order = np.empty(ntiles, np.int64)
    order[slots] = np.arange(ntiles)
    assert np.all(np.diff(cls[order]) <= 0), "the order is not heaviest class first"
