"""Pins of oracle.append_aliasing, the append write-aliasing rule (CPU only).

Worked tables check each clause by hand. A second, independent check runs the
oracle's own append on a pool whose every slot holds a distinct marker: a call
aliases exactly when, afterwards, some live position or some new token of the
batch no longer reads back its own marker.
"""
import numpy as np
import pytest

import oracle

PAGE = oracle.PAGE


def table(rows, width=4):
    bt = np.full((len(rows), width), -1, np.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    return bt


def cu(ns):
    return np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)


def check(rows, lens, ns, num_pages=16, max_new=64, msl=64):
    return oracle.append_aliasing(table(rows), lens, cu(ns), num_pages, max_new, msl)


def test_worked_tables():
    # separate pages: no aliasing
    assert not check([[0, 1], [2, 3]], [10, 20], [5, 7])
    # a session's table lists one page twice and its new tokens reach both entries
    assert check([[4, 4]], [10], [10])
    # ... but not when the new tokens stay on the first entry
    assert not check([[4, 4]], [3], [5])
    # session 1 appends into session 0's partly filled page at live slots
    assert check([[5], [5]], [10, 3], [0, 4])
    # session 1 appends into session 0's page at slots session 0 does not hold
    assert not check([[5], [5]], [3, 8], [0, 4])
    # a full, block-aligned prefix page shared by both sessions, each appending to a page of its own
    assert not check([[6, 7], [6, 8]], [16, 16], [5, 9])
    # both append into the shared page's successor they both map (their own tokens collide)
    assert check([[6, 7], [6, 7]], [16, 16], [1, 1])
    # two sessions start one page at the same slots: new tokens collide
    assert check([[9], [9]], [0, 0], [4, 4])
    # ... or one writes above the other's live tokens, the other over them
    assert check([[9], [9]], [0, 8], [4, 4])
    # a new token over the writing session's own live token (its table repeats a page)
    assert check([[3, 3]], [20], [1])


def test_skipped_writes():
    # out-of-range page ids write nothing (the append reports them)
    assert not check([[99], [99]], [0, 0], [2, 2], num_pages=16)
    # a session whose lengths the append rejects writes nothing
    assert not check([[1], [1]], [0, 0], [70, 2], max_new=64)
    # a session whose seq_lens exceeds max_seq_len holds no live slots for the rule
    assert not check([[2], [2]], [80, 0], [0, 3], msl=64)


def _markers_survive(bt, lens, ns, num_pages):
    """Append distinct markers over a pool of distinct markers; True if every live
    position and every new token reads back its own marker afterwards."""
    shape = oracle.PoolShape(1, num_pages, 1, 64)
    pool = np.zeros(shape.elems, np.uint16)
    k0 = oracle.k_offset
    for pid in range(num_pages):
        base = oracle.tile_start(0, pid, 0, num_pages, 1, 64)
        for t in range(PAGE):
            pool[base + k0(t, 0)] = 0x4000 + pid * PAGE + t
    c = cu(ns)
    total = int(c[-1])
    k_new = np.zeros((total, 1, 64), np.uint16)
    k_new[:, 0, 0] = 1 + np.arange(total)
    after = oracle.append(pool, shape, 0, k_new, np.zeros_like(k_new), c, bt, lens)

    def read(b, p):
        pid = int(bt[b, p // PAGE])
        return after[oracle.tile_start(0, pid, 0, num_pages, 1, 64) + k0(p % PAGE, 0)]

    for b in range(len(lens)):
        for q in range(lens[b]):
            pid = int(bt[b, q // PAGE])
            if read(b, q) != 0x4000 + pid * PAGE + q % PAGE:
                return False
        for j in range(ns[b]):
            if read(b, lens[b] + j) != 1 + c[b] + j:
                return False
    return True


@pytest.mark.parametrize("seed", range(40))
def test_rule_equals_marker_readback(seed):
    rng = np.random.default_rng(seed)
    B, num_pages, width = int(rng.integers(1, 4)), int(rng.integers(2, 9)), 3
    bt = rng.integers(0, num_pages, size=(B, width)).astype(np.int32)
    lens = [int(x) for x in rng.integers(0, 2 * PAGE, size=B)]
    ns = [int(rng.integers(0, width * PAGE - L + 1)) for L in lens]
    got = oracle.append_aliasing(bt, lens, cu(ns), num_pages, width * PAGE, width * PAGE)
    assert got == (not _markers_survive(bt, lens, ns, num_pages))
