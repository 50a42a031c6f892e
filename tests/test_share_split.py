"""The stream-K share boundaries of the decode kernels, checked on the CPU.

A call cuts T tiles into n shares (n = 4 x workgroups, a multiple of 32, at
most 1024), WPG consecutive shares per workgroup, workgroup i on XCD i % 8.  A
share on an even XCD weighs `even`, one on an odd XCD 512 - even; the weight
before share k, scaled to a whole of 2^18 by mult = floor(2^26 / n), gives
share_start(k) = (W(k) * T) >> 18, with share_start(n) = T.  The kernels rely on:
the shares tile 0 .. T in order; share_of(t) is the share holding tile t; and
when T * floor(min(even, 512 - even) * mult / 2^16) >= 2^18, no share is empty
(the merge tree then skips its search for shares with tiles).  At n = 1024 the
scaling is the identity.  This model restates the arithmetic; the GPU tests
run the kernels on forced grids against the oracle.
"""
import itertools

import numpy as np
import pytest


def weight_before(k, n, even, wpg):
    per = 8 * wpg
    odd = 512 - even
    r, g = k % per, (k % per) // wpg
    prev = ((g + 1) >> 1) * even + (g >> 1) * odd
    raw = (k // per) * wpg * 4 * 512 + wpg * prev + (r % wpg) * (odd if g & 1 else even)
    return (raw * ((1 << 26) // n)) >> 16


def share_start(k, T, n, even, wpg):
    return T if k >= n else (weight_before(k, n, even, wpg) * T) >> 18


def share_of(t, T, n, even, wpg):
    lo, hi = 0, n
    while hi - lo > 1:
        mid = (lo + hi) >> 1
        if weight_before(mid, n, even, wpg) * T < (t + 1) << 18:
            lo = mid
        else:
            hi = mid
    return lo


@pytest.mark.parametrize("wg,even,wpg", list(itertools.product([8, 24, 64, 200, 248, 256], [1, 236, 256, 276, 511],
                                                                [1, 4])))
def test_shares_tile_the_list(wg, even, wpg):
    n = 4 * wg
    mult = (1 << 26) // n
    assert weight_before(n, n, even, wpg) <= 1 << 18
    if n == 1024:
        assert mult == 1 << 16
    for T in (1, 7, 31, n - 1, n, 3 * n + 5, 100003, 1 << 22):
        starts = [share_start(k, T, n, even, wpg) for k in range(n + 1)]
        assert starts[0] == 0 and starts[-1] == T
        assert all(a <= b for a, b in zip(starts, starts[1:]))
        sizes = np.diff(starts)
        dense = T * ((min(even, 512 - even) * mult) >> 16) >= 1 << 18
        if dense:
            assert sizes.min() >= 1, (T, n, even)
        # share_of inverts share_start on every tile (sampled on large T)
        ts = range(T) if T <= 5000 else np.random.default_rng(T).integers(0, T, 2000)
        for t in ts:
            k = share_of(int(t), T, n, even, wpg)
            assert starts[k] <= t < starts[k + 1], (t, k)


def test_full_grid_scaling_is_exact():
    """At 1024 shares the scaled weights equal the plain ones: the boundaries are
    (weight before k) * T / 2^18 with the weights summing to exactly 2^18."""
    for even in (256, 276):
        for k in range(0, 1025, 37):
            per = 32
            odd = 512 - even
            g = (k % per) // 4
            raw = (k // per) * 4 * 4 * 512 + 4 * (((g + 1) >> 1) * even + (g >> 1) * odd) + \
                (k % 4) * (odd if g & 1 else even)
            assert weight_before(k, 1024, even, 4) == raw
