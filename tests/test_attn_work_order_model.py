"""CPU model of the attention kernels' work order with several prompts
(``work_item`` in csrc/tg_common.h), checked against a sort.

A grid slot of rank r (dispatch order) takes the r-th existing (prompt,
query tile) pair in the order tile index descending, then prompt ascending;
ranks past the last pair are empty.  The model follows the kernel's steps:
S(t) = sum_b max(0, n_b - t) counts the pairs with tile index >= t, a
binary search finds the largest t with S(t) > r, and the prompt is the
(r - S(t + 1))-th one, in prompt order, among those with n_b > t, found 64
prompts at a time as the kernel's ballots do.  Every existing pair must be
taken exactly once, in that order, and every later rank must be empty.
"""

import numpy as np
import pytest


def _tiles_of(cu, b, bq):
    return (int(cu[b + 1]) - int(cu[b]) + bq - 1) // bq


def _S(cu, B, bq, t):
    return sum(max(0, _tiles_of(cu, b, bq) - t) for b in range(B))


def _work_item(cu, B, n_qt, bq, r):
    if _S(cu, B, bq, 0) <= r:
        return None
    lo, hi = 0, n_qt
    while hi - lo > 1:
        mid = (lo + hi) >> 1
        if _S(cu, B, bq, mid) > r:
            lo = mid
        else:
            hi = mid
    j = r - _S(cu, B, bq, lo + 1)
    for b0 in range(0, B, 64):
        has = [bb < B and _tiles_of(cu, bb, bq) > lo for bb in range(b0, b0 + 64)]
        c = sum(has)
        if j < c:
            return b0 + [i for i, h in enumerate(has) if h][j], lo
        j -= c
    raise AssertionError("rank inside the pairs but no prompt found")


@pytest.mark.parametrize("seed", range(40))
def test_work_order_matches_sort(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(2, 150))
    bq = int(rng.choice([128, 256]))
    lens = rng.integers(0, 3000, B)
    lens[rng.random(B) < 0.1] = 0
    if lens.max() == 0:
        lens[0] = 1
    cu = np.concatenate([[0], np.cumsum(lens)])
    n_qt = (int(lens.max()) + bq - 1) // bq
    got = [_work_item(cu, B, n_qt, bq, r) for r in range(B * n_qt)]
    want = sorted(((b, t) for b in range(B) for t in range(_tiles_of(cu, b, bq))), key=lambda p: (-p[1], p[0]))
    assert got[:len(want)] == want
    assert all(g is None for g in got[len(want):])
