"""Pins of the oracle's contract for one batch of block copies
(oracle.pool.copy_batch_violations): hand-worked batches, and the property
the contract exists for -- a batch with no violation has the same effect in
any order of its copies."""
import itertools

import numpy as np
import pytest

from oracle import pool as OPL
from oracle.pool import SlotPool

NB = 10


@pytest.mark.parametrize("pairs,want", [
    ([], 0),
    ([(1, 2), (3, 4)], 0),                       # independent copies
    ([(1, 2), (3, 2)], 2),                       # one destination written twice: both pairs
    ([(1, 2), (2, 3)], 1),                       # the first destination is read by the second
    ([(2, 3), (1, 2)], 1),                       # the same, listed the other way round
    ([(5, 5)], 1),                               # a block copied onto itself
    ([(1, 2), (3, 4), (4, 1)], 2),               # 4 and 1 are destinations that are read
    ([(1, 2), (1, 3), (1, 4)], 0),               # one source read by several copies
    ([(1, NB), (NB, 2), (-1, 3), (2, 4)], 0),    # out-of-pool pairs are skipped, not counted,
    ([(1, NB), (4, 2), (2, 5)], 1),              # and take no part in other pairs' checks
    ([(7, -1), (3, 7)], 0),
])
def test_hand_worked_batches(pairs, want):
    assert OPL.copy_batch_violations(pairs, NB) == want


def _apply(pairs, order, nb=NB):
    pool = SlotPool(nb, 2)
    for blk in range(nb):
        pool.write(2 * blk, ("tok", blk))
    for i in order:
        s, d = pairs[i]
        if 0 <= s < nb and 0 <= d < nb:
            pool.copy(s, d)
    return pool.slots


def test_valid_batches_are_order_independent():
    """The contract's point: with no violation, every order of the copies
    gives the same pool (small batches, all orders)."""
    rng = np.random.default_rng(11)
    seen = 0
    for _ in range(400):
        n = int(rng.integers(1, 5))
        pairs = [(int(rng.integers(0, NB)), int(rng.integers(0, NB))) for _ in range(n)]
        if OPL.copy_batch_violations(pairs, NB):
            continue
        seen += 1
        ref = _apply(pairs, range(n))
        for order in itertools.permutations(range(n)):
            assert _apply(pairs, order) == ref
    assert seen > 50


def test_each_violation_kind_can_change_the_result():
    """A duplicate destination or a destination that is read makes the
    outcome depend on the order (distinct block contents)."""
    for pairs in ([(1, 2), (3, 2)], [(1, 2), (2, 3)]):
        assert OPL.copy_batch_violations(pairs, NB) > 0
        assert _apply(pairs, [0, 1]) != _apply(pairs, [1, 0])


def test_count_is_order_invariant():
    rng = np.random.default_rng(12)
    for _ in range(200):
        n = int(rng.integers(0, 12))
        pairs = [(int(rng.integers(-2, NB + 2)), int(rng.integers(-2, NB + 2))) for _ in range(n)]
        want = OPL.copy_batch_violations(pairs, NB)
        perm = list(rng.permutation(n))
        assert OPL.copy_batch_violations([pairs[i] for i in perm], NB) == want
