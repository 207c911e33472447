"""Pins for oracle.paging: address translation, slots and waste arithmetic.

Pinned to values printed on "Inside vLLM and TGI", section "Block addresses
and fragmentation arithmetic" (worked example, waste bound, capacity
exercise) via tests/golden/, to exact rational closed forms, and to brute
force enumeration of slots.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import paging

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_example_fifty_tokens():
    g = _golden("worked_example.json")
    b = g["block_width"]
    r = g["fifty_token_request"]
    table = r["table"]
    assert paging.blocks_needed(r["tokens"], b) == r["blocks"] == len(table)
    assert paging.tail_waste(r["tokens"], b) == r["unused_slots"]
    assert paging.allocated_slots(r["tokens"], b) - r["tokens"] == r["unused_slots"]
    t = r["next_token_position"]
    j, o = paging.logical_address(t, b)
    assert o == r["next_token_offset"]
    assert paging.physical_block(table, t, b) == r["next_token_physical_block"]
    # flat slot of that position: block 5, offset 2 -> 5 * 16 + 2
    assert paging.slot(table, t, b) == r["next_token_physical_block"] * b + r["next_token_offset"] == 82


def test_worked_example_other_requests():
    g = _golden("worked_example.json")
    b = g["block_width"]
    assert paging.blocks_needed(g["sixty_five_token_request"]["tokens"], b) == 5
    # the 65th token (position 64) is the first of logical block 4: a fifth block
    assert paging.logical_address(64, b) == (4, 0)
    r = g["twenty_token_request"]
    assert paging.allocated_slots(r["tokens"], b) == r["allocated_slots"]
    assert paging.tail_waste(r["tokens"], b) == r["unused_slots"]


def test_slots_brute_force_enumeration():
    """Slots of a table are exactly the enumeration of its blocks' offsets in order."""
    rng = np.random.default_rng(0)
    for b in (1, 4, 16, 32):
        table = [int(x) for x in rng.permutation(50)[:7]]
        expected = [blk * b + o for blk in table for o in range(b)]
        got = [paging.slot(table, t, b) for t in range(len(table) * b)]
        assert got == expected


def test_waste_bound_and_range():
    rng = np.random.default_rng(1)
    for b in (1, 3, 16, 64):
        L = [int(x) for x in rng.integers(1, 5000, size=300)]
        for x in L:
            w = paging.tail_waste(x, b)
            assert 0 <= w <= b - 1
            assert (x + w) % b == 0
            assert paging.allocated_slots(x, b) == x + w
        total = sum(paging.tail_waste(x, b) for x in L)
        assert total < b * len(L)
    assert paging.tail_waste(0, 16) == 0 and paging.blocks_needed(0, 16) == 0


def test_capacity_exercise_printed_values():
    g = _golden("capacity_u200_2000.json")
    lengths = range(g["lengths"]["lo"], g["lengths"]["hi"] + 1)
    b = g["block_width"]
    rep = paging.waste_report(lengths, b)
    p = g["printed"]

    def close(x, key):
        assert abs(float(x) - p[key]["value"]) <= p[key]["abs_tol"], (key, float(x))

    close(rep["mean_length"], "mean_length")
    close(paging.reservation_utilisation(lengths, 2000), "used_fraction_reserve_2000")
    close(rep["mean_waste"], "mean_rounding_waste_slots")
    close(rep["utilisation_ratio_of_sums"], "payload_utilisation")
    close(paging.reservation_utilisation(lengths, 4096), "used_fraction_reserve_4096")
    # the exhaustive loop's own assertion: allocated - used < b * count
    assert rep["allocated"] - rep["used"] < b * rep["n"]


def test_capacity_exact_closed_forms():
    """Exact rationals for U{200..2000}, b = 16, computed by hand-countable sums."""
    lengths = list(range(200, 2001))
    rep = paging.waste_report(lengths, 16)
    assert rep["n"] == 1801 and rep["mean_length"] == 1100
    # 1801 = 112 * 16 + 9 lengths.  Lengths 200..1991 form 112 runs of 16 consecutive
    # integers, each run covering every residue once: waste 0+1+...+15 = 120 per run.
    # The 9 lengths 1992..2000 have residues 8..15, 0: wastes 8,7,...,1,0 = 36.
    assert rep["waste"] == 112 * 120 + 36
    assert rep["mean_waste"] == Fraction(112 * 120 + 36, 1801)
    assert rep["utilisation_ratio_of_sums"] == Fraction(1100 * 1801, 1100 * 1801 + 112 * 120 + 36)
    # the two ratios the page says to keep apart do differ
    assert rep["utilisation_mean_of_ratios"] != rep["utilisation_ratio_of_sums"]
    assert abs(float(rep["utilisation_mean_of_ratios"]) - 0.990620) < 5e-7
    assert paging.reservation_utilisation(lengths, 4096) == Fraction(1100, 4096)


def test_logical_address_rejects_bad_input():
    with pytest.raises(ValueError):
        paging.logical_address(-1, 16)
    with pytest.raises(ValueError):
        paging.logical_address(3, 0)
    # divmod identity
    for t in range(200):
        j, o = paging.logical_address(t, 16)
        assert j * 16 + o == t and 0 <= o < 16
