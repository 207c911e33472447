"""Address translation and waste arithmetic (oracle).

Source: "Inside vLLM and TGI: Paging, Versioned Schedulers and Operations",
section "Block addresses and fragmentation arithmetic":
  * position t of a request maps to logical block t // b, offset t % b,
    and physical block table[t // b];
  * a request of T tokens occupies ceil(T / b) blocks, b * ceil(T / b)
    slots; its waste is (-T) mod b, in [0, b - 1]; the total over requests is
    below b times the number of non-empty requests;
  * a max-reservation allocator uses N * T_max slots instead.
The slot index (physical block * b + offset) is the flat position of a token
in the pool when blocks are numbered in order; the pages give the parts, the
flat form is the plainest way to name one slot.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Dict, Iterable, Sequence, Tuple


def logical_address(t: int, b: int) -> Tuple[int, int]:
    """(logical block, offset) of zero-based position t with block width b."""
    if t < 0 or b < 1:
        raise ValueError("position must be >= 0 and block width >= 1")
    return t // b, t % b


def physical_block(table: Sequence[int], t: int, b: int) -> int:
    """Physical block holding position t: table[logical block]."""
    j, _ = logical_address(t, b)
    return table[j]


def slot(table: Sequence[int], t: int, b: int) -> int:
    """Flat pool slot of position t: physical block * b + offset."""
    j, o = logical_address(t, b)
    return table[j] * b + o


def blocks_needed(T: int, b: int) -> int:
    """Blocks a T-token request occupies: ceil(T / b) (0 for T = 0)."""
    return -(-T // b)


def allocated_slots(T: int, b: int) -> int:
    return b * blocks_needed(T, b)


def tail_waste(T: int, b: int) -> int:
    """Unused slots of the last block: (-T) mod b."""
    return (-T) % b


def waste_report(lengths: Iterable[int], b: int) -> Dict[str, Fraction]:
    """Exact (rational) capacity figures for a set of live lengths.

    used / allocated is the ratio of sums (equivalently of means); the mean
    of per-request ratios is reported separately, since the page asks which
    one is meant and notes they differ.
    """
    L = [int(x) for x in lengths]
    n = len(L)
    used = sum(L)
    alloc = sum(allocated_slots(x, b) for x in L)
    waste = sum(tail_waste(x, b) for x in L)
    return {
        "n": Fraction(n),
        "used": Fraction(used),
        "allocated": Fraction(alloc),
        "waste": Fraction(waste),
        "mean_length": Fraction(used, n),
        "mean_waste": Fraction(waste, n),
        "utilisation_ratio_of_sums": Fraction(used, alloc),
        "utilisation_mean_of_ratios": sum(Fraction(x, allocated_slots(x, b)) for x in L) / n,
    }


def reservation_utilisation(lengths: Iterable[int], reserve: int) -> Fraction:
    """Used fraction when every request reserves `reserve` slots (N * T_max)."""
    L = [int(x) for x in lengths]
    return Fraction(sum(L), reserve * len(L))
