"""Host-side block manager: tables, reference counts, growth and copy-on-write.

Behaviour follows "Inside vLLM and TGI: Paging, Versioned Schedulers and
Operations", section "Exact CPU block manager and copy-on-write", and the
"vLLM and PagedAttention" transcript, paragraphs 3-4:
  * blocks are taken from the end of the free list and freed blocks are
    appended to it;
  * a request of T tokens holds ceil(T / b) blocks; growth takes a block only
    when the last one is full;
  * forks share every block (reference counts); appending to a shared,
    partially filled last block first copies it to a fresh block;
  * admission and growth fail with MemoryError before any change when no
    block is free;
  * swapping (transcript, paragraph 5): a live sequence moves to host blocks
    (its own free list, taken at the end) and its device blocks are released;
    swapping in takes fresh device blocks for every host block and returns the
    host blocks in table order; both fail before any change without space.
The manager keeps only counts (token contents live in the device pool) and
reports the device work each operation implies: token writes by slot and
block copies, which `paged_cache.PagedKV` turns into pa_write_kv and
pa_copy_blocks calls, and (device, host) block pairs for pa_swap_blocks.
"""
from __future__ import annotations

from typing import Dict, Hashable, List, Optional, Sequence, Tuple

import numpy as np


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order: Optional[Sequence[int]] = None, host_blocks: int = 0):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.b = block_size
        self.refs = np.zeros(num_blocks, dtype=np.int64)
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if len(order) != num_blocks or len(set(order)) != num_blocks or \
                min(order) < 0 or max(order) >= num_blocks:
            raise ValueError("free_order must be a permutation of the block ids")
        self.free: List[int] = order
        self.tables: Dict[Hashable, List[int]] = {}
        self.lengths: Dict[Hashable, int] = {}
        self.host_blocks = host_blocks
        self.host_free: List[int] = list(range(host_blocks))
        self.swapped: Dict[Hashable, List[int]] = {}

    # -- helpers ------------------------------------------------------------
    def _take(self) -> int:
        blk = self.free.pop()
        self.refs[blk] = 1
        return blk

    def _drop(self, blk: int) -> None:
        self.refs[blk] -= 1
        if self.refs[blk] == 0:
            self.free.append(blk)

    def slot(self, name: Hashable, pos: int) -> int:
        t = self.tables[name]
        return t[pos // self.b] * self.b + pos % self.b

    # -- operations -------------------------------------------------------------
    def create(self, name: Hashable, num_tokens: int) -> List[int]:
        """Admit a request with `num_tokens` tokens; returns the slots to write, in order."""
        if name in self.tables or num_tokens < 1:
            raise ValueError("duplicate name or empty request")
        need = (num_tokens + self.b - 1) // self.b
        if need > len(self.free):
            raise MemoryError("pool full")
        table = [self._take() for _ in range(need)]
        self.tables[name] = table
        self.lengths[name] = num_tokens
        arr = np.asarray(table, dtype=np.int64)
        pos = np.arange(num_tokens, dtype=np.int64)
        return list(arr[pos // self.b] * self.b + pos % self.b)

    def fork(self, src: Hashable, name: Hashable) -> None:
        if name in self.tables:
            raise ValueError("duplicate name")
        table = list(self.tables[src])
        for blk in table:
            self.refs[blk] += 1
        self.tables[name] = table
        self.lengths[name] = self.lengths[src]

    def append(self, name: Hashable) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Grow by one token.  Returns (slot of the new token, (src, dst) copy or None)."""
        table = self.tables[name]
        n = self.lengths[name]
        fill = n - (len(table) - 1) * self.b          # tokens in the last block
        last = table[-1]
        full = fill == self.b
        shared_partial = (not full) and self.refs[last] > 1
        if (full or shared_partial) and not self.free:
            raise MemoryError("no free block")
        copy = None
        if full:
            table.append(self._take())
        elif shared_partial:
            dst = self._take()
            self._drop(last)
            table[-1] = dst
            copy = (last, dst)
        self.lengths[name] = n + 1
        return self.slot(name, n), copy

    def release(self, name: Hashable) -> None:
        for blk in self.tables.pop(name):
            self._drop(blk)
        del self.lengths[name]

    def swap_out(self, name: Hashable) -> List[Tuple[int, int]]:
        """Evict a live sequence to host blocks; returns the (device, host) block
        pairs to copy before the device blocks are reused."""
        table = self.tables[name]
        if len(table) > len(self.host_free):
            raise MemoryError("host swap space full")
        host = [self.host_free.pop() for _ in table]
        for blk in self.tables.pop(name):
            self._drop(blk)
        self.swapped[name] = host
        return list(zip(table, host))

    def swap_in(self, name: Hashable) -> List[Tuple[int, int]]:
        """Restore a swapped sequence; returns the (host, device) block pairs to copy."""
        host = self.swapped[name]
        if name in self.tables:
            raise ValueError("duplicate name")
        if len(host) > len(self.free):
            raise MemoryError("pool full")
        table = [self._take() for _ in host]
        self.host_free.extend(host)
        del self.swapped[name]
        self.tables[name] = table
        return list(zip(host, table))

    # -- device views ---------------------------------------------------------
    def table_array(self, names: Sequence[Hashable], width: Optional[int] = None,
                    pad: int = 0x7FFFFFFF) -> np.ndarray:
        """int32 [len(names)][width] block tables, entries past each table = pad."""
        if width is None:
            width = max((len(self.tables[n]) for n in names), default=1)
        out = np.full((len(names), max(width, 1)), pad, dtype=np.int32)
        for i, n in enumerate(names):
            t = self.tables[n]
            if len(t) > width:
                raise ValueError("table wider than the requested width")
            out[i, :len(t)] = t
        return out

    def length_array(self, names: Sequence[Hashable]) -> np.ndarray:
        return np.asarray([self.lengths[n] for n in names], dtype=np.int32)

    def check(self) -> None:
        """Structural invariant: counts equal table occurrences; free = zero-count set."""
        counts = np.zeros(self.num_blocks, dtype=np.int64)
        for t in self.tables.values():
            np.add.at(counts, np.asarray(t, dtype=np.int64), 1)
        assert np.array_equal(counts, self.refs)
        assert len(set(self.free)) == len(self.free)
        assert set(self.free) == set(np.nonzero(self.refs == 0)[0].tolist())
        for name, t in self.tables.items():
            assert len(t) == (self.lengths[name] + self.b - 1) // self.b
        held = [hb for t in self.swapped.values() for hb in t]
        assert sorted(held + self.host_free) == list(range(self.host_blocks))
        for name, t in self.swapped.items():
            assert len(t) == (self.lengths[name] + self.b - 1) // self.b
