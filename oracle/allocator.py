"""Reference-counted block allocator with copy-on-write (oracle).

Source: "Inside vLLM and TGI", section "Exact CPU block manager and
copy-on-write", and the polomodov.tech transcript, paragraphs 3-4.  The
behaviour restated here:
  * a pool of `count` equal blocks of width b; a free list from which blocks
    are taken at its end and to which freed blocks are appended;
  * every block has a reference count = number of tables that list it;
  * create: a non-empty request gets ceil(T / b) fresh blocks filled in token
    order; if fewer blocks are free, it fails with MemoryError before any
    change (atomic admission);
  * fork: a new table listing the same blocks; each block's count rises by 1;
  * append: if the last block is full a fresh block is added; if it is not
    full but shared (count > 1) it is first copied into a fresh block, the old
    block loses one reference and the table points at the copy; either case
    fails with MemoryError, leaving everything unchanged, when no block is
    free; then the token goes into the (now private) last block;
  * release: every block of the table loses one reference; at zero it is
    emptied and returned to the free list;
  * structural invariant after every operation: counts equal table
    occurrences, the free list has no duplicates and equals the zero-count
    set, every non-last block of a table is full and the last one holds
    1..b tokens.
Swapping (transcript, paragraph 5: when the pool is empty a whole sequence
is evicted, its K/V moved to CPU memory and restored later; "Inside vLLM and
TGI", section "Read the vLLM0.11.0 scheduler": host swap costs the cache
bytes in both directions):
  * swap_out: every block of the table is copied to a fresh HOST block (host
    blocks come from their own free list, taken at its end), then the table
    is released as by `release`; fails with MemoryError before any change
    when too few host blocks are free;
  * swap_in: every host block of the sequence is copied into a fresh device
    block (atomic: MemoryError before any change when too few are free), the
    host blocks return to the end of the host free list in table order, and
    the sequence is live again with its old length.
Reading (the pages are silent): each sequence is swapped on its own; a block
it shared with another live sequence is copied out for it, and after swap-in
it holds private copies (sharing is not restored).

The page's own model stores token ids; this one stores opaque payload
references (whatever the caller passes), and additionally records the device
side effects each operation implies -- token writes by flat slot and
whole-block copies -- so that a pool can replay them.

Readings (the pages are silent): taking from the END of the free list is
the first page's rule (the third page takes from the front; its code is not
followed).  Slot = physical block * b + offset names one pool position.
"""
from __future__ import annotations

from collections import Counter
from typing import Any, Dict, List, Optional, Sequence, Tuple

# ("write", slot, payload) | ("copy", src, dst) | ("swap_out", dev, host) | ("swap_in", host, dev)
Event = Tuple[str, int, Any]


class BlockModel:
    def __init__(self, count: int, width: int, free_order: Optional[Sequence[int]] = None,
                 checked: bool = True, host_count: int = 0):
        if not isinstance(count, int) or not isinstance(width, int) or count < 1 or width < 1:
            raise ValueError("pool size and block width must be positive integers")
        self.width = width
        self.count = count
        self.contents: List[List[Any]] = [[] for _ in range(count)]
        self.refcount: List[int] = [0] * count
        if free_order is None:
            free_order = range(count)
        self.free: List[int] = list(free_order)
        if sorted(self.free) != list(range(count)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.tables: Dict[Any, List[int]] = {}
        self.events: List[Event] = []
        self.checked = checked
        self.host_count = host_count
        self.host_contents: List[List[Any]] = [[] for _ in range(host_count)]
        self.host_free: List[int] = list(range(host_count))
        self.swapped: Dict[Any, List[int]] = {}          # name -> host blocks, in table order

    # -- block ownership ---------------------------------------------------
    def _fresh_block(self) -> int:
        blk = self.free.pop()                 # the end of the free list
        assert self.refcount[blk] == 0
        self.refcount[blk] = 1
        self.contents[blk] = []
        return blk

    def _unref(self, blk: int) -> None:
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            self.contents[blk] = []
            self.free.append(blk)

    def _put(self, blk: int, payload: Any) -> None:
        offset = len(self.contents[blk])
        self.contents[blk].append(payload)
        self.events.append(("write", blk * self.width + offset, payload))

    # -- operations ----------------------------------------------------------
    def create(self, name: Any, payloads: Sequence[Any]) -> None:
        if name in self.tables or len(payloads) == 0:
            raise ValueError("name already live, or no tokens")
        want = -(-len(payloads) // self.width)
        if want > len(self.free):
            raise MemoryError("pool full")
        table: List[int] = []
        for pos, payload in enumerate(payloads):
            if pos % self.width == 0:
                table.append(self._fresh_block())
            self._put(table[-1], payload)
        self.tables[name] = table
        self._verify()

    def fork(self, src: Any, name: Any) -> None:
        if name in self.tables:
            raise ValueError("name already live")
        table = list(self.tables[src])
        for blk in table:
            self.refcount[blk] += 1
        self.tables[name] = table
        self._verify()

    def append(self, name: Any, payload: Any) -> Optional[Tuple[int, int]]:
        """Grow by one token; returns the (src, dst) block copy it made, if any."""
        table = self.tables[name]
        last = table[-1]
        is_full = len(self.contents[last]) == self.width
        is_shared_partial = (not is_full) and self.refcount[last] > 1
        if (is_full or is_shared_partial) and not self.free:
            raise MemoryError("no free block for growth or copy")
        copied = None
        if is_full:
            table.append(self._fresh_block())
        elif is_shared_partial:
            dst = self._fresh_block()
            self.contents[dst] = list(self.contents[last])
            self.events.append(("copy", last, dst))
            self._unref(last)
            table[-1] = dst
            copied = (last, dst)
        self._put(table[-1], payload)
        self._verify()
        return copied

    def release(self, name: Any) -> None:
        for blk in self.tables.pop(name):
            self._unref(blk)
        self._verify()

    def swap_out(self, name: Any) -> List[Tuple[int, int]]:
        """Move a live sequence to host blocks; returns its (device, host) copies."""
        table = self.tables[name]
        if len(table) > len(self.host_free):
            raise MemoryError("host swap space full")
        pairs = []
        host_table = []
        for blk in table:
            hb = self.host_free.pop()
            self.host_contents[hb] = list(self.contents[blk])
            self.events.append(("swap_out", blk, hb))
            pairs.append((blk, hb))
            host_table.append(hb)
        for blk in self.tables.pop(name):
            self._unref(blk)
        self.swapped[name] = host_table
        self._verify()
        return pairs

    def swap_in(self, name: Any) -> List[Tuple[int, int]]:
        """Bring a swapped sequence back into fresh device blocks; returns its
        (host, device) copies."""
        host_table = self.swapped[name]
        if name in self.tables:
            raise ValueError("name already live")
        if len(host_table) > len(self.free):
            raise MemoryError("pool full")
        table, pairs = [], []
        for hb in host_table:
            blk = self._fresh_block()
            self.contents[blk] = list(self.host_contents[hb])
            self.events.append(("swap_in", hb, blk))
            pairs.append((hb, blk))
            table.append(blk)
        for hb in host_table:
            self.host_contents[hb] = []
            self.host_free.append(hb)
        del self.swapped[name]
        self.tables[name] = table
        self._verify()
        return pairs

    # -- views ---------------------------------------------------------------
    def read(self, name: Any) -> List[Any]:
        """Payloads of a table in logical order (walks the table)."""
        return [p for blk in self.tables[name] for p in self.contents[blk]]

    def length(self, name: Any) -> int:
        table = self.tables[name]
        return (len(table) - 1) * self.width + len(self.contents[table[-1]])

    # -- invariant -----------------------------------------------------------
    def _verify(self) -> None:
        if self.checked:
            self.check()

    def check(self) -> None:
        seen = Counter(blk for table in self.tables.values() for blk in table)
        assert all(self.refcount[i] == seen.get(i, 0) for i in range(self.count)), "refcounts"
        assert len(set(self.free)) == len(self.free), "duplicate free id"
        assert set(self.free) == {i for i in range(self.count) if self.refcount[i] == 0}, "free set"
        for table in self.tables.values():
            assert all(len(self.contents[blk]) == self.width for blk in table[:-1]), "gap"
            assert 1 <= len(self.contents[table[-1]]) <= self.width, "last block fill"
        held = [hb for t in self.swapped.values() for hb in t]
        assert len(set(self.host_free)) == len(self.host_free), "duplicate host free id"
        assert sorted(held + self.host_free) == list(range(self.host_count)), "host blocks"
        assert not set(self.swapped) & set(self.tables), "swapped and live"


def run_script(ops, num_blocks: int, width: int, free_order: Sequence[int],
               checked: bool = True, host_blocks: int = 0) -> BlockModel:
    """Replay an op script.  Each op has .kind in {create, fork, append, release,
    swap_out, swap_in}, .name, and for create .count/.key (payload rows
    (key, 0..count-1)), for fork .src, for append .key/.index (payload (key, index))."""
    model = BlockModel(num_blocks, width, free_order, checked=checked, host_count=host_blocks)
    for op in ops:
        if op.kind == "create":
            model.create(op.name, [(op.key, r) for r in range(op.count)])
        elif op.kind == "fork":
            model.fork(op.src, op.name)
        elif op.kind == "append":
            model.append(op.name, (op.key, op.index))
        elif op.kind == "release":
            model.release(op.name)
        elif op.kind == "swap_out":
            model.swap_out(op.name)
        elif op.kind == "swap_in":
            model.swap_in(op.name)
        else:
            raise ValueError(op.kind)
    return model
