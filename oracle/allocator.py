"""Reference-counted block allocator with copy-on-write (oracle).
Test infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline use it.

Source: "Inside vLLM and TGI", section "Exact CPU block manager and
copy-on-write", and the polomodov.tech transcript, paragraphs 3-4.  Rules
this model keeps (restated from the prose, not from the page's listing):
  R1  the pool is `count` equal blocks of b token slots; free blocks wait in
      a list, a block is handed out from the END of that list and a block
      whose last reference goes away is put back at the end;
  R2  a block's reference count is the number of tables that list it;
  R3  token p of a sequence lives at offset p % b of the block its table
      lists at index p // b (section "Block addresses and fragmentation
      arithmetic");
  R4  growth: a token whose offset is 0 opens a new logical block, so a
      fresh block is appended to the table; otherwise the token goes into
      the block already listed there, and if that block is shared
      (count > 1) the sequence first receives a private copy of it (the
      shared block loses this sequence's reference) -- a shared block is
      read-only;
  R5  create = an empty table grown by the request's tokens in order (it
      needs ceil(T / b) fresh blocks; T = 0 is rejected); fork = a new
      table listing the same blocks (each count + 1); release = every block
      of the table loses one reference (in table order);
  R6  an operation that cannot get the blocks it needs fails with
      MemoryError and leaves no trace: tables, counts, free list, contents
      and the recorded device effects are exactly as before it;
  R7  after every operation: counts equal table occurrences, the free list
      holds each zero-count block once, every table's blocks except the
      last are full and the last holds 1..b tokens.
Swapping (transcript, paragraph 5: a sequence evicted when the pool runs
out has its K/V moved to CPU memory and brought back later; "Inside vLLM and
TGI", section "Read the vLLM0.11.0 scheduler": a swap moves the cache bytes
each way):
  S1  swap_out: each block of the table, in order, is copied to a fresh host
      block (host blocks have their own free list, handed out from its end),
      then the table is released as in R5;
  S2  swap_in: each host block of the sequence, in order, is copied into a
      fresh device block; the host blocks go back to the end of the host free
      list in table order; the sequence is live again with its old length.
  Reading (the pages are silent): each sequence is swapped on its own; a
  block it shared with a live sequence is copied out for it, and after
  swap-in it holds private copies (sharing is not restored).

Structure: every state change goes through a handful of journaled
primitives (claim a block, drop a reference, place a token, clone a block,
...), each of which records how to undo itself; a public operation runs
inside `_atomic()`, which rolls the journal back if the operation raises.
R6 therefore holds by construction, whatever step runs out of blocks.

The page's own model stores token ids; this one stores opaque payload
references (whatever the caller passes) and records the device side effects
each operation implies -- token writes by flat slot, whole-block copies and
swaps -- so that a pool can replay them.  Taking blocks from the END of the
free list is the first page's rule (the third page takes from the front; its
code is not followed).
"""
from __future__ import annotations

from collections import Counter
from contextlib import contextmanager
from typing import Any, Callable, Dict, List, Optional, Sequence, Tuple

# ("write", slot, payload) | ("copy", src, dst) | ("swap_out", dev, host) | ("swap_in", host, dev)
Event = Tuple[str, int, Any]


class BlockModel:
    def __init__(self, count: int, width: int, free_order: Optional[Sequence[int]] = None,
                 checked: bool = True, host_count: int = 0):
        if not isinstance(count, int) or not isinstance(width, int) or count < 1 or width < 1:
            raise ValueError("pool size and block width must be positive integers")
        self.width = width
        self.count = count
        self.free: List[int] = list(range(count) if free_order is None else free_order)
        if sorted(self.free) != list(range(count)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.refcount: List[int] = [0] * count
        self.contents: List[List[Any]] = [[] for _ in range(count)]   # tokens, by offset
        self.tables: Dict[Any, List[int]] = {}
        self.events: List[Event] = []
        self.checked = checked
        self.host_count = host_count
        self.host_free: List[int] = list(range(host_count))
        self.host_contents: List[List[Any]] = [[] for _ in range(host_count)]
        self.swapped: Dict[Any, List[int]] = {}          # name -> host blocks, in table order
        self._undo: List[Callable[[], None]] = []
        self._depth = 0

    # -- journal (R6) -----------------------------------------------------------
    @contextmanager
    def _atomic(self):
        mark = len(self._undo)
        self._depth += 1
        try:
            yield
        except BaseException:
            while len(self._undo) > mark:
                self._undo.pop()()
            raise
        finally:
            self._depth -= 1
        if self._depth == 0:
            self._undo.clear()
            if self.checked:
                self.check()

    def _record(self, kind: str, a: int, c: Any) -> None:
        self.events.append((kind, a, c))
        self._undo.append(self.events.pop)

    def _set_table(self, name: Any, table: Optional[List[int]]) -> None:
        """Bind `name` to `table` (None unbinds it)."""
        had = name in self.tables
        old = self.tables.get(name)
        if table is None:
            del self.tables[name]
        else:
            self.tables[name] = table

        def undo():
            if had:
                self.tables[name] = old
            else:
                self.tables.pop(name, None)
        self._undo.append(undo)

    def _set_entry(self, table: List[int], index: int, blk: int) -> None:
        """table[index] = blk, or append when index == len(table)."""
        if index == len(table):
            table.append(blk)
            self._undo.append(table.pop)
        else:
            old = table[index]
            table[index] = blk
            self._undo.append(lambda: table.__setitem__(index, old))

    # -- device blocks (R1, R2) ---------------------------------------------------
    def _claim(self) -> int:
        """A fresh block from the end of the free list, holding one reference."""
        if not self.free:
            raise MemoryError("no free device block")
        blk = self.free.pop()
        assert self.refcount[blk] == 0, "a listed free block is still referenced"
        stale = self.contents[blk]
        self.refcount[blk], self.contents[blk] = 1, []

        def undo():
            self.refcount[blk], self.contents[blk] = 0, stale
            self.free.append(blk)
        self._undo.append(undo)
        return blk

    def _add_ref(self, blk: int) -> None:
        self.refcount[blk] += 1
        self._undo.append(lambda: self.refcount.__setitem__(blk, self.refcount[blk] - 1))

    def _drop_ref(self, blk: int) -> None:
        """One reference fewer; a block nobody lists goes back to the free list's end."""
        self.refcount[blk] -= 1
        if self.refcount[blk] > 0:
            self._undo.append(lambda: self.refcount.__setitem__(blk, self.refcount[blk] + 1))
            return
        held = self.contents[blk]
        self.contents[blk] = []
        self.free.append(blk)

        def undo():
            assert self.free.pop() == blk
            self.contents[blk] = held
            self.refcount[blk] = 1
        self._undo.append(undo)

    def _place(self, blk: int, payload: Any) -> None:
        """Store a token at the next offset of a block; records the slot write."""
        offset = len(self.contents[blk])
        assert offset < self.width, "block overflow"
        self.contents[blk].append(payload)
        self._undo.append(self.contents[blk].pop)
        self._record("write", blk * self.width + offset, payload)

    def _fill(self, blk: int, tokens: List[Any]) -> None:
        """Replace a claimed block's tokens wholesale."""
        before = self.contents[blk]
        self.contents[blk] = tokens
        self._undo.append(lambda: self.contents.__setitem__(blk, before))

    def _clone(self, src: int, dst: int) -> None:
        """dst receives src's tokens (a whole-block device copy)."""
        self._fill(dst, list(self.contents[src]))
        self._record("copy", src, dst)

    # -- host blocks (S1, S2) -------------------------------------------------------
    def _claim_host(self) -> int:
        if not self.host_free:
            raise MemoryError("no free host block")
        hb = self.host_free.pop()
        self._undo.append(lambda: self.host_free.append(hb))
        return hb

    def _set_host(self, hb: int, tokens: List[Any]) -> None:
        before = self.host_contents[hb]
        self.host_contents[hb] = tokens
        self._undo.append(lambda: self.host_contents.__setitem__(hb, before))

    def _return_host(self, hb: int) -> None:
        self._set_host(hb, [])
        self.host_free.append(hb)
        self._undo.append(self.host_free.pop)

    def _set_swapped(self, name: Any, host_table: Optional[List[int]]) -> None:
        had = name in self.swapped
        old = self.swapped.get(name)
        if host_table is None:
            del self.swapped[name]
        else:
            self.swapped[name] = host_table

        def undo():
            if had:
                self.swapped[name] = old
            else:
                self.swapped.pop(name, None)
        self._undo.append(undo)

    # -- growth (R3, R4) -------------------------------------------------------------
    def _grow(self, name: Any, payload: Any) -> Optional[Tuple[int, int]]:
        table = self.tables[name]
        j, offset = divmod(self.length(name), self.width)
        copied = None
        if offset == 0:
            self._set_entry(table, j, self._claim())
        elif self.refcount[table[j]] > 1:
            shared = table[j]
            private = self._claim()
            self._clone(shared, private)
            self._set_entry(table, j, private)
            self._drop_ref(shared)
            copied = (shared, private)
        self._place(table[j], payload)
        return copied

    # -- operations (R5, S1, S2) ------------------------------------------------------
    def create(self, name: Any, payloads: Sequence[Any]) -> None:
        if name in self.tables or name in self.swapped or len(payloads) == 0:
            raise ValueError("name already in use, or no tokens")
        with self._atomic():
            self._set_table(name, [])
            for payload in payloads:
                self._grow(name, payload)

    def fork(self, src: Any, name: Any) -> None:
        if name in self.tables or name in self.swapped:
            raise ValueError("name already in use")
        with self._atomic():
            table = list(self.tables[src])
            for blk in table:
                self._add_ref(blk)
            self._set_table(name, table)

    def append(self, name: Any, payload: Any) -> Optional[Tuple[int, int]]:
        """Grow by one token; returns the (shared, private) block copy it made, if any."""
        with self._atomic():
            return self._grow(name, payload)

    def release(self, name: Any) -> None:
        with self._atomic():
            for blk in self.tables[name]:
                self._drop_ref(blk)
            self._set_table(name, None)

    def swap_out(self, name: Any) -> List[Tuple[int, int]]:
        """Move a live sequence to host blocks; returns its (device, host) copies."""
        with self._atomic():
            table = self.tables[name]
            host_table = []
            for blk in table:
                hb = self._claim_host()
                self._set_host(hb, list(self.contents[blk]))
                self._record("swap_out", blk, hb)
                host_table.append(hb)
            for blk in table:
                self._drop_ref(blk)
            self._set_table(name, None)
            self._set_swapped(name, host_table)
            return list(zip(table, host_table))

    def swap_in(self, name: Any) -> List[Tuple[int, int]]:
        """Bring a swapped sequence back into fresh device blocks; returns its
        (host, device) copies."""
        if name in self.tables:
            raise ValueError("name already live")
        with self._atomic():
            host_table = self.swapped[name]
            table = []
            for hb in host_table:
                blk = self._claim()
                self._fill(blk, list(self.host_contents[hb]))
                self._record("swap_in", hb, blk)
                table.append(blk)
            for hb in host_table:
                self._return_host(hb)
            self._set_swapped(name, None)
            self._set_table(name, table)
            return list(zip(host_table, table))

    # -- views ------------------------------------------------------------------------
    def read(self, name: Any) -> List[Any]:
        """Payloads of a table in logical order (walks the table)."""
        return [p for blk in self.tables[name] for p in self.contents[blk]]

    def length(self, name: Any) -> int:
        """Tokens held: every block but the last is full (R7)."""
        table = self.tables[name]
        return (len(table) - 1) * self.width + len(self.contents[table[-1]]) if table else 0

    # -- invariant (R7) -------------------------------------------------------------------
    def check(self) -> None:
        listed = Counter(blk for table in self.tables.values() for blk in table)
        for blk in range(self.count):
            assert self.refcount[blk] == listed[blk], f"refcount of block {blk}"
        assert sorted(self.free) == [b for b in range(self.count) if listed[b] == 0], "free list"
        for name, table in self.tables.items():
            fills = [len(self.contents[blk]) for blk in table]
            assert table and all(f == self.width for f in fills[:-1]), f"gap in {name!r}"
            assert 1 <= fills[-1] <= self.width, f"last block of {name!r}"
        parked = [hb for t in self.swapped.values() for hb in t]
        assert sorted(parked + self.host_free) == list(range(self.host_count)), "host blocks"
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
