"""The paged K/V pool as the kernels see it (oracle).

Source: transcript paragraph 3 (equal blocks anywhere in a shared pool, a
table per request) and "Inside vLLM and TGI", section "Block addresses and
fragmentation arithmetic" (block, offset addressing).

The pool is `num_blocks * b` slots; slot s is offset s % b of block s // b.
Each slot holds an opaque payload reference or None (never written: its
device bytes are whatever the pool was filled with).  Two operations change
it, mirroring the device side effects of the allocator:
  write(slot, payload)   one token's K and V rows for every KV head
  copy(src, dst)         every slot of block src into block dst (all b slots,
                         written or not)
and two move whole blocks to and from a host pool of the same shape
(swapping, transcript paragraph 5):
  swap_out(dev, host)    every slot of device block dev into host block host
  swap_in(host, dev)     every slot of host block host into device block dev
Values are resolved only when asked, in fp64, in the layout
[block][offset][kv head][dim] -- deliberately not the device layout.
"""
from __future__ import annotations

from typing import Any, Callable, Iterable, List, Optional, Sequence, Tuple

import numpy as np


class SlotPool:
    def __init__(self, num_blocks: int, width: int, host_blocks: int = 0):
        self.num_blocks = num_blocks
        self.width = width
        self.slots: List[Optional[Any]] = [None] * (num_blocks * width)
        self.host_blocks = host_blocks
        self.host: List[Optional[Any]] = [None] * (host_blocks * width)

    def write(self, slot: int, payload: Any) -> None:
        if slot < 0:
            return                                  # negative slot: nothing written
        self.slots[slot] = payload

    def copy(self, src: int, dst: int) -> None:
        b = self.width
        self.slots[dst * b:(dst + 1) * b] = self.slots[src * b:(src + 1) * b]

    def swap_out(self, dev: int, host: int) -> None:
        b = self.width
        self.host[host * b:(host + 1) * b] = self.slots[dev * b:(dev + 1) * b]

    def swap_in(self, host: int, dev: int) -> None:
        b = self.width
        self.slots[dev * b:(dev + 1) * b] = self.host[host * b:(host + 1) * b]

    def replay(self, events: Iterable[Tuple[str, int, Any]]) -> None:
        for kind, a, c in events:
            if kind == "write":
                self.write(a, c)
            elif kind == "copy":
                self.copy(a, c)
            elif kind == "swap_out":
                self.swap_out(a, c)
            elif kind == "swap_in":
                self.swap_in(a, c)
            else:
                raise ValueError(kind)

    def host_block_payloads(self, hb: int) -> List[Optional[Any]]:
        b = self.width
        return self.host[hb * b:(hb + 1) * b]

    def block_payloads(self, blk: int) -> List[Optional[Any]]:
        b = self.width
        return self.slots[blk * b:(blk + 1) * b]

    def materialize(self, resolve: Callable[[Any], Tuple[np.ndarray, np.ndarray]],
                    num_kv_heads: int, head_dim: int,
                    blocks: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
        """fp64 K, V of the listed blocks (all by default) as [n][b][Hkv][d]; NaN where unwritten."""
        blocks = range(self.num_blocks) if blocks is None else blocks
        blocks = list(blocks)
        shape = (len(blocks), self.width, num_kv_heads, head_dim)
        K = np.full(shape, np.nan)
        V = np.full(shape, np.nan)
        for i, blk in enumerate(blocks):
            for o, p in enumerate(self.block_payloads(blk)):
                if p is not None:
                    k, v = resolve(p)
                    K[i, o] = k
                    V[i, o] = v
        return K, V


def copy_batch_violations(pairs: Sequence[Tuple[int, int]], num_blocks: int) -> int:
    """Pairs of one batched block copy that break the batch's contract.

    Source: "Inside vLLM and TGI", section "Exact CPU block manager and
    copy-on-write" -- a copy-on-write fills a block just taken from the free
    list (never shared, never read in the same step) with the contents of the
    old block -- and transcript paragraph 4.  A batch of such copies issued
    at once has the meaning of the copies applied one after another only when
    no block is written twice and no written block is read: every destination
    distinct, and no destination also a source (its own pair's included).

    A pair with an id outside [0, num_blocks) is skipped by the copy and is
    not counted, nor does it take part in the checks of other pairs.  Among the
    remaining pairs, pair i counts once when its destination is the
    destination of another remaining pair, or the source of any remaining pair.
    """
    live = [(int(s), int(d)) for s, d in pairs
            if 0 <= int(s) < num_blocks and 0 <= int(d) < num_blocks]
    bad = 0
    for i, (_, di) in enumerate(live):
        dup = any(dj == di for j, (_, dj) in enumerate(live) if j != i)
        read = any(sj == di for sj, _ in live)
        bad += 1 if (dup or read) else 0
    return bad
