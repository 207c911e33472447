"""Device-side paged KV cache and a driver that builds a decode batch.

`PagedKV` owns the two pools (torch allocations, laid out as `include/pa.h`
specifies) and issues pa_write_kv / pa_copy_blocks.  `build_batch` replays a
workload's allocator script with the host `BlockManager`, turning each
operation's device work into batched library calls in an order that keeps
copy-on-write correct (a copy runs after every earlier write to its source
block and before every later write to its source or destination), then
uploads tables, lengths and queries.  `DecodeStep` is one decode iteration
over the batch: slot mapping and write of each sequence's current token,
then decode attention.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

from . import binding as B
from .blocks import BlockManager
from .workloads import (APPEND, CREATE, DTYPES, FORK, RELEASE, SWAP_IN, SWAP_OUT, TABLE_PAD,
                        Workload)

class PagedKV:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str,
                 device: str = "cuda", poison: bool = True, block_size: int = 16,
                 host_blocks: int = 0, kv_scales=None):
        # FP8 pools: per-KV-head scales live on the device beside the pools
        self.k_scales = self.v_scales = None
        if dtype == "fp8":
            ks, vs = kv_scales
            self.k_scales = torch.tensor(ks, dtype=torch.float32, device=device)
            self.v_scales = torch.tensor(vs, dtype=torch.float32, device=device)
        self.desc = B.make_desc(num_blocks, num_kv_heads, head_dim, dtype, block_size,
                                self.k_scales, self.v_scales)
        self.dtype = dtype
        self.block_size = block_size
        elems = num_blocks * num_kv_heads * block_size * head_dim
        self.k = torch.empty(elems, dtype=DTYPES[dtype], device=device)
        self.v = torch.empty(elems, dtype=DTYPES[dtype], device=device)
        nan = 0x7F if dtype == "fp8" else float("nan")     # the E4M3 NaN code
        if poison:                                   # stale/unused slots read as NaN
            self.k.fill_(nan)
            self.v.fill_(nan)
        # host swap space: pinned (page-locked) memory in the same block layout
        self.host_blocks = host_blocks
        helems = host_blocks * num_kv_heads * block_size * head_dim
        self.host_k = torch.empty(helems, dtype=DTYPES[dtype], pin_memory=host_blocks > 0)
        self.host_v = torch.empty(helems, dtype=DTYPES[dtype], pin_memory=host_blocks > 0)
        if poison:
            self.host_k.fill_(nan)
            self.host_v.fill_(nan)

    @property
    def num_blocks(self) -> int:
        return self.desc.num_blocks

    def write(self, k_new: torch.Tensor, v_new: torch.Tensor, slots: torch.Tensor) -> None:
        B.write_kv_t(self.desc, self.k, self.v, k_new, v_new, slots)

    def copy(self, pairs: torch.Tensor) -> None:
        B.copy_blocks_t(self.desc, self.k, self.v, pairs)

    def swap(self, pairs: torch.Tensor, direction: int) -> None:
        """(src, dst) block pairs: device -> host (B.PA_SWAP_OUT) or host -> device."""
        B.swap_blocks_t(self.desc, self.k, self.v, self.host_k, self.host_v, self.host_blocks,
                        pairs, direction)


@dataclass
class Batch:
    w: Workload
    kv: PagedKV
    bm: BlockManager
    tables: torch.Tensor          # int32 [S][M] (device)
    lens: torch.Tensor            # int32 [S]    (device)
    q: torch.Tensor               # [S][Hq][D]   (device, pool dtype)
    max_len: int
    last_payload: Dict[int, Tuple[int, int]]
    step_k: torch.Tensor          # [S][Hkv][D] current token's K per sequence (host)
    step_v: torch.Tensor
    copies: List[Tuple[int, int]]
    write_calls: int
    copy_calls: int


class _Flusher:
    """Accumulates writes and copies; flushes copies first, then writes.

    A flush happens before a copy whose source has a pending write or is a
    pending copy's destination, and before a second write to a pending slot,
    so every batched call is order-independent."""

    def __init__(self, w: Workload, kv: PagedKV, device: str, max_tokens: int = 1 << 16):
        self.w, self.kv, self.device, self.max_tokens = w, kv, device, max_tokens
        self.writes: List[Tuple[int, int, int]] = []      # (slot, key, row)
        self.write_slots = set()
        self.write_blocks = set()
        self.pairs: List[Tuple[int, int]] = []
        self.copy_dsts = set()
        self.write_calls = 0
        self.copy_calls = 0
        self.swap_calls = 0

    def add_write(self, slot: int, key: int, row: int) -> None:
        # one call must not write a slot twice (which write lands is unspecified)
        if slot in self.write_slots:
            self.flush()
        self.writes.append((slot, key, row))
        self.write_slots.add(slot)
        self.write_blocks.add(slot // self.kv.block_size)

    def add_copy(self, src: int, dst: int) -> None:
        # copies run before writes: flush first when the copy reads a block with
        # pending writes or another copy's output, or overwrites a block that
        # pending writes (an earlier tenant's) would land in afterwards
        if src in self.write_blocks or src in self.copy_dsts or dst in self.write_blocks:
            self.flush()
        self.pairs.append((src, dst))
        self.copy_dsts.add(dst)

    def swap(self, pairs: List[Tuple[int, int]], direction: int) -> None:
        """Swaps are issued at once, in order, after everything pending."""
        self.flush()
        if pairs:
            self.kv.swap(torch.tensor(pairs, dtype=torch.int32).to(self.device), direction)
            self.swap_calls += 1

    def flush(self) -> None:
        if self.pairs:
            pairs = torch.tensor(self.pairs, dtype=torch.int32).to(self.device)
            self.kv.copy(pairs)
            self.copy_calls += 1
        for a in range(0, len(self.writes), self.max_tokens):
            chunk = self.writes[a:a + self.max_tokens]
            self._write_chunk(chunk)
        self.writes, self.write_slots, self.write_blocks = [], set(), set()
        self.pairs, self.copy_dsts = [], set()

    def _write_chunk(self, chunk) -> None:
        arr = np.asarray(chunk, dtype=np.int64)
        slots, keys, rows = arr[:, 0], arr[:, 1], arr[:, 2]
        order = np.argsort(keys, kind="stable")
        ks, vs, ss = [], [], []
        for key in np.unique(keys):
            sel = order[keys[order] == key]
            k, v = self.w.kv(int(key))
            idx = torch.from_numpy(rows[sel])
            ks.append(k.index_select(0, idx))
            vs.append(v.index_select(0, idx))
            ss.append(slots[sel])
        k_new = torch.cat(ks).to(self.device)
        v_new = torch.cat(vs).to(self.device)
        sl = torch.from_numpy(np.concatenate(ss).astype(np.int32)).to(self.device)
        self.kv.write(k_new, v_new, sl)
        self.write_calls += 1


def build_batch(w: Workload, device: str = "cuda", poison: bool = True,
                table_width: Optional[int] = None, drop_payload_cache: bool = True) -> Batch:
    kv = PagedKV(w.num_blocks, w.num_kv_heads, w.head_dim, w.dtype, device, poison, w.block_size,
                 w.host_blocks, w.kv_scales() if w.dtype == "fp8" else None)
    bm = BlockManager(w.num_blocks, w.block_size, w.free_order, host_blocks=w.host_blocks)
    fl = _Flusher(w, kv, device)
    last: Dict[int, Tuple[int, int]] = {}
    copies: List[Tuple[int, int]] = []
    for op in w.ops:
        if op.kind == CREATE:
            for r, s in enumerate(bm.create(op.name, op.count)):
                fl.add_write(int(s), op.key, r)
            last[op.name] = (op.key, op.count - 1)
        elif op.kind == FORK:
            bm.fork(op.src, op.name)
            last[op.name] = last[op.src]
        elif op.kind == APPEND:
            s, cp = bm.append(op.name)
            if cp is not None:
                fl.add_copy(*cp)
                copies.append(cp)
            fl.add_write(int(s), op.key, op.index)
            last[op.name] = (op.key, op.index)
        elif op.kind == RELEASE:
            bm.release(op.name)
        elif op.kind == SWAP_OUT:
            fl.swap(bm.swap_out(op.name), B.PA_SWAP_OUT)
        elif op.kind == SWAP_IN:
            fl.swap(bm.swap_in(op.name), B.PA_SWAP_IN)
        else:
            raise ValueError(op.kind)
    fl.flush()
    names = w.seq_names
    tab = bm.table_array(names, width=table_width, pad=TABLE_PAD)
    lens = bm.length_array(names)
    q = w.queries().to(device)
    shape = (len(names), w.num_kv_heads, w.head_dim)
    step_k = torch.empty(shape, dtype=DTYPES[w.input_dtype])
    step_v = torch.empty(shape, dtype=DTYPES[w.input_dtype])
    for i, n in enumerate(names):
        key, row = last[n]
        k, v = w.kv(key)
        step_k[i], step_v[i] = k[row], v[row]
    if drop_payload_cache:
        w.drop_cache()
    return Batch(w=w, kv=kv, bm=bm, tables=torch.from_numpy(tab).to(device),
                 lens=torch.from_numpy(lens).to(device), q=q,
                 max_len=int(lens.max()) if len(lens) else 0, last_payload=last,
                 step_k=step_k, step_v=step_v, copies=copies,
                 write_calls=fl.write_calls, copy_calls=fl.copy_calls)


class DecodeStep:
    """One decode iteration over a batch: write every sequence's current token
    (position L - 1) and attend.  fused=True issues pa_decode_step (one launch);
    fused=False issues pa_slot_mapping, pa_write_kv and pa_decode_attention."""

    def __init__(self, batch: Batch, partition_size: int = 0, out_dtype=torch.float32,
                 fused: bool = True):
        self.b = batch
        self.fused = fused
        w = batch.w
        dev = batch.q.device
        S = w.num_seqs
        self.partition_size = partition_size
        self.seq_ids = torch.arange(S, dtype=torch.int32, device=dev)
        pos = batch.bm.length_array(w.seq_names) - 1
        self.positions = torch.from_numpy(pos.astype(np.int32)).to(dev)
        self.slots = torch.empty(S, dtype=torch.int32, device=dev)
        self.k_new = batch.step_k.to(dev)
        self.v_new = batch.step_v.to(dev)
        # NaN until a launch writes it: a row no kernel writes cannot pass for a result
        self.out = torch.full((S, w.num_q_heads, w.head_dim), float("nan"), dtype=out_dtype,
                              device=dev)
        nbytes = B.workspace_size(batch.kv.desc, S, w.num_q_heads, batch.max_len, partition_size)
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)

    def write_current(self) -> None:
        B.slot_mapping_t(self.b.tables, self.seq_ids, self.positions, self.slots,
                         self.b.kv.block_size)
        self.b.kv.write(self.k_new, self.v_new, self.slots)

    def attend(self) -> None:
        b = self.b
        B.decode_attention_t(b.kv.desc, b.kv.k, b.kv.v, b.q, self.out, b.tables, b.lens,
                             b.w.scale, b.max_len, self.partition_size, self.workspace)

    def fused_step(self) -> None:
        b = self.b
        B.decode_step_t(b.kv.desc, b.kv.k, b.kv.v, self.k_new, self.v_new, b.q, self.out,
                        b.tables, b.lens, b.w.scale, b.max_len, self.partition_size,
                        self.workspace)

    def __call__(self) -> torch.Tensor:
        if self.fused:
            self.fused_step()
        else:
            self.write_current()
            self.attend()
        return self.out


class PrefillStep:
    """One multi-token step over a batch built from a chunked workload: write
    every chunk's K/V (pa_slot_mapping + pa_write_kv), then pa_prefill_attention."""

    def __init__(self, batch: Batch, out_dtype=torch.float32):
        self.b = batch
        w = batch.w
        if w.chunk_lens is None:
            raise ValueError("workload has no chunks")
        dev = batch.q.device
        lens = batch.bm.length_array(w.seq_names).astype(np.int64)
        chunk = np.asarray(w.chunk_lens, dtype=np.int64)
        starts = np.concatenate([[0], np.cumsum(chunk)])
        self.max_chunk = int(chunk.max()) if len(chunk) else 0
        self.q = w.chunk_queries().to(dev)
        self.q_start = torch.from_numpy(starts.astype(np.int32)).to(dev)
        seq = np.repeat(np.arange(w.num_seqs), chunk)
        pos = np.concatenate([np.arange(L - n, L) for L, n in zip(lens, chunk)]) if len(chunk) \
            else np.zeros(0, dtype=np.int64)
        self.seq_ids = torch.from_numpy(seq.astype(np.int32)).to(dev)
        self.positions = torch.from_numpy(pos.astype(np.int32)).to(dev)
        self.slots = torch.empty(len(pos), dtype=torch.int32, device=dev)
        ks, vs = [], []
        for name, L, n in zip(w.seq_names, lens, chunk):     # chunk rows: payload key = name
            k, v = w.kv(name)
            ks.append(k[L - n:L])
            vs.append(v[L - n:L])
        self.k_new = torch.cat(ks).to(dev)
        self.v_new = torch.cat(vs).to(dev)
        self.out = torch.full(self.q.shape, float("nan"), dtype=out_dtype, device=dev)

    def write_chunks(self) -> None:
        B.slot_mapping_t(self.b.tables, self.seq_ids, self.positions, self.slots,
                         self.b.kv.block_size)
        self.b.kv.write(self.k_new, self.v_new, self.slots)

    def attend(self) -> None:
        b = self.b
        B.prefill_attention_t(b.kv.desc, b.kv.k, b.kv.v, self.q, self.out, self.q_start,
                              b.tables, b.lens, b.w.scale, self.max_chunk, b.max_len)

    def __call__(self) -> torch.Tensor:
        self.write_chunks()
        self.attend()
        return self.out
