"""Glue that feeds a seeded workload to the oracle (test-side only).

The oracle receives only what the workload generator produced: the op
script, the free list and the payload values (upcast exactly to fp64).
"""
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

from oracle.allocator import BlockModel, run_script
from oracle.pool import SlotPool
from oracle import attention as OA
from oracle import prefill as OPF


class OracleRun:
    def __init__(self, w, checked: bool = False):
        self.w = w
        self.model: BlockModel = run_script(w.ops, w.num_blocks, w.block_size, w.free_order,
                                            checked=checked, host_blocks=w.host_blocks)
        self.pool = SlotPool(w.num_blocks, w.block_size, w.host_blocks)
        self.pool.replay(self.model.events)
        self._f64: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}

    def resolve(self, payload):
        key, row = payload
        if key not in self._f64:
            k, v = self.w.kv(key)
            self._f64[key] = (k.to(torch.float64).numpy(), v.to(torch.float64).numpy())
        k, v = self._f64[key]
        return k[row], v[row]

    @property
    def tables(self):
        return [self.model.tables[n] for n in self.w.seq_names]

    @property
    def lengths(self):
        return [self.model.length(n) for n in self.w.seq_names]

    def q64(self) -> np.ndarray:
        return self.w.queries().to(torch.float64).numpy()

    def decode(self, rows: Optional[Sequence[int]] = None, q: Optional[np.ndarray] = None):
        q = self.q64() if q is None else q
        return OA.paged_decode(self.pool, self.resolve, self.tables, self.lengths, q,
                               self.w.num_kv_heads, self.w.scale, rows=rows)

    def chunk_q64(self) -> np.ndarray:
        return self.w.chunk_queries().to(torch.float64).numpy()

    def prefill(self, seqs: Optional[Sequence[int]] = None, q: Optional[np.ndarray] = None):
        q = self.chunk_q64() if q is None else q
        return OPF.paged_prefill(self.pool, self.resolve, self.tables, self.lengths,
                                 self.w.chunk_lens, q, self.w.num_kv_heads, self.w.scale,
                                 seqs=seqs)

    def logical_kv(self, i: int):
        return OA.gather_kv(self.pool, self.resolve, self.tables[i], self.lengths[i],
                            self.w.num_kv_heads, self.w.head_dim)

    def copies(self):
        return [(a, b) for kind, a, b in self.model.events if kind == "copy"]
