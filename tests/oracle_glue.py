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
from oracle import fp8 as OF8
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
        """fp64 K, V rows of a payload as the pool holds them: the generated
        values, or for FP8 pools value(code) * scale of each KV head."""
        key, row = payload
        if key not in self._f64:
            k, v = self.w.kv(key)
            k, v = k.to(torch.float64).numpy(), v.to(torch.float64).numpy()
            if self.w.dtype == "fp8":
                ks, vs = self.w.kv_scales()
                k, v = k.copy(), v.copy()
                for g in range(self.w.num_kv_heads):
                    k[:, g] = OF8.dequantize(OF8.quantize(k[:, g], ks[g]), ks[g])
                    v[:, g] = OF8.dequantize(OF8.quantize(v[:, g], vs[g]), vs[g])
            self._f64[key] = (k, v)
        k, v = self._f64[key]
        return k[row], v[row]

    def resolve_codes(self, payload):
        """FP8 pools: the E4M3 codes of a payload's K, V rows, as floats with
        the NaN codes as NaN (for bit-exact pool comparison)."""
        key, row = payload
        k, v = self.w.kv(key)
        ks, vs = self.w.kv_scales()
        kc = np.stack([OF8.quantize(k[row, g].float().numpy(), ks[g])
                       for g in range(self.w.num_kv_heads)]).astype(np.float64)
        vc = np.stack([OF8.quantize(v[row, g].float().numpy(), vs[g])
                       for g in range(self.w.num_kv_heads)]).astype(np.float64)
        kc[(kc == 0x7F) | (kc == 0xFF)] = np.nan
        vc[(vc == 0x7F) | (vc == 0xFF)] = np.nan
        return kc, vc

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


_FULL_DECODE: Dict[tuple, np.ndarray] = {}


def full_decode(w) -> np.ndarray:
    """Every row of the oracle's decode of workload `w` ([S][Hq][d] fp64),
    computed once per workload per test session (several launch
    configurations of one batch compare against the same rows)."""
    key = (w.name, w.seed, w.dtype, w.block_size, w.num_seqs, w.num_blocks)
    if key not in _FULL_DECODE:
        _FULL_DECODE[key] = OracleRun(w).decode()
    return _FULL_DECODE[key]
