"""Single-query decode attention read through a block table (oracle, fp64).

Sources: the polomodov.tech transcript, paragraph 3 (a table maps a
request's logical blocks to physical blocks anywhere in a shared pool, the
attention kernel reads through that mapping and token order stays correct)
and paragraph 1 (decode reads the stored keys and values of all earlier
tokens); "Inside vLLM and TGI", section "Block addresses and fragmentation
arithmetic" (logical block t // b, offset t % b, physical table[t // b]).

The pages never write the attention formula.  Plain reading used here:
ordinary scaled dot-product softmax attention of one query vector over the
sequence's L stored tokens, no mask other than the length; query head h
reads KV head h // G where G = Hq / Hkv (contiguous groups; with Hq = Hkv
this is multi-head attention); scale is passed in (1/sqrt(d) rounded to fp32
by the workloads).  The split-context form computes, per partition of
consecutive positions, the running maximum m_p, the sum of exponentials l_p
and the unnormalised weighted sum o_p, and combines them by rescaling with
exp(m_p - max_p m_p); that equals the unsplit result algebraically.
"""
from __future__ import annotations

from typing import Any, Callable, List, Sequence, Tuple

import numpy as np

from .pool import SlotPool


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query q [d], keys/values [L, d] (fp64)."""
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w / w.sum()) @ V


def table_walk(pool: SlotPool, table: Sequence[int], length: int) -> List[Any]:
    """Payload of positions 0..length-1, fetched block by block through the table."""
    b = pool.width
    out: List[Any] = []
    for j in range(-(-length // b)):
        phys = int(table[j])
        filled = min(b, length - j * b)
        out.extend(pool.block_payloads(phys)[:filled])
    return out


def gather_kv(pool: SlotPool, resolve: Callable[[Any], Tuple[np.ndarray, np.ndarray]],
              table: Sequence[int], length: int, num_kv_heads: int,
              head_dim: int) -> Tuple[np.ndarray, np.ndarray]:
    """Logical K, V [L, Hkv, d] of one sequence (NaN rows where a slot was never written)."""
    payloads = table_walk(pool, table, length)
    if len(payloads) != length:
        raise AssertionError("table walk returned a different number of tokens than the length")
    K = np.full((length, num_kv_heads, head_dim), np.nan)
    V = np.full((length, num_kv_heads, head_dim), np.nan)
    for t, p in enumerate(payloads):
        if p is not None:
            K[t], V[t] = resolve(p)
    return K, V


def decode_sequence(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """All query heads of one sequence: q [Hq, d], K/V [L, Hkv, d] -> [Hq, d]."""
    num_q_heads = q.shape[0]
    num_kv_heads = K.shape[1]
    if num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    group = num_q_heads // num_kv_heads
    out = np.empty(q.shape, dtype=np.float64)
    for h in range(num_q_heads):
        g = h // group
        out[h] = softmax_attention(q[h], K[:, g, :], V[:, g, :], scale)
    return out


def paged_decode(pool: SlotPool, resolve: Callable[[Any], Tuple[np.ndarray, np.ndarray]],
                 tables: Sequence[Sequence[int]], lengths: Sequence[int], q: np.ndarray,
                 num_kv_heads: int, scale: float, rows: Sequence[int] = None) -> np.ndarray:
    """Decode attention for the sequences in `rows` (all by default).

    q is [S, Hq, d] fp64; returns [len(rows), Hq, d].  A sequence of length 0
    has no tokens to attend to; its output is defined as zeros.
    """
    rows = range(len(lengths)) if rows is None else rows
    head_dim = q.shape[2]
    out = []
    for i in rows:
        L = int(lengths[i])
        if L == 0:
            out.append(np.zeros(q.shape[1:]))
            continue
        K, V = gather_kv(pool, resolve, tables[i], L, num_kv_heads, head_dim)
        out.append(decode_sequence(q[i], K, V, scale))
    return np.stack(out) if out else np.zeros((0,) + q.shape[1:])


# -- split-context form ---------------------------------------------------

def partition_state(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                    scale: float) -> Tuple[float, float, np.ndarray]:
    """(m, l, o) of one partition: max score, sum of exp(s - m), sum of exp(s - m) * V."""
    s = scale * (K @ q)
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ V


def combine_partitions(states: Sequence[Tuple[float, float, np.ndarray]]) -> np.ndarray:
    """Rescale every partition to the global maximum and normalise once."""
    M = max(m for m, _, _ in states)
    num = sum(np.exp(m - M) * o for m, _, o in states)
    den = sum(np.exp(m - M) * l for m, l, _ in states)
    return num / den


def split_decode_sequence(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                          partition: int) -> np.ndarray:
    """decode_sequence computed over consecutive `partition`-token slices of positions."""
    num_q_heads = q.shape[0]
    group = num_q_heads // K.shape[1]
    L = K.shape[0]
    out = np.empty(q.shape, dtype=np.float64)
    for h in range(num_q_heads):
        g = h // group
        states = [partition_state(q[h], K[a:a + partition, g], V[a:a + partition, g], scale)
                  for a in range(0, L, partition)]
        out[h] = combine_partitions(states)
    return out
