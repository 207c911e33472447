"""Multi-token (prefill and chunked-prefill) attention read through a block
table -- oracle, fp64.  Test infrastructure: only tests/, the smoke check and
the benchmark's CPU baseline use it.

Sources: the polomodov.tech transcript, paragraph 1 (in prefill every prompt
token is known at once, so the work is large matrix products; decode then
attends to the stored keys and values of earlier tokens) and paragraph 3
(attention reads K/V through the block table, token order kept); "Inside
vLLM and TGI", section "Read the vLLM0.11.0 scheduler" (the scheduler tracks
how many of a request's tokens are computed; admissions may reuse a computed
prefix) and section "Observability and debugging runbook" (a prompt longer
than the per-step token budget is processed in chunks); same page, "Worked
recall", item 3 (a reused prefix saves its prefill, the new suffix still
costs work).

The pages give no formula.  Plain reading used here: a chunk is the n newest
of a sequence's L stored tokens (positions L-n .. L-1, their K/V already in
the pool); the L-n older tokens are the computed prefix.  Query row j of the
chunk sits at position p = L - n + j and attends causally to positions
0..p with ordinary scaled dot-product softmax attention; query head h reads
KV head h // G as in decode.  n = L is a whole prompt; n = 1 is one decode
step.  Each row is computed on its own (no blocking).
"""
from __future__ import annotations

from typing import Any, Callable, Sequence, Tuple

import numpy as np

from .attention import decode_sequence, gather_kv
from .pool import SlotPool


def causal_chunk(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Rows of one chunk: q_rows [n, Hq, d] for positions L-n..L-1 of K/V [L, Hkv, d]."""
    n = q_rows.shape[0]
    L = K.shape[0]
    if n > L:
        raise ValueError("a chunk cannot hold more tokens than the sequence")
    out = np.empty(q_rows.shape, dtype=np.float64)
    for j in range(n):
        p = L - n + j
        out[j] = decode_sequence(q_rows[j], K[:p + 1], V[:p + 1], scale)
    return out


def paged_prefill(pool: SlotPool, resolve: Callable[[Any], Tuple[np.ndarray, np.ndarray]],
                  tables: Sequence[Sequence[int]], lengths: Sequence[int],
                  chunk_lens: Sequence[int], q: np.ndarray, num_kv_heads: int, scale: float,
                  seqs: Sequence[int] = None) -> np.ndarray:
    """Chunk attention for the sequences in `seqs` (all by default).

    q is [T, Hq, d] fp64 with the chunks of sequences 0..S-1 back to back
    (sequence i's rows start at sum(chunk_lens[:i])); returns the rows of the
    selected sequences, in order, as [sum of their chunk lengths, Hq, d].
    """
    starts = np.concatenate([[0], np.cumsum(np.asarray(chunk_lens, dtype=np.int64))])
    seqs = range(len(lengths)) if seqs is None else seqs
    head_dim = q.shape[2]
    out = []
    for i in seqs:
        n, L = int(chunk_lens[i]), int(lengths[i])
        if n == 0:
            continue
        K, V = gather_kv(pool, resolve, tables[i], L, num_kv_heads, head_dim)
        out.append(causal_chunk(q[starts[i]:starts[i + 1]], K, V, scale))
    return np.concatenate(out) if out else np.zeros((0,) + q.shape[1:])
