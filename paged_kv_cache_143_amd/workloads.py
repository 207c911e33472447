"""Seeded synthetic workloads for paged decode attention.

This module is the only code shared by the HIP path's tests/bench and the
CPU oracle.  It draws random numbers and describes *what happens* to a pool
of blocks (which sequences are created, forked, grown, released, and the
order of the free list); it performs none of the method's arithmetic: no
block/offset/slot computation, no copy-on-write decision, no attention.

Workload shapes follow the pages:
  * lengths uniform over the integers 200..2000 and 16-token blocks
    ("Inside vLLM and TGI", section "Block addresses and fragmentation
    arithmetic");
  * the OPT-13B head shape (40 heads x 128, FP16) from the polomodov.tech
    transcript, second paragraph;
  * the worked table [7, 3, 12, 5] for a 50-token request (same section of
    "Inside vLLM and TGI");
  * forks sharing a prompt, as in the copy-on-write discussion of both the
    "Exact CPU block manager and copy-on-write" section and the transcript's
    fourth paragraph.

Values of q, K and V are N(0, 1) drawn in fp32 by torch's CPU generator and
rounded (round-to-nearest-even) to the storage dtype.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

# Table padding value for entries past a sequence's last block; it is never a
# valid block id, so any read through it would be an out-of-range access.
TABLE_PAD = 0x7FFFFFFF

# Storage dtypes.  FP8 pools store E4M3 codes (as bytes on the device); their
# inputs (q, new K/V) are bf16.
DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
          "fp8": torch.uint8}
INPUT_DTYPE = {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8": "bf16"}

# Op kinds of an allocator script.
CREATE, FORK, APPEND, RELEASE = "create", "fork", "append", "release"
SWAP_OUT, SWAP_IN = "swap_out", "swap_in"


def _mix(*parts: int) -> int:
    """Deterministic 63-bit seed from integer parts (splitmix64 finaliser)."""
    x = 0x243F6A8885A308D3
    for p in parts:
        x = (x ^ (int(p) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        x = (x + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        x = z ^ (z >> 31)
    return x & 0x7FFFFFFFFFFFFFFF


def normal(shape, seed_parts: Sequence[int], dtype: str) -> torch.Tensor:
    """N(0,1) in fp32 from a seeded CPU generator, rounded RNE to `dtype`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(_mix(*seed_parts))
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    return x.to(DTYPES[dtype])


@dataclass(frozen=True)
class Op:
    """One allocator action.

    create:  name gets `count` tokens whose payload rows are data[key][0:count]
    fork:    name becomes a sharer of every block of `src`
    append:  name grows by one token whose payload row is data[key][index]
    release: name is dropped
    swap_out / swap_in: name moves to host blocks / back to device blocks
    """
    kind: str
    name: int
    count: int = 0
    src: int = -1
    key: int = -1
    index: int = 0


@dataclass
class Workload:
    """Everything needed to build one batch of paged decode input."""
    name: str
    seed: int
    dtype: str
    num_blocks: int
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    ops: List[Op]
    free_order: List[int]          # free list; allocators take from the END
    seq_names: List[int]           # batch order of the live sequences
    data_len: Dict[int, int]       # payload key -> number of rows
    partition_size: int = 0
    notes: str = ""
    # Multi-token workloads: the chunk of sequence i is its chunk_lens[i]
    # newest tokens (payload rows L-n .. L-1 of key i); None for decode.
    chunk_lens: Optional[List[int]] = None
    host_blocks: int = 0            # host swap space, in blocks
    # FP8 pools: per-KV-head scales (fp32 values); drawn from the seed when None
    k_scales: Optional[List[float]] = None
    v_scales: Optional[List[float]] = None
    _cache: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = field(default_factory=dict, repr=False)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_names)

    @property
    def input_dtype(self) -> str:
        return INPUT_DTYPE[self.dtype]

    def kv_scales(self) -> Tuple[List[float], List[float]]:
        """FP8 pools: (K, V) scale per KV head.  Default: (3 + 2u) / 448 with u
        uniform per head, i.e. about 3..5 standard deviations map to the
        largest code, so a few of the N(0,1) values saturate."""
        if self.k_scales is not None and self.v_scales is not None:
            return list(self.k_scales), list(self.v_scales)
        rng = np.random.default_rng(_mix(self.seed, 5))
        u = rng.random((2, self.num_kv_heads))
        sc = ((3.0 + 2.0 * u) / 448.0).astype(np.float32)
        return [float(x) for x in sc[0]], [float(x) for x in sc[1]]

    @property
    def scale(self) -> float:
        # 1/sqrt(head_dim) rounded to fp32: the value both sides are handed.
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    def kv(self, key: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """Payload rows (K, V) for `key`, each [rows, Hkv, d] in the dtype."""
        if key not in self._cache:
            n = self.data_len[key]
            shape = (n, self.num_kv_heads, self.head_dim)
            k = normal(shape, (self.seed, 1, key), self.input_dtype)
            v = normal(shape, (self.seed, 2, key), self.input_dtype)
            self._cache[key] = (k, v)
        return self._cache[key]

    def drop_cache(self) -> None:
        self._cache.clear()

    def queries(self) -> torch.Tensor:
        """q [num_seqs, Hq, d] in the dtype, one draw per sequence name."""
        rows = [normal((self.num_q_heads, self.head_dim), (self.seed, 3, n), self.input_dtype)
                for n in self.seq_names]
        return torch.stack(rows) if rows else torch.empty(
            (0, self.num_q_heads, self.head_dim), dtype=DTYPES[self.input_dtype])

    def chunk_queries(self) -> torch.Tensor:
        """q rows [sum(chunk_lens), Hq, d] of the chunks, sequence by sequence."""
        rows = [normal((int(n), self.num_q_heads, self.head_dim), (self.seed, 4, name),
                       self.input_dtype)
                for name, n in zip(self.seq_names, self.chunk_lens)]
        return torch.cat(rows) if rows else torch.empty(
            (0, self.num_q_heads, self.head_dim), dtype=DTYPES[self.input_dtype])


def _uniform_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> List[int]:
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


def _shuffled(rng: np.random.Generator, ids: Sequence[int]) -> List[int]:
    ids = list(ids)
    perm = rng.permutation(len(ids))
    return [ids[i] for i in perm]


def independent(name: str, seed: int, dtype: str, lengths: Sequence[int], num_q_heads: int,
                num_kv_heads: int, head_dim: int, num_blocks: int, block_size: int = 16,
                pinned_first: Optional[Sequence[int]] = None, last_token_append: bool = True,
                partition_size: int = 0, ghosts: Sequence[int] = (),
                notes: str = "", in_order: bool = False) -> Workload:
    """Independent sequences (no sharing) on a seeded, shuffled free list.

    Sequence i is created with its first L_i - 1 tokens and then grows by one
    appended token (the current decode token), so `context length` L_i counts
    the token written in the step itself.  `pinned_first` places those block
    ids at the end of the free list, in order, so the first sequence takes them.
    `ghosts` are lengths of earlier tenants that are created and released
    first, so that recycled blocks hold their stale tokens.  `in_order` hands out
    block ids 0, 1, 2, ... (each sequence's blocks then lie back to back: the
    identity table, no indirection scatter) instead of a shuffled list.
    """
    rng = np.random.default_rng(seed)
    ids = list(range(num_blocks))
    pinned = list(pinned_first or [])
    rest = [i for i in ids if i not in set(pinned)]
    rest = list(reversed(rest)) if in_order else _shuffled(rng, rest)
    free_order = rest + list(reversed(pinned))
    ops: List[Op] = []
    data_len: Dict[int, int] = {}
    for k, G in enumerate(ghosts):
        gname = 2_000_000 + k
        data_len[gname] = int(G)
        ops.append(Op(CREATE, name=gname, count=int(G), key=gname))
    for k in range(len(ghosts)):
        ops.append(Op(RELEASE, name=2_000_000 + k))
    for i, L in enumerate(lengths):
        data_len[i] = int(L)
        if last_token_append and L >= 2:
            ops.append(Op(CREATE, name=i, count=int(L) - 1, key=i))
            ops.append(Op(APPEND, name=i, key=i, index=int(L) - 1))
        else:
            ops.append(Op(CREATE, name=i, count=int(L), key=i))
    return Workload(name=name, seed=seed, dtype=dtype, num_blocks=num_blocks,
                    block_size=block_size, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, ops=ops,
                    free_order=free_order, seq_names=list(range(len(lengths))),
                    data_len=data_len, partition_size=partition_size, notes=notes)


def shared_prefix(name: str, seed: int, dtype: str, groups: int, forks: int, prompt_len: int,
                  tail_lo: int, tail_hi: int, num_q_heads: int, num_kv_heads: int,
                  head_dim: int, num_blocks: int, block_size: int = 16,
                  partition_size: int = 0, notes: str = "") -> Workload:
    """Parallel sampling: per group a parent prompt, `forks` sharers, parent dropped.

    Then decode rounds: in round r every fork whose private tail is longer
    than r appends one token, forks in order.  The first appends hit the
    shared last block of the prompt when the prompt does not end on a block
    boundary.
    """
    rng = np.random.default_rng(seed)
    free_order = _shuffled(rng, range(num_blocks))
    ops: List[Op] = []
    data_len: Dict[int, int] = {}
    tails: Dict[int, int] = {}
    fork_names: List[int] = []
    for g in range(groups):
        parent = 1_000_000 + g
        pkey = 1_000_000 + g
        data_len[pkey] = prompt_len
        ops.append(Op(CREATE, name=parent, count=prompt_len, key=pkey))
        for f in range(forks):
            fname = g * forks + f
            ops.append(Op(FORK, name=fname, src=parent))
            fork_names.append(fname)
            tails[fname] = int(rng.integers(tail_lo, tail_hi + 1))
            data_len[fname] = tails[fname]
        ops.append(Op(RELEASE, name=parent))
    longest = max(tails.values()) if tails else 0
    for r in range(longest):
        for fname in fork_names:
            if tails[fname] > r:
                ops.append(Op(APPEND, name=fname, key=fname, index=r))
    return Workload(name=name, seed=seed, dtype=dtype, num_blocks=num_blocks,
                    block_size=block_size, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, ops=ops,
                    free_order=free_order, seq_names=fork_names, data_len=data_len,
                    partition_size=partition_size, notes=notes)


def fork_payload_rows(w: Workload) -> Dict[int, List[Tuple[int, int]]]:
    """For each live name, the payload (key, row) of every token in logical order.

    This is bookkeeping of the op script itself (what each sequence was told
    to contain), used by tests as the un-paged "contiguous" view.
    """
    seqs: Dict[int, List[Tuple[int, int]]] = {}
    parked: Dict[int, List[Tuple[int, int]]] = {}          # swapped out
    for op in w.ops:
        if op.kind == CREATE:
            seqs[op.name] = [(op.key, r) for r in range(op.count)]
        elif op.kind == FORK:
            seqs[op.name] = list(seqs[op.src])
        elif op.kind == APPEND:
            seqs[op.name].append((op.key, op.index))
        elif op.kind == RELEASE:
            del seqs[op.name]
        elif op.kind == SWAP_OUT:
            parked[op.name] = seqs.pop(op.name)
        elif op.kind == SWAP_IN:
            seqs[op.name] = parked.pop(op.name)
    return seqs


# --------------------------------------------------------------------------
# The five decode workloads: shapes of the pages' examples, fixed seeds 1..5.
# --------------------------------------------------------------------------

def tiny_f32() -> Workload:
    """4 sequences {50, 20, 65, 16}, 12 heads x 64, fp32, 64-block pool;
    the 50-token sequence sits on blocks [7, 3, 12, 5]."""
    return independent("tiny-f32", 1, "f32", [50, 20, 65, 16], 12, 12, 64, 64,
                       pinned_first=[7, 3, 12, 5])


def recycled_f32() -> Workload:
    """Tiny fp32 shapes on a pool whose every block first served released tenants,
    so unused tail slots hold other requests' stale tokens (not poison)."""
    return independent("recycled-f32", 6, "f32", [50, 20, 65, 16, 1, 33], 4, 2, 64, 24,
                       ghosts=[16 * 24 - 5])


def _pool_for(lengths: Sequence[int], block_size: int, extra: float) -> int:
    # Generous size: every sequence may waste a block, plus `extra` spare.
    return int((sum(lengths) / block_size + len(lengths)) * (1.0 + extra)) + 1


def opt13b_f16(num_seqs: int = 64, seed: int = 2) -> Workload:
    """OPT-13B-shaped layer: 64 sequences, L ~ U{200..2000}, 40/40 heads x 128, fp16,
    pool sized to fit plus about 10 % shuffled free blocks."""
    rng = np.random.default_rng(seed + 100)
    lengths = _uniform_lengths(rng, num_seqs, 200, 2000)
    return independent("opt13b-mha-f16", seed, "f16", lengths, 40, 40, 128,
                       _pool_for(lengths, 16, 0.10))


def gqa_bf16(num_seqs: int = 256, seed: int = 3) -> Workload:
    """Batch-256 GQA decode: L ~ U{200..2000}, 32 q / 8 kv heads x 128, bf16,
    randomly permuted physical blocks, one new token written per sequence."""
    rng = np.random.default_rng(seed + 100)
    lengths = _uniform_lengths(rng, num_seqs, 200, 2000)
    return independent("gqa-bf16-b256", seed, "bf16", lengths, 32, 8, 128,
                       _pool_for(lengths, 16, 0.0))


def chunked(name: str, seed: int, dtype: str, prefix_lens: Sequence[int],
            chunk_lens: Sequence[int], num_q_heads: int, num_kv_heads: int, head_dim: int,
            block_size: int = 16, extra_blocks: float = 0.1) -> Workload:
    """Multi-token step: sequence i holds prefix_lens[i] computed tokens plus a
    chunk of chunk_lens[i] new ones (prefill when the prefix is 0), all stored
    in the pool (shuffled free list); the chunk's rows are the queries."""
    lengths = [int(p) + int(c) for p, c in zip(prefix_lens, chunk_lens)]
    w = independent(name, seed, dtype, lengths, num_q_heads, num_kv_heads, head_dim,
                    _pool_for(lengths, block_size, extra_blocks), block_size=block_size,
                    last_token_append=False)
    w.chunk_lens = [int(c) for c in chunk_lens]
    return w


def prefill_bf16(num_seqs: int = 16, prompt_len: int = 2048, seed: int = 6) -> Workload:
    """Whole-prompt prefill: 16 prompts of 2048 tokens, 32 q / 8 kv heads x 128, bf16."""
    return chunked("prefill-bf16", seed, "bf16", [0] * num_seqs, [prompt_len] * num_seqs,
                   32, 8, 128)


def prefill_fp8(num_seqs: int = 16, prompt_len: int = 2048, seed: int = 6) -> Workload:
    """The whole-prompt prefill workload (same prompts and values) on an FP8 E4M3 cache."""
    return chunked("prefill-fp8", seed, "fp8", [0] * num_seqs, [prompt_len] * num_seqs,
                   32, 8, 128)


def prefill_opt13b_f16(num_seqs: int = 8, prompt_len: int = 2048, seed: int = 8) -> Workload:
    """OPT-13B-shaped whole-prompt prefill: 8 prompts of 2048 tokens, 40 heads
    (MHA) x 128, fp16."""
    return chunked("prefill-opt13b-f16", seed, "f16", [0] * num_seqs, [prompt_len] * num_seqs,
                   40, 40, 128)


def chunked_prefill_bf16(num_seqs: int = 32, chunk: int = 512, seed: int = 7) -> Workload:
    """Chunked prefill: 32 sequences with cached prefixes U{512..4096} and a
    512-token chunk each (a 16K-token step), 32 q / 8 kv heads x 128, bf16."""
    rng = np.random.default_rng(seed + 100)
    prefix = _uniform_lengths(rng, num_seqs, 512, 4096)
    return chunked("chunked-prefill-bf16", seed, "bf16", prefix, [chunk] * num_seqs, 32, 8, 128)


def swap_cycle(name: str, seed: int, dtype: str, lengths: Sequence[int], num_q_heads: int,
               num_kv_heads: int, head_dim: int, block_size: int = 16,
               every: int = 3) -> Workload:
    """Preemption by swapping: every `every`-th sequence is swapped out after
    its prompt, other requests (fillers) then occupy the freed blocks while the
    rest decode one token, the fillers finish, and the swapped sequences come
    back (into other blocks) and decode their token.  Sequence i holds L_i
    tokens at the end; the batch is every original sequence."""
    rng = np.random.default_rng(seed)
    lengths = [int(L) for L in lengths]
    b = block_size
    need = sum(-(-L // b) for L in lengths)
    num_blocks = int(need * 1.15) + 4
    ops: List[Op] = []
    data_len: Dict[int, int] = {}
    for i, L in enumerate(lengths):
        data_len[i] = L
        ops.append(Op(CREATE, name=i, count=max(L - 1, 1), key=i))
    out = [i for i in range(len(lengths)) if i % every == 0 and lengths[i] >= 2]
    for i in out:
        ops.append(Op(SWAP_OUT, name=i))
    fillers = []
    for k, i in enumerate(out):
        f = 1_000_000 + k
        data_len[f] = lengths[i]
        ops.append(Op(CREATE, name=f, count=lengths[i], key=f))
        fillers.append(f)
    for i, L in enumerate(lengths):
        if i not in out and L >= 2:
            ops.append(Op(APPEND, name=i, key=i, index=L - 1))
    for f in fillers:
        ops.append(Op(RELEASE, name=f))
    for i in out:
        ops.append(Op(SWAP_IN, name=i))
        ops.append(Op(APPEND, name=i, key=i, index=lengths[i] - 1))
    host = sum(-(-lengths[i] // b) for i in out) + 2      # room for a second cycle at L
    return Workload(name=name, seed=seed, dtype=dtype, num_blocks=num_blocks, block_size=b,
                    num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    ops=ops, free_order=_shuffled(rng, range(num_blocks)),
                    seq_names=list(range(len(lengths))), data_len=data_len, host_blocks=host)


def swap_gqa_bf16(num_seqs: int = 256, seed: int = 8) -> Workload:
    """The batch-256 GQA shape (L ~ U{200..2000}, 32 q / 8 kv heads x 128,
    bf16) with a third of the sequences swapped out and back."""
    rng = np.random.default_rng(seed + 100)
    lengths = _uniform_lengths(rng, num_seqs, 200, 2000)
    return swap_cycle("swap-gqa-bf16", seed, "bf16", lengths, 32, 8, 128)


def gqa_fp8(num_seqs: int = 256, seed: int = 3) -> Workload:
    """The batch-256 GQA workload (same lengths and values) on an FP8 E4M3 cache."""
    rng = np.random.default_rng(seed + 100)
    lengths = _uniform_lengths(rng, num_seqs, 200, 2000)
    return independent("gqa-fp8-b256", seed, "fp8", lengths, 32, 8, 128,
                       _pool_for(lengths, 16, 0.0))


def gqa_bf16_in_order(num_seqs: int = 256, seed: int = 3) -> Workload:
    """The batch-256 GQA workload with every sequence on consecutive physical
    blocks (same lengths and values): the cost of the table indirection."""
    rng = np.random.default_rng(seed + 100)
    lengths = _uniform_lengths(rng, num_seqs, 200, 2000)
    return independent("gqa-bf16-b256-in-order", seed, "bf16", lengths, 32, 8, 128,
                       _pool_for(lengths, 16, 0.0), in_order=True)


def shared_prefix_bf16(groups: int = 32, forks: int = 8, prompt_len: int = 1024,
                       seed: int = 4) -> Workload:
    """Parallel sampling: 32 groups x 8 forks of a shared prompt, private tails
    U{1..512}, 32 q / 8 kv heads x 128, bf16.  prompt_len=1016 leaves a shared
    partial last block, which the first appends copy on write."""
    per_group = (prompt_len + 15) // 16 + forks * (512 // 16 + 2)
    return shared_prefix(f"shared-prefix-bf16-p{prompt_len}", seed, "bf16", groups, forks,
                         prompt_len, 1, 512, 32, 8, 128, groups * per_group + 16)


def long_ctx_bf16(num_seqs: int = 16, seed: int = 5, partition_size: int = 512) -> Workload:
    """Long context: 16 sequences, L ~ U{8192..32768}, 64 q / 8 kv heads x 128,
    bf16, split into 512-token partitions and reduced."""
    rng = np.random.default_rng(seed + 100)
    lengths = _uniform_lengths(rng, num_seqs, 8192, 32768)
    return independent("long-ctx-splitk-bf16", seed, "bf16", lengths, 64, 8, 128,
                       _pool_for(lengths, 16, 0.0), partition_size=partition_size)


def long_ctx_single_bf16(length: int = 32768, seed: int = 9) -> Workload:
    """Single-sequence long-context decode (the latency case): one sequence of
    32768 tokens, 64 q / 8 kv heads x 128, bf16; too few (sequence, KV head)
    pairs to fill the GPU, so the split is planned from the length."""
    return independent("long-ctx-1x32k-bf16", seed, "bf16", [length], 64, 8, 128,
                       _pool_for([length], 16, 0.0), partition_size=-1)


def scaled(kind: str, seed: int, num_seqs: int, lo: int, hi: int, num_q_heads: int,
           num_kv_heads: int, head_dim: int, dtype: str, extra_blocks: float = 0.1,
           partition_size: int = 0, block_size: int = 16) -> Workload:
    """A reduced-size variant of a workload family (same distributions)."""
    rng = np.random.default_rng(seed + 100)
    lengths = _uniform_lengths(rng, num_seqs, lo, hi)
    return independent(kind, seed, dtype, lengths, num_q_heads, num_kv_heads, head_dim,
                       _pool_for(lengths, block_size, extra_blocks), block_size=block_size,
                       partition_size=partition_size)


def gqa_bf16_block(block_size: int, num_seqs: int = 256, seed: int = 3) -> Workload:
    """The batch-256 GQA workload (same lengths and values) on blocks of another size."""
    rng = np.random.default_rng(seed + 100)
    lengths = _uniform_lengths(rng, num_seqs, 200, 2000)
    return independent(f"gqa-bf16-b256-bs{block_size}", seed, "bf16", lengths, 32, 8, 128,
                       _pool_for(lengths, block_size, 0.0), block_size=block_size)


def head_shard(w: Workload, ways: int, name: str) -> Workload:
    """One GPU's share of `w` when its KV heads are split `ways` ways (tensor
    parallel by head): the same sequences, lengths, block size and pool, with
    Hq / ways query heads on Hkv / ways KV heads.  Payload values are drawn
    for the shard's own shape (seeded like the whole workload)."""
    if w.num_kv_heads % ways:
        raise ValueError(f"{w.num_kv_heads} KV heads do not split {ways} ways")
    return Workload(name=name, seed=w.seed, dtype=w.dtype, num_blocks=w.num_blocks,
                    block_size=w.block_size, num_q_heads=w.num_q_heads // ways,
                    num_kv_heads=w.num_kv_heads // ways, head_dim=w.head_dim, ops=w.ops,
                    free_order=w.free_order, seq_names=w.seq_names, data_len=w.data_len,
                    partition_size=-1, notes=f"{ways}-way head shard of {w.name}")


def gqa_bf16_tp8() -> Workload:
    """Batch-256 GQA step as one of 8 GPUs sees it under head sharding: 4 q / 1 kv heads."""
    return head_shard(gqa_bf16(), 8, "gqa-bf16-b256-tp8")


def long_ctx_bf16_tp8() -> Workload:
    """Long-context batch as one of 8 GPUs sees it under head sharding: 8 q / 1 kv heads."""
    return head_shard(long_ctx_bf16(), 8, "long-ctx-splitk-bf16-tp8")


def opt13b_f16_tp8() -> Workload:
    """OPT-13B-shaped layer as one of 8 GPUs sees it under head sharding: 5 / 5 heads."""
    return head_shard(opt13b_f16(), 8, "opt13b-mha-f16-tp8")


def gqa_bf16_dp8() -> Workload:
    """Batch-256 GQA step as one of 8 GPUs sees it under sequence sharding:
    every eighth sequence of the batch (32, the same lengths), all 32 / 8 heads."""
    rng = np.random.default_rng(3 + 100)
    lengths = _uniform_lengths(rng, 256, 200, 2000)[::8]
    w = independent("gqa-bf16-b256-dp8", 3, "bf16", lengths, 32, 8, 128,
                    _pool_for(lengths, 16, 0.0))
    w.partition_size = -1
    return w
