#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

Workload: the batch-256 GQA decode layer -- 256 sequences with lengths
uniform over 200..2000, 32 query / 8 KV heads of 128, bf16 pools of 16-token
blocks on randomly permuted physical blocks (shapes of the pages' capacity
exercise and of a GQA model; synthetic N(0,1) data, seed 3).

One step = the whole decode hot path over the batch: address translation of
the 256 current tokens (positions L_i - 1), their K/V written into the pool,
and decode attention for every sequence and head through its table.  By
default this is one pa_decode_step launch (slot computed in-kernel, write
fused, the written token patched into registers); --unfused issues
pa_slot_mapping + pa_write_kv + pa_decode_attention instead.  Inputs are
resident in HBM before the timed region.  `value` is KV bytes read per step /
step time (whole step); the roofline block reports the launch that reads the
KV (the fused step, or the decode call), timed with HIP events on the stream
it runs on.

  python bench.py [--steps K] [--warmup W] [--partition P] [--unfused] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
DEFAULT_PARTITION = 0
# rocprofv3 FETCH_SIZE / WRITE_SIZE record of a workload's KV-reading launch
COUNTERS = os.path.join(ROOT, "profiles", "decode_step_{}_counters.json")
KERNEL_SOURCES = ("paged_kv_cache_143_amd/csrc/pa_decode.hip",
                  "paged_kv_cache_143_amd/csrc/pa_tile.h",
                  "paged_kv_cache_143_amd/csrc/pa_internal.h")
PCIE_PEAK_GBS = 64.0            # host link: PCIe 5.0 x16, one direction, published
# dense, published; FP8 caches are computed on bf16 matrix cores (codes widened in registers)
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 2500.0, "f32": 157.3}


# name -> (constructor, default partition size, length description, headline?)
def _workloads():
    from paged_kv_cache_143_amd import workloads as W
    return {
        "gqa-bf16-b256": (W.gqa_bf16, 0, "uniform int 200..2000"),
        "opt13b-mha-f16": (W.opt13b_f16, 0, "uniform int 200..2000"),
        "shared-prefix-bf16-p1024": (lambda: W.shared_prefix_bf16(prompt_len=1024), 0,
                                     "1024-token prompt + tails uniform 1..512"),
        "shared-prefix-bf16-p1016": (lambda: W.shared_prefix_bf16(prompt_len=1016), 0,
                                     "1016-token prompt + tails uniform 1..512"),
        "long-ctx-splitk-bf16": (W.long_ctx_bf16, -1, "uniform int 8192..32768"),
        "long-ctx-1x32k-bf16": (W.long_ctx_single_bf16, -1, "one sequence of 32768 tokens"),
        "gqa-fp8-b256": (W.gqa_fp8, 0, "uniform int 200..2000, FP8 E4M3 cache"),
        "gqa-bf16-b256-in-order": (W.gqa_bf16_in_order, 0,
                                   "uniform int 200..2000, consecutive physical blocks"),
        "gqa-bf16-b256-bs8": (lambda: W.gqa_bf16_block(8), 0,
                              "uniform int 200..2000, 8-token blocks"),
        "gqa-bf16-b256-bs32": (lambda: W.gqa_bf16_block(32), 0,
                               "uniform int 200..2000, 32-token blocks"),
        # one GPU's share under 8-way head sharding (tensor parallel by KV head)
        "gqa-bf16-b256-tp8": (W.gqa_bf16_tp8, -1, "uniform int 200..2000, 4 q / 1 kv heads"),
        "long-ctx-splitk-bf16-tp8": (W.long_ctx_bf16_tp8, -1,
                                     "uniform int 8192..32768, 8 q / 1 kv heads"),
        "opt13b-mha-f16-tp8": (W.opt13b_f16_tp8, -1, "uniform int 200..2000, 5 / 5 heads"),
        # one GPU's share under 8-way sequence sharding
        "gqa-bf16-b256-dp8": (W.gqa_bf16_dp8, -1, "every 8th sequence of gqa-bf16-b256 (32)"),
        "tiny-f32": (W.tiny_f32, 0, "{50, 20, 65, 16}"),
        "swap-gqa-bf16": (W.swap_gqa_bf16, 0,
                          "uniform int 200..2000; every third sequence swapped out and back"),
        "prefill-bf16": (W.prefill_bf16, 0, "16 prompts x 2048 tokens, no cached prefix"),
        "prefill-fp8": (W.prefill_fp8, 0, "16 prompts x 2048 tokens, no cached prefix, FP8 E4M3 cache"),
        "prefill-opt13b-f16": (W.prefill_opt13b_f16, 0,
                               "8 prompts x 2048 tokens, no cached prefix, 40/40 heads x 128 fp16"),
        "chunked-prefill-bf16": (W.chunked_prefill_bf16, 0,
                                 "32 x 512-token chunks over cached prefixes U{512..4096}"),
    }


def _code_text(src: str) -> str:
    """The source with C/C++ comments removed and whitespace runs collapsed:
    what the compiler sees, so that editing a comment does not count as
    changing the kernel."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest() -> str:
    """sha256 over the decode kernel's sources (comments and whitespace runs
    removed), the key of the committed counter record."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_text(fh.read()).encode())
        h.update(b"\0")
    return h.hexdigest()


def _measured_traffic(workload: str, fused: bool, partition: int):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    record of this workload (a split launch: the decode and combine kernels
    together), only while the kernel sources are the ones it was taken on and
    for the configuration it was taken in (fused step, same partition
    setting); otherwise None."""
    try:
        rec = json.load(open(COUNTERS.format(workload.replace("-", "_"))))
    except (OSError, ValueError):
        return None
    if (rec.get("kernel_source_sha256") != kernel_source_digest() or not fused
            or partition != rec.get("partition_size", 0)):
        return None
    return rec.get("traffic_bytes_per_launch")


def _unique_kv_bytes(w, batch, lens):
    """KV bytes of the distinct physical tiles the launch reads: a block listed
    by several tables (forks sharing a prompt) counts once, with the most
    tokens any of them attends in it."""
    import numpy as np
    b = w.block_size
    tab = batch.tables.cpu().numpy()
    used = {}
    for i, L in enumerate(np.asarray(lens, dtype=np.int64)):
        for j in range(int((L + b - 1) // b)):
            blk = int(tab[i, j])
            n = int(min(b, L - j * b))
            if n > used.get(blk, 0):
                used[blk] = n
    es = {"bf16": 2, "f16": 2, "f32": 4, "fp8": 1}[w.dtype]
    return sum(used.values()) * w.num_kv_heads * w.head_dim * 2 * es


def _algorithmic_bytes(w, lens, fused):
    """Bytes the KV-reading launch must move at minimum (each byte once): the
    KV of every valid (token, KV head) -- 2 * head_dim * 2 B = 512 B each for
    bf16 -- plus q, out, tables and lengths, plus (fused step) the current
    tokens' K/V read from k_new/v_new and written to the pool."""
    import numpy as np
    L = np.asarray(lens, dtype=np.int64)
    es = {"bf16": 2, "f16": 2, "f32": 4, "fp8": 1}[w.dtype]          # stored element
    ies = 4 if w.dtype == "f32" else 2                                 # q, new K/V inputs
    kv = int(L.sum()) * w.num_kv_heads * w.head_dim * 2 * es
    q = w.num_seqs * w.num_q_heads * w.head_dim * ies
    out = w.num_seqs * w.num_q_heads * w.head_dim * 4
    b = w.block_size
    tables = int(((L + b - 1) // b).sum()) * 4 + w.num_seqs * 4
    new = (w.num_seqs * w.num_kv_heads * w.head_dim * 2 * (ies + es)) if fused else 0
    return {"kv": kv, "q": q, "out": out, "tables_lens": tables, "new_tokens": new,
            "total": kv + q + out + tables + new}


def _walk_keys(pool, table, length):
    from oracle.attention import table_walk
    return [p for p in table_walk(pool, table, length) if p is not None]


def cpu_baseline(w, budget_s: float):
    """Time the fp64 oracle (as it stands) on the same batch: whole passes over its
    sequences until `budget_s` of oracle time, the last pass possibly partial."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    from oracle.allocator import run_script
    from oracle.attention import paged_decode
    from oracle.pool import SlotPool

    model = run_script(w.ops, w.num_blocks, w.block_size, w.free_order, checked=False)
    pool = SlotPool(w.num_blocks, w.block_size)
    pool.replay(model.events)
    tables = [model.tables[n] for n in w.seq_names]
    lens = [model.length(n) for n in w.seq_names]
    q64 = w.queries().to(torch.float64).numpy()
    elapsed, kv_bytes, done, tokens = 0.0, 0, 0, 0
    cache = {}

    def resolve(p):                     # payload (key, row) -> fp64 K, V rows (input prep)
        if p[0] not in cache:
            k, v = w.kv(p[0])
            cache[p[0]] = (k.to(torch.float64).numpy(), v.to(torch.float64).numpy())
        kk, vv = cache[p[0]]
        return kk[p[1]], vv[p[1]]

    es = {"bf16": 2, "f16": 2, "f32": 4, "fp8": 1}[w.dtype]
    with threadpool_limits(limits=1):
        while elapsed < budget_s:
            for i in range(w.num_seqs):
                # materialise this sequence's payloads first: only the oracle is timed
                for p in set(x[0] for x in _walk_keys(pool, tables[i], lens[i])):
                    resolve((p, 0))
                t0 = time.perf_counter()
                paged_decode(pool, resolve, tables, lens, q64, w.num_kv_heads, w.scale, rows=[i])
                elapsed += time.perf_counter() - t0
                if len(cache) > 4:
                    cache.clear()
                    w.drop_cache()
                kv_bytes += lens[i] * w.num_kv_heads * w.head_dim * 2 * es
                tokens += lens[i]
                done += 1
                if elapsed >= budget_s:
                    break
    return {"value": kv_bytes / elapsed / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} sequence decodes = {done / w.num_seqs:.2f} passes over the "
                      f"{w.num_seqs}-sequence batch ({tokens} context tokens, all "
                      f"{w.num_q_heads} query heads), fp64 NumPy oracle, 1 thread, "
                      f"{elapsed:.1f} s",
            "seconds": elapsed, "sequences": done,
            "host_cores": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_worker(job):
    """One process of the all-core oracle figure: rebuild the workload's pool
    (untimed), then decode its share of the sequences, one thread, until the
    budget; returns (KV bytes, oracle seconds, decodes)."""
    name, share, budget_s = job
    from threadpoolctl import threadpool_limits
    import torch
    from oracle.allocator import run_script
    from oracle.attention import paged_decode
    from oracle.pool import SlotPool

    torch.set_num_threads(1)
    w = _workloads()[name][0]()
    model = run_script(w.ops, w.num_blocks, w.block_size, w.free_order, checked=False)
    pool = SlotPool(w.num_blocks, w.block_size)
    pool.replay(model.events)
    tables = [model.tables[n] for n in w.seq_names]
    lens = [model.length(n) for n in w.seq_names]
    q64 = w.queries().to(torch.float64).numpy()
    es = {"bf16": 2, "f16": 2, "f32": 4, "fp8": 1}[w.dtype]
    cache = {}

    def resolve(p):
        if p[0] not in cache:
            k, v = w.kv(p[0])
            cache[p[0]] = (k.to(torch.float64).numpy(), v.to(torch.float64).numpy())
        kk, vv = cache[p[0]]
        return kk[p[1]], vv[p[1]]

    elapsed, kv_bytes, done = 0.0, 0, 0
    with threadpool_limits(limits=1):
        while elapsed < budget_s:
            for i in share:
                for key in set(x[0] for x in _walk_keys(pool, tables[i], lens[i])):
                    resolve((key, 0))
                t0 = time.perf_counter()
                paged_decode(pool, resolve, tables, lens, q64, w.num_kv_heads, w.scale, rows=[i])
                elapsed += time.perf_counter() - t0
                cache.clear()
                w.drop_cache()
                kv_bytes += lens[i] * w.num_kv_heads * w.head_dim * 2 * es
                done += 1
                if elapsed >= budget_s:
                    break
    return kv_bytes, elapsed, done


def cpu_baseline_all_cores(name: str, num_seqs: int, budget_s: float, max_procs: int = 16):
    """The same oracle on every host core this process may use (one process per
    core, capped at the machine's CPU share), sequences dealt round-robin; rate =
    all processes' KV bytes / the longest process's oracle time."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    cores = len(os.sched_getaffinity(0))
    procs = max(1, min(cores, max_procs, num_seqs))
    shares = [list(range(r, num_seqs, procs)) for r in range(procs)]
    ctx = mp.get_context("spawn")                  # fresh interpreters: no GPU state inherited
    env_keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in env_keys}
    for k in env_keys:
        os.environ[k] = "1"
    try:
        # a worker that dies raises here instead of being replaced
        with ProcessPoolExecutor(max_workers=procs, mp_context=ctx) as ex:
            res = list(ex.map(_cpu_worker, [(name, sh, budget_s) for sh in shares],
                              timeout=budget_s * 4 + 300))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    kv = sum(r[0] for r in res)
    secs = max(r[1] for r in res)
    done = sum(r[2] for r in res)
    return {"value": kv / secs / 1e9, "unit": "GB/s", "cores": procs, "kind": "oracle",
            "sample": f"{done} sequence decodes over {procs} processes (one thread each, "
                      f"sequences dealt round-robin), about {budget_s:.0f} s of oracle time "
                      f"per process"}


def device_copy_gbs(reps: int = 10) -> float:
    """A plain 1 GiB device-to-device copy on the same GPU: (read + write bytes) /
    median time.  The ceiling a bandwidth-bound kernel is compared with besides
    the published peak."""
    import numpy as np
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for k in range(reps):
        dst.copy_(src)
        ev[k + 1].record()
    torch.cuda.synchronize()
    ms = np.median([ev[k].elapsed_time(ev[k + 1]) for k in range(reps)])
    del src, dst
    return 2 * (1 << 30) / (ms / 1e3) / 1e9


def _prefill_flops(w, lens, chunk_lens=None):
    """Algorithmic flops of the chunks: per (row at position p, query head),
    (p + 1) keys x (2d for q.k + 2d for P.V)."""
    total = 0
    for L, n in zip(lens, w.chunk_lens if chunk_lens is None else chunk_lens):
        L, n = int(L), int(n)
        keys = n * (L - n) + n * (n + 1) // 2            # sum over rows of (p + 1)
        total += keys * w.num_q_heads * 4 * w.head_dim
    return total


def cpu_baseline_prefill(w, budget_s: float):
    """The fp64 oracle (as it stands) on whole chunks of the same batch, sequence
    by sequence, until `budget_s` of oracle time; flops as the GPU line counts them."""
    import torch
    from threadpoolctl import threadpool_limits
    from oracle.allocator import run_script
    from oracle.attention import gather_kv
    from oracle.pool import SlotPool
    from oracle.prefill import causal_chunk

    model = run_script(w.ops, w.num_blocks, w.block_size, w.free_order, checked=False)
    pool = SlotPool(w.num_blocks, w.block_size)
    pool.replay(model.events)
    q = w.chunk_queries().to(torch.float64).numpy()
    starts = [0]
    for n in w.chunk_lens:
        starts.append(starts[-1] + n)
    elapsed, flops, rows = 0.0, 0, 0

    def resolve(p):
        k, v = w.kv(p[0])
        return k[p[1]].to(torch.float64).numpy(), v[p[1]].to(torch.float64).numpy()

    with threadpool_limits(limits=1):
        for i, name in enumerate(w.seq_names):
            L, n = model.length(name), w.chunk_lens[i]
            K, V = gather_kv(pool, resolve, model.tables[name], L, w.num_kv_heads, w.head_dim)
            t0 = time.perf_counter()
            causal_chunk(q[starts[i]:starts[i + 1]], K, V, w.scale)
            elapsed += time.perf_counter() - t0
            flops += _prefill_flops(w, [L], [n])
            rows += n
            w.drop_cache()
            if elapsed >= budget_s:
                break
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{i + 1} of {w.num_seqs} chunks ({rows} rows, all {w.num_q_heads} "
                      f"query heads), fp64 NumPy oracle, 1 thread, {elapsed:.1f} s",
            "seconds": elapsed}


def run_prefill(args, w, length_desc):
    """Multi-token step: chunk K/V written (pa_slot_mapping + pa_write_kv), then
    pa_prefill_attention; TFLOP/s of algorithmic flops over the whole step."""
    import numpy as np
    import torch
    from paged_kv_cache_143_amd.paged_cache import PrefillStep, build_batch

    batch = build_batch(w, device="cuda")
    lens = batch.bm.length_array(w.seq_names)
    step = PrefillStep(batch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev_w = [mk() for _ in range(args.steps)]
    ev_a = [mk() for _ in range(args.steps)]
    ev_end = mk()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev_w[k].record()
        step.write_chunks()
        ev_a[k].record()
        step.attend()
    ev_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nxt = [ev_w[k + 1] if k + 1 < args.steps else ev_end for k in range(args.steps)]
    att_ms = np.array([ev_a[k].elapsed_time(nxt[k]) for k in range(args.steps)])
    wr_ms = np.array([ev_w[k].elapsed_time(ev_a[k]) for k in range(args.steps)])
    ms_step = wall / args.steps * 1e3
    flops = _prefill_flops(w, lens)
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    att_tf = flops / (att_ms.mean() / 1e3) / 1e12
    value = flops / (ms_step / 1e3) / 1e12
    rows = int(sum(w.chunk_lens))
    print(f"[bench] prefill step {ms_step:.4f} ms, attention launch median "
          f"{np.median(att_ms) * 1e3:.1f} us, chunk write median {np.median(wr_ms) * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    line = {
        "metric": "paged prefill attention TFLOP/s (algorithmic, causal) + rows/s, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "num_seqs": w.num_seqs, "chunks": length_desc,
                   "rows": rows, "context_tokens": int(lens.sum()),
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "out_dtype": "f32",
                   "seed": w.seed,
                   "step": "pa_slot_mapping + pa_write_kv(chunk rows) + pa_prefill_attention"},
        "rows_per_s": round(rows / (ms_step / 1e3), 1),
        "kernels_us": {"chunk_write_median": round(float(np.median(wr_ms)) * 1e3, 2),
                       "attention_median": round(float(np.median(att_ms)) * 1e3, 2),
                       "attention_mean": round(float(att_ms.mean()) * 1e3, 2),
                       "attention_min": round(float(att_ms.min()) * 1e3, 2),
                       "attention_p90": round(float(np.percentile(att_ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "mfma", "achieved": round(att_tf, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(att_tf / peak, 4), "traffic": None,
                     "kernel": "pa_prefill_attention (" + ("prefill_ring_kernel" if w.dtype in ("bf16", "f16", "fp8")
                                                         else "prefill_kernel") + ")",
                     "algorithmic_flops": flops},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


def run_swap(args, w, length_desc):
    """Swap every block of the workload's swapped sequences out to pinned host
    memory and back (pa_swap_blocks both ways), and the pages' cost check: the
    swap time against recomputing those sequences' attention by prefill."""
    import numpy as np
    import torch
    from paged_kv_cache_143_amd import binding as B
    from paged_kv_cache_143_amd import workloads as W
    from paged_kv_cache_143_amd.paged_cache import PrefillStep, build_batch

    batch = build_batch(w, device="cuda")
    names = sorted({op.name for op in w.ops if op.kind == W.SWAP_OUT})
    dev_blocks = [blk for n in names for blk in batch.bm.tables[n]]
    nb = len(dev_blocks)
    if nb > w.host_blocks:
        raise RuntimeError("host swap space smaller than the swapped sequences")
    out_pairs = torch.tensor([[d, h] for h, d in enumerate(dev_blocks)], dtype=torch.int32,
                             device="cuda")
    in_pairs = out_pairs.flip(1).contiguous()
    kv = batch.kv
    block_bytes = w.num_kv_heads * w.block_size * w.head_dim * {"bf16": 2, "f16": 2, "f32": 4, "fp8": 1}[w.dtype]
    moved = nb * 2 * block_bytes                      # K and V, one direction
    for _ in range(args.warmup):
        kv.swap(out_pairs, B.PA_SWAP_OUT)
        kv.swap(in_pairs, B.PA_SWAP_IN)
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev = [(mk(), mk(), mk()) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b_, c in ev:
        a.record()
        kv.swap(out_pairs, B.PA_SWAP_OUT)
        b_.record()
        kv.swap(in_pairs, B.PA_SWAP_IN)
        c.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_out = np.array([a.elapsed_time(b_) for a, b_, _ in ev])
    t_in = np.array([b_.elapsed_time(c) for _, b_, c in ev])
    ms_step = wall / args.steps * 1e3
    gbs_out = moved / (np.median(t_out) / 1e3) / 1e9
    gbs_in = moved / (np.median(t_in) / 1e3) / 1e9
    # recompute alternative: prefill attention over the same sequences (attention only)
    lens = [int(batch.bm.lengths[n]) for n in names]
    pw = W.chunked("recompute", 9, w.dtype, [0] * len(lens), lens, w.num_q_heads,
                   w.num_kv_heads, w.head_dim, block_size=w.block_size)
    pstep = PrefillStep(build_batch(pw, device="cuda"))
    pstep.attend()
    torch.cuda.synchronize()
    pe = [(mk(), mk()) for _ in range(5)]
    for a, b_ in pe:
        a.record()
        pstep.attend()
        b_.record()
    torch.cuda.synchronize()
    t_rec = float(np.median([a.elapsed_time(b_) for a, b_ in pe]))
    t_swap = float(np.median(t_out) + np.median(t_in))
    line = {
        "metric": "KV swap GB/s (device->host + host->device, pinned host pools), 1 GPU",
        "value": round(2 * moved / (t_swap / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "lengths": length_desc,
                   "swapped_sequences": len(names), "blocks": nb,
                   "bytes_each_way": moved, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size,
                   "step": "pa_swap_blocks out + pa_swap_blocks in"},
        "kernels_us": {"swap_out_median": round(float(np.median(t_out)) * 1e3, 1),
                       "swap_in_median": round(float(np.median(t_in)) * 1e3, 1)},
        "swap_out_gbs": round(gbs_out, 2), "swap_in_gbs": round(gbs_in, 2),
        "cost_check": {"t_swap_ms": round(t_swap, 3),
                       "t_swap_formula_ms": round(2 * moved / (min(gbs_out, gbs_in) * 1e9) * 1e3, 3),
                       "t_recompute_attention_only_ms": round(t_rec, 3),
                       "note": "recompute would also redo every layer's projections and MLP "
                               "for these tokens; only the attention part is timed here"},
        "roofline": {"bound": "link", "achieved": round(min(gbs_out, gbs_in), 2),
                     "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": round(min(gbs_out, gbs_in) / PCIE_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pa_swap_blocks (swap_blocks_kernel)"},
    }
    print(json.dumps(line), flush=True)


def run(args):
    import numpy as np
    import torch
    from paged_kv_cache_143_amd import binding
    from paged_kv_cache_143_amd import workloads as W
    from paged_kv_cache_143_amd.paged_cache import DecodeStep, build_batch

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    binding.lib()
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        # A plain copy of known size (read 512 MiB + write 512 MiB per launch):
        # hardware byte counters read on it give their scale to true bytes.
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    make, default_ps, length_desc = _workloads()[args.workload]
    w = make()
    if w.chunk_lens is not None:
        return run_prefill(args, w, length_desc)
    if w.host_blocks > 0:
        return run_swap(args, w, length_desc)
    if args.partition is None:
        args.partition = default_ps
    t_setup = time.perf_counter()
    batch = build_batch(w, device="cuda")
    lens = batch.bm.length_array(w.seq_names)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    print(f"[bench] setup {setup_s:.1f}s: {w.name}, {int(lens.sum())} context tokens, "
          f"{w.num_blocks} blocks", file=sys.stderr, flush=True)

    results = {}
    partitions = args.sweep if args.sweep else [args.partition]
    for ps in partitions:
        step = DecodeStep(batch, partition_size=ps, fused=not args.unfused)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        # One event per boundary: before every launch and after the last, so
        # the markers add as little as possible between kernels.
        mk = lambda: torch.cuda.Event(enable_timing=True)
        ev_kv = [mk() for _ in range(args.steps)]          # before each KV-reading launch
        ev_w = [mk() for _ in range(args.steps)] if args.unfused else None
        ev_end = mk()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            if args.unfused:
                ev_w[k].record()
                step.write_current()
                ev_kv[k].record()
                step.attend()
            else:
                ev_kv[k].record()
                step.fused_step()
        ev_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        nxt = [(ev_w[k + 1] if args.unfused else ev_kv[k + 1]) if k + 1 < args.steps else ev_end
               for k in range(args.steps)]
        dec_ms = np.array([ev_kv[k].elapsed_time(nxt[k]) for k in range(args.steps)])
        write_ms = (np.array([ev_w[k].elapsed_time(ev_kv[k]) for k in range(args.steps)])
                    if args.unfused else np.zeros(args.steps))
        results[ps] = (wall / args.steps * 1e3, write_ms, dec_ms)
        print(f"[bench] partition {ps}{' unfused' if args.unfused else ''}: step "
              f"{wall / args.steps * 1e3:.4f} ms, KV-reading launch median "
              f"{np.median(dec_ms) * 1e3:.1f} us, separate write+slots median "
              f"{np.median(write_ms) * 1e3:.1f} us", file=sys.stderr, flush=True)

    ps = partitions[0] if not args.sweep else min(results, key=lambda p: results[p][0])
    ms_step, write_ms, dec_ms = results[ps]
    alg = _algorithmic_bytes(w, lens, not args.unfused)
    dec_mean_s = float(dec_ms.mean()) / 1e3
    achieved = alg["total"] / dec_mean_s / 1e9
    kv_gbs = alg["kv"] / (ms_step / 1e3) / 1e9
    reserved = int(((lens + w.block_size - 1) // w.block_size).sum()) * w.block_size
    line = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) + tokens/s at batch 256, 1 GPU",
        "value": round(kv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "num_seqs": w.num_seqs,
                   "lengths": length_desc, "context_tokens": int(lens.sum()),
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size,
                   "partition_size": ps, "out_dtype": "f32", "seed": w.seed,
                   "reserved_tokens": reserved, "tail_waste_frac": round(1 - lens.sum() / reserved, 4),
                   "step": ("pa_slot_mapping + pa_write_kv(256 tokens) + pa_decode_attention"
                            if args.unfused else
                            "pa_decode_step (slot + write of 256 tokens + decode, one launch)")},
        "pct_hbm_peak": round(100.0 * kv_gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.num_seqs / (ms_step / 1e3), 1),
        "context_tokens_per_s": round(float(lens.sum()) / (ms_step / 1e3), 1),
        # decode tokens per second over the KV-reading launch alone (attention
        # only when the write runs separately)
        ("attention_only_tokens_per_s" if args.unfused else "kv_launch_tokens_per_s"):
            round(w.num_seqs / (float(np.median(dec_ms)) / 1e3), 1),
        # q.k and P.V: 4 d flops per (context token, query head), plus one exp each
        "algorithmic_gflop": round(float(lens.sum()) * w.num_q_heads * 4 * w.head_dim / 1e9, 4),
        "kernels_us": {"separate_write_and_slots_median":
                           round(float(np.median(write_ms)) * 1e3, 2) if args.unfused else 0.0,
                       "kv_launch_median": round(float(np.median(dec_ms)) * 1e3, 2),
                       "kv_launch_mean": round(dec_mean_s * 1e6, 2),
                       "kv_launch_min": round(float(dec_ms.min()) * 1e3, 2),
                       "kv_launch_p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _measured_traffic(args.workload, not args.unfused, ps),
                     "kernel": ("pa_decode_attention" if args.unfused else "pa_decode_step")
                     + " (decode_kernel" + (" + reduce_kernel" if step.workspace.numel() > 1
                                            else "") + ")",
                     "algorithmic_bytes": alg},
    }
    if w.name.startswith("shared-prefix"):
        # Forks read their shared prompt tiles once per fork (logical bytes) but
        # the caches serve some of those reads; the fetched-byte figure comes from
        # the committed counter record of this workload.
        uniq = _unique_kv_bytes(w, batch, lens)
        line["config"]["unique_kv_bytes"] = uniq
        traffic = line["roofline"]["traffic"]
        if traffic:
            fetched = traffic / dec_mean_s / 1e9
            line["roofline_fetched"] = {"bound": "hbm", "achieved": round(fetched, 1),
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": round(fetched / HBM_PEAK_GBS, 4),
                                        "bytes_per_launch": traffic}
    copy = device_copy_gbs()
    line["device_copy_gbs"] = round(copy, 1)
    line["pct_device_copy"] = round(100.0 * kv_gbs / copy, 2)
    if args.sweep:
        line["sweep_ms_per_step"] = {str(p): round(v[0], 5) for p, v in results.items()}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(make(), args.cpu_budget)
        if not args.no_all_core_baseline:
            line["cpu_baseline"]["all_cores"] = cpu_baseline_all_cores(
                args.workload, w.num_seqs, args.cpu_budget * 2 / 3)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gqa-bf16-b256", choices=sorted(_workloads()),
                    help="the headline metric is quoted on gqa-bf16-b256 (the default)")
    ap.add_argument("--partition", type=int, default=None,
                    help="partition size in tokens (0 = one work unit per sequence and KV head, "
                         "-1 = library's choice; default: 0, or -1 for the long-context workload)")
    ap.add_argument("--sweep", type=int, nargs="*", default=None,
                    help="time several partition sizes and report the fastest")
    ap.add_argument("--unfused", action="store_true",
                    help="three launches per step instead of pa_decode_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all-core-baseline", action="store_true",
                    help="skip the all-core oracle figure (the one-thread figure still runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run three plain 512 MiB device copies (counter calibration)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work in the CPU baseline sample")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decode path here is built and timed on a "
              "single MI355X (no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
