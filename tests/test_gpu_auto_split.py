"""GPU parity of automatic partitioning (PA_PARTITION_AUTO) when the split is
planned from the lengths.

With fewer (sequence, KV head) pairs than resident workgroups, both kernels of
the split derive the same plan from the context lengths: a sequence of n tiles
gets ceil(n / u) units of near-equal tile ranges, u the smallest size (at
least 512 tokens) that keeps one KV head's units within its share of the
resident workgroups.  The cases cover every pool dtype, head dims 64 and 128,
block sizes 8, 16 and 32 (8-token blocks pair up into 16-token tiles), more
than 64 sequences (the plan's scans then take several rounds), batches whose
plan collapses to one unit per sequence, enough rows for the combine kernel's
one-wavefront-per-row form, zero-length rows, and the fused step.
Each output is checked against the fp64 oracle (1e-5 per row for fp32 pools,
2e-3 otherwise) and against the unsplit kernel (partition_size 0).
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_143_amd import binding as B
from paged_kv_cache_143_amd import workloads as W
from paged_kv_cache_143_amd.paged_cache import DecodeStep, build_batch
from tests.gpu_util import announce, require_gpu, row_rel_err, tol_for
from tests.oracle_glue import OracleRun

pytestmark = pytest.mark.gpu

AUTO = B.PA_PARTITION_AUTO


@pytest.fixture(autouse=True)
def _gpu(request):
    require_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _blocks(lengths, b, spare=8):
    return sum((L + b - 1) // b for L in lengths) + spare


MIXED = [1, 15, 16, 17, 511, 512, 513, 1029, 3000, 7001, 12345]


def _mixed(name, seed, dtype, hq, hkv, d, b):
    return W.independent(name, seed, dtype, MIXED, hq, hkv, d, _blocks(MIXED, b), block_size=b)


CASES = {
    "bf16-d128-b16-mixed": lambda: _mixed("as-bf16", 201, "bf16", 32, 8, 128, 16),
    "f16-d64-b16-mixed": lambda: _mixed("as-f16", 202, "f16", 16, 2, 64, 16),
    "bf16-d128-b8-mixed": lambda: _mixed("as-b8", 203, "bf16", 16, 2, 128, 8),
    "f16-d128-b32-mixed": lambda: _mixed("as-b32", 204, "f16", 12, 2, 128, 32),
    "fp8-d128-b16-mixed": lambda: _mixed("as-fp8", 205, "fp8", 32, 8, 128, 16),
    "fp8-d64-b8-mixed": lambda: _mixed("as-fp8b8", 206, "fp8", 8, 1, 64, 8),
    "f32-d128-b16-mixed": lambda: _mixed("as-f32", 207, "f32", 6, 2, 128, 16),
    "f32-d64-b32-mixed": lambda: _mixed("as-f32b", 208, "f32", 4, 4, 64, 32),
    # 70 sequences, one KV head: scans over two rounds of 64 lanes
    "bf16-70seqs": lambda: W.scaled("as-70", 209, 70, 1, 2600, 4, 1, 128, "bf16"),
    # 90 x 8 units just under 768 resident: the plan keeps one unit per sequence
    "bf16-90seqs-no-room": lambda: W.scaled("as-90", 210, 90, 600, 2000, 32, 8, 128, "bf16"),
    # 64 x 64 = 4096 rows of about 1.5 units: combined one wavefront per row
    "bf16-64seqs-4096rows": lambda: W.scaled("as-64", 214, 64, 600, 3000, 64, 8, 128, "bf16"),
    # one long sequence over many units
    "bf16-one-long": lambda: W.independent("as-one", 211, "bf16", [20011], 16, 2, 128,
                                           _blocks([20011], 16)),
}


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_auto_split_matches_oracle_and_unsplit(name, fused):
    w = CASES[name]()
    batch = build_batch(w, drop_payload_cache=False)
    nbytes = B.workspace_size(batch.kv.desc, w.num_seqs, w.num_q_heads, batch.max_len, AUTO)
    assert nbytes > 0                                  # these batches take the planned split
    got = DecodeStep(batch, partition_size=AUTO, fused=fused)().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    whole = DecodeStep(batch, partition_size=0, fused=False)().cpu().numpy().astype(np.float64)
    ref = OracleRun(w).decode()
    err = row_rel_err(got, ref)
    announce(f"{name} auto fused={fused}: max row rel err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= tol_for(w.dtype)
    assert row_rel_err(got, whole) <= 1e-5


def test_auto_split_long_row_past_one_chunk():
    """One 40000-token sequence among 255 of 50 tokens, one KV head, 16 query
    heads: 4096 rows, so the combine kernel runs one wavefront per row, and the
    long sequence's 79 units take it past its first 64 partitions."""
    lens = [50] * 256
    lens[77] = 40000
    w = W.independent("as-chunk", 215, "bf16", lens, 16, 1, 128, _blocks(lens, 16))
    batch = build_batch(w, drop_payload_cache=False)
    got = DecodeStep(batch, partition_size=AUTO, fused=True)().cpu().numpy().astype(np.float64)
    whole = DecodeStep(batch, partition_size=0, fused=False)().cpu().numpy().astype(np.float64)
    err = row_rel_err(got, OracleRun(w).decode())
    announce(f"long row among short ones: max row rel err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= 2e-3
    assert row_rel_err(got, whole) <= 1e-5


def test_auto_split_zero_length_rows_and_clipping():
    """Zero-length rows come out zero, lengths above max_context_len are clipped,
    and both count as the plan's units without disturbing the other rows."""
    w = _mixed("as-zero", 212, "bf16", 16, 2, 128, 16)
    batch = build_batch(w, drop_payload_cache=False)
    lens = batch.lens.clone()
    lens[0] = 0
    lens[4] = 0
    lens[9] = -5
    nbytes = B.workspace_size(batch.kv.desc, w.num_seqs, w.num_q_heads, batch.max_len, AUTO)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.full((w.num_seqs, w.num_q_heads, w.head_dim), 7.0, device="cuda")
    B.decode_attention_t(batch.kv.desc, batch.kv.k, batch.kv.v, batch.q, out, batch.tables,
                         lens, w.scale, batch.max_len, partition_size=AUTO, workspace=ws)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert (o[[0, 4, 9]] == 0).all()
    keep = [i for i in range(w.num_seqs) if i not in (0, 4, 9)]
    ref = OracleRun(w).decode(rows=keep)
    assert row_rel_err(o[keep], ref) <= 2e-3
    # a length far above max_context_len attends to max_context_len positions
    lens2 = batch.lens.clone()
    lens2[10] = 10 ** 9
    B.decode_attention_t(batch.kv.desc, batch.kv.k, batch.kv.v, batch.q, out, batch.tables,
                         lens2, w.scale, batch.max_len, partition_size=AUTO, workspace=ws)
    torch.cuda.synchronize()
    assert row_rel_err(out.cpu().numpy().astype(np.float64)[keep], ref) <= 2e-3


def test_auto_split_repeatable_across_calls():
    """The same call twice gives bit-identical outputs (the plan is a function of
    the lengths; nothing carries over between calls)."""
    w = _mixed("as-rep", 213, "bf16", 32, 8, 128, 16)
    batch = build_batch(w, drop_payload_cache=False)
    step = DecodeStep(batch, partition_size=AUTO, fused=False)
    a = step().clone()
    b = step().clone()
    assert torch.equal(a, b)
