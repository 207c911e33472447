"""GPU parity of pa_decode_attention against the fp64 oracle.

Tolerance (per row = (sequence, query head): max_d |gpu - ref| / max_d |ref|):
1e-5 for fp32 pools and 2e-3 for fp16/bf16 pools, fp32 output.  Cases cover
several tiles and ragged tails, every GQA group size up to 16, head_dim 64
and 128, NaN poison in unused slots and free blocks, padded table entries,
recycled blocks with stale tenants, split-context partitions, forks sharing
blocks before and after copy-on-write, zero-length rows, lengths clipped by
max_context_len in the fused step, batches of up to 700 sequences with tied
lengths under longest-first dispatch, maximum sizes (4096 sequences; one
65,536-token sequence in 1024 partitions), and every full-size workload
(every row of the batch against the oracle) in the launch configuration the
benchmark times.  Outputs start as NaN, so a row that no kernel writes fails.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_143_amd import binding as B
from paged_kv_cache_143_amd import workloads as W
from paged_kv_cache_143_amd.paged_cache import DecodeStep, build_batch
from tests.gpu_util import announce, frob_rel_err, require_gpu, row_rel_err, tol_for
from oracle import attention as OA
from tests.oracle_glue import OracleRun, full_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(request):
    require_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _run(w, partition_size=0, out_dtype=torch.float32, rows=None):
    batch = build_batch(w, drop_payload_cache=False)
    step = DecodeStep(batch, partition_size=partition_size, out_dtype=out_dtype)
    out = step().float().cpu().numpy()
    torch.cuda.synchronize()
    run = OracleRun(w)
    ref = run.decode(rows=rows)
    got = out if rows is None else out[list(rows)]
    return got, ref, batch, run


CASES = {
    "tiny-f32": W.tiny_f32,
    "recycled-f32": W.recycled_f32,
    "mha-f16-d128": lambda: W.scaled("mha", 51, 6, 1, 300, 4, 4, 128, "f16"),
    "gqa4-bf16-d128": lambda: W.scaled("g4", 52, 9, 1, 700, 32, 8, 128, "bf16"),
    "gqa8-bf16-d64": lambda: W.scaled("g8", 53, 7, 1, 500, 16, 2, 64, "bf16"),
    "gqa16-f16-d64": lambda: W.scaled("g16", 54, 5, 1, 400, 16, 1, 64, "f16"),
    "gqa2-bf16-d128": lambda: W.scaled("g2", 55, 5, 200, 600, 4, 2, 128, "bf16"),
    "gqa3-f32-d128": lambda: W.scaled("g3", 56, 4, 1, 300, 6, 2, 128, "f32"),
    "mha-f32-d64": lambda: W.scaled("m32", 57, 4, 1, 300, 5, 5, 64, "f32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name):
    w = CASES[name]()
    got, ref, _, _ = _run(w)
    assert np.isfinite(got).all()
    err = row_rel_err(got, ref)
    announce(f"{name}: max row rel err {err:.3e}")
    assert err <= tol_for(w.dtype)


@pytest.mark.parametrize("ps", [16, 32, 48, 512])
def test_split_context_matches_oracle_and_unsplit(ps):
    w = W.scaled("split", 61, 6, 1, 900, 16, 4, 128, "bf16")
    got, ref, batch, _ = _run(w, partition_size=ps)
    err = row_rel_err(got, ref)
    announce(f"ps={ps}: max row rel err {err:.3e}")
    assert err <= tol_for(w.dtype)
    whole = DecodeStep(batch, partition_size=0)()
    assert row_rel_err(got, whole.cpu().numpy().astype(np.float64)) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_more_partitions_than_one_chunk(dtype):
    """16-token partitions over up to 5000 tokens: 313 partitions in a row, so
    the combine kernel's workgroup walks them in two chunks of 256."""
    lens = [5000, 4100, 300, 17]
    w = W.independent(f"ps16-{dtype}", 69, dtype, lens, 8, 2, 128, sum(-(-L // 16) for L in lens) + 4)
    got, ref, batch, _ = _run(w, partition_size=16)
    err = row_rel_err(got, ref)
    announce(f"313 partitions {dtype}: max row rel err {err:.3e}")
    assert err <= tol_for(w.dtype)
    whole = DecodeStep(batch, partition_size=0)().cpu().numpy().astype(np.float64)
    assert row_rel_err(got, whole) <= 1e-5


def test_split_context_fp32():
    w = W.scaled("split32", 62, 3, 40, 300, 4, 2, 64, "f32")
    got, ref, _, _ = _run(w, partition_size=64)
    assert row_rel_err(got, ref) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_pool_dtype_output_is_a_rounded_fp32_result(dtype):
    """A 16-bit output is the round-to-nearest of some value within the fp32 row
    bound of the reference: |got - ref| <= ulp(got) + 1e-5 * max|ref row|.  (A pure
    1-ulp test against RNE(ref) is too strict for elements far below the row's
    magnitude, whose ulp is smaller than the fp32 accumulation error.)"""
    w = W.scaled("out16", 63, 5, 1, 400, 8, 2, 128, dtype)
    got, ref, _, _ = _run(w, out_dtype=W.DTYPES[dtype])
    tdt = W.DTYPES[dtype]
    g16 = torch.from_numpy(got).to(tdt)
    assert torch.equal(g16.to(torch.float64), torch.from_numpy(got))    # exactly 16-bit values
    up = g16.view(torch.int16).add(1).view(tdt).to(torch.float64).numpy()
    ulp = np.abs(up - got)
    rowmax = np.abs(ref).max(axis=-1, keepdims=True)
    assert (np.abs(got - ref) <= ulp + 1e-5 * rowmax).all()


def test_tail_and_length_edges():
    """Lengths 1, 15, 16, 17, 31, 32, 33 (partial last blocks on both sides of a
    boundary), poison everywhere else."""
    w = W.independent("edges", 64, "bf16", [1, 15, 16, 17, 31, 32, 33, 2], 8, 2, 128, 40)
    got, ref, _, _ = _run(w)
    assert np.isfinite(got).all()
    assert row_rel_err(got, ref) <= 2e-3
    w1 = W.independent("edges32", 65, "f32", [1, 2, 16, 17, 48], 4, 4, 64, 20)
    got, ref, _, _ = _run(w1)
    # one token: softmax weight exactly 1, output = that V row (fp32 arithmetic)
    assert row_rel_err(got, ref) <= 1e-5


def test_zero_length_rows_and_bad_entries():
    w = W.scaled("zero", 66, 4, 20, 80, 8, 2, 64, "bf16", extra_blocks=0.5)
    batch = build_batch(w, drop_payload_cache=False)
    lens = batch.lens.clone()
    lens[1] = 0
    out = torch.full((w.num_seqs, w.num_q_heads, w.head_dim), 7.0, device="cuda")
    B.decode_attention_t(batch.kv.desc, batch.kv.k, batch.kv.v, batch.q, out, batch.tables,
                         lens, w.scale, batch.max_len)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert (o[1] == 0).all()
    run = OracleRun(w)
    ref = run.decode(rows=[0, 2, 3])
    assert row_rel_err(o[[0, 2, 3]], ref) <= 2e-3
    # a length above max_context_len is clipped to it; a table entry out of range
    # contributes nothing -- both without faults (finite output)
    lens2 = batch.lens.clone()
    lens2[0] = 10_000
    tab = batch.tables.clone()
    tab[2, 0] = w.num_blocks + 5
    B.decode_attention_t(batch.kv.desc, batch.kv.k, batch.kv.v, batch.q, out, tab, lens2,
                         w.scale, batch.max_len)
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()


def test_forks_identical_before_and_correct_after_cow():
    """Forks sharing every block give bit-identical outputs for the same query; after
    copy-on-write and divergence each fork matches its own oracle result."""
    groups, forks = 2, 4
    w = W.shared_prefix("forkcow", 67, "bf16", groups, forks, 1016, 1, 50, 8, 2, 128, 400)
    # before divergence: keep only create + forks + parent release
    pre = [op for op in w.ops if op.kind != W.APPEND]
    w_pre = W.Workload(**{**w.__dict__, "ops": pre, "_cache": {}})
    batch = build_batch(w_pre, drop_payload_cache=False)
    q_same = batch.q.clone()
    for g in range(groups):
        q_same[g * forks:(g + 1) * forks] = batch.q[g * forks]
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), device="cuda")
    B.decode_attention_t(batch.kv.desc, batch.kv.k, batch.kv.v, q_same, out, batch.tables,
                         batch.lens, w.scale, batch.max_len)
    torch.cuda.synchronize()
    o = out.cpu()
    for g in range(groups):
        for f in range(1, forks):
            assert torch.equal(o[g * forks], o[g * forks + f])
    # after: the full script (7 copies per group would be 3 here: forks - 1)
    got, ref, b2, run = _run(w)
    assert len(b2.copies) == groups * (forks - 1)
    assert row_rel_err(got, ref) <= 2e-3


def test_shared_prefix_full_block_prompt():
    w = W.shared_prefix("fullp", 68, "bf16", 2, 8, 1024, 1, 64, 32, 8, 128, 400)
    got, ref, b, _ = _run(w)
    assert not b.copies
    assert row_rel_err(got, ref) <= 2e-3


@pytest.mark.parametrize("ps", [0, 256, 512])
def test_gqa_batch256_full_size_all_rows(ps):
    """The batch-256 GQA bf16 workload at full size: every row vs the oracle."""
    w = W.gqa_bf16()
    batch = build_batch(w, drop_payload_cache=False)
    got = DecodeStep(batch, partition_size=ps, fused=False)().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    ref = full_decode(w)
    err = row_rel_err(got, ref)
    announce(f"gqa-bf16-b256 ps={ps}: all {w.num_seqs} rows max row rel err {err:.3e}, "
             f"Frobenius {frob_rel_err(got, ref):.3e}")
    assert err <= 2e-3


MANY_ROWS = {
    # 256 x 32 = 8192 rows of up to 8 partitions: one wavefront per row combines them
    "gqa-bf16-b256-ps256": (W.gqa_bf16, 256, torch.float32),
    "gqa-bf16-b256-ps512-bf16out": (W.gqa_bf16, 512, torch.bfloat16),
    # 256 x 16 = 4096 rows, head_dim 64, up to 10 partitions of 32 tokens
    "f16-d64-4096rows": (lambda: W.scaled("mr64", 79, 256, 20, 300, 16, 2, 64, "f16"), 32,
                         torch.float32),
}


@pytest.mark.parametrize("name", list(MANY_ROWS))
def test_many_rows_split_matches_unsplit(name):
    """Every row of a many-row split (the combine kernel's one-wavefront-per-row
    form) against the unsplit kernel and against the oracle."""
    make, ps, odt = MANY_ROWS[name]
    w = make()
    batch = build_batch(w, drop_payload_cache=False)
    got = DecodeStep(batch, partition_size=ps, out_dtype=odt)().float().cpu().numpy()
    whole = DecodeStep(batch, partition_size=0, out_dtype=torch.float32)().cpu().numpy()
    assert w.num_seqs * w.num_q_heads >= 4096
    assert np.isfinite(got).all()
    if odt == torch.float32:
        assert row_rel_err(got.astype(np.float64), whole.astype(np.float64)) <= 1e-5
    else:                                           # a rounding of a value within 1e-5
        want = torch.from_numpy(whole).to(odt).float().numpy()
        ulp = np.abs(want) * 2.0 ** -7 + 1e-30
        assert (np.abs(got - whole) <= ulp + 1e-5 * np.abs(whole).max(axis=-1, keepdims=True)).all()
    # vs the oracle, every row: the fp32-output split (the same combine path; a
    # 16-bit output adds its own rounding, checked above)
    got32 = got if odt == torch.float32 else \
        DecodeStep(batch, partition_size=ps, out_dtype=torch.float32)().cpu().numpy()
    assert np.isfinite(got32).all()
    err = row_rel_err(got32.astype(np.float64), full_decode(w))
    announce(f"{name}: all rows max row rel err {err:.3e}")
    assert err <= tol_for(w.dtype)


def _poison_current_tokens(batch):
    """Overwrite every sequence's current token (position L-1) in the pool with NaN."""
    w = batch.w
    slots = [batch.bm.slot(n, batch.bm.lengths[n] - 1) for n in w.seq_names]
    shape = (len(slots), w.num_kv_heads, w.head_dim)
    nan = torch.full(shape, float("nan"), dtype=W.DTYPES[w.input_dtype], device="cuda")
    batch.kv.write(nan, nan, torch.tensor(slots, dtype=torch.int32, device="cuda"))


def _tied(name, seed, values, n, dtype="bf16"):
    """n sequences whose lengths are drawn from a few values (ties in the
    ranking's length bins)."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.choice(values, n)]
    return W.independent(name, seed, dtype, lengths, 4, 2, 64, W._pool_for(lengths, 16, 0.1))


# Longest-first dispatch ranks the sequences in every workgroup: pairwise up
# to 128 sequences, by counting above (several passes over the lengths once
# there are more sequences than a workgroup has threads).  Every row of each
# batch is checked, so a rank that is not a bijection (a row never written,
# or written twice) fails.
RANKED = {
    "100seqs-tied-pairwise": lambda: _tied("rk-pw", 94, [33, 34, 200], 100),
    "300seqs-one-bin": lambda: _tied("rk-one", 93, [100, 101, 127], 300),
    "600seqs-U1..300": lambda: W.scaled("rk600", 91, 600, 1, 300, 4, 2, 64, "bf16"),
    "700seqs-tied-bins-f16": lambda: _tied("rk-tie", 92, [17, 160, 161, 300], 700, "f16"),
}


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", list(RANKED))
def test_longest_first_ranking_covers_every_row(name, fused):
    w = RANKED[name]()
    batch = build_batch(w, drop_payload_cache=False)
    got = DecodeStep(batch, partition_size=0, fused=fused)().float().cpu().numpy()
    torch.cuda.synchronize()
    assert np.isfinite(got).all()
    err = row_rel_err(got, full_decode(w))
    announce(f"{name} fused={fused}: all {w.num_seqs} rows max row rel err {err:.3e}")
    assert err <= tol_for(w.dtype)


# Maximum sizes: 4096 sequences (32768 workgroups; the counting ranking makes
# 16 passes over the lengths), and one 65,536-token sequence split by the
# library's plan or into 1024 partitions of 64 tokens per row.
@pytest.mark.parametrize("fused", [True, False])
def test_4096_sequences_every_row(fused):
    w = W.scaled("max-s", 401, 4096, 1, 64, 8, 2, 64, "bf16")
    batch = build_batch(w, drop_payload_cache=False)
    got = DecodeStep(batch, partition_size=0, fused=fused)().float().cpu().numpy()
    torch.cuda.synchronize()
    assert np.isfinite(got).all()
    err = row_rel_err(got, full_decode(w))
    announce(f"4096 sequences fused={fused}: max row rel err {err:.3e}")
    assert err <= tol_for(w.dtype)


@pytest.mark.parametrize("ps", [B.PA_PARTITION_AUTO, 64])
def test_one_64k_token_sequence(ps):
    w = W.independent("max-l", 402, "bf16", [65536], 32, 8, 128, 65536 // 16 + 20)
    batch = build_batch(w, drop_payload_cache=False)
    got = DecodeStep(batch, partition_size=ps)().float().cpu().numpy()
    torch.cuda.synchronize()
    assert np.isfinite(got).all()
    err = row_rel_err(got, full_decode(w))
    announce(f"65536 tokens ps={ps}: max row rel err {err:.3e}")
    assert err <= tol_for(w.dtype)


FUSED = {
    "tiny-f32": (W.tiny_f32, 0),
    "gqa4-bf16-d128": (lambda: W.scaled("fg4", 71, 9, 1, 700, 32, 8, 128, "bf16"), 0),
    "gqa2-f16-d64-split": (lambda: W.scaled("fg2", 72, 6, 1, 500, 4, 2, 64, "f16"), 32),
    "gqa3-f32-d128-split": (lambda: W.scaled("fg3", 73, 4, 1, 300, 6, 2, 128, "f32"), 64),
    "cow-bf16": (lambda: W.shared_prefix("fcow", 74, "bf16", 2, 8, 1016, 1, 40, 8, 2, 64, 200), 0),
    "edges-bf16": (lambda: W.independent("fedge", 75, "bf16", [1, 15, 16, 17, 31, 32, 33, 2],
                                          8, 2, 128, 40), 0),
}


@pytest.mark.parametrize("name", list(FUSED))
def test_fused_step_equals_three_calls_and_oracle(name):
    make, ps = FUSED[name]
    w = make()
    outs, pools = [], []
    for fused in (False, True):
        batch = build_batch(w, drop_payload_cache=False)
        _poison_current_tokens(batch)
        step = DecodeStep(batch, partition_size=ps, fused=fused)
        outs.append(step().clone())
        torch.cuda.synchronize()
        pools.append((batch.kv.k.clone(), batch.kv.v.clone()))
    assert torch.equal(outs[0], outs[1])
    bits = lambda t: t.view(torch.int16 if t.element_size() == 2 else torch.int32)
    for a, b in zip(pools[0], pools[1]):
        assert torch.equal(bits(a), bits(b))
    ref = OracleRun(w).decode()
    err = row_rel_err(outs[1].cpu().numpy().astype(np.float64), ref)
    announce(f"fused {name}: max row rel err {err:.3e}")
    assert err <= tol_for(w.dtype)


@pytest.mark.parametrize("ps", [0, 32])
@pytest.mark.parametrize("clip", ["longest", "all", "zero"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_fused_step_with_clipped_lengths(dtype, clip, ps):
    """Lengths above max_context_len.  The three-call form writes each current
    token at its true position L_i - 1 (slot mapping + write) and attends the
    clipped range; the fused step must do the same: bit-identical pools and
    outputs, and the outputs equal the oracle over the clipped lengths (the
    current token of a clipped sequence is written but not attended)."""
    w = W.scaled(f"clip-{dtype}", 76, 6, 20, 200, 8, 2, 128, dtype)
    lens = [len(r) for r in W.fork_payload_rows(w).values()]
    cap = {"longest": max(lens) - 7, "all": min(lens) - 3, "zero": 0}[clip]
    outs, pools = [], []
    for fused in (False, True):
        batch = build_batch(w, drop_payload_cache=False)
        _poison_current_tokens(batch)
        batch.max_len = cap
        step = DecodeStep(batch, partition_size=ps, fused=fused)
        outs.append(step().clone())
        torch.cuda.synchronize()
        pools.append((batch.kv.k.clone(), batch.kv.v.clone()))
    assert torch.equal(outs[0], outs[1])
    bits = lambda t: t.view(torch.uint8 if t.element_size() == 1 else torch.int16)
    for a, b in zip(pools[0], pools[1]):
        assert torch.equal(bits(a), bits(b))
    # every current token is in the pool (nothing poisoned is left at L_i - 1)
    run = OracleRun(w)
    got = outs[1].cpu().numpy().astype(np.float64)
    clipped = [min(L, cap) for L in run.lengths]
    ref = OA.paged_decode(run.pool, run.resolve, run.tables, clipped, run.q64(), w.num_kv_heads,
                          w.scale)
    assert np.isfinite(got).all()
    err = row_rel_err(got, ref)
    announce(f"clipped {dtype} {clip} ps={ps}: max row rel err {err:.3e}")
    assert err <= tol_for(w.dtype)
    if clip == "zero":
        assert (got == 0).all()


def test_fused_step_full_size_all_rows():
    """The batch-256 GQA workload in the benchmark's launch configuration
    (pa_decode_step, one pass), every row vs the oracle."""
    w = W.gqa_bf16()
    batch = build_batch(w, drop_payload_cache=False)
    _poison_current_tokens(batch)
    out = DecodeStep(batch, partition_size=0, fused=True)().cpu().numpy().astype(np.float64)
    assert np.isfinite(out).all()
    ref = full_decode(w)
    err = row_rel_err(out, ref)
    announce(f"fused gqa-bf16-b256: all rows max row rel err {err:.3e}, "
             f"Frobenius {frob_rel_err(out, ref):.3e}")
    assert err <= 2e-3


FULL = {
    "opt13b-mha-f16": (W.opt13b_f16, 0, None),
    "shared-prefix-p1024": (lambda: W.shared_prefix_bf16(prompt_len=1024), 0, 0),
    "shared-prefix-p1016": (lambda: W.shared_prefix_bf16(prompt_len=1016), 0, 32 * 7),
    "gqa-in-order": (W.gqa_bf16_in_order, 0, None),
    "long-ctx-splitk": (W.long_ctx_bf16, 512, None),
    "long-ctx-auto": (W.long_ctx_bf16, -1, None),
    # one GPU's share under 8-way head sharding
    "gqa-b256-tp8": (W.gqa_bf16_tp8, -1, None),
    "long-ctx-tp8": (W.long_ctx_bf16_tp8, -1, None),
    "opt13b-tp8": (W.opt13b_f16_tp8, -1, None),
    # one GPU's share under 8-way sequence sharding
    "gqa-b256-dp8": (W.gqa_bf16_dp8, -1, None),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_workloads_all_rows(name):
    """The other workloads at full size, in the benchmark's step (pa_decode_step with
    the current tokens first poisoned in the pool), every row vs the oracle."""
    make, ps, copies = FULL[name]
    w = make()
    batch = build_batch(w, drop_payload_cache=False)
    if copies is not None:
        assert len(batch.copies) == copies
    _poison_current_tokens(batch)
    out = DecodeStep(batch, partition_size=ps, fused=True)().cpu().numpy().astype(np.float64)
    assert np.isfinite(out).all()
    ref = full_decode(w)
    err = row_rel_err(out, ref)
    announce(f"{name} ps={ps}: all {w.num_seqs} rows max row rel err {err:.3e}, "
             f"Frobenius {frob_rel_err(out, ref):.3e}")
    assert err <= tol_for(w.dtype)
