"""ctypes binding of libpa.so (argument marshalling only).

Functions named like the C entry points take the same arguments (integers
for device pointers and streams).  The `*_t` helpers accept torch tensors,
check dtype/device/contiguity, and pass `data_ptr()` and torch's current
stream.  Every computation happens in the HIP library; when it is missing
`lib()` raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(5)
PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
PA_PARTITION_AUTO = -1
DTYPE_CODES = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16, "fp8": PA_FP8_E4M3}

EXPORTS = ("pa_status_string", "pa_version", "pa_slot_mapping", "pa_write_kv",
           "pa_copy_blocks", "pa_decode_workspace_size", "pa_decode_attention",
           "pa_decode_step", "pa_prefill_attention", "pa_swap_blocks", "pa_validate_tables",
           "pa_decode_step_noalloc", "pa_validate_copy_pairs")
PA_NOALLOC_SCRATCH_BYTES = 64 << 20
PA_SWAP_OUT, PA_SWAP_IN = 0, 1


class PaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k_scales", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p)]


_lib: Optional[ctypes.CDLL] = None
P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64


def _hip_runtimes_loaded():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def lib() -> ctypes.CDLL:
    """Load libpa.so once (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Load a libpa build and declare its entry points."""
    import torch  # noqa: F401  -- loads the HIP runtime torch was built with
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m paged_kv_cache_143_amd.build`")
    L = ctypes.CDLL(path)
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_status_string.argtypes = [I32]
    L.pa_version.restype = I32
    L.pa_version.argtypes = []
    L.pa_slot_mapping.restype = I32
    L.pa_slot_mapping.argtypes = [P, I32, I32, P, P, I32, I32, P, P]
    L.pa_write_kv.restype = I32
    L.pa_write_kv.argtypes = [ctypes.POINTER(PoolDesc), P, P, P, P, I64, P, I32, P]
    L.pa_copy_blocks.restype = I32
    L.pa_copy_blocks.argtypes = [ctypes.POINTER(PoolDesc), P, P, P, I32, P]
    L.pa_decode_workspace_size.restype = I32
    L.pa_decode_workspace_size.argtypes = [ctypes.POINTER(PoolDesc), I32, I32, I32, I32,
                                           ctypes.POINTER(ctypes.c_size_t)]
    L.pa_decode_attention.restype = I32
    L.pa_decode_attention.argtypes = [ctypes.POINTER(PoolDesc), P, P, P, P, I32, P, I32, P,
                                      I32, I32, ctypes.c_float, I32, I32, P, ctypes.c_size_t, P]
    L.pa_decode_step.restype = I32
    L.pa_decode_step.argtypes = [ctypes.POINTER(PoolDesc), P, P, P, P, I64, P, P, I32, P, I32,
                                 P, I32, I32, ctypes.c_float, I32, I32, P, ctypes.c_size_t, P]
    L.pa_decode_step_noalloc.restype = I32
    L.pa_decode_step_noalloc.argtypes = [ctypes.POINTER(PoolDesc), P, P, P, P, I64, P, P, I32,
                                         P, I32, P, I32, I32, ctypes.c_float, I32, I32, P]
    L.pa_prefill_attention.restype = I32
    L.pa_prefill_attention.argtypes = [ctypes.POINTER(PoolDesc), P, P, P, P, I32, P, P, I32, P,
                                       I32, I32, ctypes.c_float, I32, I32, P]
    L.pa_swap_blocks.restype = I32
    L.pa_swap_blocks.argtypes = [ctypes.POINTER(PoolDesc), P, P, P, P, I32, P, I32, I32, P]
    L.pa_validate_tables.restype = I32
    L.pa_validate_tables.argtypes = [ctypes.POINTER(PoolDesc), P, I32, P, I32, I32, P, P]
    L.pa_validate_copy_pairs.restype = I32
    L.pa_validate_copy_pairs.argtypes = [ctypes.POINTER(PoolDesc), P, I32, P, P]
    return L


def single_hip_runtime() -> bool:
    """True when exactly one libamdhip64 is mapped into this process."""
    return len(_hip_runtimes_loaded()) == 1


def status_string(s: int) -> str:
    return lib().pa_status_string(s).decode()


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PaError(fn, status)


# ---- raw entry points (same names and arguments as the C ABI) -------------

def pa_version() -> int:
    return lib().pa_version()


def pa_slot_mapping(block_tables, max_blocks_per_seq, num_seqs, seq_ids, positions, n,
                    block_size, slots, stream) -> int:
    return lib().pa_slot_mapping(block_tables, max_blocks_per_seq, num_seqs, seq_ids, positions,
                                 n, block_size, slots, stream)


def pa_write_kv(desc, k_pool, v_pool, k_new, v_new, new_stride, slot_mapping, n, stream) -> int:
    return lib().pa_write_kv(ctypes.byref(desc), k_pool, v_pool, k_new, v_new, new_stride,
                             slot_mapping, n, stream)


def pa_copy_blocks(desc, k_pool, v_pool, block_pairs, n_pairs, stream) -> int:
    return lib().pa_copy_blocks(ctypes.byref(desc), k_pool, v_pool, block_pairs, n_pairs, stream)


def pa_decode_workspace_size(desc, num_seqs, num_q_heads, max_context_len, partition_size):
    out = ctypes.c_size_t(0)
    st = lib().pa_decode_workspace_size(ctypes.byref(desc), num_seqs, num_q_heads,
                                        max_context_len, partition_size, ctypes.byref(out))
    return st, out.value


def pa_decode_attention(desc, k_pool, v_pool, q, out, out_dtype, block_tables,
                        max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale,
                        max_context_len, partition_size, workspace, workspace_bytes,
                        stream) -> int:
    return lib().pa_decode_attention(ctypes.byref(desc), k_pool, v_pool, q, out, out_dtype,
                                     block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                     num_q_heads, scale, max_context_len, partition_size,
                                     workspace, workspace_bytes, stream)


def pa_decode_step(desc, k_pool, v_pool, k_new, v_new, new_stride, q, out, out_dtype,
                   block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale,
                   max_context_len, partition_size, workspace, workspace_bytes, stream) -> int:
    return lib().pa_decode_step(ctypes.byref(desc), k_pool, v_pool, k_new, v_new, new_stride, q,
                                out, out_dtype, block_tables, max_blocks_per_seq, context_lens,
                                num_seqs, num_q_heads, scale, max_context_len, partition_size,
                                workspace, workspace_bytes, stream)


def pa_decode_step_noalloc(desc, k_pool, v_pool, k_new, v_new, new_stride, q, out, out_dtype,
                           block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                           scale, max_context_len, partition_size, stream) -> int:
    return lib().pa_decode_step_noalloc(ctypes.byref(desc), k_pool, v_pool, k_new, v_new,
                                        new_stride, q, out, out_dtype, block_tables,
                                        max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                        scale, max_context_len, partition_size, stream)


def pa_prefill_attention(desc, k_pool, v_pool, q, out, out_dtype, q_start, block_tables,
                         max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale,
                         max_chunk_len, max_context_len, stream) -> int:
    return lib().pa_prefill_attention(ctypes.byref(desc), k_pool, v_pool, q, out, out_dtype,
                                      q_start, block_tables, max_blocks_per_seq, context_lens,
                                      num_seqs, num_q_heads, scale, max_chunk_len,
                                      max_context_len, stream)


def pa_swap_blocks(desc, k_pool, v_pool, host_k, host_v, host_num_blocks, block_pairs, n_pairs,
                   direction, stream) -> int:
    return lib().pa_swap_blocks(ctypes.byref(desc), k_pool, v_pool, host_k, host_v,
                                host_num_blocks, block_pairs, n_pairs, direction, stream)


def pa_validate_tables(desc, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       max_context_len, bad_count, stream) -> int:
    return lib().pa_validate_tables(ctypes.byref(desc), block_tables, max_blocks_per_seq,
                                    context_lens, num_seqs, max_context_len, bad_count, stream)


def pa_validate_copy_pairs(desc, block_pairs, n_pairs, bad_count, stream) -> int:
    return lib().pa_validate_copy_pairs(ctypes.byref(desc), block_pairs, n_pairs, bad_count, stream)


# ---- torch-tensor helpers ------------------------------------------------------

def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _dev_i32(t, name):
    import torch
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 CUDA tensor")


def make_desc(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str,
              block_size: int = 16, k_scales=None, v_scales=None) -> PoolDesc:
    """k_scales / v_scales: device float32 tensors [Hkv] for FP8 pools (kept
    alive by the caller), else None."""
    return PoolDesc(num_blocks, block_size, num_kv_heads, head_dim, DTYPE_CODES[dtype],
                    _ptr(k_scales) or None, _ptr(v_scales) or None)


def slot_mapping_t(block_tables, seq_ids, positions, slots, block_size: int) -> None:
    for t, nm in ((block_tables, "block_tables"), (seq_ids, "seq_ids"),
                  (positions, "positions"), (slots, "slots")):
        _dev_i32(t, nm)
    n = seq_ids.numel()
    if positions.numel() != n or slots.numel() != n:
        raise ValueError("seq_ids, positions and slots must have one entry per token")
    S, M = block_tables.shape
    _check("pa_slot_mapping", pa_slot_mapping(_ptr(block_tables), M, S, _ptr(seq_ids),
                                               _ptr(positions), n, block_size, _ptr(slots),
                                               _stream()))


def write_kv_t(desc, k_pool, v_pool, k_new, v_new, slots) -> None:
    _dev_i32(slots, "slots")
    n = slots.numel()
    if k_new.shape[0] != n or v_new.shape[0] != n:
        raise ValueError("k_new/v_new need one row per slot")
    if k_new.stride() != v_new.stride() or k_new.stride(-1) != 1:
        raise ValueError("k_new and v_new must share a row stride with contiguous dims")
    _check("pa_write_kv", pa_write_kv(desc, _ptr(k_pool), _ptr(v_pool), _ptr(k_new),
                                       _ptr(v_new), k_new.stride(0), _ptr(slots), n, _stream()))


def copy_blocks_t(desc, k_pool, v_pool, pairs) -> None:
    _dev_i32(pairs, "pairs")
    n = pairs.numel() // 2
    _check("pa_copy_blocks", pa_copy_blocks(desc, _ptr(k_pool), _ptr(v_pool), _ptr(pairs), n,
                                             _stream()))


def workspace_size(desc, num_seqs, num_q_heads, max_context_len, partition_size) -> int:
    st, nbytes = pa_decode_workspace_size(desc, num_seqs, num_q_heads, max_context_len,
                                          partition_size)
    _check("pa_decode_workspace_size", st)
    return nbytes


def decode_attention_t(desc, k_pool, v_pool, q, out, block_tables, context_lens, scale,
                       max_context_len, partition_size=0, workspace=None) -> None:
    import torch
    _dev_i32(block_tables, "block_tables")
    _dev_i32(context_lens, "context_lens")
    if not q.is_contiguous() or not out.is_contiguous():
        raise ValueError("q and out must be contiguous")
    S, Hq, D = q.shape
    out_code = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}[out.dtype]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode_attention",
           pa_decode_attention(desc, _ptr(k_pool), _ptr(v_pool), _ptr(q), _ptr(out), out_code,
                               _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                               S, Hq, float(scale), int(max_context_len), int(partition_size),
                               _ptr(workspace), ws_bytes, _stream()))


def decode_step_t(desc, k_pool, v_pool, k_new, v_new, q, out, block_tables, context_lens, scale,
                  max_context_len, partition_size=0, workspace=None) -> None:
    import torch
    _dev_i32(block_tables, "block_tables")
    _dev_i32(context_lens, "context_lens")
    if not q.is_contiguous() or not out.is_contiguous():
        raise ValueError("q and out must be contiguous")
    if k_new.stride() != v_new.stride() or k_new.stride(-1) != 1:
        raise ValueError("k_new and v_new must share a row stride with contiguous dims")
    S, Hq, D = q.shape
    if k_new.shape[0] != S or v_new.shape[0] != S:
        raise ValueError("k_new / v_new need one row per sequence")
    out_code = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}[out.dtype]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode_step",
           pa_decode_step(desc, _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new),
                          k_new.stride(0), _ptr(q), _ptr(out), out_code, _ptr(block_tables),
                          block_tables.shape[1], _ptr(context_lens), S, Hq, float(scale),
                          int(max_context_len), int(partition_size), _ptr(workspace), ws_bytes,
                          _stream()))


def prefill_attention_t(desc, k_pool, v_pool, q, out, q_start, block_tables, context_lens, scale,
                        max_chunk_len, max_context_len) -> None:
    import torch
    _dev_i32(q_start, "q_start")
    _dev_i32(block_tables, "block_tables")
    _dev_i32(context_lens, "context_lens")
    if not q.is_contiguous() or not out.is_contiguous():
        raise ValueError("q and out must be contiguous")
    if q.shape != out.shape:
        raise ValueError("out must have q's shape")
    S, M = block_tables.shape
    if q_start.numel() != S + 1 or context_lens.numel() != S:
        raise ValueError("q_start needs num_seqs + 1 entries, context_lens num_seqs")
    out_code = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}[out.dtype]
    _check("pa_prefill_attention",
           pa_prefill_attention(desc, _ptr(k_pool), _ptr(v_pool), _ptr(q), _ptr(out), out_code,
                                _ptr(q_start), _ptr(block_tables), M, _ptr(context_lens), S,
                                q.shape[1], float(scale), int(max_chunk_len),
                                int(max_context_len), _stream()))


def swap_blocks_t(desc, k_pool, v_pool, host_k, host_v, host_num_blocks, pairs,
                  direction) -> None:
    _dev_i32(pairs, "pairs")
    if host_k.is_cuda or host_v.is_cuda or not host_k.is_pinned() or not host_v.is_pinned():
        raise ValueError("host pools must be pinned host tensors")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n][2]")
    _check("pa_swap_blocks",
           pa_swap_blocks(desc, _ptr(k_pool), _ptr(v_pool), host_k.data_ptr(), host_v.data_ptr(),
                          int(host_num_blocks), _ptr(pairs), pairs.shape[0], int(direction),
                          _stream()))


def validate_copy_pairs_t(desc, pairs, bad_count) -> None:
    _dev_i32(pairs, "pairs")
    _dev_i32(bad_count, "bad_count")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n][2]")
    _check("pa_validate_copy_pairs", pa_validate_copy_pairs(desc, _ptr(pairs), pairs.shape[0],
                                                             _ptr(bad_count), _stream()))


def validate_tables_t(desc, block_tables, context_lens, max_context_len, bad_count) -> None:
    _dev_i32(block_tables, "block_tables")
    _dev_i32(context_lens, "context_lens")
    _dev_i32(bad_count, "bad_count")
    S, M = block_tables.shape
    _check("pa_validate_tables", pa_validate_tables(desc, _ptr(block_tables), M, _ptr(context_lens),
                                                     S, int(max_context_len), _ptr(bad_count),
                                                     _stream()))
