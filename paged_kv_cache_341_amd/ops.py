"""ctypes binding of libpagedattn.so: torch tensors in, C-ABI calls out.

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
The functions carry the C names (pa_decode, pa_prefill_chunk, kv_append, cow_copy_blocks) and
enqueue on torch's current HIP stream of the tensors' device.  A missing library or a non-zero
status raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PA_OK = 0
PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_INVALID_ARGUMENT", 2: "PA_ERR_UNSUPPORTED",
                3: "PA_ERR_WORKSPACE_TOO_SMALL", 4: "PA_ERR_DEVICE"}

EXPORTED = ("pa_decode", "pa_decode_workspace_size", "pa_decode_contiguous", "pa_decode_noalloc",
            "pa_decode_grouped",
            "pa_decode_grouped_workspace_size", "pa_mixed_step", "pa_mixed_workspace_size",
            "pa_prefill_chunk",
            "pa_prefill_workspace_size", "kv_append", "cow_copy_blocks", "pa_status_string",
            "pa_last_error", "pa_hbm_read_probe", "swap_blocks", "pa_set_checked_mode",
            "pa_checked_mode", "pa_mfma_probe")
# the native block manager (include/block_manager.h), bound in native_block_manager.py
BM_EXPORTED = ("pa_bm_create", "pa_bm_destroy", "pa_bm_add_sequence", "pa_bm_append",
               "pa_bm_fork", "pa_bm_free", "pa_bm_blocks_needed", "pa_bm_seq_info",
               "pa_bm_table", "pa_bm_block_tables", "pa_bm_refcount", "pa_bm_preempt_latest",
               "pa_bm_swap_in_earliest", "pa_bm_resume_recompute", "pa_bm_request_members",
               "pa_bm_get_stats", "pa_bm_last_error", "pa_sp_create", "pa_sp_destroy",
               "pa_sp_set_limits", "pa_sp_add_request", "pa_sp_finish", "pa_sp_counts", "pa_sp_step")


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None

_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t


class MixedBatch(ctypes.Structure):
    """pa_mixed_batch (pagedattn.h), field for field."""
    _fields_ = [
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("slot_mapping", ctypes.c_void_p),
        ("num_new_tokens", ctypes.c_int32),
        ("chunk_out", ctypes.c_void_p), ("chunk_q", ctypes.c_void_p),
        ("chunk_tables", ctypes.c_void_p), ("chunk_seq_lens", ctypes.c_void_p),
        ("query_start_loc", ctypes.c_void_p), ("num_chunks", ctypes.c_int32),
        ("chunk_total_q", ctypes.c_int32), ("chunk_max_q_len", ctypes.c_int32),
        ("chunk_max_seq_len", ctypes.c_int32), ("chunk_max_blocks_per_seq", ctypes.c_int32),
        ("dec_out", ctypes.c_void_p), ("dec_q", ctypes.c_void_p), ("dec_tables", ctypes.c_void_p),
        ("dec_seq_lens", ctypes.c_void_p), ("num_seqs", ctypes.c_int32),
        ("dec_max_seq_len", ctypes.c_int32), ("dec_max_blocks_per_seq", ctypes.c_int32),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("scale", ctypes.c_float), ("dtype", ctypes.c_int),
    ]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the C ABI.  Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m paged_kv_cache_341_amd.build_lib` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                              _i32, _i32, _f32, ctypes.c_int, _vp, _sz, _vp]
    lib.pa_decode_workspace_size.restype = _sz
    lib.pa_decode_workspace_size.argtypes = [_i32] * 6
    lib.pa_decode_contiguous.restype = ctypes.c_int
    lib.pa_decode_contiguous.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _f32, ctypes.c_int, _vp, _sz, _vp]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _f32, ctypes.c_int, _vp]
    lib.pa_decode_grouped.restype = ctypes.c_int
    lib.pa_decode_grouped.argtypes = [_vp] * 8 + [_i32] * 10 + [_f32, ctypes.c_int, _vp, _sz,
                                                                _vp]
    lib.pa_decode_grouped_workspace_size.restype = _sz
    lib.pa_decode_grouped_workspace_size.argtypes = [_i32] * 6
    lib.pa_prefill_chunk.restype = ctypes.c_int
    lib.pa_prefill_chunk.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp] + [_i32] * 10 + \
        [_f32, ctypes.c_int, _vp, _sz, _vp]
    lib.pa_prefill_workspace_size.restype = _sz
    lib.pa_prefill_workspace_size.argtypes = [_i32] * 5
    lib.kv_append.restype = ctypes.c_int
    lib.kv_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                              ctypes.c_int, _vp]
    lib.cow_copy_blocks.restype = ctypes.c_int
    lib.cow_copy_blocks.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_int,
                                    _vp]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_mixed_step.restype = ctypes.c_int
    lib.pa_mixed_step.argtypes = [ctypes.POINTER(MixedBatch), _vp, _sz, _vp]
    lib.pa_mixed_workspace_size.restype = _sz
    lib.pa_mixed_workspace_size.argtypes = [_i32] * 6
    lib.swap_blocks.restype = ctypes.c_int
    lib.swap_blocks.argtypes = [_vp] * 5 + [_i32] * 6 + [ctypes.c_int, _vp]
    lib.pa_hbm_read_probe.restype = ctypes.c_int
    lib.pa_hbm_read_probe.argtypes = [_vp, _sz, _vp, _i32, _vp]
    lib.pa_mfma_probe.restype = ctypes.c_int
    lib.pa_mfma_probe.argtypes = [_vp, _i32, _i32, _vp]
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_set_checked_mode.restype = ctypes.c_int
    lib.pa_set_checked_mode.argtypes = [ctypes.c_int]
    lib.pa_checked_mode.restype = ctypes.c_int
    lib.pa_checked_mode.argtypes = []
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != PA_OK:
        msg = load_library().pa_last_error().decode()
        raise PagedAttnError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    if t.dtype == torch.float32:
        return PA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor, stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    if t.is_cuda:
        return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _need(cond: bool, what: str) -> None:
    if not cond:
        raise ValueError(what)


def _contig(*ts) -> None:
    for t in ts:
        _need(t.is_contiguous(), "tensors must be contiguous")


def pa_decode_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                             block_size: int, max_seq_len: int) -> int:
    return int(load_library().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                       head_dim, block_size, max_seq_len))


def pa_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, scale: float,
              workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[s, h] = attention of q[s, h] over sequence s's cached tokens (see pagedattn.h)."""
    lib = load_library()
    _contig(out, q, k_cache, v_cache, block_tables, seq_lens)
    _need(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32,
          "block_tables and seq_lens must be int32")
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    _need(D2 == D and tuple(v_cache.shape) == tuple(k_cache.shape), "cache shape mismatch")
    _need(tuple(out.shape) == tuple(q.shape), "out must match q")
    _need(out.dtype == q.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
    ws_need = pa_decode_workspace_size(S, Hq, Hkv, D, B, max_seq_len)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                       _ptr(seq_lens), S, Hq, Hkv, D, B, NB, block_tables.shape[1],
                       int(max_seq_len), float(scale), _dtype_code(q), _ptr(workspace),
                       ws_bytes, _stream(q, stream))
    _check(st)
    return out


def pa_decode_contiguous(out: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode over contiguous KV: k, v [num_seqs, num_kv_heads, capacity, head_dim], row j of
    (s, kv head) is token j (see pagedattn.h)."""
    lib = load_library()
    _contig(out, q, k, v, seq_lens)
    _need(seq_lens.dtype == torch.int32, "seq_lens must be int32")
    S, Hq, D = q.shape
    S2, Hkv, cap, D2 = k.shape
    _need(S2 == S and D2 == D and tuple(v.shape) == tuple(k.shape), "k/v shape mismatch")
    _need(tuple(out.shape) == tuple(q.shape), "out must match q")
    _need(out.dtype == q.dtype == k.dtype == v.dtype, "dtypes must match")
    ws_need = pa_decode_workspace_size(S, Hq, Hkv, D, 16, max_seq_len)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_decode_contiguous(_ptr(out), _ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), S, Hq,
                                  Hkv, D, cap, int(max_seq_len), float(scale), _dtype_code(q),
                                  _ptr(workspace), ws_bytes, _stream(q, stream))
    _check(st)
    return out


# Bytes of the library's static scratch behind pa_decode_noalloc (PA_DECODE_NOALLOC_SCRATCH_BYTES
# in pagedattn.h).
DECODE_NOALLOC_SCRATCH_BYTES = 128 << 20


def pa_decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                      max_seq_len: int, scale: float, stream=None) -> torch.Tensor:
    """pa_decode without a workspace: the split partials go to the library's static scratch
    (see pagedattn.h).  Allocates nothing; calls that overlap on one GPU race."""
    lib = load_library()
    _contig(out, q, k_cache, v_cache, block_tables, seq_lens)
    _need(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32,
          "block_tables and seq_lens must be int32")
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    _need(D2 == D and tuple(v_cache.shape) == tuple(k_cache.shape), "cache shape mismatch")
    _need(tuple(out.shape) == tuple(q.shape), "out must match q")
    _need(out.dtype == q.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
    st = lib.pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_tables), _ptr(seq_lens), S, Hq, Hkv, D, B, NB,
                               block_tables.shape[1], int(max_seq_len), float(scale),
                               _dtype_code(q), _stream(q, stream))
    _check(st)
    return out


def pa_decode_grouped_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                    head_dim: int, block_size: int, max_seq_len: int) -> int:
    return int(load_library().pa_decode_grouped_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len))


def pa_decode_grouped(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                      group_start: torch.Tensor, shared_blocks: torch.Tensor,
                      max_group_size: int, max_seq_len: int, scale: float,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_decode for sequences grouped by a shared block prefix (see pagedattn.h)."""
    lib = load_library()
    _contig(out, q, k_cache, v_cache, block_tables, seq_lens, group_start, shared_blocks)
    _need(all(t.dtype == torch.int32 for t in (block_tables, seq_lens, group_start,
                                                shared_blocks)),
          "block_tables, seq_lens, group_start and shared_blocks must be int32")
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    _need(D2 == D and tuple(v_cache.shape) == tuple(k_cache.shape), "cache shape mismatch")
    _need(tuple(out.shape) == tuple(q.shape), "out must match q")
    _need(out.dtype == q.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
    _need(shared_blocks.numel() == S, "shared_blocks needs one entry per sequence")
    ws_need = pa_decode_grouped_workspace_size(S, Hq, Hkv, D, B, max_seq_len)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_decode_grouped(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_tables), _ptr(seq_lens), _ptr(group_start),
                               _ptr(shared_blocks), S, group_start.numel() - 1,
                               int(max_group_size), Hq, Hkv, D, B, NB, block_tables.shape[1],
                               int(max_seq_len), float(scale), _dtype_code(q), _ptr(workspace),
                               ws_bytes, _stream(q, stream))
    _check(st)
    return out


def pa_mixed_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            block_size: int, dec_max_seq_len: int) -> int:
    return int(load_library().pa_mixed_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                       head_dim, block_size, dec_max_seq_len))


def pa_mixed_step(k_cache: torch.Tensor, v_cache: torch.Tensor, scale: float, *,
                  k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                  slot_mapping: Optional[torch.Tensor] = None,
                  chunk_out: Optional[torch.Tensor] = None, chunk_q: Optional[torch.Tensor] = None,
                  chunk_tables: Optional[torch.Tensor] = None,
                  chunk_seq_lens: Optional[torch.Tensor] = None,
                  query_start_loc: Optional[torch.Tensor] = None, chunk_max_q_len: int = 0,
                  chunk_max_seq_len: int = 0, dec_out: Optional[torch.Tensor] = None,
                  dec_q: Optional[torch.Tensor] = None, dec_tables: Optional[torch.Tensor] = None,
                  dec_seq_lens: Optional[torch.Tensor] = None, dec_max_seq_len: int = 0,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Append, chunk attention and decode attention of one iteration (see pagedattn.h)."""
    lib = load_library()
    _contig(k_cache, v_cache)
    NB, Hkv, B, D = k_cache.shape
    b = MixedBatch()
    b.k_cache, b.v_cache = _ptr(k_cache), _ptr(v_cache)
    b.num_kv_heads, b.head_dim, b.block_size, b.num_blocks = Hkv, D, B, NB
    b.scale, b.dtype = float(scale), _dtype_code(k_cache)
    Hq = None
    if slot_mapping is not None and slot_mapping.numel() > 0:
        _contig(k_new, v_new, slot_mapping)
        _need(slot_mapping.dtype == torch.int64, "slot_mapping must be int64")
        b.k_new, b.v_new, b.slot_mapping = _ptr(k_new), _ptr(v_new), _ptr(slot_mapping)
        b.num_new_tokens = slot_mapping.numel()
    if chunk_q is not None and chunk_q.shape[0] > 0:
        _contig(chunk_out, chunk_q, chunk_tables, chunk_seq_lens, query_start_loc)
        _need(all(t.dtype == torch.int32 for t in (chunk_tables, chunk_seq_lens,
                                                    query_start_loc)), "chunk indices must be int32")
        Hq = chunk_q.shape[1]
        b.chunk_out, b.chunk_q = _ptr(chunk_out), _ptr(chunk_q)
        b.chunk_tables, b.chunk_seq_lens = _ptr(chunk_tables), _ptr(chunk_seq_lens)
        b.query_start_loc = _ptr(query_start_loc)
        b.num_chunks, b.chunk_total_q = chunk_seq_lens.numel(), chunk_q.shape[0]
        b.chunk_max_q_len, b.chunk_max_seq_len = int(chunk_max_q_len), int(chunk_max_seq_len)
        b.chunk_max_blocks_per_seq = chunk_tables.shape[1]
    if dec_q is not None and dec_q.shape[0] > 0:
        _contig(dec_out, dec_q, dec_tables, dec_seq_lens)
        _need(dec_tables.dtype == torch.int32 and dec_seq_lens.dtype == torch.int32,
              "decode indices must be int32")
        _need(Hq is None or Hq == dec_q.shape[1], "chunk and decode head counts differ")
        Hq = dec_q.shape[1]
        b.dec_out, b.dec_q = _ptr(dec_out), _ptr(dec_q)
        b.dec_tables, b.dec_seq_lens = _ptr(dec_tables), _ptr(dec_seq_lens)
        b.num_seqs, b.dec_max_seq_len = dec_seq_lens.numel(), int(dec_max_seq_len)
        b.dec_max_blocks_per_seq = dec_tables.shape[1]
    b.num_q_heads = Hkv if Hq is None else Hq
    need = pa_mixed_workspace_size(b.num_seqs, b.num_q_heads, Hkv, D, B, b.dec_max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=k_cache.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.pa_mixed_step(ctypes.byref(b), _ptr(workspace), ws_bytes, _stream(k_cache, stream)))


def pa_prefill_chunk(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                     v_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                     query_start_loc: torch.Tensor, max_q_len: int, max_seq_len: int,
                     scale: float, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Chunk attention over paged prefixes, causal inside each chunk (see pagedattn.h)."""
    lib = load_library()
    _contig(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc)
    _need(block_tables.dtype == seq_lens.dtype == query_start_loc.dtype == torch.int32,
          "index tensors must be int32")
    T, Hq, D = q.shape
    NB, Hkv, B, _ = k_cache.shape
    C = seq_lens.shape[0]
    _need(query_start_loc.shape[0] == C + 1, "query_start_loc must have num_chunks + 1 entries")
    _need(tuple(out.shape) == tuple(q.shape), "out must match q")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_prefill_chunk(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_tables), _ptr(seq_lens), _ptr(query_start_loc), C, T,
                              int(max_q_len), int(max_seq_len), Hq, Hkv, D, B, NB,
                              block_tables.shape[1], float(scale), _dtype_code(q),
                              _ptr(workspace), ws_bytes, _stream(q, stream))
    _check(st)
    return out


def kv_append(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
              v_new: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Write k_new[t], v_new[t] into slot slot_mapping[t] of the pool (see pagedattn.h)."""
    lib = load_library()
    _contig(k_cache, v_cache, k_new, v_new, slot_mapping)
    _need(slot_mapping.dtype == torch.int64, "slot_mapping must be int64")
    NB, Hkv, B, D = k_cache.shape
    T = k_new.shape[0]
    _need(tuple(k_new.shape) == (T, Hkv, D) and tuple(v_new.shape) == (T, Hkv, D),
          "k_new/v_new must be [T, num_kv_heads, head_dim]")
    _need(slot_mapping.shape[0] == T, "slot_mapping must have one entry per token")
    st = lib.kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                       _ptr(slot_mapping), T, Hkv, D, B, NB, _dtype_code(k_cache),
                       _stream(k_cache, stream))
    _check(st)


def cow_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_pairs: torch.Tensor,
                    stream=None) -> None:
    """k_cache[dst] = k_cache[src] (and V) for every (src, dst) pair (see pagedattn.h)."""
    lib = load_library()
    _contig(k_cache, v_cache, block_pairs)
    _need(block_pairs.dtype == torch.int64, "block_pairs must be int64 [P, 2]")
    NB, Hkv, B, D = k_cache.shape
    P = block_pairs.shape[0]
    st = lib.cow_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_pairs), P, Hkv, D, B, NB,
                             _dtype_code(k_cache), _stream(k_cache, stream))
    _check(st)


def swap_blocks(dst_k: torch.Tensor, dst_v: torch.Tensor, src_k: torch.Tensor,
                src_v: torch.Tensor, block_pairs: torch.Tensor, stream=None) -> None:
    """dst[pairs[p][1]] = src[pairs[p][0]] (K and V) between a device pool and a pinned host
    pool, either direction (see pagedattn.h); enqueued on the device pool's stream."""
    lib = load_library()
    _contig(dst_k, dst_v, src_k, src_v, block_pairs)
    _need(block_pairs.dtype == torch.int64, "block_pairs must be int64 [P, 2]")
    _need(tuple(dst_k.shape[1:]) == tuple(src_k.shape[1:]) and dst_k.shape == dst_v.shape
          and src_k.shape == src_v.shape, "pool shapes differ")
    _need(dst_k.dtype == src_k.dtype == dst_v.dtype == src_v.dtype, "dtypes must match")
    dev = dst_k if dst_k.is_cuda else src_k
    host = src_k if dst_k.is_cuda else dst_k
    _need(dev.is_cuda and (host.is_cuda or host.is_pinned()),
          "one pool must be on the device and the other on the device or in pinned host memory")
    _need(block_pairs.is_cuda or block_pairs.is_pinned(),
          "block_pairs must be device or pinned host memory")
    _, Hkv, B, D = dst_k.shape
    st = lib.swap_blocks(_ptr(dst_k), _ptr(dst_v), _ptr(src_k), _ptr(src_v), _ptr(block_pairs),
                         block_pairs.shape[0], Hkv, D, B, src_k.shape[0], dst_k.shape[0],
                         _dtype_code(dev), _stream(dev, stream))
    _check(st)


def pa_hbm_read_probe(src: torch.Tensor, sink: torch.Tensor, num_workgroups: int,
                      stream=None) -> None:
    """Stream all of `src` through the read probe; `sink` holds num_workgroups * 256 int32."""
    lib = load_library()
    _contig(src, sink)
    nbytes = src.numel() * src.element_size()
    _need(sink.numel() * sink.element_size() >= num_workgroups * 256 * 4, "sink too small")
    _check(lib.pa_hbm_read_probe(_ptr(src), nbytes, _ptr(sink), int(num_workgroups),
                                 _stream(src, stream)))


def set_checked_mode(enable: bool) -> bool:
    """Turn the library's checked mode on or off (see pagedattn.h); returns the previous
    setting."""
    return bool(load_library().pa_set_checked_mode(1 if enable else 0))


def checked_mode() -> bool:
    return bool(load_library().pa_checked_mode())


def pa_mfma_probe(sink: torch.Tensor, num_workgroups: int, iters: int, stream=None) -> None:
    """Diagnostic: matrix-core loop of num_workgroups x 512 lanes (see pagedattn.h)."""
    lib = load_library()
    _need(sink.dtype == torch.float32 and sink.numel() >= num_workgroups * 512,
          "sink must hold num_workgroups * 512 floats")
    _check(lib.pa_mfma_probe(_ptr(sink), int(num_workgroups), int(iters), _stream(sink, stream)))


def status_string(status: int) -> str:
    return load_library().pa_status_string(status).decode()


def to_device_index(a: np.ndarray, device, dtype=torch.int32) -> torch.Tensor:
    """Host index array -> contiguous device tensor of the given integer type."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype=dtype).to(device)
