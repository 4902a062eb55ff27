"""ctypes binding of the native block manager (include/block_manager.h).

``NativeBlockManager`` has the interface of ``block_manager.BlockManager`` (admission, append
with copy-on-write pairs, fork, free, preemption by swap or recompute, swap-in, counters) and
the same semantics; the tests drive both with the same operations and compare every result.
The binding only marshals arguments: all of the bookkeeping runs in the C++ library.
"""
from __future__ import annotations

import ctypes
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from . import ops
from .block_manager import (RECOMPUTE_MODE, SWAP, BlockStats, NoVictim, OutOfBlocks,
                            blocks_for)

BM_OK, BM_INVALID, BM_OUT_OF_BLOCKS, BM_NO_VICTIM, BM_WRONG_STATE = 0, 1, 2, 3, 4

_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
_P64 = ctypes.POINTER(ctypes.c_int64)
_P32 = ctypes.POINTER(ctypes.c_int32)


class _Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_blocks", "free_blocks", "num_cpu_blocks", "free_cpu_blocks",
        "allocation_failures", "cow_copies", "blocks_allocated", "blocks_freed",
        "preemptions_swap", "preemptions_recompute", "blocks_swapped_out", "blocks_swapped_in",
        "tail_waste_slots", "num_sequences", "num_requests")]


class _Plan(ctypes.Structure):
    """pa_sp_plan (block_manager.h), field for field."""
    _fields_ = [("chunk_seqs", _vp), ("chunk_lens", _vp), ("chunk_capacity", _i32),
                ("num_chunks", _i32), ("decode_seqs", _vp), ("decode_capacity", _i32),
                ("num_decodes", _i32), ("slot_mapping", _vp), ("slot_capacity", _i32),
                ("num_slots", _i32), ("cow_pairs", _vp), ("cow_capacity", _i32),
                ("num_cow", _i32)]


_LIB = None


def _bind(lib):
    sig = {
        "pa_bm_create": (_vp, [_i32, _i32, _i32, _vp, _vp]),
        "pa_bm_destroy": (None, [_vp]),
        "pa_bm_add_sequence": (ctypes.c_int, [_vp, _i64, _i64, _vp]),
        "pa_bm_append": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i32, _P32]),
        "pa_bm_fork": (ctypes.c_int, [_vp, _i64, _i64]),
        "pa_bm_free": (ctypes.c_int, [_vp, _i64]),
        "pa_bm_blocks_needed": (_i64, [_vp, _i64, _i64]),
        "pa_bm_seq_info": (ctypes.c_int, [_vp, _i64, _P64, _P32, _P32, _P64, _P64]),
        "pa_bm_table": (ctypes.c_int, [_vp, _i64, _vp, _i32]),
        "pa_bm_block_tables": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp]),
        "pa_bm_refcount": (_i32, [_vp, _i32, _i32]),
        "pa_bm_preempt_latest": (ctypes.c_int, [_vp, _i32, _i64, _P64, _vp, _i32, _P32]),
        "pa_bm_swap_in_earliest": (ctypes.c_int, [_vp, _P64, _vp, _i32, _P32]),
        "pa_bm_resume_recompute": (ctypes.c_int, [_vp, _i64]),
        "pa_bm_request_members": (ctypes.c_int, [_vp, _i64, _vp, _i32, _P32]),
        "pa_bm_get_stats": (ctypes.c_int, [_vp, ctypes.POINTER(_Stats)]),
        "pa_bm_last_error": (ctypes.c_char_p, []),
        "pa_sp_create": (_vp, [_vp, _i32, _i32]),
        "pa_sp_destroy": (None, [_vp]),
        "pa_sp_set_limits": (ctypes.c_int, [_vp, _i32, _i32]),
        "pa_sp_add_request": (ctypes.c_int, [_vp, _i64, _i64]),
        "pa_sp_finish": (ctypes.c_int, [_vp, _i64]),
        "pa_sp_counts": (ctypes.c_int, [_vp, _P32, _P32]),
        "pa_sp_step": (ctypes.c_int, [_vp, ctypes.POINTER(_Plan)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def _lib():
    global _LIB
    if _LIB is None:
        _LIB = _bind(ops.load_library())
    return _LIB


def use_library(path: str) -> None:
    """Bind the block manager to another build of block_manager.cpp (for example one built
    with host sanitizers); it must export the pa_bm_* functions of block_manager.h."""
    global _LIB
    _LIB = _bind(ctypes.CDLL(path))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class NativeBlockManager:
    """The C++ block manager behind the Python ``BlockManager`` interface."""

    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order: Optional[Sequence[int]] = None, num_cpu_blocks: int = 0,
                 cpu_free_order: Optional[Sequence[int]] = None):
        lib = _lib()
        fo = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        co = None if cpu_free_order is None else np.ascontiguousarray(cpu_free_order,
                                                                       dtype=np.int32)
        if fo is not None and fo.size != num_blocks:
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        if co is not None and co.size != num_cpu_blocks:
            raise ValueError("cpu_free_order must be a permutation of range(num_cpu_blocks)")
        h = lib.pa_bm_create(int(num_blocks), int(num_cpu_blocks), int(block_size), _ptr(fo),
                             _ptr(co))
        if not h:
            raise ValueError(lib.pa_bm_last_error().decode())
        self._h = ctypes.c_void_p(h)
        self.num_blocks = int(num_blocks)
        self.num_cpu_blocks = int(num_cpu_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _LIB is not None:
            _LIB.pa_bm_destroy(h)
            self._h = None

    # ------------------------------------------------------------------ helpers
    def _check(self, st: int) -> None:
        if st == BM_OK:
            return
        msg = _lib().pa_bm_last_error().decode()
        if st == BM_OUT_OF_BLOCKS:
            raise OutOfBlocks(msg)
        if st == BM_NO_VICTIM:
            raise NoVictim(msg)
        if st == BM_WRONG_STATE:
            raise ValueError(msg)
        if "unknown sequence" in msg:
            raise KeyError(msg)
        raise ValueError(msg)

    def _info(self, seq_id: int):
        L, n, st, r, rt = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32(), \
            ctypes.c_int64(), ctypes.c_int64()
        self._check(_lib().pa_bm_seq_info(self._h, int(seq_id), ctypes.byref(L), ctypes.byref(n),
                                          ctypes.byref(st), ctypes.byref(r), ctypes.byref(rt)))
        return L.value, n.value, st.value, r.value, rt.value

    def _stats(self) -> _Stats:
        s = _Stats()
        self._check(_lib().pa_bm_get_stats(self._h, ctypes.byref(s)))
        return s

    # ------------------------------------------------------------------ queries
    @property
    def num_free(self) -> int:
        return int(self._stats().free_blocks)

    @property
    def num_used(self) -> int:
        return self.num_blocks - self.num_free

    @property
    def num_free_cpu(self) -> int:
        return int(self._stats().free_cpu_blocks)

    @property
    def stats(self) -> BlockStats:
        s = self._stats()
        return BlockStats(allocation_failures=s.allocation_failures, cow_copies=s.cow_copies,
                          blocks_allocated=s.blocks_allocated, blocks_freed=s.blocks_freed,
                          preemptions_swap=s.preemptions_swap,
                          preemptions_recompute=s.preemptions_recompute,
                          blocks_swapped_out=s.blocks_swapped_out,
                          blocks_swapped_in=s.blocks_swapped_in)

    def refcount(self, block: int) -> int:
        return int(_lib().pa_bm_refcount(self._h, int(block), 0))

    def cpu_refcount(self, block: int) -> int:
        return int(_lib().pa_bm_refcount(self._h, int(block), 1))

    def seq_len(self, seq_id: int) -> int:
        return self._info(seq_id)[0]

    def state(self, seq_id: int) -> int:
        return self._info(seq_id)[2]

    def request_of(self, seq_id: int) -> int:
        return self._info(seq_id)[3]

    def recompute_tokens(self, seq_id: int) -> int:
        return self._info(seq_id)[4]

    def has(self, seq_id: int) -> bool:
        return _lib().pa_bm_seq_info(self._h, int(seq_id), None, None, None, None, None) == 0

    def table(self, seq_id: int) -> List[int]:
        n = self._info(seq_id)[1]
        out = np.empty(max(n, 1), dtype=np.int32)
        self._check(_lib().pa_bm_table(self._h, int(seq_id), _ptr(out), n))
        return out[:n].tolist()

    def members(self, request: int) -> List[int]:
        cnt = ctypes.c_int32()
        _lib().pa_bm_request_members(self._h, int(request), None, 0, ctypes.byref(cnt))
        out = np.empty(max(cnt.value, 1), dtype=np.int64)
        self._check(_lib().pa_bm_request_members(self._h, int(request), _ptr(out), cnt.value,
                                                 ctypes.byref(cnt)))
        return out[:cnt.value].tolist()

    def tail_waste_total(self) -> int:
        return int(self._stats().tail_waste_slots)

    def block_tables(self, seq_ids: Iterable[int], width: Optional[int] = None) -> np.ndarray:
        ids = np.ascontiguousarray(list(seq_ids), dtype=np.int64)
        if width is None:
            width = max((self._info(s)[1] for s in ids), default=0)
        out = np.full((ids.size, max(int(width), 1)), -1, dtype=np.int32)
        self._check(_lib().pa_bm_block_tables(self._h, _ptr(ids), ids.size, out.shape[1],
                                              _ptr(out)))
        return out

    def blocks_needed(self, seq_id: int, num_new: int) -> int:
        n = int(_lib().pa_bm_blocks_needed(self._h, int(seq_id), int(num_new)))
        if n < 0:
            raise ValueError(f"sequence {seq_id} unknown or not resident")
        return n

    def can_allocate(self, num_tokens: int) -> bool:
        return blocks_for(num_tokens, self.block_size) <= self.num_free

    # ------------------------------------------------------------- allocation
    def add_sequence(self, seq_id: int, num_tokens: int = 0) -> List[int]:
        slots = np.empty(max(int(num_tokens), 1), dtype=np.int64)
        self._check(_lib().pa_bm_add_sequence(self._h, int(seq_id), int(num_tokens),
                                              _ptr(slots)))
        return slots[:int(num_tokens)].tolist()

    def append_tokens(self, seq_id: int, num_new: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        slots = np.empty(max(int(num_new), 1), dtype=np.int64)
        pairs = np.empty(2, dtype=np.int64)
        n = ctypes.c_int32(0)
        self._check(_lib().pa_bm_append(self._h, int(seq_id), int(num_new), _ptr(slots),
                                        _ptr(pairs), 1, ctypes.byref(n)))
        return slots[:int(num_new)].tolist(), [(int(pairs[0]), int(pairs[1]))][:n.value]

    def fork(self, parent: int, child: int) -> None:
        self._check(_lib().pa_bm_fork(self._h, int(parent), int(child)))

    def free(self, seq_id: int) -> None:
        self._check(_lib().pa_bm_free(self._h, int(seq_id)))

    # -------------------------------------------------------------- preemption
    def _pairs_call(self, fn, *args) -> Tuple[int, List[Tuple[int, int]]]:
        cap = self.num_blocks + self.num_cpu_blocks
        buf = np.empty(2 * max(cap, 1), dtype=np.int64)
        r = ctypes.c_int64(-1)
        n = ctypes.c_int32(0)
        self._check(fn(self._h, *args, ctypes.byref(r), _ptr(buf), cap, ctypes.byref(n)))
        p = buf[:2 * n.value].reshape(-1, 2)
        return r.value, [(int(a), int(b)) for a, b in p]

    def preempt_latest(self, mode: int = SWAP,
                       protect: Optional[int] = None) -> Tuple[int, List[Tuple[int, int]]]:
        if mode not in (SWAP, RECOMPUTE_MODE):
            raise ValueError("mode must be SWAP or RECOMPUTE_MODE")
        return self._pairs_call(_lib().pa_bm_preempt_latest, int(mode),
                                -1 if protect is None else int(protect))

    def swap_in_earliest(self) -> Tuple[int, List[Tuple[int, int]]]:
        return self._pairs_call(_lib().pa_bm_swap_in_earliest)

    def resume_recompute(self, request: int) -> List[Tuple[int, int]]:
        self._check(_lib().pa_bm_resume_recompute(self._h, int(request)))
        return [(s, self.recompute_tokens(s)) for s in self.members(request)]


class NativeStepPlanner:
    """The C++ step planner (pa_sp_*) behind the interface of ``step_planner.StepPlanner``:
    add_request, finish and step() returning a ``StepPlan``."""

    def __init__(self, bm: NativeBlockManager, max_tokens_per_step: int,
                 max_chunk: Optional[int] = None):
        lib = _lib()
        h = lib.pa_sp_create(bm._h, int(max_tokens_per_step),
                             0 if max_chunk is None else int(max_chunk))
        if not h:
            raise ValueError(lib.pa_bm_last_error().decode())
        self._h = ctypes.c_void_p(h)
        self.bm = bm                      # keeps the manager alive as long as the planner
        self.max_tokens = int(max_tokens_per_step)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _LIB is not None:
            _LIB.pa_sp_destroy(h)
            self._h = None

    def counts(self) -> Tuple[int, int]:
        d, p = ctypes.c_int32(), ctypes.c_int32()
        self.bm._check(_lib().pa_sp_counts(self._h, ctypes.byref(d), ctypes.byref(p)))
        return d.value, p.value

    def set_limits(self, max_tokens_per_step: int, max_chunk: Optional[int] = None) -> None:
        self.bm._check(_lib().pa_sp_set_limits(self._h, int(max_tokens_per_step),
                                               0 if max_chunk is None else int(max_chunk)))
        self.max_tokens = int(max_tokens_per_step)

    def add_request(self, seq_id: int, prompt_len: int) -> None:
        self.bm._check(_lib().pa_sp_add_request(self._h, int(seq_id), int(prompt_len)))

    def finish(self, seq_id: int) -> None:
        self.bm._check(_lib().pa_sp_finish(self._h, int(seq_id)))

    def step(self):
        from .step_planner import StepPlan
        nd, npre = self.counts()
        cs = np.empty(max(npre, 1), np.int64)
        cl = np.empty(max(npre, 1), np.int64)
        ds = np.empty(max(nd, 1), np.int64)
        ns = max(nd, self.max_tokens)
        sm = np.empty(max(ns, 1), np.int64)
        cp = np.empty(2 * max(nd + npre, 1), np.int64)
        plan = _Plan(_ptr(cs), _ptr(cl), npre, 0, _ptr(ds), nd, 0, _ptr(sm), ns, 0, _ptr(cp),
                     nd + npre, 0)
        self.bm._check(_lib().pa_sp_step(self._h, ctypes.byref(plan)))
        return StepPlan(chunk_seqs=cs[:plan.num_chunks].tolist(),
                        chunk_lens=cl[:plan.num_chunks].tolist(),
                        decode_seqs=ds[:plan.num_decodes].tolist(),
                        slot_mapping=sm[:plan.num_slots].copy(),
                        cow_pairs=[(int(a), int(b)) for a, b in
                                   cp[:2 * plan.num_cow].reshape(-1, 2)])
