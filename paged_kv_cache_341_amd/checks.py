"""Host-side checks of the device-content preconditions the kernels rely on.

The C ABI validates scalars only; table entries, lengths, slots and copy pairs are read on the
device without bounds checks.  These functions check them on host copies and raise ValueError,
so a caller (and every GPU test) can refuse a launch that would read or write out of range.
"""
from __future__ import annotations

import numpy as np


def check_tables(block_tables: np.ndarray, seq_lens: np.ndarray, num_blocks: int,
                 block_size: int, max_seq_len: int) -> None:
    bt = np.asarray(block_tables)
    sl = np.asarray(seq_lens)
    if bt.ndim != 2 or sl.ndim != 1 or bt.shape[0] != sl.shape[0]:
        raise ValueError("block_tables must be [S, MB] and seq_lens [S]")
    if sl.size and (sl.min() < 1 or sl.max() > max_seq_len):
        raise ValueError("seq_lens must lie in [1, max_seq_len]")
    if max_seq_len > bt.shape[1] * block_size:
        raise ValueError("max_seq_len exceeds the table width")
    for s, L in enumerate(sl):
        used = bt[s, :-(-int(L) // block_size)]
        if used.size and (used.min() < 0 or used.max() >= num_blocks):
            raise ValueError(f"sequence {s}: block id out of range")


def check_groups(group_start: np.ndarray, shared_blocks: np.ndarray, block_tables: np.ndarray,
                 seq_lens: np.ndarray, block_size: int, max_group_size: int) -> None:
    """The grouped decode's preconditions: groups cover the batch in order, and each group's
    members agree on the shared prefix and its block ids, which are full blocks of every
    member.  (The kernels clamp what they read, so a breach gives wrong values, not faults.)"""
    gs = np.asarray(group_start, dtype=np.int64)
    sb = np.asarray(shared_blocks, dtype=np.int64)
    bt = np.asarray(block_tables)
    sl = np.asarray(seq_lens, dtype=np.int64)
    S = sl.shape[0]
    if gs.ndim != 1 or gs.size < 2 or gs[0] != 0 or gs[-1] != S or np.any(np.diff(gs) < 1):
        raise ValueError("group_start must rise strictly from 0 to num_seqs")
    if np.diff(gs).max() > max_group_size:
        raise ValueError("a group is larger than max_group_size")
    if sb.shape != (S,) or sb.min() < 0 or np.any(sb * block_size > sl):
        raise ValueError("shared_blocks must lie in [0, seq_len // block_size]")
    for g in range(gs.size - 1):
        a, b = int(gs[g]), int(gs[g + 1])
        n = int(sb[a])
        if np.any(sb[a:b] != n):
            raise ValueError(f"group {g}: members disagree on shared_blocks")
        if n and np.any(bt[a:b, :n] != bt[a, :n]):
            raise ValueError(f"group {g}: members' shared table entries differ")


def check_chunks(query_start_loc: np.ndarray, seq_lens: np.ndarray, total_q: int,
                 max_q_len: int) -> None:
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    if qsl[0] != 0 or qsl[-1] != total_q or np.any(np.diff(qsl) < 0):
        raise ValueError("query_start_loc must rise from 0 to total_q")
    n = np.diff(qsl)
    if n.size and n.max() > max_q_len:
        raise ValueError("a chunk has more rows than max_q_len")
    if np.any(n > np.asarray(seq_lens)):
        raise ValueError("a chunk has more rows than its sequence")


def check_slots(slot_mapping: np.ndarray, num_blocks: int, block_size: int) -> None:
    s = np.asarray(slot_mapping, dtype=np.int64)
    live = s[s >= 0]
    if live.size and live.max() >= num_blocks * block_size:
        raise ValueError("slot out of range")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slots")


def check_pairs(pairs: np.ndarray, num_blocks: int) -> None:
    p = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if p.size == 0:
        return
    if p.min() < 0 or p.max() >= num_blocks:
        raise ValueError("block id out of range")
    if np.unique(p[:, 1]).size != p.shape[0]:
        raise ValueError("duplicate destination")
    if np.intersect1d(p[:, 0], p[:, 1]).size:
        raise ValueError("a destination is also a source")


def check_swap_pairs(pairs: np.ndarray, num_src_blocks: int, num_dst_blocks: int) -> None:
    p = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if p.size == 0:
        return
    if p[:, 0].min() < 0 or p[:, 0].max() >= num_src_blocks:
        raise ValueError("source block id out of range")
    if p[:, 1].min() < 0 or p[:, 1].max() >= num_dst_blocks:
        raise ValueError("destination block id out of range")
    if np.unique(p[:, 1]).size != p.shape[0]:
        raise ValueError("duplicate destination")
