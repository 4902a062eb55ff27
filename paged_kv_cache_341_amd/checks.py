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
