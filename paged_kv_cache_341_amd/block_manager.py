"""Host-side allocator for a paged KV pool: free list, block tables, refcounts, fork, copy-on-write.

What the pages describe, restated:
  * The pool is a set of equal, fixed-size physical blocks (16 tokens by default).  A sequence
    sees logical blocks filled left to right; a per-sequence block table maps each logical block
    to the physical block that holds it.  (study-docs "PagedAttention & Continuous Batching",
    section "Block tables"; cloudmash "Batching and PagedAttention", section "PagedAttention",
    numbered steps 1-2.)
  * Blocks are taken one at a time as the current one fills, nothing is reserved for a maximum
    length, and a finished sequence hands its blocks back to the free list.  (cloudmash,
    "PagedAttention" step 3; study-docs "Block tables"; llmdeepdive "Concept", paging paragraph.)
  * Forking copies the parent's block ids and raises each block's reference count; the first
    write into a shared block takes a fresh block, copies the old one into it and then writes.
    A block goes back to the pool when its count reaches zero.  (study-docs "Copy-on-write";
    cloudmash "Sharing blocks"; llmdeepdive "Concept", sharing paragraph.)
  * Capacity is countable in blocks, so admission can refuse a request early, before any work is
    done for it.  (llmdeepdive "Concept", continuous-batching paragraph.)

Readings where the pages are silent:
  * A write into a shared block is a copy for every holder but the last one: a writer that finds
    the block's count above one copies; a writer that finds it at one writes in place.
  * The copy covers the whole block (every head, every slot), not only the filled slots.
  * The flat slot index that the device append consumes is ``physical_block * block_size +
    offset``; a negative slot marks a padding token that is not written.

This module only produces the integer inputs of the device path (tables, slots, copy pairs); it
moves no KV bytes itself.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


class OutOfBlocks(RuntimeError):
    """Raised before any state changes when a request needs more free blocks than the pool has."""


def blocks_for(num_tokens: int, block_size: int) -> int:
    """Number of blocks that hold ``num_tokens`` tokens (round up)."""
    if num_tokens < 0:
        raise ValueError("num_tokens must be >= 0")
    return -(-num_tokens // block_size)


def tail_waste(num_tokens: int, block_size: int) -> int:
    """Unfilled slots in the last block of a sequence of ``num_tokens`` tokens.

    Waste under paging is at most this one partly filled block per sequence, so the value is
    always below ``block_size`` (cloudmash "PagedAttention", paragraph after the steps).
    """
    return blocks_for(num_tokens, block_size) * block_size - num_tokens


@dataclass
class BlockStats:
    """Operational counters (llmdeepdive "Concept", metrics paragraph)."""

    allocation_failures: int = 0
    cow_copies: int = 0
    blocks_allocated: int = 0
    blocks_freed: int = 0


@dataclass
class _Seq:
    blocks: List[int] = field(default_factory=list)
    length: int = 0


class BlockManager:
    """Free list + per-sequence block tables + reference counts for one KV pool.

    ``free_order`` fixes which physical ids are handed out first (index 0 first).  A seeded
    permutation here is what scatters a sequence's blocks across the pool.  Freed blocks are
    pushed on top of the free stack and are the next ones reused.
    """

    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self._free: List[int] = order[::-1]           # top of the stack is order[0]
        self._ref = np.zeros(num_blocks, dtype=np.int64)
        self._seqs: Dict[int, _Seq] = {}
        self.stats = BlockStats()

    # ------------------------------------------------------------------ queries
    @property
    def num_free(self) -> int:
        return len(self._free)

    @property
    def num_used(self) -> int:
        return self.num_blocks - len(self._free)

    def refcount(self, block: int) -> int:
        return int(self._ref[block])

    def seq_len(self, seq_id: int) -> int:
        return self._seqs[seq_id].length

    def table(self, seq_id: int) -> List[int]:
        return list(self._seqs[seq_id].blocks)

    def has(self, seq_id: int) -> bool:
        return seq_id in self._seqs

    def tail_waste_total(self) -> int:
        return sum(tail_waste(s.length, self.block_size) for s in self._seqs.values())

    def block_tables(self, seq_ids: Iterable[int], width: Optional[int] = None) -> np.ndarray:
        """int32 [len(seq_ids), width] table; entries past a sequence's blocks are -1."""
        rows = [self._seqs[s].blocks for s in seq_ids]
        w = max((len(r) for r in rows), default=0) if width is None else int(width)
        out = np.full((len(rows), max(w, 1)), -1, dtype=np.int32)
        for i, r in enumerate(rows):
            if len(r) > w:
                raise ValueError("table width smaller than a sequence's block count")
            out[i, :len(r)] = r
        return out

    # ------------------------------------------------------------- allocation
    def _pop(self) -> int:
        b = self._free.pop()
        self._ref[b] = 1
        self.stats.blocks_allocated += 1
        return b

    def _release(self, b: int) -> None:
        self._ref[b] -= 1
        if self._ref[b] < 0:
            raise AssertionError("negative reference count")
        if self._ref[b] == 0:
            self._free.append(b)
            self.stats.blocks_freed += 1

    def blocks_needed(self, seq_id: int, num_new: int) -> int:
        """Free blocks an append of ``num_new`` tokens would take (new blocks + a CoW copy)."""
        s = self._seqs[seq_id]
        b = self.block_size
        need = blocks_for(s.length + num_new, b) - len(s.blocks)
        if num_new > 0 and s.length % b != 0 and self._ref[s.blocks[-1]] > 1:
            need += 1
        return need

    def can_allocate(self, num_tokens: int) -> bool:
        return blocks_for(num_tokens, self.block_size) <= self.num_free

    def add_sequence(self, seq_id: int, num_tokens: int = 0) -> List[int]:
        """Admit a new sequence holding ``num_tokens`` tokens; returns their slots."""
        if seq_id in self._seqs:
            raise ValueError(f"sequence {seq_id} already exists")
        if not self.can_allocate(num_tokens):
            self.stats.allocation_failures += 1
            raise OutOfBlocks(f"need {blocks_for(num_tokens, self.block_size)} blocks, "
                              f"{self.num_free} free")
        self._seqs[seq_id] = _Seq()
        slots, pairs = self.append_tokens(seq_id, num_tokens)
        assert not pairs
        return slots

    def reserve_sequence(self, seq_id: int, reserve_tokens: int) -> None:
        """Contiguous-reservation policy: take blocks for ``reserve_tokens`` up front.

        The pages contrast this with paging; it exists here so the same allocator can count both
        policies (cloudmash "KV cache fragmentation", "Try it").
        """
        if seq_id in self._seqs:
            raise ValueError(f"sequence {seq_id} already exists")
        n = blocks_for(reserve_tokens, self.block_size)
        if n > self.num_free:
            self.stats.allocation_failures += 1
            raise OutOfBlocks(f"need {n} blocks, {self.num_free} free")
        self._seqs[seq_id] = _Seq(blocks=[self._pop() for _ in range(n)], length=0)

    def append_tokens(self, seq_id: int, num_new: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Grow a sequence by ``num_new`` tokens.

        Returns (slots, cow_pairs).  ``slots[i]`` is the flat pool slot of the i-th new token.
        ``cow_pairs`` lists (src, dst) block copies that must run on the device before the
        append writes these slots.  Raises OutOfBlocks (state unchanged) if the pool is short.
        """
        s = self._seqs[seq_id]
        b = self.block_size
        need = self.blocks_needed(seq_id, num_new)
        if need > self.num_free:
            self.stats.allocation_failures += 1
            raise OutOfBlocks(f"need {need} blocks, {self.num_free} free")
        pairs: List[Tuple[int, int]] = []
        slots: List[int] = []
        for _ in range(num_new):
            lb, off = divmod(s.length, b)
            if lb == len(s.blocks):
                s.blocks.append(self._pop())
            elif self._ref[s.blocks[lb]] > 1:
                src = s.blocks[lb]
                dst = self._pop()
                self._ref[src] -= 1
                s.blocks[lb] = dst
                pairs.append((src, dst))
                self.stats.cow_copies += 1
            slots.append(s.blocks[lb] * b + off)
            s.length += 1
        return slots, pairs

    def fork(self, parent: int, child: int) -> None:
        """Child shares every block of the parent; each shared block's count goes up by one."""
        if child in self._seqs:
            raise ValueError(f"sequence {child} already exists")
        p = self._seqs[parent]
        for blk in p.blocks:
            self._ref[blk] += 1
        self._seqs[child] = _Seq(blocks=list(p.blocks), length=p.length)

    def free(self, seq_id: int) -> None:
        """Return a finished sequence's blocks (each block is freed when its count hits 0)."""
        s = self._seqs.pop(seq_id)
        for blk in s.blocks:
            self._release(blk)


def shared_prefix_groups(block_tables: np.ndarray, seq_lens: np.ndarray, block_size: int,
                         max_group: int = 64) -> Tuple[np.ndarray, np.ndarray, int]:
    """Group a decode batch by shared leading blocks, for the grouped decode.

    Consecutive sequences whose first table entries are the same physical block (forks of one
    parent: parallel samples, beams) form a group; its shared prefix is the number of leading
    entries equal across all members, limited to each member's full blocks (a partly filled
    block is never shared by the time its holders decode: the first write copied it).  Groups
    are cut at ``max_group`` members.  Sequences with no shared full block stay in groups of
    one with a prefix of 0.  Returns (group_start [G+1], shared_blocks [S], largest group).
    """
    tables = np.asarray(block_tables)
    lens = np.asarray(seq_lens, dtype=np.int64)
    S = lens.shape[0]
    full = lens // block_size
    starts = [0]
    shared = np.zeros(S, dtype=np.int32)
    i = 0
    while i < S:
        j = i + 1
        while (j < S and j - i < max_group and full[i] > 0 and full[j] > 0
               and tables[j, 0] == tables[i, 0]):
            j += 1
        if j - i > 1:
            n = int(min(full[i:j]))
            same = np.all(tables[i:j, :n] == tables[i, :n], axis=0)
            n = int(np.argmin(same)) if not same.all() else n
            shared[i:j] = n
        starts.append(j)
        i = j
    gs = np.asarray(starts, dtype=np.int32)
    return gs, shared, int(np.max(np.diff(gs))) if S else 0


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int, num_layers: int = 1) -> int:
    """K plus V bytes one token occupies across ``num_layers`` layers."""
    return 2 * num_kv_heads * head_dim * elem_bytes * num_layers
