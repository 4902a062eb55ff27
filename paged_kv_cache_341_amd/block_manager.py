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

  * Requests are served in arrival order; when allocation runs dry mid-generation, preemption
    takes the newest request first and moves all of its blocks at once: they go to the host
    pool, or they are dropped and the request's tokens are run again later.  (cloudmash, "When
    blocks run out".)
  * The counters to watch: free and used blocks, allocation failures, tail waste, preemptions.
    (llmdeepdive "Concept", metrics paragraph.)

Readings where the pages are silent:
  * A write into a shared block is a copy for every holder but the last one: a writer that finds
    the block's count above one copies; a writer that finds it at one writes in place.
  * The copy covers the whole block (every head, every slot), not only the filled slots.
  * The flat slot index that the device append consumes is ``physical_block * block_size +
    offset``; a negative slot marks a padding token that is not written.
  * A request is a sequence admitted with ``add_sequence`` together with every fork of it
    (samples, beams); preemption evicts a whole request, since its members share blocks.
    Arrival order is admission order.
  * Swap-out gives each distinct GPU block of the request one CPU block (members in request
    order, each member's blocks in table order, first appearance), carrying its reference
    count, so sharing survives the round trip; swap-in is the mirror image and takes the
    earliest-arrived swapped request first.  Either direction fails, changing nothing, when the
    other pool has too few free blocks.
  * Recompute frees the blocks and keeps each member's token count; on resume every member
    re-appends its tokens into private blocks (sharing is not rebuilt).

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


class NoVictim(RuntimeError):
    """Raised by a preemption when no running request other than the protected one exists."""


RUNNING, SWAPPED, RECOMPUTE = 0, 1, 2
SWAP, RECOMPUTE_MODE = 0, 1


@dataclass
class BlockStats:
    """Operational counters (llmdeepdive "Concept", metrics paragraph)."""

    allocation_failures: int = 0
    cow_copies: int = 0
    blocks_allocated: int = 0
    blocks_freed: int = 0
    preemptions_swap: int = 0
    preemptions_recompute: int = 0
    blocks_swapped_out: int = 0
    blocks_swapped_in: int = 0


@dataclass
class _Seq:
    blocks: List[int] = field(default_factory=list)
    length: int = 0
    request: int = -1
    state: int = RUNNING
    recompute_tokens: int = 0


class BlockManager:
    """Free list + per-sequence block tables + reference counts for one KV pool.

    ``free_order`` fixes which physical ids are handed out first (index 0 first).  A seeded
    permutation here is what scatters a sequence's blocks across the pool.  Freed blocks are
    pushed on top of the free stack and are the next ones reused.
    """

    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order: Optional[Sequence[int]] = None, num_cpu_blocks: int = 0,
                 cpu_free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0 or num_cpu_blocks < 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.num_cpu_blocks = int(num_cpu_blocks)
        self.block_size = int(block_size)
        self._free = self._stack(num_blocks, free_order)
        self._cpu_free = self._stack(num_cpu_blocks, cpu_free_order)
        self._ref = np.zeros(num_blocks, dtype=np.int64)
        self._cpu_ref = np.zeros(num_cpu_blocks, dtype=np.int64)
        self._seqs: Dict[int, _Seq] = {}
        self._requests: Dict[int, List[int]] = {}      # request id (= arrival) -> members
        self._next_request = 0
        self.stats = BlockStats()

    @staticmethod
    def _stack(n: int, order: Optional[Sequence[int]]) -> List[int]:
        o = list(range(n)) if order is None else [int(b) for b in order]
        if sorted(o) != list(range(n)):
            raise ValueError("a free order must be a permutation of range(num_blocks)")
        return o[::-1]                                # top of the stack is order[0]

    # ------------------------------------------------------------------ queries
    @property
    def num_free(self) -> int:
        return len(self._free)

    @property
    def num_used(self) -> int:
        return self.num_blocks - len(self._free)

    @property
    def num_free_cpu(self) -> int:
        return len(self._cpu_free)

    def refcount(self, block: int) -> int:
        return int(self._ref[block])

    def cpu_refcount(self, block: int) -> int:
        return int(self._cpu_ref[block])

    def state(self, seq_id: int) -> int:
        return self._seqs[seq_id].state

    def request_of(self, seq_id: int) -> int:
        return self._seqs[seq_id].request

    def recompute_tokens(self, seq_id: int) -> int:
        return self._seqs[seq_id].recompute_tokens

    def members(self, request: int) -> List[int]:
        return list(self._requests[request])

    def seq_len(self, seq_id: int) -> int:
        return self._seqs[seq_id].length

    def table(self, seq_id: int) -> List[int]:
        return list(self._seqs[seq_id].blocks)

    def has(self, seq_id: int) -> bool:
        return seq_id in self._seqs

    def tail_waste_total(self) -> int:
        """Unfilled slots in the last blocks of the sequences resident on the GPU."""
        return sum(tail_waste(s.length, self.block_size) for s in self._seqs.values()
                   if s.state == RUNNING)

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
        if s.state != RUNNING:
            raise ValueError(f"sequence {seq_id} is not resident (preempted)")
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
        self._seqs[seq_id] = _Seq(request=self._new_request(seq_id))
        slots, pairs = self.append_tokens(seq_id, num_tokens)
        assert not pairs
        return slots

    def _new_request(self, seq_id: int) -> int:
        r = self._next_request
        self._next_request += 1
        self._requests[r] = [seq_id]
        return r

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
        self._seqs[seq_id] = _Seq(blocks=[self._pop() for _ in range(n)], length=0,
                                  request=self._new_request(seq_id))

    def append_tokens(self, seq_id: int, num_new: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Grow a sequence by ``num_new`` tokens.

        Returns (slots, cow_pairs).  ``slots[i]`` is the flat pool slot of the i-th new token.
        ``cow_pairs`` lists (src, dst) block copies that must run on the device before the
        append writes these slots.  Raises OutOfBlocks (state unchanged) if the pool is short.
        """
        s = self._seqs[seq_id]
        if s.state != RUNNING:
            raise ValueError(f"sequence {seq_id} is not resident (preempted)")
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
        if p.state != RUNNING:
            raise ValueError(f"sequence {parent} is not resident (preempted)")
        for blk in p.blocks:
            self._ref[blk] += 1
        self._seqs[child] = _Seq(blocks=list(p.blocks), length=p.length, request=p.request)
        self._requests[p.request].append(child)

    def free(self, seq_id: int) -> None:
        """Return a finished sequence's blocks (each block is freed when its count hits 0)."""
        s = self._seqs.pop(seq_id)
        for blk in s.blocks:
            if s.state == SWAPPED:
                self._cpu_ref[blk] -= 1
                if self._cpu_ref[blk] == 0:
                    self._cpu_free.append(blk)
            else:
                self._release(blk)
        members = self._requests[s.request]
        members.remove(seq_id)
        if not members:
            del self._requests[s.request]

    # -------------------------------------------------------------- preemption
    def _distinct_blocks(self, request: int) -> List[int]:
        seen, order = set(), []
        for sid in self._requests[request]:
            for blk in self._seqs[sid].blocks:
                if blk not in seen:
                    seen.add(blk)
                    order.append(blk)
        return order

    def _request_state(self, request: int) -> int:
        return self._seqs[self._requests[request][0]].state

    def preempt_latest(self, mode: int = SWAP,
                       protect: Optional[int] = None) -> Tuple[int, List[Tuple[int, int]]]:
        """Evict the most recently arrived running request other than ``protect``.

        ``mode`` SWAP moves all its blocks to the CPU pool and returns the (gpu, cpu) block
        pairs to copy device-to-host before the GPU blocks are reused; RECOMPUTE frees them
        and returns no pairs.  Raises NoVictim, or OutOfBlocks (nothing changed) when the CPU
        pool cannot take a swap.
        """
        cands = [r for r in self._requests
                 if r != protect and self._request_state(r) == RUNNING]
        if not cands:
            raise NoVictim("no running request to preempt")
        r = max(cands)
        if mode == SWAP:
            blocks = self._distinct_blocks(r)
            if len(blocks) > self.num_free_cpu:
                raise OutOfBlocks(f"swap needs {len(blocks)} CPU blocks, "
                                  f"{self.num_free_cpu} free")
            remap, pairs = {}, []
            for g in blocks:
                c = self._cpu_free.pop()
                self._cpu_ref[c] = self._ref[g]
                self._ref[g] = 0
                self._free.append(g)
                self.stats.blocks_freed += 1
                remap[g] = c
                pairs.append((g, c))
            for sid in self._requests[r]:
                s = self._seqs[sid]
                s.blocks = [remap[g] for g in s.blocks]
                s.state = SWAPPED
            self.stats.preemptions_swap += 1
            self.stats.blocks_swapped_out += len(pairs)
            return r, pairs
        if mode != RECOMPUTE_MODE:
            raise ValueError("mode must be SWAP or RECOMPUTE_MODE")
        for sid in self._requests[r]:
            s = self._seqs[sid]
            for blk in s.blocks:
                self._release(blk)
            s.recompute_tokens, s.length, s.blocks, s.state = s.length, 0, [], RECOMPUTE
        self.stats.preemptions_recompute += 1
        return r, []

    def swap_in_earliest(self) -> Tuple[int, List[Tuple[int, int]]]:
        """Bring back the earliest-arrived swapped request: returns it and the (cpu, gpu)
        block pairs to copy host-to-device.  Raises NoVictim when none is swapped, or
        OutOfBlocks (nothing changed) when the GPU pool is short."""
        cands = [r for r in self._requests if self._request_state(r) == SWAPPED]
        if not cands:
            raise NoVictim("no swapped request")
        r = min(cands)
        blocks = self._distinct_blocks(r)
        if len(blocks) > self.num_free:
            self.stats.allocation_failures += 1
            raise OutOfBlocks(f"swap-in needs {len(blocks)} blocks, {self.num_free} free")
        remap, pairs = {}, []
        for c in blocks:
            g = self._pop()
            self._ref[g] = self._cpu_ref[c]
            self._cpu_ref[c] = 0
            self._cpu_free.append(c)
            remap[c] = g
            pairs.append((c, g))
        for sid in self._requests[r]:
            s = self._seqs[sid]
            s.blocks = [remap[c] for c in s.blocks]
            s.state = RUNNING
        self.stats.blocks_swapped_in += len(pairs)
        return r, pairs

    def resume_recompute(self, request: int) -> List[Tuple[int, int]]:
        """Make a recompute-preempted request resident again, empty: returns (seq, tokens)
        for each member, the tokens the caller re-appends (re-prefills).  The counts stay
        readable through ``recompute_tokens`` (the length each member had when preempted)."""
        if request not in self._requests or self._request_state(request) != RECOMPUTE:
            raise ValueError(f"request {request} is not waiting for recompute")
        out = []
        for sid in self._requests[request]:
            s = self._seqs[sid]
            s.state = RUNNING
            out.append((sid, s.recompute_tokens))
        return out


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
