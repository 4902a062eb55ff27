"""Seeded synthetic inputs for the paged KV-cache hot path.

This module draws inputs only; it holds no attention, append or copy arithmetic.  Both the HIP
path and the fp64 oracle are fed the exact bytes made here.

Recipe (the same for every workload):
  * Structure first, with ``numpy.random.default_rng(seed)``: sequence lengths, then the seeded
    permutation that orders the free list (so physical block ids are scattered), then any other
    integer choices.  Block tables, slot mappings and copy pairs come from ``BlockManager``.
  * Values second, with ``torch.Generator(device).manual_seed(seed)``: standard normal fp32, in
    the order q, K pool, V pool, then new K, new V.  bf16 values are the fp32 draws rounded to
    nearest-even by torch's cast.  The K/V pools are drawn directly in pool order (every block,
    owned or not); slots that hold no token are then set to NaN when ``poison`` is on, so any
    read of them shows up in the result.
  * ``seed = 3410 + k`` for the k-th standard workload.

Standard workloads (names give the sizes):
  1 ``tiny_f32``      4 sequences, lengths {1,17,40,100}, 2 q heads / 1 kv head, head_dim 64,
                      fp32, pool of 64 blocks, the sequences take the first 13 ids of a seeded
                      permutation in order, scale 1/8.
  2 ``decode_bf16``   64 sequences, lengths uniform integers in [128, 4096], 32/8 heads,
                      head_dim 128, bf16, pool = ceil(1.2 x blocks needed), permuted ids.
  3 ``long_bf16``     32 sequences of 32768 tokens, 16/4 heads, head_dim 256, bf16, pool
                      ceil(1.2 x 65536) = 78644 blocks.
  4 ``mixed_bf16``    8 prefill chunks of 512 tokens over resident prefixes uniform in [0, 8192]
                      plus 192 decode sequences with lengths round(lognormal(ln 2000, 1)) clipped
                      to [1, 16384]; 32/8 heads, head_dim 128, bf16; 4288 new tokens appended.
  5 ``beams_bf16``    16 prompts x 8 beams; each prompt shares 4096 + s tokens (s uniform in
                      [1, 15], so the last shared block is partly filled) across its beams; each
                      beam then appends a tail uniform in [1, 256]; 7 copy-on-write pairs per
                      prompt; 32/8 heads, head_dim 128, bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

from .block_manager import BlockManager, blocks_for, shared_prefix_groups

SEED_BASE = 3410
BLOCK_SIZE = 16

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class PoolSpec:
    num_blocks: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str


@dataclass
class DecodeBatch:
    """Inputs of one paged decode call."""

    q: torch.Tensor                 # [S, Hq, D]
    k_cache: torch.Tensor           # [NB, Hkv, B, D]
    v_cache: torch.Tensor
    block_tables: np.ndarray        # int32 [S, MB], -1 padded
    seq_lens: np.ndarray            # int32 [S]
    scale: float                    # an fp32 value
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    name: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())


@dataclass
class ContiguousDecode:
    """Inputs of one decode over KV kept without paging: k, v [S, Hkv, capacity, D], row j of
    (s, kv head) holds token j."""

    q: torch.Tensor                 # [S, Hq, D]
    k: torch.Tensor                 # [S, Hkv, capacity, D]
    v: torch.Tensor
    seq_lens: np.ndarray            # int32 [S]
    scale: float
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    name: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    @property
    def capacity(self) -> int:
        return int(self.k.shape[2])


@dataclass
class MixedStep:
    """One continuous-batching iteration: append, then prefill chunks and decodes."""

    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_new: torch.Tensor             # [T, Hkv, D]
    v_new: torch.Tensor
    slot_mapping: np.ndarray        # int64 [T]
    # chunks
    q_chunk: torch.Tensor           # [total_q, Hq, D]
    chunk_tables: np.ndarray        # int32 [C, MB]
    chunk_seq_lens: np.ndarray      # int32 [C], prefix + chunk (after the append)
    query_start_loc: np.ndarray     # int32 [C + 1]
    # decodes
    q_decode: torch.Tensor          # [Sd, Hq, D]
    decode_tables: np.ndarray
    decode_seq_lens: np.ndarray     # int32 [Sd], after the append
    # copy-on-write pairs that must run before the append (may be empty)
    cow_pairs: np.ndarray           # int64 [P, 2]
    scale: float
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    name: str = ""
    extra: dict = field(default_factory=dict)


def f32(x: float) -> float:
    """Round a Python float to the nearest fp32 value."""
    return float(np.float32(x))


def default_scale(head_dim: int) -> float:
    return f32(1.0 / math.sqrt(head_dim))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, gen: torch.Generator, dtype: str, device) -> torch.Tensor:
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32, device=device)
    return x.to(TORCH_DTYPES[dtype])


def _poison_pool(cache: torch.Tensor, filled: np.ndarray) -> None:
    """NaN every slot whose ``filled`` entry ([NB, B] bool) is False."""
    mask = torch.from_numpy(~filled).to(cache.device)
    cache.masked_fill_(mask[:, None, :, None], float("nan"))


def _filled_slots(bm: BlockManager, seq_ids: Sequence[int], num_blocks: int, block_size: int,
                  lengths: Optional[Sequence[int]] = None) -> np.ndarray:
    """[NB, B] bool: slots holding one of the first ``lengths[i]`` tokens of ``seq_ids[i]``."""
    filled = np.zeros((num_blocks, block_size), dtype=bool)
    for i, s in enumerate(seq_ids):
        n = bm.seq_len(s) if lengths is None else int(lengths[i])
        tab = bm.table(s)
        for lb in range(blocks_for(n, block_size)):
            filled[tab[lb], :min(block_size, n - lb * block_size)] = True
    return filled


def _permuted_manager(rng: np.random.Generator, num_blocks: int, block_size: int,
                      scatter: bool = True) -> BlockManager:
    """Free list in a seeded random order (scattered physical ids), or in id order, which lays
    every sequence's blocks out contiguously (the permutation is drawn either way, so the
    values drawn afterwards do not depend on the choice)."""
    order = rng.permutation(num_blocks)
    return BlockManager(num_blocks, block_size,
                        free_order=order if scatter else np.arange(num_blocks))


def make_decode(seq_lens: Sequence[int], num_q_heads: int, num_kv_heads: int, head_dim: int,
                dtype: str, seed: int, *, block_size: int = BLOCK_SIZE,
                num_blocks: Optional[int] = None, pool_factor: float = 1.2,
                rng: Optional[np.random.Generator] = None, poison: bool = True,
                device="cpu", scale: Optional[float] = None, name: str = "",
                scatter: bool = True) -> DecodeBatch:
    """A decode batch over the given lengths, blocks handed out from a permuted free list
    (``scatter=False``: in id order, so each sequence's blocks are physically contiguous)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lens = [int(x) for x in seq_lens]
    need = sum(blocks_for(n, block_size) for n in lens)
    nb = int(num_blocks) if num_blocks is not None else max(1, math.ceil(pool_factor * need))
    bm = _permuted_manager(rng, nb, block_size, scatter)
    for i, n in enumerate(lens):
        bm.add_sequence(i, n)
    tables = bm.block_tables(range(len(lens)))
    gen = _gen(seed, device)
    q = _randn((len(lens), num_q_heads, head_dim), gen, dtype, device)
    k = _randn((nb, num_kv_heads, block_size, head_dim), gen, dtype, device)
    v = _randn((nb, num_kv_heads, block_size, head_dim), gen, dtype, device)
    if poison:
        filled = _filled_slots(bm, range(len(lens)), nb, block_size)
        _poison_pool(k, filled)
        _poison_pool(v, filled)
    return DecodeBatch(q=q, k_cache=k, v_cache=v, block_tables=tables,
                       seq_lens=np.asarray(lens, dtype=np.int32),
                       scale=default_scale(head_dim) if scale is None else f32(scale),
                       num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                       block_size=block_size, dtype=dtype, name=name)


def make_contiguous_decode(seq_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                           head_dim: int, dtype: str, seed: int, *, capacity: Optional[int] = None,
                           poison: bool = True, device="cpu", name: str = "") -> ContiguousDecode:
    """A decode batch with contiguous KV: q, then K and V drawn directly in the
    [S, Hkv, capacity, D] layout (capacity: the longest length rounded up to 16 unless given).
    Rows past a sequence's length are NaN when ``poison`` is on."""
    lens = np.asarray([int(x) for x in seq_lens], dtype=np.int32)
    cap = int(capacity) if capacity is not None else int(-(-int(lens.max()) // 16) * 16)
    gen = _gen(seed, device)
    S = len(lens)
    q = _randn((S, num_q_heads, head_dim), gen, dtype, device)
    k = _randn((S, num_kv_heads, cap, head_dim), gen, dtype, device)
    v = _randn((S, num_kv_heads, cap, head_dim), gen, dtype, device)
    if poison:
        past = torch.from_numpy(np.arange(cap)[None, :] >= lens[:, None]).to(device)
        k.masked_fill_(past[:, None, :, None], float("nan"))
        v.masked_fill_(past[:, None, :, None], float("nan"))
    return ContiguousDecode(q=q, k=k, v=v, seq_lens=lens, scale=default_scale(head_dim),
                            num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                            head_dim=head_dim, dtype=dtype, name=name)


def make_grouped_decode(groups: Sequence[tuple], num_q_heads: int, num_kv_heads: int,
                        head_dim: int, seed: int, *, dtype: str = "bf16", poison: bool = True,
                        device="cpu") -> DecodeBatch:
    """A decode batch of forked groups: ``groups`` lists (prefix_len, [tail_len per member]).
    Each group's parent holds ``prefix_len`` tokens, is forked to the other members, and then
    every member appends its tail (members 1.. first, the parent last, as in a beam step), so
    a partly filled last prefix block is copied for all members but the parent.  Block ids come
    from a permuted free list.  ``extra`` holds the group plan of ``shared_prefix_groups``."""
    rng = np.random.default_rng(seed)
    need = 0
    for prefix, tails in groups:
        need += blocks_for(prefix, BLOCK_SIZE)
        need += sum(blocks_for(prefix + t, BLOCK_SIZE) - prefix // BLOCK_SIZE for t in tails)
    nb = max(1, math.ceil(1.2 * need) + 1)
    bm = _permuted_manager(rng, nb, BLOCK_SIZE)
    seq_ids = []
    sid = 0
    for prefix, tails in groups:
        root = sid
        bm.add_sequence(root, prefix)
        members = [root + m for m in range(len(tails))]
        for m in members[1:]:
            bm.fork(root, m)
        for m, t in list(zip(members, tails))[1:] + [(root, tails[0])]:
            if t:
                bm.append_tokens(m, int(t))
        seq_ids += members
        sid += len(tails)
    tables = bm.block_tables(seq_ids)
    lens = np.asarray([bm.seq_len(s) for s in seq_ids], dtype=np.int32)
    gen = _gen(seed, device)
    q = _randn((len(seq_ids), num_q_heads, head_dim), gen, dtype, device)
    k = _randn((nb, num_kv_heads, BLOCK_SIZE, head_dim), gen, dtype, device)
    v = _randn((nb, num_kv_heads, BLOCK_SIZE, head_dim), gen, dtype, device)
    if poison:
        filled = _filled_slots(bm, seq_ids, nb, BLOCK_SIZE)
        _poison_pool(k, filled)
        _poison_pool(v, filled)
    group_start, shared_blocks, max_group = shared_prefix_groups(tables, lens, BLOCK_SIZE)
    return DecodeBatch(q=q, k_cache=k, v_cache=v, block_tables=tables, seq_lens=lens,
                       scale=default_scale(head_dim), num_q_heads=num_q_heads,
                       num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=BLOCK_SIZE,
                       dtype=dtype, name="grouped",
                       extra={"group_start": group_start, "shared_blocks": shared_blocks,
                              "max_group_size": max_group})


def tiny_f32(device="cpu", poison: bool = True, seed: int = SEED_BASE + 1) -> DecodeBatch:
    """Workload 1: 4 sequences {1,17,40,100}, fp32, 64-block pool, first 13 permuted ids."""
    rng = np.random.default_rng(seed)
    return make_decode([1, 17, 40, 100], 2, 1, 64, "f32", seed, num_blocks=64, rng=rng,
                       poison=poison, device=device, scale=0.125, name="tiny_f32")


def decode_bf16(device="cpu", poison: bool = True, seed: int = SEED_BASE + 2,
                num_seqs: int = 64, lo: int = 128, hi: int = 4096,
                block_size: int = BLOCK_SIZE, scatter: bool = True) -> DecodeBatch:
    """Workload 2: 64 sequences, lengths U[128, 4096], 32/8 heads, head_dim 128, bf16."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=num_seqs)
    return make_decode(lens, 32, 8, 128, "bf16", seed, rng=rng, poison=poison, device=device,
                       name="decode_bf16", block_size=block_size, scatter=scatter)


def decode_bf16_contiguous(device="cpu", poison: bool = True,
                           seed: int = SEED_BASE + 2) -> ContiguousDecode:
    """Workload 2's lengths (the same draw) and heads, with contiguous KV of capacity 4096."""
    lens = np.random.default_rng(seed).integers(128, 4097, size=64)
    return make_contiguous_decode(lens, 32, 8, 128, "bf16", seed, capacity=4096, poison=poison,
                                  device=device, name="decode_bf16_contiguous")


def long_bf16_contiguous(device="cpu", poison: bool = True,
                         seed: int = SEED_BASE + 3) -> ContiguousDecode:
    """Workload 3's shape (32 x 32768 tokens, 16/4 heads, head_dim 256) with contiguous KV."""
    return make_contiguous_decode([32768] * 32, 16, 4, 256, "bf16", seed, poison=poison,
                                  device=device, name="long_bf16_contiguous")


def long_bf16(device="cpu", poison: bool = True, seed: int = SEED_BASE + 3,
              num_seqs: int = 32, seq_len: int = 32768, block_size: int = BLOCK_SIZE,
              scatter: bool = True) -> DecodeBatch:
    """Workload 3: 32 sequences x 32768 tokens, 16/4 heads, head_dim 256, bf16."""
    rng = np.random.default_rng(seed)
    return make_decode([seq_len] * num_seqs, 16, 4, 256, "bf16", seed, rng=rng, poison=poison,
                       device=device, name="long_bf16", block_size=block_size,
                       scatter=scatter)


def mixed_bf16(device="cpu", poison: bool = True, seed: int = SEED_BASE + 4,
               num_chunks: int = 8, chunk_len: int = 512, max_prefix: int = 8192,
               num_decode: int = 192, median: float = 2000.0, sigma: float = 1.0,
               cap: int = 16384, num_q_heads: int = 32, num_kv_heads: int = 8,
               head_dim: int = 128, dtype: str = "bf16",
               chunk_lens: Optional[Sequence[int]] = None,
               prefixes: Optional[Sequence[int]] = None) -> MixedStep:
    """Workload 4: chunked prefills over resident prefixes plus single-token decodes.

    Before the step, chunk c holds ``prefix[c]`` tokens and decode sequence d holds
    ``L[d] - 1``.  The step appends ``chunk_len`` tokens to each chunk and one to each decode,
    all through one slot mapping ordered chunks first, then decodes.  ``chunk_lens`` overrides
    the per-chunk query count (ragged chunks) and ``prefixes`` the resident prefix lengths.
    """
    rng = np.random.default_rng(seed)
    drawn = rng.integers(0, max_prefix + 1, size=num_chunks)
    prefixes = drawn if prefixes is None else np.asarray(prefixes, dtype=np.int64)
    dec = np.rint(np.exp(rng.normal(math.log(median), sigma, size=num_decode)))
    dec = np.clip(dec, 1, cap).astype(np.int64)
    clens = [chunk_len] * num_chunks if chunk_lens is None else [int(x) for x in chunk_lens]
    need = sum(blocks_for(int(p) + n, BLOCK_SIZE) for p, n in zip(prefixes, clens))
    need += sum(blocks_for(int(n), BLOCK_SIZE) for n in dec)
    nb = math.ceil(1.2 * need)
    bm = _permuted_manager(rng, nb, BLOCK_SIZE)
    chunk_ids = list(range(num_chunks))
    dec_ids = list(range(num_chunks, num_chunks + num_decode))
    for c, p in zip(chunk_ids, prefixes):
        bm.add_sequence(c, int(p))
    for d, n in zip(dec_ids, dec):
        bm.add_sequence(d, int(n) - 1)
    filled_before = _filled_slots(bm, chunk_ids + dec_ids, nb, BLOCK_SIZE)
    slots: List[int] = []
    for c, n in zip(chunk_ids, clens):
        s, pairs = bm.append_tokens(c, n)
        assert not pairs
        slots += s
    for d in dec_ids:
        s, pairs = bm.append_tokens(d, 1)
        assert not pairs
        slots += s
    width = max(len(bm.table(s)) for s in chunk_ids + dec_ids)
    gen = _gen(seed, device)
    total_q = sum(clens)
    T = len(slots)
    q_chunk = _randn((total_q, num_q_heads, head_dim), gen, dtype, device)
    q_dec = _randn((num_decode, num_q_heads, head_dim), gen, dtype, device)
    k = _randn((nb, num_kv_heads, BLOCK_SIZE, head_dim), gen, dtype, device)
    v = _randn((nb, num_kv_heads, BLOCK_SIZE, head_dim), gen, dtype, device)
    k_new = _randn((T, num_kv_heads, head_dim), gen, dtype, device)
    v_new = _randn((T, num_kv_heads, head_dim), gen, dtype, device)
    if poison:
        _poison_pool(k, filled_before)
        _poison_pool(v, filled_before)
    qsl = np.zeros(num_chunks + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(clens)
    return MixedStep(
        k_cache=k, v_cache=v, k_new=k_new, v_new=v_new,
        slot_mapping=np.asarray(slots, dtype=np.int64),
        q_chunk=q_chunk, chunk_tables=bm.block_tables(chunk_ids, width),
        chunk_seq_lens=np.asarray([bm.seq_len(c) for c in chunk_ids], dtype=np.int32),
        query_start_loc=qsl,
        q_decode=q_dec, decode_tables=bm.block_tables(dec_ids, width),
        decode_seq_lens=np.asarray([bm.seq_len(d) for d in dec_ids], dtype=np.int32),
        cow_pairs=np.zeros((0, 2), dtype=np.int64), scale=default_scale(head_dim),
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        block_size=BLOCK_SIZE, dtype=dtype, name="mixed_bf16",
        extra={"prefixes": prefixes.astype(np.int64), "decode_lens": dec, "num_blocks": nb})


def beams_bf16(device="cpu", poison: bool = True, seed: int = SEED_BASE + 5,
               num_prompts: int = 16, beams: int = 8, prefix: int = 4096,
               partial_shared: bool = True, tail_lo: int = 1, tail_hi: int = 256,
               num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
               dtype: str = "bf16") -> MixedStep:
    """Workload 5: beams sharing a prompt, copy-on-write of the shared partial block, append, decode.

    Each prompt's region of ``prefix + s`` tokens (s uniform in [1, 15] when
    ``partial_shared``; s = 0 otherwise) is owned by beam 0 and forked to beams 1..7.  Beams
    then append their tails in the order 1..7, 0: each of beams 1..7 finds the last shared
    block still shared and copies it; beam 0 finds it private and writes in place.  The copy
    pairs, the slot mapping of all tails and the final tables are returned; only the decode
    part of ``MixedStep`` is populated (no chunks).
    """
    rng = np.random.default_rng(seed)
    extra_shared = rng.integers(1, BLOCK_SIZE, size=num_prompts) if partial_shared \
        else np.zeros(num_prompts, dtype=np.int64)
    tails = rng.integers(tail_lo, tail_hi + 1, size=(num_prompts, beams))
    need = 0
    for p in range(num_prompts):
        shared = prefix + int(extra_shared[p])
        need += blocks_for(shared, BLOCK_SIZE)
        for b in range(beams):
            need += blocks_for(shared + int(tails[p, b]), BLOCK_SIZE) - shared // BLOCK_SIZE
    nb = math.ceil(1.2 * need)
    bm = _permuted_manager(rng, nb, BLOCK_SIZE)
    seq_ids = []
    for p in range(num_prompts):
        root = p * beams
        bm.add_sequence(root, prefix + int(extra_shared[p]))
        for b in range(1, beams):
            bm.fork(root, root + b)
        seq_ids += [root + b for b in range(beams)]
    filled_before = _filled_slots(bm, seq_ids, nb, BLOCK_SIZE)
    slots: List[int] = []
    pairs: List[tuple] = []
    order = []
    for p in range(num_prompts):
        order += [p * beams + b for b in list(range(1, beams)) + [0]]
    tail_of = {p * beams + b: int(tails[p, b]) for p in range(num_prompts) for b in range(beams)}
    for sid in order:
        s, pr = bm.append_tokens(sid, tail_of[sid])
        slots += s
        pairs += pr
    width = max(len(bm.table(s)) for s in seq_ids)
    gen = _gen(seed, device)
    T = len(slots)
    q_dec = _randn((len(seq_ids), num_q_heads, head_dim), gen, dtype, device)
    k = _randn((nb, num_kv_heads, BLOCK_SIZE, head_dim), gen, dtype, device)
    v = _randn((nb, num_kv_heads, BLOCK_SIZE, head_dim), gen, dtype, device)
    k_new = _randn((T, num_kv_heads, head_dim), gen, dtype, device)
    v_new = _randn((T, num_kv_heads, head_dim), gen, dtype, device)
    if poison:
        _poison_pool(k, filled_before)
        _poison_pool(v, filled_before)
    empty_q = torch.empty((0, num_q_heads, head_dim), dtype=TORCH_DTYPES[dtype], device=device)
    return MixedStep(
        k_cache=k, v_cache=v, k_new=k_new, v_new=v_new,
        slot_mapping=np.asarray(slots, dtype=np.int64),
        q_chunk=empty_q, chunk_tables=np.zeros((0, width), dtype=np.int32),
        chunk_seq_lens=np.zeros(0, dtype=np.int32), query_start_loc=np.zeros(1, dtype=np.int32),
        q_decode=q_dec, decode_tables=bm.block_tables(seq_ids, width),
        decode_seq_lens=np.asarray([bm.seq_len(s) for s in seq_ids], dtype=np.int32),
        cow_pairs=np.asarray(pairs, dtype=np.int64).reshape(-1, 2),
        scale=default_scale(head_dim), num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=BLOCK_SIZE, dtype=dtype, name="beams_bf16",
        extra={"shared_lens": prefix + extra_shared, "tails": tails, "num_blocks": nb,
               "refcount_max": beams})


WORKLOADS = {1: tiny_f32, 2: decode_bf16, 3: long_bf16, 4: mixed_bf16, 5: beams_bf16}
