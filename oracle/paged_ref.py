"""fp64 CPU oracle for paged attention, KV append and copy-on-write block copies.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this
module; only the tests, the package smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP path and imports nothing from it.

What it computes is the plain definition, evaluated through the block table:

  * Where a token lives.  A sequence's tokens fill its logical blocks left to right; the block
    table maps logical block i to a physical block of the pool.  Token j therefore sits in
    physical block ``table[j // B]`` at offset ``j % B``.  (study-docs "PagedAttention &
    Continuous Batching", "Block tables"; cloudmash "Batching and PagedAttention",
    "PagedAttention" steps 1-2 and 4.)
  * Attention gathers K and V through that mapping and is otherwise ordinary scaled dot-product
    attention: x_j = scale * <q, K_j>, w = softmax(x), out = sum_j w_j V_j.  Paging changes where
    keys and values are stored, never the result.  (cloudmash "PagedAttention" step 4;
    llmdeepdive "Concept", paging paragraph.)
  * Decode: every sequence contributes one query token that sees all of its seq_len keys
    (cloudmash "Continuous batching"; llmdeepdive "Concept", continuous-batching paragraph).
  * Prefill chunk: a chunk of n new tokens at the end of a sequence of length L; row i sits at
    position L - n + i and sees keys 0 .. L - n + i, i.e. the whole resident prefix plus the
    chunk causally (cloudmash "Continuous batching", chunked prefill).
  * Append: new token t goes to slot ``slot_mapping[t]`` = block * B + offset; negative slots are
    padding (study-docs "Block tables": a sequence grows into its current block).
  * Copy-on-write: the whole destination block becomes a byte copy of the source block, K and V
    (study-docs "Copy-on-write"; cloudmash "Sharing blocks").
  * Swap: a preempted request's blocks move to CPU memory and back, whole blocks, all of a
    sequence's blocks together (cloudmash "Batching and PagedAttention", "When blocks run out");
    a swap is a byte copy of each source block of one pool into its destination block of the
    other pool.

Readings taken where the pages are silent: the pool layout is [blocks, kv_heads, B, head_dim];
query head h reads kv head h // (Hq / Hkv); seq_lens count the tokens appended in the same step
(append runs before attention); seq_len 0, duplicate slots and overlapping copy pairs are
invalid and raise.

Precision: inputs are widened exactly to fp64 (bf16 by placing its 16 bits on top of an fp32
bit pattern); ``scale`` is taken as the fp32 value the caller passes.  Nothing is rounded back.
"""
from __future__ import annotations

import numpy as np

BF16 = "bf16"
F32 = "f32"


class OracleInputError(ValueError):
    """An input the method does not define (empty sequence, duplicate slot, bad copy pair)."""


# ----------------------------------------------------------------------------- value widening
def to_f64(a, dtype: str) -> np.ndarray:
    """Exact widening to fp64.  bf16 arrives as raw uint16 bits, fp32 as float32."""
    a = np.asarray(a)
    if dtype == BF16:
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be passed as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == F32:
        if a.dtype != np.float32:
            raise TypeError("f32 data must be float32")
        return a.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def scale_f64(scale: float) -> float:
    return float(np.float32(scale))


# --------------------------------------------------------------------------- small definitions
def token_position(j, block_size: int):
    """(logical block, offset inside it) of token index j: blocks fill left to right."""
    return j // block_size, j % block_size


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """kv head read by query head h: contiguous groups of Hq / Hkv query heads."""
    return h // (num_q_heads // num_kv_heads)


def visible_keys(position: int) -> int:
    """Number of keys a query at absolute position ``position`` sees (itself included)."""
    return position + 1


def softmax_weights(x: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, max-shifted (shift-invariant, exact up to rounding)."""
    m = np.max(x, axis=-1, keepdims=True)
    w = np.exp(x - m)
    return w / np.sum(w, axis=-1, keepdims=True)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           visible=None) -> np.ndarray:
    """Scaled dot-product attention of query rows q [..., D] over K, V [L, D] (fp64).

    ``visible`` (optional, bool, broadcast against the scores [..., L]) names the keys each row
    may see; the others get score -inf, i.e. weight exactly 0.  Every row must see a key.
    """
    x = scale * (q @ K.T)
    if visible is not None:
        x = np.where(visible, x, -np.inf)
    return softmax_weights(x) @ V


def selected(count: int, wanted=None, first: int = 0) -> list:
    """Indices i in [0, count) whose global index first + i is wanted (all when wanted is None).
    The oracle computes only those rows; the rest of its output stays NaN."""
    if wanted is None:
        return list(range(count))
    w = set(int(x) for x in wanted)
    return [i for i in range(count) if first + i in w]


# ---------------------------------------------------------------------------------- gathering
def gather_tokens(cache: np.ndarray, table_row: np.ndarray, length: int,
                  block_size: int) -> np.ndarray:
    """Raw [length, Hkv, D] rows of one sequence, read through its block table."""
    if length < 1:
        raise OracleInputError("a sequence must hold at least one token")
    j = np.arange(length)
    lb, off = token_position(j, block_size)
    if lb.max() >= table_row.shape[0]:
        raise OracleInputError("block table too short for seq_len")
    phys = np.asarray(table_row)[lb].astype(np.int64)
    if phys.min() < 0 or phys.max() >= cache.shape[0]:
        raise OracleInputError("block table entry out of range")
    return cache[phys, :, off, :]


# ----------------------------------------------------------------------------------- decoding
def decode_ref(q, k_cache, v_cache, block_tables, seq_lens, scale: float, dtype: str,
               block_size: int = 16, seqs=None) -> np.ndarray:
    """fp64 decode output [S, Hq, D].

    q [S, Hq, D]; k_cache, v_cache [NB, Hkv, B, D]; block_tables int [S, MB]; seq_lens [S].
    ``seqs`` (optional) restricts the work to those sequence indices; the rows of the others
    stay NaN.
    """
    q = np.asarray(q)
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv != 0:
        raise OracleInputError("num_q_heads must be a multiple of num_kv_heads")
    sc = scale_f64(scale)
    out = np.full((S, Hq, D), np.nan)
    for s in selected(S, seqs):
        L = int(seq_lens[s])
        K = to_f64(gather_tokens(k_cache, block_tables[s], L, block_size), dtype)
        V = to_f64(gather_tokens(v_cache, block_tables[s], L, block_size), dtype)
        qs = to_f64(q[s], dtype)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[s, h] = attend(qs[h], K[:, g, :], V[:, g, :], sc)
    return out


def decode_contiguous_ref(q, k, v, seq_lens, scale: float, dtype: str, seqs=None) -> np.ndarray:
    """fp64 decode output [S, Hq, D] over KV kept without paging: k, v [S, Hkv, capacity, D],
    row j < seq_lens[s] of (s, kv head) is token j.  This is the contiguous layout the pages
    weigh paging against (cloudmash "Batching and PagedAttention", "The indirection has a
    cost"); the attention is the same definition as decode_ref's, minus the table.
    ``seqs`` restricts the work as in decode_ref."""
    q = np.asarray(q)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise OracleInputError("num_q_heads must be a multiple of num_kv_heads")
    sc = scale_f64(scale)
    out = np.full((S, Hq, D), np.nan)
    for s in selected(S, seqs):
        L = int(seq_lens[s])
        if L < 1 or L > k.shape[2]:
            raise OracleInputError("seq_len outside [1, capacity]")
        K = to_f64(k[s, :, :L, :], dtype)
        V = to_f64(v[s, :, :L, :], dtype)
        qs = to_f64(q[s], dtype)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[s, h] = attend(qs[h], K[g], V[g], sc)
    return out


# ------------------------------------------------------------------------------ prefill chunks
def prefill_ref(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale: float,
                dtype: str, block_size: int = 16, rows=None) -> np.ndarray:
    """fp64 chunk output [total_q, Hq, D].

    Chunk c owns packed query rows qsl[c] .. qsl[c+1]-1 and ends its sequence of seq_lens[c]
    tokens.  ``rows`` (optional) restricts the work to the given packed row indices; other rows
    stay NaN.
    """
    q = np.asarray(q)
    T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv != 0:
        raise OracleInputError("num_q_heads must be a multiple of num_kv_heads")
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    if qsl[0] != 0 or qsl[-1] != T or np.any(np.diff(qsl) < 0):
        raise OracleInputError("query_start_loc must rise from 0 to total_q")
    sc = scale_f64(scale)
    out = np.full((T, Hq, D), np.nan)
    for c in range(len(qsl) - 1):
        n = int(qsl[c + 1] - qsl[c])
        if n == 0:
            continue
        L = int(seq_lens[c])
        prefix = L - n
        if prefix < 0:
            raise OracleInputError("chunk longer than its sequence")
        idx = selected(n, rows, first=int(qsl[c]))
        if not idx:
            continue
        K = to_f64(gather_tokens(k_cache, block_tables[c], L, block_size), dtype)
        V = to_f64(gather_tokens(v_cache, block_tables[c], L, block_size), dtype)
        r = int(qsl[c]) + np.asarray(idx)
        # row i (at position prefix + i) sees keys 0 .. prefix + i
        nk = np.array([visible_keys(prefix + i) for i in idx])
        visible = np.arange(L)[None, :] < nk[:, None]
        qc = to_f64(q[r], dtype)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[r, h] = attend(qc[:, h], K[:, g, :], V[:, g, :], sc, visible)
    return out


# --------------------------------------------------------------------------- append and copies
def append_ref(k_cache, v_cache, k_new, v_new, slot_mapping, block_size: int = 16):
    """New (k_cache, v_cache) after writing token t's rows to slot_mapping[t] (bit copies)."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    nb = kc.shape[0]
    live = slots[slots >= 0]
    if live.size and (live.max() >= nb * block_size):
        raise OracleInputError("slot out of range")
    if np.unique(live).size != live.size:
        raise OracleInputError("duplicate slot in slot_mapping")
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        b, o = token_position(int(slot), block_size)
        kc[b, :, o, :] = k_new[t]
        vc[b, :, o, :] = v_new[t]
    return kc, vc


def validate_cow_pairs(pairs, num_blocks: int) -> np.ndarray:
    p = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if p.size == 0:
        return p
    src, dst = p[:, 0], p[:, 1]
    if p.min() < 0 or p.max() >= num_blocks:
        raise OracleInputError("copy pair block id out of range")
    if np.unique(dst).size != dst.size:
        raise OracleInputError("two copies into one destination block")
    if np.any(src == dst):
        raise OracleInputError("copy pair with src == dst")
    if np.intersect1d(src, dst).size:
        raise OracleInputError("a destination block is also a source")
    return p


def cow_ref(k_cache, v_cache, pairs):
    """New (k_cache, v_cache) with every destination block a byte copy of its source block."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    p = validate_cow_pairs(pairs, kc.shape[0])
    for src, dst in p:
        kc[dst] = k_cache[src]
        vc[dst] = v_cache[src]
    return kc, vc


def swap_ref(dst_k, dst_v, src_k, src_v, pairs):
    """New (dst_k, dst_v): destination block pairs[p][1] becomes a byte copy of source block
    pairs[p][0] of the other pool (K and V); no other destination block changes.  Destination
    ids must be distinct and every id in range."""
    dk = np.array(dst_k, copy=True)
    dv = np.array(dst_v, copy=True)
    p = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if p.size and (p.min() < 0 or p[:, 0].max() >= src_k.shape[0]
                   or p[:, 1].max() >= dk.shape[0]):
        raise OracleInputError("swap block id out of range")
    if np.unique(p[:, 1]).size != p.shape[0]:
        raise OracleInputError("duplicate swap destination")
    for src, dst in p:
        dk[dst] = src_k[src]
        dv[dst] = src_v[src]
    return dk, dv
