"""Pins for the fp64 oracle: each check takes the oracle module and raises AssertionError if it
disagrees with something the pages or the mathematics fix independently of the oracle.

The same checks run against deliberately broken copies of the oracle (tests/test_oracle_mutations.py)
to show that a plausible mistake anywhere in it fails at least one of them.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import brute


# ---------------------------------------------------------------------------- tiny builders
def _rng(seed):
    return np.random.default_rng(seed)


def scatter(logical, tables, block_size, num_blocks, fill=np.nan):
    """Pool [NB, Hkv, B, D] holding sequence s's token j at (tables[s][j // B], j % B).

    ``logical`` is a list of per-sequence float32 arrays [L_s, Hkv, D].
    """
    Hkv, D = logical[0].shape[1:]
    pool = np.full((num_blocks, Hkv, block_size, D), fill, dtype=np.float32)
    for s, rows in enumerate(logical):
        for j in range(rows.shape[0]):
            pool[tables[s][j // block_size], :, j % block_size, :] = rows[j]
    return pool


def tables_for(lengths, block_size, num_blocks, rng):
    """Random distinct physical ids for every sequence's blocks (scattered)."""
    ids = rng.permutation(num_blocks)
    out, k = [], 0
    nblk = [-(-n // block_size) for n in lengths]
    width = max(nblk)
    t = np.full((len(lengths), width), -1, dtype=np.int32)
    for s, n in enumerate(nblk):
        t[s, :n] = ids[k:k + n]
        k += n
    return t


class Tiny:
    """Tiny fp32 decode/prefill inputs with the logical K/V kept beside the pool."""

    def __init__(self, lengths, Hq, Hkv, D, block_size, seed, num_blocks=None, q=None,
                 kscale=1.0):
        rng = _rng(seed)
        self.lengths = list(lengths)
        self.B = block_size
        need = sum(-(-n // block_size) for n in lengths)
        self.NB = num_blocks or need + 3
        self.Hq, self.Hkv, self.D = Hq, Hkv, D
        self.tables = tables_for(lengths, block_size, self.NB, _rng(seed + 7919))
        self.K = [(kscale * rng.standard_normal((n, Hkv, D))).astype(np.float32) for n in lengths]
        self.V = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lengths]
        self.q = rng.standard_normal((len(lengths), Hq, D)).astype(np.float32) if q is None else q
        self.scale = float(np.float32(1.0 / math.sqrt(D)))
        self.build()

    def build(self, fill=np.nan):
        self.kc = scatter(self.K, self.tables, self.B, self.NB, fill)
        self.vc = scatter(self.V, self.tables, self.B, self.NB, fill)
        return self

    def decode(self, ref):
        return ref.decode_ref(self.q, self.kc, self.vc, self.tables,
                              np.asarray(self.lengths, np.int32), self.scale, "f32", self.B)


# --------------------------------------------------------------------------------- the pins
def check_hand_example(ref):
    """Two keys worked by hand: q=(1,0), K=((1,0),(0,1)), V=((1,2),(3,4)), scale 1.

    Scores (1, 0) give weights (e, 1)/(1+e), so out = ((e+3)/(1+e), (2e+4)/(1+e)).
    """
    q = np.array([[[1.0, 0.0]]], np.float32)
    kc = np.array([[[[1, 0], [0, 1]]]], np.float32)     # one block of 2 slots, one head
    vc = np.array([[[[1, 2], [3, 4]]]], np.float32)
    out = ref.decode_ref(q, kc, vc, np.array([[0]], np.int32), np.array([2], np.int32), 1.0,
                         "f32", block_size=2)
    e = math.e
    want = np.array([(e + 3) / (1 + e), (2 * e + 4) / (1 + e)])
    assert np.allclose(out[0, 0], want, rtol=0, atol=1e-15), (out[0, 0], want)


def check_brute_force(ref):
    """Paged oracle == loop-based contiguous attention on the logical rows (S1)."""
    for B in (4, 16):
        t = Tiny([1, 7, 33, 16], Hq=4, Hkv=2, D=8, block_size=B, seed=11)
        out = t.decode(ref)
        for s, L in enumerate(t.lengths):
            for h in range(t.Hq):
                g = h // (t.Hq // t.Hkv)
                want = brute.attention_row(t.q[s, h].tolist(), t.K[s][:, g].tolist(),
                                           t.V[s][:, g].tolist(), t.scale, L)
                assert np.max(np.abs(out[s, h] - want)) <= 1e-12, (B, s, h)
    # a chunk of 5 rows at the end of a 14-token sequence, and a prefix-0 chunk of 6
    for L, n in ((14, 5), (6, 6)):
        t = Tiny([L], Hq=2, Hkv=1, D=8, block_size=4, seed=12 + L)
        qc = _rng(99).standard_normal((n, 2, 8)).astype(np.float32)
        out = ref.prefill_ref(qc, t.kc, t.vc, t.tables, np.array([L], np.int32),
                              np.array([0, n], np.int32), t.scale, "f32", 4)
        for i in range(n):
            for h in range(2):
                want = brute.attention_row(qc[i, h].tolist(), t.K[0][:, 0].tolist(),
                                           t.V[0][:, 0].tolist(), t.scale, L - n + i + 1)
                assert np.max(np.abs(out[i, h] - want)) <= 1e-12, (L, n, i, h)


def check_permutation(ref):
    """Relabelling physical blocks (pool and table together) leaves the output bit-identical (S2)."""
    t = Tiny([5, 16, 17, 50], Hq=2, Hkv=1, D=16, block_size=16, seed=21, num_blocks=12)
    a = t.decode(ref)
    pi = _rng(22).permutation(t.NB)
    kc2 = np.empty_like(t.kc)
    vc2 = np.empty_like(t.vc)
    kc2[pi] = t.kc
    vc2[pi] = t.vc
    tab2 = np.where(t.tables >= 0, pi[np.maximum(t.tables, 0)], -1).astype(np.int32)
    b = ref.decode_ref(t.q, kc2, vc2, tab2, np.asarray(t.lengths, np.int32), t.scale, "f32", 16)
    assert np.array_equal(a, b)


def check_block_size_invariance(ref):
    """Block size 1, 4 and 16 over the same logical rows give bit-identical outputs (S3)."""
    outs = []
    for B in (1, 4, 16):
        t = Tiny([3, 16, 29], Hq=4, Hkv=1, D=8, block_size=B, seed=31)
        outs.append(t.decode(ref))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def check_row_sums(ref):
    """Softmax weights are non-negative and every row sums to 1 (S4)."""
    x = _rng(41).standard_normal((7, 123)) * 5
    w = ref.softmax_weights(x)
    assert np.all(w >= 0)
    assert np.max(np.abs(w.sum(axis=-1) - 1)) <= 1e-12
    # shift-invariance of the definition
    assert np.allclose(ref.softmax_weights(x + 3.25), w, rtol=0, atol=1e-15)


def check_single_token(ref):
    """A length-1 sequence returns its only V row exactly (S5)."""
    t = Tiny([1, 1], Hq=4, Hkv=2, D=8, block_size=16, seed=51)
    out = t.decode(ref)
    for s in range(2):
        for h in range(4):
            assert np.array_equal(out[s, h], t.V[s][0, h // 2].astype(np.float64))


def check_zero_query(ref):
    """q = 0 makes every weight equal: out is the mean of the visible V rows (S6)."""
    t = Tiny([9, 40], Hq=2, Hkv=1, D=8, block_size=16, seed=61,
             q=np.zeros((2, 2, 8), np.float32))
    out = t.decode(ref)
    for s, L in enumerate(t.lengths):
        want = t.V[s][:, 0].astype(np.float64).mean(axis=0)
        assert np.max(np.abs(out[s, 0] - want)) <= 1e-13


def check_constant_values(ref):
    """All V rows equal c gives c for any query (S7)."""
    t = Tiny([23], Hq=2, Hkv=1, D=4, block_size=16, seed=71)
    c = np.array([1.5, -2.0, 0.25, 7.0], np.float32)
    t.V = [np.broadcast_to(c, t.V[0].shape).copy()]
    t.build()
    out = t.decode(ref)
    assert np.max(np.abs(out[0] - c)) <= 1e-14 * 8


def check_needle(ref):
    """A key whose score towers 40+ over the rest pulls out its V row, at block edges (S8)."""
    L, B, D = 40, 16, 16
    for jstar in (0, 15, 16, L - 2, L - 1):
        t = Tiny([L], Hq=1, Hkv=1, D=D, block_size=B, seed=81 + jstar, kscale=0.05)
        qv = t.q[0, 0].astype(np.float64)
        t.K[0][jstar, 0] = (60.0 / (t.scale * float(qv @ qv)) * qv).astype(np.float32)
        t.build()
        out = t.decode(ref)
        assert np.max(np.abs(out[0, 0] - t.V[0][jstar, 0])) <= 1e-12, jstar


def check_sdpa(ref):
    """Grouped decode and a prefix-0 causal chunk equal torch's scaled_dot_product_attention (S9)."""
    F = torch.nn.functional
    L, Hq, Hkv, D = 37, 6, 2, 16
    t = Tiny([L], Hq=Hq, Hkv=Hkv, D=D, block_size=16, seed=91)
    Kc = torch.from_numpy(t.K[0].astype(np.float64)).permute(1, 0, 2)   # [Hkv, L, D]
    Vc = torch.from_numpy(t.V[0].astype(np.float64)).permute(1, 0, 2)
    Kr = Kc.repeat_interleave(Hq // Hkv, dim=0)[None]
    Vr = Vc.repeat_interleave(Hq // Hkv, dim=0)[None]
    qd = torch.from_numpy(t.q[0].astype(np.float64))[None, :, None, :]   # [1, Hq, 1, D]
    want = F.scaled_dot_product_attention(qd, Kr, Vr, scale=t.scale)[0, :, 0, :].numpy()
    got = t.decode(ref)[0]
    assert np.max(np.abs(got - want)) <= 1e-12
    qc = _rng(92).standard_normal((L, Hq, D)).astype(np.float32)
    got = ref.prefill_ref(qc, t.kc, t.vc, t.tables, np.array([L], np.int32),
                          np.array([0, L], np.int32), t.scale, "f32", 16)
    qt = torch.from_numpy(qc.astype(np.float64)).permute(1, 0, 2)[None]
    want = F.scaled_dot_product_attention(qt, Kr, Vr, is_causal=True, scale=t.scale)
    want = want[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(got - want)) <= 1e-12


def check_chunk_positions(ref):
    """Chunk row i (of n, ending a length-L sequence) equals a decode at length L - n + i + 1
    (S10), and it ignores later keys while seeing every prefix key.

    The chunk is evaluated as one masked product per head and the decode as one vector product
    per row, so the two agree to fp64 rounding (1e-13 here), not bit for bit; moving the causal
    bound by one key changes a row by about 1/L, some 1e-2 at these sizes."""
    L, n = 45, 12
    t = Tiny([L], Hq=2, Hkv=1, D=8, block_size=16, seed=101)
    qc = _rng(102).standard_normal((n, 2, 8)).astype(np.float32)
    ch = ref.prefill_ref(qc, t.kc, t.vc, t.tables, np.array([L], np.int32),
                         np.array([0, n], np.int32), t.scale, "f32", 16)
    for i in range(n):
        d = ref.decode_ref(qc[i:i + 1], t.kc, t.vc, t.tables, np.array([L - n + i + 1], np.int32),
                           t.scale, "f32", 16)
        assert np.max(np.abs(ch[i] - d[0])) <= 1e-13, i
    # a later key changes nothing for row 0; the first prefix key changes it
    i = 0
    kc, vc = t.kc.copy(), t.vc.copy()
    pos = L - n + i + 1
    kc[t.tables[0][pos // 16], :, pos % 16, :] += 3.0
    vc[t.tables[0][pos // 16], :, pos % 16, :] += 3.0
    ch2 = ref.prefill_ref(qc, kc, vc, t.tables, np.array([L], np.int32),
                          np.array([0, n], np.int32), t.scale, "f32", 16)
    assert np.array_equal(ch[i], ch2[i])
    vc = t.vc.copy()
    vc[t.tables[0][0], :, 0, :] += 3.0
    ch3 = ref.prefill_ref(qc, t.kc, vc, t.tables, np.array([L], np.int32),
                          np.array([0, n], np.int32), t.scale, "f32", 16)
    assert not np.array_equal(ch[i], ch3[i])


def check_append_roundtrip(ref):
    """Appending rows then reading them back through the table returns them bit-exactly,
    padding slots are skipped, and every other byte of the pool is unchanged (S11)."""
    B, NB, Hkv, D = 4, 9, 2, 3
    rng = _rng(111)
    kc = rng.standard_normal((NB, Hkv, B, D)).astype(np.float32)
    vc = rng.standard_normal((NB, Hkv, B, D)).astype(np.float32)
    table = np.array([7, 3, 5], np.int32)   # a sequence that already holds 5 tokens
    new_pos = [5, 6, 7, 8, 9]               # positions of its new tokens
    slots = [int(table[p // B]) * B + p % B for p in new_pos]
    slots.insert(2, -1)                      # a padding token in the middle
    T = len(slots)
    kn = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    k2, v2 = ref.append_ref(kc, vc, kn, vn, np.array(slots, np.int64), B)
    kg = ref.gather_tokens(k2, table, 10, B)
    vg = ref.gather_tokens(v2, table, 10, B)
    real = [t for t, s in enumerate(slots) if s >= 0]
    assert np.array_equal(kg[5:], kn[real]) and np.array_equal(vg[5:], vn[real])
    touched = np.zeros((NB, B), bool)
    for s in slots:
        if s >= 0:
            touched[s // B, s % B] = True
    def untouched(a):
        return a.transpose(0, 2, 1, 3)[~touched]
    assert np.array_equal(untouched(k2), untouched(kc))
    assert np.array_equal(untouched(v2), untouched(vc))
    try:
        ref.append_ref(kc, vc, kn[:2], vn[:2], np.array([4, 4], np.int64), B)
    except ref.OracleInputError:
        pass
    else:
        raise AssertionError("duplicate slots accepted")


def check_cow(ref):
    """After the copy each destination block equals its source byte for byte, K and V, and no
    other block changes; malformed pair sets are refused (S11)."""
    rng = _rng(121)
    kc = rng.standard_normal((10, 2, 4, 3)).astype(np.float32)
    vc = rng.standard_normal((10, 2, 4, 3)).astype(np.float32)
    pairs = np.array([[1, 6], [4, 2], [1, 9]], np.int64)
    k2, v2 = ref.cow_ref(kc, vc, pairs)
    for src, dst in pairs:
        assert k2[dst].tobytes() == kc[src].tobytes() and v2[dst].tobytes() == vc[src].tobytes()
    other = [b for b in range(10) if b not in (6, 2, 9)]
    assert np.array_equal(k2[other], kc[other]) and np.array_equal(v2[other], vc[other])
    for bad in ([[1, 1]], [[1, 6], [2, 6]], [[1, 6], [6, 3]], [[0, 10]]):
        try:
            ref.cow_ref(kc, vc, np.array(bad, np.int64))
        except ref.OracleInputError:
            continue
        raise AssertionError(f"bad pairs accepted: {bad}")


def check_swap(ref):
    """A swap-out and swap-in round trip through a smaller second pool restores every swapped
    block byte for byte in its new place, leaves the rest alone, and refuses bad pairs."""
    rng = _rng(127)
    gk = rng.standard_normal((8, 2, 4, 3)).astype(np.float32)
    gv = rng.standard_normal((8, 2, 4, 3)).astype(np.float32)
    ck = np.full((5, 2, 4, 3), np.nan, np.float32)
    cv = np.full((5, 2, 4, 3), np.nan, np.float32)
    out = np.array([[6, 3], [1, 0], [4, 4]], np.int64)        # (gpu, cpu)
    ck2, cv2 = ref.swap_ref(ck, cv, gk, gv, out)
    assert ck2[3].tobytes() == gk[6].tobytes() and cv2[0].tobytes() == gv[1].tobytes()
    assert np.all(np.isnan(ck2[[1, 2]])) and np.all(np.isnan(cv2[[1, 2]]))
    back = np.array([[3, 2], [0, 7], [4, 5]], np.int64)       # (cpu, gpu), new places
    gk2, gv2 = ref.swap_ref(gk, gv, ck2, cv2, back)
    for (g, c), (c2, g2) in zip(out, back):
        assert c == c2 and gk2[g2].tobytes() == gk[g].tobytes()
        assert gv2[g2].tobytes() == gv[g].tobytes()
    keep = [b for b in range(8) if b not in (2, 7, 5)]
    assert np.array_equal(gk2[keep], gk[keep]) and np.array_equal(gv2[keep], gv[keep])
    for bad in ([[0, 5]], [[8, 0]], [[1, 2], [3, 2]], [[-1, 0]]):
        try:
            ref.swap_ref(ck, cv, gk, gv, np.array(bad, np.int64))
        except ref.OracleInputError:
            continue
        raise AssertionError(f"bad pairs accepted: {bad}")


def check_nan_poison(ref):
    """NaN in every slot no sequence owns leaves the output finite and unchanged (S13)."""
    t = Tiny([5, 16, 30], Hq=2, Hkv=1, D=8, block_size=16, seed=131)
    a = t.build(fill=0.0).decode(ref)
    b = t.build(fill=np.nan).decode(ref)
    assert np.all(np.isfinite(b)) and np.array_equal(a, b)


def check_bf16_widening(ref):
    """bf16 bit patterns widen to the values IEEE bfloat16 assigns them."""
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0x3EAB, 0x8000], np.uint16)
    got = ref.to_f64(bits, "bf16")
    want = [1.0, -2.0, 2.0 ** -133, math.inf, (1 + 0x2B / 128) * 2.0 ** -2, -0.0]
    assert got[:5].tolist() == want[:5]
    assert got[5] == 0.0 and math.copysign(1, got[5]) == -1
    assert np.isnan(ref.to_f64(np.array([0x7FC0], np.uint16), "bf16")[0])


def check_bf16_decode(ref):
    """bf16 storage is read at its exact value: a bf16 pool gives the fp32 pool's answer when
    the fp32 values are exactly representable in bf16."""
    t = Tiny([19], Hq=2, Hkv=1, D=8, block_size=16, seed=141)
    # round every value to bf16 first, so both encodings hold the same numbers
    def to_bits(a):
        u = a.astype(np.float32).view(np.uint32)
        return (u >> 16).astype(np.uint16)        # truncation is exact for bf16-valued data
    def trunc(a):
        return (a.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    t.K = [trunc(t.K[0])]
    t.V = [trunc(t.V[0])]
    t.q = trunc(t.q)
    t.build()
    f = t.decode(ref)
    b = ref.decode_ref(to_bits(t.q), to_bits(t.kc), to_bits(t.vc), t.tables,
                       np.array([19], np.int32), t.scale, "bf16", 16)
    assert np.array_equal(f, b)


def check_subsets(ref):
    """Asking for a subset of rows (the full-size GPU comparisons do) computes exactly those
    rows, each equal to the same row of the full evaluation, and leaves every other row NaN:
    decode by sequence, chunks by packed row, including rows at chunk edges."""
    t = Tiny([5, 16, 17, 50, 3], Hq=4, Hkv=2, D=8, block_size=4, seed=151)
    full = t.decode(ref)
    lens = np.asarray(t.lengths, np.int32)
    for seqs in ([0], [4], [1, 3], [3, 1, 1], [0, 2, 4], []):
        part = ref.decode_ref(t.q, t.kc, t.vc, t.tables, lens, t.scale, "f32", 4, seqs=seqs)
        want = sorted(set(seqs))
        assert np.max(np.abs(part[want] - full[want]), initial=0.0) <= 1e-13, seqs
        rest = [s for s in range(len(lens)) if s not in want]
        assert np.all(np.isnan(part[rest])), seqs
    # two chunks: rows 0..5 end a 14-token sequence, rows 6..12 a 7-token one (prefix 0)
    t2 = Tiny([14, 7], Hq=2, Hkv=1, D=8, block_size=4, seed=152)
    qc = _rng(153).standard_normal((13, 2, 8)).astype(np.float32)
    sl, qsl = np.array([14, 7], np.int32), np.array([0, 6, 13], np.int32)
    full = ref.prefill_ref(qc, t2.kc, t2.vc, t2.tables, sl, qsl, t2.scale, "f32", 4)
    assert np.all(np.isfinite(full))
    for rows in ([0], [5], [6], [12], [5, 6], [0, 3, 7, 12], list(range(13)), []):
        part = ref.prefill_ref(qc, t2.kc, t2.vc, t2.tables, sl, qsl, t2.scale, "f32", 4,
                               rows=rows)
        assert np.max(np.abs(part[rows] - full[rows]), initial=0.0) <= 1e-13, rows
        rest = [r for r in range(13) if r not in rows]
        assert np.all(np.isnan(part[rest])), rows


def check_contiguous(ref):
    """The contiguous-KV decode equals loop brute force on the logical rows (S1 for the
    unpaged layout), ignores rows past each length (NaN there), and equals the paged oracle on
    the same rows scattered through a table."""
    t = Tiny([1, 7, 33, 16], Hq=4, Hkv=2, D=8, block_size=4, seed=161)
    cap = 48
    k = np.full((4, 2, cap, 8), np.nan, np.float32)
    v = np.full((4, 2, cap, 8), np.nan, np.float32)
    for s, L in enumerate(t.lengths):
        k[s, :, :L] = t.K[s].transpose(1, 0, 2)
        v[s, :, :L] = t.V[s].transpose(1, 0, 2)
    lens = np.asarray(t.lengths, np.int32)
    out = ref.decode_contiguous_ref(t.q, k, v, lens, t.scale, "f32")
    for s, L in enumerate(t.lengths):
        for h in range(4):
            g = h // 2
            want = brute.attention_row(t.q[s, h].tolist(), t.K[s][:, g].tolist(),
                                       t.V[s][:, g].tolist(), t.scale, L)
            assert np.max(np.abs(out[s, h] - want)) <= 1e-12, (s, h)
    assert np.max(np.abs(out - t.decode(ref))) <= 1e-13


ALL_CHECKS = [check_hand_example, check_brute_force, check_permutation,
              check_block_size_invariance, check_row_sums, check_single_token, check_zero_query,
              check_constant_values, check_needle, check_sdpa, check_chunk_positions,
              check_append_roundtrip, check_cow, check_swap, check_nan_poison,
              check_bf16_widening,
              check_bf16_decode, check_subsets, check_contiguous]
