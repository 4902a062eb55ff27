"""HIP path vs the fp64 oracle on one MI355X, through the C ABI.

Tolerances: bf16 KV with fp32 accumulation, |gpu - ref| <= 5e-3 + 1e-2 |ref| per element;
fp32 throughout, 2e-5 + 2e-5 |ref|; append and copy-on-write, the whole pool bit-exact.
Unfilled and unowned slots hold NaN, so any read of them shows up as a non-finite output.
"""
import numpy as np
import pytest
import torch

from oracle import paged_ref as ref
from paged_kv_cache_341_amd import workloads as W
from paged_kv_cache_341_amd import checks, ops
from paged_kv_cache_341_amd.block_manager import shared_prefix_groups
from tests.gpu_util import (ATOL, F32_ATOL, F32_RTOL, RTOL, assert_close, compact, dev_i32,
                            dev_i64, raw,
                            run_append, run_cow, run_decode, run_decode_grouped, run_mixed_step,
                            run_prefill, say, widen)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def oracle_decode(batch, seqs=None):
    return ref.decode_ref(raw(batch.q), raw(batch.k_cache), raw(batch.v_cache),
                          batch.block_tables, batch.seq_lens, batch.scale, batch.dtype,
                          batch.block_size, seqs=seqs)


# ------------------------------------------------------------------------------ decode
def test_decode_tiny_f32():
    say("case: tiny_f32 decode (4 seqs {1,17,40,100}, 2q/1kv, D64, fp32)")
    b = W.tiny_f32(device=DEV)
    out = run_decode(b)
    want = oracle_decode(b)
    assert_close(widen(out), want, F32_ATOL, F32_RTOL, "tiny_f32")
    # a length-1 sequence returns its V row bit for bit
    v0 = b.v_cache[int(b.block_tables[0, 0]), 0, 0]
    assert torch.equal(out[0, 0], v0) and torch.equal(out[0, 1], v0)


@pytest.mark.parametrize("G,D", [(1, 64), (2, 128), (4, 128), (8, 128), (4, 256), (4, 64)])
def test_decode_bf16_ragged(G, D):
    lens = [1, 2, 15, 16, 17, 31, 33, 100, 257, 512, 513, 1000, 1500, 2049]
    say(f"case: bf16 decode ragged lens G={G} D={D}")
    b = W.make_decode(lens, 2 * G, 2, D, "bf16", seed=500 + G + D, device=DEV)
    out = run_decode(b)
    assert_close(widen(out), oracle_decode(b), ATOL, RTOL, f"ragged G{G} D{D}")
    # length-1 rows are exact
    tab = int(b.block_tables[0, 0])
    for h in range(2 * G):
        assert torch.equal(out[0, h], b.v_cache[tab, h // G, 0])


@pytest.mark.parametrize("G,D", [(2, 64), (4, 128), (8, 256)])
def test_decode_f32_ragged(G, D):
    lens = [1, 16, 17, 300, 1025]
    say(f"case: f32 decode ragged lens G={G} D={D}")
    b = W.make_decode(lens, G, 1, D, "f32", seed=600 + G + D, device=DEV)
    out = run_decode(b)
    assert_close(widen(out), oracle_decode(b), F32_ATOL, F32_RTOL, f"f32 G{G} D{D}")


@pytest.mark.parametrize("B", [1, 4, 8, 32, 64])
def test_decode_other_block_sizes(B):
    """Block sizes 1, 4, 8, 32 and 64 (16 is the default everywhere else): ragged lengths
    around block edges, NaN in every unfilled slot, G = 4, and an fp32 case."""
    lens = sorted(set(max(1, x) for x in [1, B - 1, B, B + 1, 3 * B + 5, 700, 2047, 4100]))
    say(f"case: bf16 decode, block size {B}")
    b = W.make_decode(lens, 16, 4, 128, "bf16", seed=1600 + B, device=DEV, block_size=B)
    out = run_decode(b)
    assert_close(widen(out), oracle_decode(b), ATOL, RTOL, f"block size {B}")
    tab = int(b.block_tables[0, 0])
    for h in range(16):
        assert torch.equal(out[0, h], b.v_cache[tab, h // 4, 0])
    f = W.make_decode(lens[:6], 4, 2, 64, "f32", seed=1700 + B, device=DEV, block_size=B)
    assert_close(widen(run_decode(f)), oracle_decode(f), F32_ATOL, F32_RTOL, f"f32 B{B}")


def _shrinking_plan_slots(max_len, G, unit):
    """Split slots of the shrinking plan the library picks for 64 sequences x 8 kv heads of up
    to max_len tokens: b = 512 tokens per split (capped at 8192 / G tokens), n = ceil(units / b),
    then max(1, n / 8) splits of 2b, two of b, then b / 2."""
    b = min(512 // unit, 8192 // G // unit)
    nb = -(-max_len // unit)
    n = -(-nb // b)
    assert 3 <= n <= 16 and 64 * 8 * n >= 2048
    s0, c0, s1, c1, s2 = min(2 * b, 8192 // G // unit), max(1, n // 8), b, 2, b // 2
    if nb <= c0 * s0:
        return -(-nb // s0)
    if nb <= c0 * s0 + c1 * s1:
        return c0 + -(-(nb - c0 * s0) // s1)
    return c0 + c1 + -(-(nb - c0 * s0 - c1 * s1) // s2)


@pytest.mark.parametrize("G,D,dtype,B", [(1, 64, "bf16", 16), (2, 256, "bf16", 16),
                                         (8, 128, "bf16", 16), (2, 128, "f32", 32),
                                         (4, 128, "bf16", 8), (4, 64, "bf16", 1),
                                         (4, 128, "bf16", 64)])
def test_decode_shrinking_split_plans(G, D, dtype, B):
    """64 sequences x 8 kv heads of up to 4096 tokens take split sizes that shrink toward the
    last splits (checked through the workspace size); every row against the oracle, with
    lengths on the plan's split edges and NaN in every unfilled slot."""
    say(f"case: shrinking split plan G={G} D={D} {dtype} B={B}")
    rng = np.random.default_rng(2600 + G + D + B)
    edges = [1, 16, 17, 1023, 1024, 1025, 1536, 1537, 2048, 2049, 3072, 4095, 4096]
    lens = edges + rng.integers(1, 4097, size=64 - len(edges)).tolist()
    b = W.make_decode(lens, 8 * G, 8, D, dtype, seed=2600 + G + D + B, device=DEV,
                      block_size=B)
    unit = B if B in (8, 16) else 16
    size = ops.pa_decode_workspace_size(64, 8 * G, 8, D, B, 4096)
    assert split_slots(size, 64 * 8 * G, D) == _shrinking_plan_slots(4096, G, unit)
    out = run_decode(b)
    atol, rtol = (ATOL, RTOL) if dtype == "bf16" else (F32_ATOL, F32_RTOL)
    assert_close(widen(out), oracle_decode(b), atol, rtol, f"plan G{G} D{D} {dtype} B{B}")
    tab = int(b.block_tables[0, 0])
    for h in range(8 * G):
        assert torch.equal(out[0, h], b.v_cache[tab, h // G, 0])


def test_decode_bf16_full_batch():
    """The 64-sequence batch at full size, every element against the oracle; then ten more
    calls that must each give the first call's bits (run-to-run identity)."""
    say("case: decode_bf16 full size (64 seqs, U[128,4096], 32/8, D128)")
    b = W.decode_bf16(device=DEV)
    out = run_decode(b)
    assert_close(widen(out), oracle_decode(b), ATOL, RTOL, "decode_bf16")
    for i in range(10):
        assert torch.equal(run_decode(b), out), f"call {i + 2} differs from call 1"


def test_decode_long_context_full_size():
    """The 32 x 32768-token batch (16/4 heads, D256) at full size: every sequence against the
    oracle, eight at a time on host copies of only the blocks they use."""
    say("case: long_bf16 full size (32 x 32768, 16/4, D256), every sequence")
    b = W.long_bf16(device=DEV)
    out = run_decode(b)
    got = widen(out)
    for first in range(0, b.num_seqs, 8):
        rows = list(range(first, min(first + 8, b.num_seqs)))
        kc, vc, tab = compact(b.k_cache, b.v_cache, b.block_tables, b.seq_lens, rows)
        want = ref.decode_ref(raw(b.q[rows]), kc, vc, tab, b.seq_lens[rows], b.scale, "bf16")
        assert_close(got[rows], want, ATOL, RTOL, f"long_bf16 sequences {rows[0]}-{rows[-1]}")
        del kc, vc


@pytest.mark.parametrize("jstar", [0, 15, 16, 1023, 1024, 2998, 2999])
def test_decode_needle(jstar):
    """One key's score towers over the rest: the output is its V row (catches gather slips)."""
    L = 3000
    say(f"case: needle at {jstar} of {L}")
    b = W.make_decode([L, 1234], 4, 1, 128, "bf16", seed=700, device=DEV)
    phys = int(b.block_tables[0, jstar // 16])
    qv = b.q[0, 0].float()
    k = (qv * (40.0 / (b.scale * float(qv @ qv)))).to(torch.bfloat16)
    b.k_cache[phys, 0, jstar % 16] = k
    out = run_decode(b)
    want = oracle_decode(b)
    assert_close(widen(out), want, ATOL, RTOL, "needle")
    target = b.v_cache[phys, 0, jstar % 16].float().cpu().numpy()
    assert np.max(np.abs(widen(out)[0, 0] - target)) < 0.05


@pytest.mark.parametrize("B", [1, 4, 32, 64])
@pytest.mark.parametrize("jstar", [0, 3, 4, 15, 16, 31, 32, 63, 64, 2999])
def test_decode_block_size_needle(B, jstar):
    """Needles at block and 16-token unit edges, with blocks smaller than a unit (each token's
    block is looked up on its own) and larger than one (a block is walked 16 tokens at a
    time)."""
    L = 3000
    say(f"case: needle at {jstar} of {L}, block size {B}")
    b = W.make_decode([L, 77], 4, 1, 128, "bf16", seed=710 + B, device=DEV, block_size=B)
    phys = int(b.block_tables[0, jstar // B])
    qv = b.q[0, 0].float()
    b.k_cache[phys, 0, jstar % B] = (qv * (40.0 / (b.scale * float(qv @ qv)))).to(torch.bfloat16)
    out = run_decode(b)
    assert_close(widen(out), oracle_decode(b), ATOL, RTOL, f"block size {B} needle")
    target = b.v_cache[phys, 0, jstar % B].float().cpu().numpy()
    assert np.max(np.abs(widen(out)[0, 0] - target)) < 0.05


# ------------------------------------------------------------------------------ contiguous KV
def run_contiguous(c):
    """pa_decode_contiguous with output and workspace between canary guard regions."""
    from tests.gpu_util import Guarded, guarded_like
    g = guarded_like(c.q)
    out = g.tensor(c.q.shape, c.q.dtype)
    n = ops.pa_decode_workspace_size(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim, 16,
                                     c.max_seq_len)
    gw = Guarded(n, device=DEV) if n else None
    ops.pa_decode_contiguous(out, c.q, c.k, c.v, dev_i32(c.seq_lens), c.max_seq_len, c.scale,
                             workspace=None if gw is None else gw.bytes())
    g.check("contiguous out")
    if gw is not None:
        gw.check("contiguous workspace")
    return out


def oracle_contiguous(c, seqs=None):
    return ref.decode_contiguous_ref(raw(c.q), raw(c.k), raw(c.v), c.seq_lens, c.scale, c.dtype,
                                     seqs=seqs)


@pytest.mark.parametrize("G,D,dtype", [(1, 64, "bf16"), (4, 128, "bf16"), (8, 128, "bf16"),
                                       (4, 256, "bf16"), (2, 128, "f32"), (8, 256, "f32")])
def test_decode_contiguous_ragged(G, D, dtype):
    """KV without paging (one slab per sequence and kv head): ragged lengths, NaN in every row
    past a length, bf16 and fp32; length-1 rows return their V row exactly."""
    say(f"case: contiguous decode G={G} D={D} {dtype}")
    lens = [1, 2, 15, 16, 17, 100, 513, 1000, 2049]
    c = W.make_contiguous_decode(lens, 2 * G, 2, D, dtype, seed=1800 + G + D, device=DEV,
                                 capacity=2064)
    out = run_contiguous(c)
    atol, rtol = (ATOL, RTOL) if dtype == "bf16" else (F32_ATOL, F32_RTOL)
    assert_close(widen(out), oracle_contiguous(c), atol, rtol, f"contiguous G{G} D{D} {dtype}")
    for h in range(2 * G):
        assert torch.equal(out[0, h], c.v[0, h // G, 0])


def test_decode_contiguous_full_size():
    """The 64-sequence batch's lengths and heads (capacity 4096) and the 32 x 32768 long
    context (16/4 heads, D256) in the contiguous layout, every sequence against the oracle."""
    say("case: contiguous decode at full size (64 x U[128,4096]; 32 x 32768 D256)")
    c = W.decode_bf16_contiguous(device=DEV)
    assert_close(widen(run_contiguous(c)), oracle_contiguous(c), ATOL, RTOL,
                 "decode_bf16 contiguous")
    del c
    torch.cuda.empty_cache()
    c = W.long_bf16_contiguous(device=DEV)
    got = widen(run_contiguous(c))
    for first in range(0, 32, 8):
        rows = list(range(first, first + 8))
        want = ref.decode_contiguous_ref(raw(c.q[rows]), raw(c.k[rows]), raw(c.v[rows]),
                                         c.seq_lens[rows], c.scale, "bf16")
        assert_close(got[rows], want, ATOL, RTOL, f"long contiguous {first}-{first + 7}")


def test_decode_permutation_invariant_and_deterministic():
    say("case: relabelled physical blocks give bit-identical output; reruns are identical")
    b = W.make_decode([77, 1000, 2500, 16], 8, 2, 128, "bf16", seed=800, device=DEV)
    a1 = run_decode(b).clone()
    a2 = run_decode(b).clone()
    assert torch.equal(a1, a2)
    nb = b.k_cache.shape[0]
    pi = np.random.default_rng(801).permutation(nb)
    pit = torch.from_numpy(pi).to(DEV)
    kc = torch.empty_like(b.k_cache)
    vc = torch.empty_like(b.v_cache)
    kc[pit] = b.k_cache
    vc[pit] = b.v_cache
    tab = np.where(b.block_tables >= 0, pi[np.maximum(b.block_tables, 0)], -1).astype(np.int32)
    b2 = W.DecodeBatch(q=b.q, k_cache=kc, v_cache=vc, block_tables=tab, seq_lens=b.seq_lens,
                       scale=b.scale, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       block_size=16, dtype="bf16")
    assert torch.equal(run_decode(b2), a1)


def test_decode_over_declared_max_len():
    """A max_seq_len larger than every length (more splits than needed) changes nothing."""
    b = W.make_decode([5, 600, 1999], 4, 1, 128, "bf16", seed=900, device=DEV)
    a = run_decode(b).clone()
    c = run_decode(b, max_seq_len=b.block_tables.shape[1] * 16)
    assert_close(widen(c), widen(a), 1e-6, 1e-6, "max_seq_len slack")


def test_decode_native_context_length():
    """The longest context the pages mention, 262,144 tokens, beside a half-length and a
    one-token sequence: 512 split slots per row, so the merge takes its general path (more
    than 64 splits, summed 64 at a time in split order)."""
    say("case: decode at 262144 tokens (512 splits per row)")
    b = W.make_decode([262144, 131073, 1], 8, 2, 128, "bf16", seed=1550, device=DEV)
    n = ops.pa_decode_workspace_size(3, 8, 2, 128, 16, 262144)
    assert n >= 3 * 8 * 512 * 130 * 4, "expected 512 split slots per row"
    out = run_decode(b)
    assert_close(widen(out), oracle_decode(b), ATOL, RTOL, "decode 262144")
    for h in range(8):
        assert torch.equal(out[2, h], b.v_cache[int(b.block_tables[2, 0]), h // 4, 0])


def test_prefill_at_native_context_length():
    """Chunks ending 262,144- and 131,000-token sequences (prefixes of 262,044 and 130,937)."""
    say("case: prefill chunks over 262k and 131k prefixes")
    _, out, want = _prefill_case(1560, [100, 63], [262044, 130937], G=4)
    assert_close(widen(out), want, ATOL, RTOL, "prefill 262k prefix")


def test_decode_workspace_reused_across_calls():
    """One uninitialised workspace serves calls of different shapes in turn (short and long
    splits), and every result matches the oracle: no workspace state carries over."""
    say("case: one decode workspace (torch.empty) reused by four calls")
    a = W.make_decode([3000, 17, 2500, 900, 4096], 8, 2, 128, "bf16", seed=950, device=DEV)
    b = W.make_decode([4000, 4000, 33], 16, 4, 128, "bf16", seed=951, device=DEV)
    c = W.make_decode([16384] * 19 + [5000], 8, 8, 64, "bf16", seed=952, device=DEV,
                      poison=False)
    size = max(ops.pa_decode_workspace_size(x.num_seqs, x.num_q_heads, x.num_kv_heads,
                                            x.head_dim, 16, x.max_seq_len) for x in (a, b, c))
    assert size > 0
    ws = torch.empty(size, dtype=torch.uint8, device=DEV).fill_(0xA5)
    for x in (a, c, b, c):
        bt, sl = dev_i32(x.block_tables), dev_i32(x.seq_lens)
        out = torch.empty_like(x.q)
        ops.pa_decode(out, x.q, x.k_cache, x.v_cache, bt, sl, x.max_seq_len, x.scale,
                      workspace=ws)
        assert_close(widen(out), oracle_decode(x), ATOL, RTOL, "reused workspace")


def split_slots(size, rows, head_dim):
    """Split slots per row of a decode workspace of `size` bytes (statistics block rounded up
    to 256 bytes, then the partial numerators)."""
    for n in range(1, 4096):
        if (rows * n * 8 + 255) // 256 * 256 + rows * n * head_dim * 4 == size:
            return n
    raise AssertionError(f"no slot count gives {size} bytes")


def test_decode_merge_ignores_unused_workspace_slots():
    """Rows with fewer splits than the workspace has slots (up to 16 slots per row: the merge
    requests every slot before it knows the row's split count) must ignore the unused slots:
    the workspace is filled with NaN bit patterns before the call.  The batch's split plan has
    sizes that shrink toward the later splits (11 slots for a 4096-token row)."""
    say("case: decode with a NaN-filled workspace, 1..11 splits per row")
    lens = [1, 15, 16, 17, 511, 512, 513, 1024, 1500, 2049, 3000, 4095, 4096]
    lens += list(range(100, 4096, 150))[:27]
    b = W.make_decode(lens, 32, 8, 128, "bf16", seed=960, device=DEV)
    size = ops.pa_decode_workspace_size(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                        16, b.max_seq_len)
    rows = b.num_seqs * b.num_q_heads
    assert split_slots(size, rows, 128) == 11, "the batch should plan 11 split slots per row"
    ws = torch.empty(size, dtype=torch.uint8, device=DEV).fill_(0xFF)
    bt, sl = dev_i32(b.block_tables), dev_i32(b.seq_lens)
    out = torch.empty_like(b.q)
    ops.pa_decode(out, b.q, b.k_cache, b.v_cache, bt, sl, b.max_seq_len, b.scale, workspace=ws)
    assert torch.isfinite(out.float()).all()
    assert_close(widen(out), oracle_decode(b), ATOL, RTOL, "NaN-filled workspace")


# ------------------------------------------------------------------------------ grouped decode
# (prefix, [tail per member]) per group: 8 forks over a 1200-token prefix with a copied partial
# block (so few rows that the prefix is cut into the shortest splits, 64 keys: 19 splits of 3 or
# 4 blocks, and every row merges more partials than one round trip takes); a single sequence;
# 3 identical forks whose every block is
# shared (no own blocks left); 4 forks that share no full block; 2 forks sharing one block;
# 5 forks over 2057 tokens (5 x G rows: two row tiles at G = 8).
GROUPS = [(1200, [5, 1, 16, 33, 100, 0, 2, 700]), (300, [20]), (640, [0, 0, 0]),
          (5, [30, 1, 2, 3]), (17, [1, 15]), (2057, [3, 64, 129, 1, 250])]


def grouped(b, **kw):
    return run_decode_grouped(b, b.extra["group_start"], b.extra["shared_blocks"],
                              b.extra["max_group_size"], **kw)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_grouped_matches_oracle(G):
    say(f"case: grouped decode, 6 groups, G={G}")
    b = W.make_grouped_decode(GROUPS, 2 * G, 2, 128, seed=1700 + G, device=DEV)
    assert b.extra["shared_blocks"].tolist()[:8] == [75] * 8
    out = grouped(b)
    assert_close(widen(out), oracle_decode(b), ATOL, RTOL, f"grouped G{G}")


@pytest.mark.parametrize("D,G", [(64, 1), (64, 4), (256, 2), (256, 4), (256, 8)])
def test_decode_grouped_head_dims(D, G):
    """The grouped decode at head_dim 64 (4 KiB key tiles) and 256 (16 KiB tiles, 32 loads per
    tile in flight) against the oracle, and equal to the plain decode when nothing is shared."""
    say(f"case: grouped decode, 6 groups, head_dim {D}, G={G}")
    b = W.make_grouped_decode(GROUPS, 2 * G, 2, D, seed=1800 + G + D, device=DEV)
    out = grouped(b)
    assert_close(widen(out), oracle_decode(b), ATOL, RTOL, f"grouped D{D} G{G}")
    s = W.make_decode([1, 17, 300, 513, 2049], 2 * G, 2, D, "bf16", seed=1850 + G + D,
                      device=DEV)
    S = s.num_seqs
    alone = run_decode_grouped(s, np.arange(S + 1, dtype=np.int32), np.zeros(S, np.int32), 1)
    assert torch.equal(alone, run_decode(s))


# 4 groups of 8 forks over prefixes up to 4100 tokens plus 32 single sequences, 32/8 heads:
# enough rows that the shared prefixes are cut into the longest splits (64 blocks of 16 keys;
# the 4096-token prefix into four such splits, the 2500-token one into three of 52 blocks)
LONG_GROUPS = ([(4100, [3, 10, 100, 1, 256, 17, 64, 33]), (2500, [5, 1, 16, 33, 100, 0, 2, 70]),
                (3000, [9, 9, 9, 9, 9, 9, 9, 9]), (1030, [1, 2, 3, 4, 5, 6, 7, 8])]
               + [(40 + 37 * i, [1 + i]) for i in range(32)])


@pytest.mark.parametrize("D", [64, 128, 256])
def test_decode_grouped_longest_shared_splits(D):
    say(f"case: grouped decode, 64 sequences over 4100-token prefixes, head_dim {D}")
    b = W.make_grouped_decode(LONG_GROUPS, 32, 8, D, seed=1900 + D, device=DEV)
    assert b.num_seqs == 64 and b.max_seq_len >= 4100
    out = grouped(b)
    assert_close(widen(out), oracle_decode(b), ATOL, RTOL, f"grouped long splits D{D}")


def test_decode_grouped_deterministic_with_dirty_workspace():
    """Two calls, the second with a workspace full of garbage, give the same bits; a larger
    declared max_seq_len (more split slots per row) gives the same bits too."""
    say("case: grouped decode, dirty workspace and declared max len")
    b = W.make_grouped_decode(GROUPS, 8, 2, 128, seed=1750, device=DEV)
    out1 = grouped(b)
    n = ops.pa_decode_grouped_workspace_size(b.num_seqs, 8, 2, 128, 16, b.max_seq_len)
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV)
    out2 = grouped(b, workspace=ws)
    assert torch.equal(out1, out2)
    b.block_tables = np.pad(b.block_tables, ((0, 0), (0, 200)), constant_values=-1)
    out3 = grouped(b, max_seq_len=b.max_seq_len + 3000)
    assert_close(widen(out3), widen(out1), 1e-6, 1e-6, "declared max len")


def test_decode_grouped_no_sharing_equals_plain():
    """With every group of one (nothing shared), the grouped call is the plain decode."""
    say("case: grouped decode with singleton groups only")
    b = W.make_decode([1, 17, 300, 513, 2049], 8, 2, 128, "bf16", seed=1760, device=DEV)
    S = b.num_seqs
    out = run_decode_grouped(b, np.arange(S + 1, dtype=np.int32), np.zeros(S, np.int32), 1)
    assert torch.equal(out, run_decode(b))


# ------------------------------------------------------------------------------ prefill
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_prefill_ragged_chunks(G):
    """Chunks of 1..300 rows over prefixes 0..~700, including a prefix-0 chunk."""
    say(f"case: prefill ragged chunks G={G}")
    m = W.mixed_bf16(device=DEV, num_chunks=5, chunk_len=0, max_prefix=700, num_decode=1,
                     median=50, cap=100, num_q_heads=2 * G, num_kv_heads=2, head_dim=128,
                     seed=1000 + G, chunk_lens=[1, 77, 300, 128, 33],
                     prefixes=[0, 5, 700, 64, 129])
    # run the append first so the chunk's own keys are in the pool
    run_append(m.k_cache, m.v_cache, m.k_new, m.v_new, m.slot_mapping)
    out = run_prefill(m.q_chunk, m.k_cache, m.v_cache, m.chunk_tables, m.chunk_seq_lens,
                      m.query_start_loc, m.scale)
    want = ref.prefill_ref(raw(m.q_chunk), raw(m.k_cache), raw(m.v_cache), m.chunk_tables,
                           m.chunk_seq_lens, m.query_start_loc, m.scale, "bf16")
    assert_close(widen(out), want, ATOL, RTOL, f"prefill G{G}")


def _prefill_case(seed, chunk_lens, prefixes, G, num_kv_heads=2, head_dim=128):
    m = W.mixed_bf16(device=DEV, num_chunks=len(chunk_lens), chunk_len=0, num_decode=1,
                     median=20, cap=40, num_q_heads=G * num_kv_heads,
                     num_kv_heads=num_kv_heads, head_dim=head_dim, seed=seed,
                     chunk_lens=list(chunk_lens), prefixes=list(prefixes))
    run_append(m.k_cache, m.v_cache, m.k_new, m.v_new, m.slot_mapping)
    out = run_prefill(m.q_chunk, m.k_cache, m.v_cache, m.chunk_tables, m.chunk_seq_lens,
                      m.query_start_loc, m.scale)
    want = ref.prefill_ref(raw(m.q_chunk), raw(m.k_cache), raw(m.v_cache), m.chunk_tables,
                           m.chunk_seq_lens, m.query_start_loc, m.scale, "bf16")
    return m, out, want


def test_prefill_many_chunks_natural_order():
    """More chunks than the kernel ranks longest-first: they are scheduled in order."""
    say("case: prefill 131 small chunks (natural order path)")
    rng = np.random.default_rng(1500)
    lens = rng.integers(1, 40, size=131)
    pre = rng.integers(0, 200, size=131)
    _, out, want = _prefill_case(1501, lens, pre, G=4)
    assert_close(widen(out), want, ATOL, RTOL, "prefill 131 chunks")


def test_prefill_short_and_tied_chunks():
    """Sequences shorter than one 64-key tile, and chunks of equal length (rank ties)."""
    say("case: prefill short sequences and tied lengths, G=8")
    m, out, want = _prefill_case(1502, [1, 3, 64, 64, 64, 17, 130], [0, 10, 100, 100, 100, 0, 0],
                                 G=8)
    assert_close(widen(out), want, ATOL, RTOL, "prefill short/tied")
    again = run_prefill(m.q_chunk, m.k_cache, m.v_cache, m.chunk_tables, m.chunk_seq_lens,
                        m.query_start_loc, m.scale)
    assert torch.equal(again, out), "prefill reruns differ"


@pytest.mark.parametrize("D,G", [(64, 1), (64, 4), (64, 8), (256, 1), (256, 2), (256, 4),
                                 (256, 8)])
def test_prefill_head_dims(D, G):
    """head_dim 64 (64-key tiles of half-width rows) and 256 (128-row work items of four waves,
    32-key tiles): ragged chunks over ragged prefixes, several row tiles per chunk, a prefix-0
    chunk and a one-row chunk."""
    say(f"case: prefill head_dim {D}, G={G}")
    _, out, want = _prefill_case(1510 + D + G, [1, 77, 300, 128, 33, 257],
                                 [0, 5, 700, 64, 129, 1000], G, head_dim=D)
    assert_close(widen(out), want, ATOL, RTOL, f"prefill D{D} G{G}")


@pytest.mark.parametrize("D", [64, 256])
def test_prefill_head_dims_long_prefix(D):
    """Chunks over 65k and 20k prefixes: hundreds of key tiles through the 4-stage ring."""
    say(f"case: prefill head_dim {D} over 65k and 20k prefixes")
    _, out, want = _prefill_case(1540 + D, [200, 31], [65000, 20011], G=4, head_dim=D)
    assert_close(widen(out), want, ATOL, RTOL, f"prefill D{D} long prefix")


@pytest.mark.parametrize("D", [64, 256])
def test_prefill_head_dims_short_tied_and_many(D):
    """Short and tied chunks (ranked path, reruns identical), then 131 chunks (in-order path)."""
    say(f"case: prefill head_dim {D}, short/tied chunks, then 131 chunks")
    m, out, want = _prefill_case(1520 + D, [1, 3, 64, 64, 64, 17, 130],
                                 [0, 10, 100, 100, 100, 0, 0], G=8, head_dim=D)
    assert_close(widen(out), want, ATOL, RTOL, f"prefill D{D} short/tied")
    again = run_prefill(m.q_chunk, m.k_cache, m.v_cache, m.chunk_tables, m.chunk_seq_lens,
                        m.query_start_loc, m.scale)
    assert torch.equal(again, out), "prefill reruns differ"
    rng = np.random.default_rng(1530 + D)
    _, out, want = _prefill_case(1531 + D, rng.integers(1, 40, size=131),
                                 rng.integers(0, 200, size=131), G=4, head_dim=D)
    assert_close(widen(out), want, ATOL, RTOL, f"prefill D{D} 131 chunks")


def test_prefill_one_row_chunk_equals_decode():
    say("case: a one-row chunk is a decode")
    b = W.make_decode([1, 40, 1000, 4095], 8, 2, 128, "bf16", seed=1100, device=DEV)
    d = run_decode(b)
    qsl = np.arange(5, dtype=np.int32)
    p = run_prefill(b.q, b.k_cache, b.v_cache, b.block_tables, b.seq_lens, qsl, b.scale)
    assert_close(widen(p), widen(d), 2e-3, 1e-2, "chunk vs decode")


# ------------------------------------------------------------------- append and CoW
def test_append_bit_exact_whole_pool():
    say("case: kv_append, reduced mixed step, whole pool bit-exact")
    m = W.mixed_bf16(device=DEV, num_chunks=3, chunk_len=100, max_prefix=300, num_decode=20,
                     seed=1200)
    before_k, before_v = raw(m.k_cache), raw(m.v_cache)
    sm = m.slot_mapping.copy()
    sm[::7] = -1                                  # padding tokens are skipped
    run_append(m.k_cache, m.v_cache, m.k_new, m.v_new, sm)
    wk, wv = ref.append_ref(before_k, before_v, raw(m.k_new), raw(m.v_new), sm)
    assert np.array_equal(raw(m.k_cache), wk) and np.array_equal(raw(m.v_cache), wv)


def test_append_f32_bit_exact():
    b = W.make_decode([40, 70], 2, 2, 64, "f32", seed=1300, device=DEV)
    T = 9
    k_new = torch.randn(T, 2, 64, device=DEV)
    v_new = torch.randn(T, 2, 64, device=DEV)
    slots = np.array([b.block_tables[0, 2] * 16 + 8 + i for i in range(8)] + [-5], np.int64)
    bk, bv = raw(b.k_cache), raw(b.v_cache)
    run_append(b.k_cache, b.v_cache, k_new, v_new, slots)
    wk, wv = ref.append_ref(bk, bv, raw(k_new), raw(v_new), slots)
    assert np.array_equal(raw(b.k_cache).view(np.uint32), wk.view(np.uint32))
    assert np.array_equal(raw(b.v_cache).view(np.uint32), wv.view(np.uint32))


def test_cow_bit_exact_whole_pool():
    say("case: cow_copy_blocks, reduced beams, whole pool bit-exact")
    m = W.beams_bf16(device=DEV, num_prompts=3, seed=1400)
    bk, bv = raw(m.k_cache), raw(m.v_cache)
    run_cow(m.k_cache, m.v_cache, m.cow_pairs)
    wk, wv = ref.cow_ref(bk, bv, m.cow_pairs)
    assert np.array_equal(raw(m.k_cache), wk) and np.array_equal(raw(m.v_cache), wv)


# ------------------------------------------------------------------- whole iterations
def test_mixed_step_full_size():
    """Full-size mixed step: append (whole pool exact), then every row of the eight chunks and
    every one of the 192 decodes against the oracle."""
    say("case: mixed_bf16 full size (8x512 chunks, 192 decodes), every row")
    m = W.mixed_bf16(device=DEV)
    bk, bv = raw(m.k_cache), raw(m.v_cache)
    run_append(m.k_cache, m.v_cache, m.k_new, m.v_new, m.slot_mapping)
    wk, wv = ref.append_ref(bk, bv, raw(m.k_new), raw(m.v_new), m.slot_mapping)
    kc, vc = raw(m.k_cache), raw(m.v_cache)
    assert np.array_equal(kc, wk) and np.array_equal(vc, wv)
    del wk, wv, bk, bv
    out = run_prefill(m.q_chunk, m.k_cache, m.v_cache, m.chunk_tables, m.chunk_seq_lens,
                      m.query_start_loc, m.scale)
    want = ref.prefill_ref(raw(m.q_chunk), kc, vc, m.chunk_tables, m.chunk_seq_lens,
                           m.query_start_loc, m.scale, "bf16")
    assert_close(widen(out), want, ATOL, RTOL, "mixed chunks, all 4096 rows")
    dec = W.DecodeBatch(q=m.q_decode, k_cache=m.k_cache, v_cache=m.v_cache,
                        block_tables=m.decode_tables, seq_lens=m.decode_seq_lens, scale=m.scale,
                        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                        dtype="bf16")
    dout = run_decode(dec)
    want = ref.decode_ref(raw(m.q_decode), kc, vc, m.decode_tables, m.decode_seq_lens, m.scale,
                          "bf16")
    assert_close(widen(dout), want, ATOL, RTOL, "mixed decodes, all 192")


def test_beam_step_full_size():
    """Full-size beam step: 112 copies, tail append (whole pool exact), decode of 128 beams."""
    say("case: beams_bf16 full size (16 prompts x 8 beams)")
    m = W.beams_bf16(device=DEV)
    assert m.cow_pairs.shape[0] == 112
    bk, bv = raw(m.k_cache), raw(m.v_cache)
    run_cow(m.k_cache, m.v_cache, m.cow_pairs)
    run_append(m.k_cache, m.v_cache, m.k_new, m.v_new, m.slot_mapping)
    wk, wv = ref.cow_ref(bk, bv, m.cow_pairs)
    wk, wv = ref.append_ref(wk, wv, raw(m.k_new), raw(m.v_new), m.slot_mapping)
    kc, vc = raw(m.k_cache), raw(m.v_cache)
    assert np.array_equal(kc, wk) and np.array_equal(vc, wv)
    dec = W.DecodeBatch(q=m.q_decode, k_cache=m.k_cache, v_cache=m.v_cache,
                        block_tables=m.decode_tables, seq_lens=m.decode_seq_lens, scale=m.scale,
                        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                        dtype="bf16")
    out = run_decode(dec)
    want = ref.decode_ref(raw(m.q_decode), kc, vc, m.decode_tables, m.decode_seq_lens, m.scale,
                          "bf16")
    assert_close(widen(out), want, ATOL, RTOL, "beams decode")
    # the grouped decode reads each prompt's shared blocks once for its 8 beams
    gs, sb, mg = shared_prefix_groups(m.decode_tables, m.decode_seq_lens, 16)
    assert gs.tolist() == list(range(0, 129, 8)) and mg == 8
    assert np.array_equal(sb, np.repeat(m.extra["shared_lens"] // 16, 8))
    gout = run_decode_grouped(dec, gs, sb, mg)
    assert_close(widen(gout), want, ATOL, RTOL, "beams grouped decode")


# ------------------------------------------------------------------------------ swap
def test_swap_out_and_in_through_pinned_host_pool():
    """The native block manager preempts the two latest requests by swapping: their blocks go
    to a pinned host pool (device-to-host swap_blocks), the freed device blocks are reused and
    overwritten, then both come back into new device blocks.  Host and device pools match the
    oracle's byte for byte after each step, and decode over the restored tables gives the same
    bits as before the swap."""
    from paged_kv_cache_341_amd.native_block_manager import NativeBlockManager
    from paged_kv_cache_341_amd.block_manager import SWAP
    say("case: swap out / in of two requests through a pinned host pool")
    rng = np.random.default_rng(1900)
    NB, NC, Hkv, D = 64, 40, 2, 128
    bm = NativeBlockManager(NB, 16, free_order=rng.permutation(NB), num_cpu_blocks=NC,
                            cpu_free_order=rng.permutation(NC))
    bm.add_sequence(0, 100)
    bm.add_sequence(1, 70)
    bm.fork(1, 2)
    _, cow = bm.append_tokens(2, 5)
    bm.add_sequence(3, 200)
    g = torch.Generator(device=DEV).manual_seed(1900)
    k = torch.randn((NB, Hkv, 16, D), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((NB, Hkv, 16, D), generator=g, device=DEV).to(torch.bfloat16)
    run_cow(k, v, np.asarray(cow, np.int64))
    seqs = [0, 1, 2, 3]
    q = torch.randn((4, 8, D), generator=g, device=DEV).to(torch.bfloat16)

    def decode():
        b = W.DecodeBatch(q=q, k_cache=k, v_cache=v, block_tables=bm.block_tables(seqs),
                          seq_lens=np.array([bm.seq_len(s) for s in seqs], np.int32),
                          scale=W.default_scale(D), num_q_heads=8, num_kv_heads=Hkv,
                          head_dim=D, block_size=16, dtype="bf16")
        return run_decode(b)

    before = decode()
    hk = torch.full((NC, Hkv, 16, D), float("nan"), dtype=torch.bfloat16).pin_memory()
    hv = torch.full((NC, Hkv, 16, D), float("nan"), dtype=torch.bfloat16).pin_memory()
    want_hk, want_hv = raw(hk), raw(hv)
    for expect in (2, 1):
        r, pairs = bm.preempt_latest(SWAP)
        assert r == expect
        p = np.asarray(pairs, np.int64)
        checks.check_swap_pairs(p, NB, NC)
        gk, gv = raw(k), raw(v)
        ops.swap_blocks(hk, hv, k, v, dev_i64(p))
        torch.cuda.synchronize()
        want_hk, want_hv = ref.swap_ref(want_hk, want_hv, gk, gv, p)
        assert np.array_equal(raw(hk), want_hk) and np.array_equal(raw(hv), want_hv)
    # the freed device blocks are reused: overwrite them
    freed = [b for b in range(NB) if bm.refcount(b) == 0]
    k[freed] = float("nan")
    v[freed] = float("nan")
    for expect in (1, 2):
        r, pairs = bm.swap_in_earliest()
        assert r == expect
        p = np.asarray(pairs, np.int64)
        checks.check_swap_pairs(p, NC, NB)
        gk, gv = raw(k), raw(v)
        ops.swap_blocks(k, v, hk, hv, dev_i64(p))
        torch.cuda.synchronize()
        wk, wv = ref.swap_ref(gk, gv, raw(hk), raw(hv), p)
        assert np.array_equal(raw(k), wk) and np.array_equal(raw(v), wv)
    assert torch.equal(decode(), before)


# ------------------------------------------------------------------------------ single launch
@pytest.mark.parametrize("G", [1, 4, 8])
def test_mixed_step_single_launch_ragged(G):
    """pa_mixed_step on a small ragged iteration: 5 chunks of {1, 37, 256, 300, 513} rows over
    prefixes {0, 5, 4000, 16, 1500} and 40 lognormal decodes.  The pool after the call is the
    oracle's append, bit for bit; every chunk and decode row matches the oracle; chunk rows
    are bit-identical to pa_prefill_chunk on the same pool (the same per-item code)."""
    say(f"case: mixed step single launch, ragged, G={G}")
    m = W.mixed_bf16(device=DEV, seed=2000 + G, num_chunks=5, chunk_lens=[1, 37, 256, 300, 513],
                     prefixes=[0, 5, 4000, 16, 1500], num_decode=40, cap=6000,
                     num_q_heads=2 * G, num_kv_heads=2)
    bk, bv = raw(m.k_cache), raw(m.v_cache)
    cout, dout = run_mixed_step(m)
    wk, wv = ref.append_ref(bk, bv, raw(m.k_new), raw(m.v_new), m.slot_mapping)
    kc, vc = raw(m.k_cache), raw(m.v_cache)
    assert np.array_equal(kc, wk) and np.array_equal(vc, wv)
    want = ref.prefill_ref(raw(m.q_chunk), kc, vc, m.chunk_tables, m.chunk_seq_lens,
                           m.query_start_loc, m.scale, "bf16")
    assert_close(widen(cout), want, ATOL, RTOL, "mixed chunks")
    alone = run_prefill(m.q_chunk, m.k_cache, m.v_cache, m.chunk_tables, m.chunk_seq_lens,
                        m.query_start_loc, m.scale)
    assert torch.equal(cout, alone)
    want = ref.decode_ref(raw(m.q_decode), kc, vc, m.decode_tables, m.decode_seq_lens, m.scale,
                          "bf16")
    assert_close(widen(dout), want, ATOL, RTOL, "mixed decodes")


@pytest.mark.parametrize("D,G", [(64, 1), (64, 8), (256, 2), (256, 4), (256, 8)])
def test_mixed_step_single_launch_head_dims(D, G):
    """pa_mixed_step at head_dim 64 (8-wave workgroups) and 256 (4-wave workgroups, 128-row
    chunk tiles): pool bit-exact after the append, chunk rows bit-identical to pa_prefill_chunk
    and within tolerance of the oracle, every decode row against the oracle."""
    say(f"case: mixed step single launch, head_dim {D}, G={G}")
    m = W.mixed_bf16(device=DEV, seed=2100 + D + G, num_chunks=4, chunk_lens=[1, 77, 300, 129],
                     prefixes=[0, 700, 33, 2000], num_decode=24, cap=5000,
                     num_q_heads=2 * G, num_kv_heads=2, head_dim=D)
    bk, bv = raw(m.k_cache), raw(m.v_cache)
    cout, dout = run_mixed_step(m)
    wk, wv = ref.append_ref(bk, bv, raw(m.k_new), raw(m.v_new), m.slot_mapping)
    kc, vc = raw(m.k_cache), raw(m.v_cache)
    assert np.array_equal(kc, wk) and np.array_equal(vc, wv)
    want = ref.prefill_ref(raw(m.q_chunk), kc, vc, m.chunk_tables, m.chunk_seq_lens,
                           m.query_start_loc, m.scale, "bf16")
    assert_close(widen(cout), want, ATOL, RTOL, f"mixed chunks D{D}")
    alone = run_prefill(m.q_chunk, m.k_cache, m.v_cache, m.chunk_tables, m.chunk_seq_lens,
                        m.query_start_loc, m.scale)
    assert torch.equal(cout, alone)
    want = ref.decode_ref(raw(m.q_decode), kc, vc, m.decode_tables, m.decode_seq_lens, m.scale,
                          "bf16")
    assert_close(widen(dout), want, ATOL, RTOL, f"mixed decodes D{D}")


def test_mixed_step_single_launch_long_decodes():
    """Two 100,000-token decodes beside two chunks: 391 decode splits per sequence (more than
    the in-kernel split-index tables would hold at one entry per thread), every row against
    the oracle."""
    say("case: mixed step single launch, two 100k-token decodes")
    m = W.mixed_bf16(device=DEV, seed=2200, num_chunks=2, chunk_lens=[40, 300],
                     prefixes=[10, 900], num_decode=2, median=100000.0, sigma=0.0, cap=131072,
                     num_q_heads=8, num_kv_heads=2)
    assert m.decode_seq_lens.tolist() == [100000, 100000]
    n = ops.pa_mixed_workspace_size(2, 8, 2, 128, 16, 100000)
    assert n > 2 * 8 * 300 * 130 * 4, "expected hundreds of split slots per row"
    cout, dout = run_mixed_step(m)
    kc, vc = raw(m.k_cache), raw(m.v_cache)
    want = ref.prefill_ref(raw(m.q_chunk), kc, vc, m.chunk_tables, m.chunk_seq_lens,
                           m.query_start_loc, m.scale, "bf16")
    assert_close(widen(cout), want, ATOL, RTOL, "mixed chunks beside long decodes")
    want = ref.decode_ref(raw(m.q_decode), kc, vc, m.decode_tables, m.decode_seq_lens, m.scale,
                          "bf16")
    assert_close(widen(dout), want, ATOL, RTOL, "mixed 100k-token decodes")


def test_mixed_step_single_launch_tied_lengths():
    """300 decodes of one length (every sequence ties on its split count) under the shrinking
    split plan: every workgroup must derive the same decode order, or items are repeated and
    others skipped; every row against the oracle, and two calls give the same bits."""
    say("case: mixed step single launch, 300 equal-length decodes")
    m = W.mixed_bf16(device=DEV, seed=2300, num_chunks=1, chunk_lens=[64], prefixes=[100],
                     num_decode=300, median=2000.0, sigma=0.0, cap=4096, num_q_heads=8,
                     num_kv_heads=2)
    assert set(m.decode_seq_lens.tolist()) == {2000}
    n = ops.pa_mixed_workspace_size(300, 8, 2, 128, 16, 2000)
    ws = torch.full((n,), 0x7F, dtype=torch.uint8, device=DEV)     # NaN partials if skipped
    cout, dout = run_mixed_step(m, workspace=ws)
    kc, vc = raw(m.k_cache), raw(m.v_cache)
    want = ref.decode_ref(raw(m.q_decode), kc, vc, m.decode_tables, m.decode_seq_lens, m.scale,
                          "bf16")
    assert_close(widen(dout), want, ATOL, RTOL, "mixed tied decodes")
    del kc, vc, want
    cout2, dout2 = run_mixed_step(m, workspace=ws)      # appends the same bytes again
    assert torch.equal(dout2, dout) and torch.equal(cout2, cout)


def test_mixed_step_single_launch_full_size():
    """The full mixed iteration (8 x 512-row chunks, 192 decodes) in one pa_mixed_step call,
    twice with the same garbage-filled workspace (the counters are reset by the call): pool
    bit-exact, every chunk row and every decode against the oracle, chunk rows bit-identical to
    pa_prefill_chunk, and the second call's outputs equal the first's."""
    say("case: mixed_bf16 full size, single launch, every row")
    m = W.mixed_bf16(device=DEV)
    bk, bv = raw(m.k_cache), raw(m.v_cache)
    n = ops.pa_mixed_workspace_size(192, 32, 8, 128, 16, int(m.decode_seq_lens.max()))
    ws = torch.full((n,), 0x7F, dtype=torch.uint8, device=DEV)
    cout, dout = run_mixed_step(m, workspace=ws)
    wk, wv = ref.append_ref(bk, bv, raw(m.k_new), raw(m.v_new), m.slot_mapping)
    kc, vc = raw(m.k_cache), raw(m.v_cache)
    assert np.array_equal(kc, wk) and np.array_equal(vc, wv)
    del wk, wv, bk, bv
    want = ref.prefill_ref(raw(m.q_chunk), kc, vc, m.chunk_tables, m.chunk_seq_lens,
                           m.query_start_loc, m.scale, "bf16")
    assert_close(widen(cout), want, ATOL, RTOL, "mixed single-launch chunks, all 4096 rows")
    alone = run_prefill(m.q_chunk, m.k_cache, m.v_cache, m.chunk_tables, m.chunk_seq_lens,
                        m.query_start_loc, m.scale)
    assert torch.equal(cout, alone)
    want = ref.decode_ref(raw(m.q_decode), kc, vc, m.decode_tables, m.decode_seq_lens, m.scale,
                          "bf16")
    assert_close(widen(dout), want, ATOL, RTOL, "mixed single-launch decodes, all 192")
    cout2, dout2 = run_mixed_step(m, workspace=ws)     # appends the same bytes again
    assert torch.equal(cout2, cout) and torch.equal(dout2, dout)


# ------------------------------------------------------------------------------ graph capture
def _replays_match(step, outs, replays=3):
    """Eager run, capture, then replays with eager work between them: every replay must give
    the eager outputs bit for bit."""
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(replays):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w)
        step()                                  # eager work between replays
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w)


def test_graph_capture_of_an_iteration():
    """kv_append, pa_prefill_chunk and pa_decode (split and merge) captured in one HIP graph,
    then the same iteration as one pa_mixed_step call captured in another: the calls allocate
    nothing, synchronise nothing and record no memset, so replays match eager runs."""
    say("case: graph capture of append + chunks + decodes, and of pa_mixed_step")
    m = W.mixed_bf16(device=DEV, seed=2100, num_chunks=3, chunk_lens=[64, 200, 7],
                     prefixes=[100, 3000, 0], num_decode=24, cap=5000)
    nb = m.k_cache.shape[0]
    checks.check_slots(m.slot_mapping, nb, 16)
    mq, msl = int(np.diff(m.query_start_loc).max()), int(m.chunk_seq_lens.max())
    dmsl = int(m.decode_seq_lens.max())
    checks.check_tables(m.chunk_tables, m.chunk_seq_lens, nb, 16, msl)
    checks.check_tables(m.decode_tables, m.decode_seq_lens, nb, 16, dmsl)
    sm = dev_i64(m.slot_mapping)
    ct, cl, qsl = dev_i32(m.chunk_tables), dev_i32(m.chunk_seq_lens), dev_i32(m.query_start_loc)
    dt, dl = dev_i32(m.decode_tables), dev_i32(m.decode_seq_lens)
    cout, dout = torch.empty_like(m.q_chunk), torch.empty_like(m.q_decode)
    dws = torch.empty(max(ops.pa_decode_workspace_size(24, 32, 8, 128, 16, dmsl), 16),
                      dtype=torch.uint8, device=DEV)

    def step():
        ops.kv_append(m.k_cache, m.v_cache, m.k_new, m.v_new, sm)
        ops.pa_prefill_chunk(cout, m.q_chunk, m.k_cache, m.v_cache, ct, cl, qsl, mq, msl, m.scale)
        ops.pa_decode(dout, m.q_decode, m.k_cache, m.v_cache, dt, dl, dmsl, m.scale,
                      workspace=dws)

    _replays_match(step, [cout, dout])
    mws = torch.empty(ops.pa_mixed_workspace_size(24, 32, 8, 128, 16, dmsl), dtype=torch.uint8,
                      device=DEV)
    cout2, dout2 = torch.empty_like(cout), torch.empty_like(dout)

    def single():
        ops.pa_mixed_step(m.k_cache, m.v_cache, m.scale, k_new=m.k_new, v_new=m.v_new,
                          slot_mapping=sm, chunk_out=cout2, chunk_q=m.q_chunk, chunk_tables=ct,
                          chunk_seq_lens=cl, query_start_loc=qsl, chunk_max_q_len=mq,
                          chunk_max_seq_len=msl, dec_out=dout2, dec_q=m.q_decode,
                          dec_tables=dt, dec_seq_lens=dl, dec_max_seq_len=dmsl, workspace=mws)

    _replays_match(single, [cout2, dout2])
    assert torch.equal(cout2, cout)


def test_graph_capture_of_grouped_decode():
    say("case: graph capture of pa_decode_grouped")
    b = W.make_grouped_decode(GROUPS, 8, 2, 128, seed=2200, device=DEV)
    msl = b.max_seq_len
    bt, sl = dev_i32(b.block_tables), dev_i32(b.seq_lens)
    gs, sb = dev_i32(b.extra["group_start"]), dev_i32(b.extra["shared_blocks"])
    out = torch.empty_like(b.q)
    ws = torch.empty(ops.pa_decode_grouped_workspace_size(b.num_seqs, 8, 2, 128, 16, msl),
                     dtype=torch.uint8, device=DEV)

    def step():
        ops.pa_decode_grouped(out, b.q, b.k_cache, b.v_cache, bt, sl, gs, sb,
                              b.extra["max_group_size"], msl, b.scale, workspace=ws)

    _replays_match(step, [out])
    assert_close(widen(out), oracle_decode(b), ATOL, RTOL, "grouped decode replayed")
