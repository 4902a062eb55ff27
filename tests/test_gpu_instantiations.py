"""Every compiled kernel instance, once, against the fp64 oracle through the C ABI.

The attention kernels are templates over element type, head_dim, query heads per kv head and
block size, and each combination is its own machine code.  The other GPU tests go deep on the
combinations the benchmark workloads use; this file runs every one of them on a small ragged
batch that still has several splits per row (so the merge runs), ragged chunks of one to a few
hundred rows over ragged prefixes, and NaN in every unfilled slot:
  * pa_decode: {bf16, fp32} x head_dim {64, 128, 256} x G {1, 2, 4, 8} x block size
    {1, 4, 8, 16, 32, 64} (144 instances);
  * pa_decode_contiguous: {bf16, fp32} x head_dim x G (24);
  * pa_prefill_chunk, pa_mixed_step and pa_decode_grouped: head_dim x G (12 each).
Tolerances are those of test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

from oracle import paged_ref as ref
from paged_kv_cache_341_amd import workloads as W
from paged_kv_cache_341_amd import ops
from tests.gpu_util import (ATOL, F32_ATOL, F32_RTOL, RTOL, Guarded, assert_close, dev_i32,
                            guarded_like, raw, run_append, run_decode, run_decode_grouped,
                            run_mixed_step, run_prefill, say, widen)

pytestmark = pytest.mark.gpu

DEV = "cuda"
GROUPS = (1, 2, 4, 8)
HEAD_DIMS = (64, 128, 256)
BLOCK_SIZES = (1, 4, 8, 16, 32, 64)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _tol(dtype):
    return (ATOL, RTOL) if dtype == "bf16" else (F32_ATOL, F32_RTOL)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", HEAD_DIMS)
def test_decode_every_group_and_block_size(dtype, D):
    """Lengths 1, B+1, 77, 300, 1100 and 2049 over 2 kv heads: about 9 splits for the longest
    row at every block size."""
    atol, rtol = _tol(dtype)
    for G in GROUPS:
        for B in BLOCK_SIZES:
            say(f"case: pa_decode {dtype} D={D} G={G} B={B}")
            lens = [1, B + 1, 77, 300, 1100, 2049]
            b = W.make_decode(lens, 2 * G, 2, D, dtype, seed=4000 + 100 * G + B + D,
                              device=DEV, block_size=B)
            n = ops.pa_decode_workspace_size(len(lens), 2 * G, 2, D, B, max(lens))
            assert n > 0, "the batch should need split partials"
            out = run_decode(b)
            want = ref.decode_ref(raw(b.q), raw(b.k_cache), raw(b.v_cache), b.block_tables,
                                  b.seq_lens, b.scale, dtype, B)
            assert_close(widen(out), want, atol, rtol, f"decode {dtype} D{D} G{G} B{B}")
            del b, out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", HEAD_DIMS)
def test_decode_contiguous_every_group(dtype, D):
    atol, rtol = _tol(dtype)
    for G in GROUPS:
        say(f"case: pa_decode_contiguous {dtype} D={D} G={G}")
        lens = [1, 17, 300, 1100, 2049]
        c = W.make_contiguous_decode(lens, 2 * G, 2, D, dtype, seed=4500 + G + D, device=DEV,
                                     capacity=2064)
        g = guarded_like(c.q)
        out = g.tensor(c.q.shape, c.q.dtype)
        n = ops.pa_decode_workspace_size(len(lens), 2 * G, 2, D, 16, c.max_seq_len)
        gw = Guarded(n, device=DEV)
        ops.pa_decode_contiguous(out, c.q, c.k, c.v, dev_i32(c.seq_lens), c.max_seq_len,
                                 c.scale, workspace=gw.bytes())
        g.check("contiguous out")
        gw.check("contiguous workspace")
        want = ref.decode_contiguous_ref(raw(c.q), raw(c.k), raw(c.v), c.seq_lens, c.scale,
                                         dtype)
        assert_close(widen(out), want, atol, rtol, f"contiguous {dtype} D{D} G{G}")


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_prefill_every_group(D):
    """Chunks of 1, 70, 200 and 33 rows over prefixes 0, 30, 500 and 1000."""
    for G in GROUPS:
        say(f"case: pa_prefill_chunk D={D} G={G}")
        m = W.mixed_bf16(device=DEV, num_chunks=4, chunk_len=0, num_decode=1, median=20, cap=40,
                         num_q_heads=2 * G, num_kv_heads=2, head_dim=D, seed=4700 + G + D,
                         chunk_lens=[1, 70, 200, 33], prefixes=[0, 30, 500, 1000])
        run_append(m.k_cache, m.v_cache, m.k_new, m.v_new, m.slot_mapping)
        out = run_prefill(m.q_chunk, m.k_cache, m.v_cache, m.chunk_tables, m.chunk_seq_lens,
                          m.query_start_loc, m.scale)
        want = ref.prefill_ref(raw(m.q_chunk), raw(m.k_cache), raw(m.v_cache), m.chunk_tables,
                               m.chunk_seq_lens, m.query_start_loc, m.scale, "bf16")
        assert_close(widen(out), want, ATOL, RTOL, f"prefill D{D} G{G}")


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_mixed_step_every_group(D):
    """Append, three chunks and 12 lognormal decodes in one pa_mixed_step call: the pool
    bit-exact, every chunk and decode row against the oracle."""
    for G in GROUPS:
        say(f"case: pa_mixed_step D={D} G={G}")
        m = W.mixed_bf16(device=DEV, seed=4900 + G + D, num_chunks=3, chunk_lens=[1, 90, 260],
                         prefixes=[0, 700, 40], num_decode=12, cap=3000, num_q_heads=2 * G,
                         num_kv_heads=2, head_dim=D)
        bk, bv = raw(m.k_cache), raw(m.v_cache)
        cout, dout = run_mixed_step(m)
        wk, wv = ref.append_ref(bk, bv, raw(m.k_new), raw(m.v_new), m.slot_mapping)
        kc, vc = raw(m.k_cache), raw(m.v_cache)
        assert np.array_equal(kc, wk) and np.array_equal(vc, wv), f"mixed pool D{D} G{G}"
        want = ref.prefill_ref(raw(m.q_chunk), kc, vc, m.chunk_tables, m.chunk_seq_lens,
                               m.query_start_loc, m.scale, "bf16")
        assert_close(widen(cout), want, ATOL, RTOL, f"mixed chunks D{D} G{G}")
        want = ref.decode_ref(raw(m.q_decode), kc, vc, m.decode_tables, m.decode_seq_lens,
                              m.scale, "bf16")
        assert_close(widen(dout), want, ATOL, RTOL, f"mixed decodes D{D} G{G}")


# (parent tokens, [tail tokens per member]): a partly filled shared block, a block-aligned
# prefix, a prefix longer than one 512-key shared split, and a group of one
FORKS = [(700, [5, 1, 16, 33]), (512, [20, 0]), (1100, [3, 90, 7]), (40, [9])]


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_decode_grouped_every_group(D):
    for G in GROUPS:
        say(f"case: pa_decode_grouped D={D} G={G}")
        b = W.make_grouped_decode(FORKS, 2 * G, 2, D, seed=5100 + G + D, device=DEV)
        out = run_decode_grouped(b, b.extra["group_start"], b.extra["shared_blocks"],
                                 b.extra["max_group_size"])
        want = ref.decode_ref(raw(b.q), raw(b.k_cache), raw(b.v_cache), b.block_tables,
                              b.seq_lens, b.scale, "bf16", b.block_size)
        assert_close(widen(out), want, ATOL, RTOL, f"grouped D{D} G{G}")
