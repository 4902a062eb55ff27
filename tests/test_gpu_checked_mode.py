"""Checked mode of the C ABI on one MI355X: calls whose index arrays break a device-content
precondition are refused before anything is enqueued, and calls with valid arrays give the same
bits as in unchecked mode.

Every refused case is built so that, even if the check failed to refuse it, the kernels would
stay inside allocated memory: the out-of-range block id still names a block of the allocation
(the pool is handed to the call as a shorter view), and the other cases break ordering or
uniqueness rules only.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_341_amd import ops
from paged_kv_cache_341_amd import workloads as W
from tests.gpu_util import dev_i32, dev_i64, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _checked():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    prev = ops.set_checked_mode(True)
    yield
    ops.set_checked_mode(prev)
    torch.cuda.synchronize()


def _refused(fn, *words):
    with pytest.raises(ops.PagedAttnError) as e:
        fn()
    assert e.value.status == 1, e.value
    msg = str(e.value)
    assert "checked mode" in msg, msg
    for w in words:
        assert w in msg, msg


def test_decode_refuses_out_of_pool_block_and_overlong_sequence():
    say("case: checked decode, block id past the declared pool; seq_len past max_seq_len")
    b = W.make_decode([40, 100, 300], 8, 2, 128, "bf16", seed=970, device=DEV, poison=False)
    nb = b.k_cache.shape[0]
    # the call sees the first nb blocks of a pool allocated with 8 more
    pad = torch.zeros((8,) + tuple(b.k_cache.shape[1:]), dtype=b.k_cache.dtype, device=DEV)
    k = torch.cat([b.k_cache, pad])[:nb]
    v = torch.cat([b.v_cache, pad])[:nb]
    bt = b.block_tables.copy()
    bt[1, 2] = nb                                       # allocated, but outside the declared pool
    sl = dev_i32(b.seq_lens)
    out = torch.empty_like(b.q)
    _refused(lambda: ops.pa_decode(out, b.q, k, v, dev_i32(bt), sl, b.max_seq_len, b.scale),
             "sequence 1", "table entry 2")
    _refused(lambda: ops.pa_decode(out, b.q, b.k_cache, b.v_cache, dev_i32(b.block_tables), sl,
                                   b.max_seq_len - 1, b.scale), "sequence 2", "seq_len 300")


def test_append_and_copy_refuse_bad_slots_and_pairs():
    say("case: checked kv_append with a repeated slot; cow with a destination that is a source")
    kc = torch.zeros(16, 2, 16, 128, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kn = torch.ones(3, 2, 128, dtype=torch.bfloat16, device=DEV)
    vn = torch.ones_like(kn)
    _refused(lambda: ops.kv_append(kc, vc, kn, vn, dev_i64(np.array([5, 6, 5]))),
             "token 2", "slot 5")
    _refused(lambda: ops.cow_copy_blocks(kc, vc, dev_i64(np.array([[1, 2], [2, 3]]))),
             "destination 2 is also a source")
    _refused(lambda: ops.cow_copy_blocks(kc, vc, dev_i64(np.array([[1, 4], [3, 4]]))),
             "destination 4 appears twice")
    assert torch.count_nonzero(kc) == 0 and torch.count_nonzero(vc) == 0, \
        "a refused call must enqueue nothing"


def test_prefill_refuses_chunk_longer_than_declared():
    say("case: checked prefill, a chunk longer than max_q_len")
    m = W.mixed_bf16(device=DEV, num_chunks=2, chunk_len=0, max_prefix=64, num_decode=1,
                     median=50, cap=100, num_q_heads=8, num_kv_heads=2, head_dim=128, seed=971,
                     chunk_lens=[10, 20], prefixes=[0, 33], poison=False)
    qsl = dev_i32(m.query_start_loc)
    out = torch.empty_like(m.q_chunk)
    _refused(lambda: ops.pa_prefill_chunk(out, m.q_chunk, m.k_cache, m.v_cache,
                                          dev_i32(m.chunk_tables), dev_i32(m.chunk_seq_lens),
                                          qsl, 15, int(m.chunk_seq_lens.max()), m.scale),
             "chunk 1 has 20 rows")


def test_valid_calls_match_unchecked_bits():
    say("case: checked mode on valid decode, prefill and append inputs")
    m = W.mixed_bf16(device=DEV, num_chunks=3, chunk_len=0, max_prefix=500, num_decode=6,
                     median=300, cap=2000, num_q_heads=8, num_kv_heads=2, head_dim=128,
                     seed=972, chunk_lens=[1, 64, 200], prefixes=[0, 100, 500])
    sm = dev_i64(m.slot_mapping)
    ops.kv_append(m.k_cache, m.v_cache, m.k_new, m.v_new, sm)
    args_c = (m.q_chunk, m.k_cache, m.v_cache, dev_i32(m.chunk_tables),
              dev_i32(m.chunk_seq_lens), dev_i32(m.query_start_loc),
              int(np.diff(m.query_start_loc).max()), int(m.chunk_seq_lens.max()), m.scale)
    args_d = (m.q_decode, m.k_cache, m.v_cache, dev_i32(m.decode_tables),
              dev_i32(m.decode_seq_lens), int(m.decode_seq_lens.max()), m.scale)
    oc1, od1 = torch.empty_like(m.q_chunk), torch.empty_like(m.q_decode)
    ops.pa_prefill_chunk(oc1, *args_c)
    ops.pa_decode(od1, *args_d)
    ops.set_checked_mode(False)
    oc2, od2 = torch.empty_like(m.q_chunk), torch.empty_like(m.q_decode)
    ops.pa_prefill_chunk(oc2, *args_c)
    ops.pa_decode(od2, *args_d)
    ops.set_checked_mode(True)
    assert torch.equal(oc1, oc2) and torch.equal(od1, od2)
