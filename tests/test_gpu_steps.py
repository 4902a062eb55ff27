"""Continuous batching under a per-step token cap, through the kernels, against the oracle.

The native step planner (pa_sp_*) plans each iteration: eight prompts arrive, are prefilled in
chunks across steps within a cap of 256 tokens per step, then decode.  Every iteration runs on
one MI355X through the C ABI (pa_mixed_step on even steps; kv_append, pa_prefill_chunk and
pa_decode on odd ones), and after each one the whole pool is compared with the oracle's append
and every chunk row and decode row with the oracle's attention over that pool."""
import numpy as np
import pytest
import torch

from oracle import paged_ref as ref
from paged_kv_cache_341_amd import workloads as W
from paged_kv_cache_341_amd.native_block_manager import NativeBlockManager, NativeStepPlanner
from tests.gpu_util import (ATOL, RTOL, assert_close, raw, run_append, run_decode,
                            run_mixed_step, run_prefill, say, widen)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def test_token_capped_iterations_match_oracle():
    NB, Hq, Hkv, D, B, CAP = 512, 8, 2, 128, 16, 256
    prompts = [100, 700, 37, 450, 16, 333, 1, 260]
    rng = np.random.default_rng(2500)
    bm = NativeBlockManager(NB, B, free_order=rng.permutation(NB))
    sp = NativeStepPlanner(bm, CAP)
    for s, n in enumerate(prompts):
        sp.add_request(s, n)
    g = torch.Generator(device=DEV).manual_seed(2500)

    def randn(*shape):
        return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)

    k = torch.full((NB, Hkv, B, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    v = torch.full_like(k, float("nan"))
    scale = W.default_scale(D)
    prefilled = {s: 0 for s in range(len(prompts))}
    step = 0
    while step < 24:
        p = sp.step()
        assert not p.cow_pairs and p.num_tokens <= CAP
        T = p.num_tokens
        say(f"case: capped step {step}: chunks {list(zip(p.chunk_seqs, p.chunk_lens))}, "
            f"{len(p.decode_seqs)} decodes, {T} tokens")
        for s, n in zip(p.chunk_seqs, p.chunk_lens):
            prefilled[s] += n
        C, S = len(p.chunk_seqs), len(p.decode_seqs)
        total_q = int(sum(p.chunk_lens))
        q_chunk = randn(total_q, Hq, D)
        q_dec = randn(S, Hq, D)
        k_new, v_new = randn(T, Hkv, D), randn(T, Hkv, D)
        ct = bm.block_tables(p.chunk_seqs) if C else np.zeros((0, 1), np.int32)
        dt = bm.block_tables(p.decode_seqs) if S else np.zeros((0, 1), np.int32)
        cl = np.array([bm.seq_len(s) for s in p.chunk_seqs], np.int32)
        dl = np.array([bm.seq_len(s) for s in p.decode_seqs], np.int32)
        qsl = p.query_start_loc()
        bk, bv = raw(k), raw(v)
        if step % 2 == 0:
            m = W.MixedStep(k_cache=k, v_cache=v, k_new=k_new, v_new=v_new,
                            slot_mapping=p.slot_mapping, q_chunk=q_chunk, chunk_tables=ct,
                            chunk_seq_lens=cl, query_start_loc=qsl, q_decode=q_dec,
                            decode_tables=dt, decode_seq_lens=dl,
                            cow_pairs=np.zeros((0, 2), np.int64), scale=scale,
                            num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                            dtype="bf16")
            cout, dout = run_mixed_step(m)
        else:
            run_append(k, v, k_new, v_new, p.slot_mapping)
            cout = run_prefill(q_chunk, k, v, ct, cl, qsl, scale) if C else None
            dout = None
            if S:
                dout = run_decode(W.DecodeBatch(q=q_dec, k_cache=k, v_cache=v, block_tables=dt,
                                                seq_lens=dl, scale=scale, num_q_heads=Hq,
                                                num_kv_heads=Hkv, head_dim=D, block_size=B,
                                                dtype="bf16"))
        wk, wv = ref.append_ref(bk, bv, raw(k_new), raw(v_new), p.slot_mapping)
        kc, vc = raw(k), raw(v)
        assert np.array_equal(kc, wk) and np.array_equal(vc, wv), f"step {step}: pool"
        if C:
            want = ref.prefill_ref(raw(q_chunk), kc, vc, ct, cl, qsl, scale, "bf16")
            assert_close(widen(cout), want, ATOL, RTOL, f"step {step} chunks")
        if S:
            want = ref.decode_ref(raw(q_dec), kc, vc, dt, dl, scale, "bf16")
            assert_close(widen(dout), want, ATOL, RTOL, f"step {step} decodes")
        step += 1
        if S == len(prompts) and not C:
            break
    assert prefilled == dict(enumerate(prompts))
    assert sp.counts() == (len(prompts), 0)
