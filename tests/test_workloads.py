"""Structure of the seeded synthetic workloads (CPU only, reduced sizes where values are drawn)."""
import math

import numpy as np
import torch

from paged_kv_cache_341_amd import workloads as W
from paged_kv_cache_341_amd.block_manager import blocks_for


def test_tiny_f32_layout():
    b = W.tiny_f32()
    assert b.seq_lens.tolist() == [1, 17, 40, 100]
    assert b.k_cache.shape == (64, 1, 16, 64) and b.k_cache.dtype == torch.float32
    assert b.scale == 0.125
    perm = np.random.default_rng(W.SEED_BASE + 1).permutation(64)
    used = [x for row in b.block_tables for x in row if x >= 0]
    assert used == perm[:13].tolist()
    # poison: exactly the unowned slots are NaN
    nan_slots = torch.isnan(b.k_cache[:, 0, :, 0]).numpy()
    assert nan_slots.sum() == 64 * 16 - 158


def test_decode_bf16_reduced():
    b = W.decode_bf16(num_seqs=6, lo=128, hi=300)
    assert b.k_cache.dtype == torch.bfloat16
    assert b.seq_lens.min() >= 128 and b.seq_lens.max() <= 300
    need = sum(blocks_for(int(n), 16) for n in b.seq_lens)
    assert b.k_cache.shape[0] == math.ceil(1.2 * need)
    assert b.scale == W.f32(1 / math.sqrt(128))


def test_mixed_reduced_structure():
    m = W.mixed_bf16(num_chunks=3, chunk_len=40, max_prefix=100, num_decode=5, median=50,
                     cap=200, num_q_heads=4, num_kv_heads=2, head_dim=64)
    assert m.query_start_loc.tolist() == [0, 40, 80, 120]
    pre = m.extra["prefixes"]
    assert m.chunk_seq_lens.tolist() == (pre + 40).tolist()
    assert len(m.slot_mapping) == 3 * 40 + 5
    assert len(set(m.slot_mapping.tolist())) == len(m.slot_mapping)
    # new-token slots are NaN-poisoned before the append
    kc = m.k_cache
    for s in m.slot_mapping[:10]:
        assert torch.isnan(kc[s // 16, :, s % 16, :]).all()
    # the decode table row reaches every token's block
    for d, L in enumerate(m.decode_seq_lens):
        assert (m.decode_tables[d, :blocks_for(int(L), 16)] >= 0).all()


def test_beams_structure():
    m = W.beams_bf16(num_prompts=3, num_q_heads=4, num_kv_heads=2, head_dim=64)
    assert m.cow_pairs.shape == (3 * 7, 2)
    src, dst = m.cow_pairs[:, 0], m.cow_pairs[:, 1]
    assert len(set(dst.tolist())) == len(dst) and not set(src.tolist()) & set(dst.tolist())
    shared = m.extra["shared_lens"]
    tails = m.extra["tails"]
    for p in range(3):
        for b in range(8):
            assert m.decode_seq_lens[p * 8 + b] == shared[p] + tails[p, b]
            # all beams of a prompt share the full prefix blocks
            assert (m.decode_tables[p * 8 + b, :shared[p] // 16]
                    == m.decode_tables[p * 8, :shared[p] // 16]).all()
    assert len(m.slot_mapping) == int(tails.sum())


def test_standard_workload_sizes():
    """Full-size structure of the standard workloads, without drawing their values."""
    rng = np.random.default_rng(W.SEED_BASE + 2)
    lens = rng.integers(128, 4097, size=64)
    assert lens.min() >= 128 and lens.max() <= 4096
    assert math.ceil(1.2 * 32 * 2048) == 78644
