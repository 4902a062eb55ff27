"""Plant plausible mistakes in the oracle (on the CPU) and show that some pin catches each one."""
import numpy as np
import pytest

from oracle import paged_ref
from tests import oracle_checks as oc

_orig_attend = paged_ref.attend
_orig_softmax = paged_ref.softmax_weights
_orig_append = paged_ref.append_ref
_orig_cow = paged_ref.cow_ref
_orig_swap = paged_ref.swap_ref
_orig_gather = paged_ref.gather_tokens
_orig_selected = paged_ref.selected
_orig_contig = paged_ref.decode_contiguous_ref


def _contig_one_row_too_many(q, k, v, seq_lens, scale, dtype, seqs=None):
    return _orig_contig(q, k, v, np.asarray(seq_lens) + 1, scale, dtype, seqs)


def _contig_heads_swapped(q, k, v, seq_lens, scale, dtype, seqs=None):
    return _orig_contig(q, k[:, ::-1], v[:, ::-1], seq_lens, scale, dtype, seqs)


def _gather_ignoring_table(cache, table_row, length, block_size):
    j = np.arange(length)
    return cache[j // block_size, :, j % block_size, :]


MUTATIONS = {
    "offset_off_by_one": ("token_position", lambda j, B: (j // B, (j + 1) % B)),
    "block_and_offset_swapped": ("token_position", lambda j, B: (j % B, j // B)),
    "gqa_modulo_map": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "causal_excludes_self": ("visible_keys", lambda p: p),
    "causal_one_too_many": ("visible_keys", lambda p: p + 2),
    "scale_dropped": ("attend", lambda q, K, V, s, vis=None: _orig_attend(q, K, V, 1.0, vis)),
    "scale_squared": ("attend", lambda q, K, V, s, vis=None: _orig_attend(q, K, V, s * s, vis)),
    "keys_used_as_values": ("attend", lambda q, K, V, s, vis=None: _orig_attend(q, K, K, s, vis)),
    "mask_ignored": ("attend", lambda q, K, V, s, vis=None: _orig_attend(q, K, V, s)),
    "subset_shifted_by_one": ("selected", lambda n, w=None, first=0:
                              _orig_selected(n, w, first + 1)),
    "subset_drops_last": ("selected", lambda n, w=None, first=0: _orig_selected(n, w, first)[:-1]),
    "subset_ignored": ("selected", lambda n, w=None, first=0: _orig_selected(n, None, first)),
    "contiguous_row_past_length": ("decode_contiguous_ref", _contig_one_row_too_many),
    "contiguous_kv_heads_swapped": ("decode_contiguous_ref", _contig_heads_swapped),
    "softmax_unnormalised": ("softmax_weights",
                             lambda x: np.exp(x - np.max(x, axis=-1, keepdims=True))),
    "softmax_sign_flipped": ("softmax_weights", lambda x: _orig_softmax(-x)),
    "softmax_drops_last_key": ("softmax_weights",
                               lambda x: _orig_softmax(x) * (np.arange(x.shape[-1]) < x.shape[-1] - 1)),
    "table_ignored": ("gather_tokens", _gather_ignoring_table),
    "append_v_gets_k": ("append_ref", lambda kc, vc, kn, vn, sm, B=16: _orig_append(kc, vc, kn, kn, sm, B)),
    "append_skips_last": ("append_ref", lambda kc, vc, kn, vn, sm, B=16:
                          _orig_append(kc, vc, kn, vn, np.where(np.arange(len(sm)) == len(sm) - 1, -1, sm), B)),
    "cow_k_only": ("cow_ref", lambda kc, vc, p: (_orig_cow(kc, vc, p)[0], np.array(vc, copy=True))),
    "swap_pairs_reversed": ("swap_ref", lambda dk, dv, sk, sv, p:
                            _orig_swap(dk, dv, sk, sv, np.asarray(p)[:, ::-1])),
    "swap_v_from_k": ("swap_ref", lambda dk, dv, sk, sv, p: _orig_swap(dk, dv, sk, sk, p)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(paged_ref, attr, fn)
    failed = []
    for check in oc.ALL_CHECKS:
        try:
            check(paged_ref)
        except (AssertionError, paged_ref.OracleInputError, IndexError, ValueError):
            failed.append(check.__name__)
    assert failed, f"mutation {name} passed every pin"
