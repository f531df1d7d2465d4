"""Pins for the KV-write oracle: the cache read back through block_table
(an independent path from slot_mapping) returns every token, nothing else
changes, and negative slots are skipped."""
import numpy as np

from chunked_prefill_attention_slot_amd.inputs import SENTINEL_K, SENTINEL_V, make_batch
from oracle.attention import gather_sequence
from oracle.kv_cache import kv_write


def test_round_trip_through_block_table():
    b = make_batch(7, num_q_heads=4, num_kv_heads=2, head_dim=16, page_size=8,
                   query_lens=[5, 1, 17], seq_lens=[12, 30, 17],
                   extra_pages=2, keep_logical=True)
    kc, vc = kv_write(b.k_cache, b.v_cache, b.k_new, b.v_new, b.slot_mapping, 8)
    for s in range(b.num_seqs):
        n = int(b.seq_lens[s])
        np.testing.assert_array_equal(gather_sequence(kc, b.block_table[s], n, 8), b.k_logical[s])
        np.testing.assert_array_equal(gather_sequence(vc, b.block_table[s], n, 8), b.v_logical[s])


def test_only_slots_change_and_negative_slots_skip():
    b = make_batch(8, num_q_heads=2, num_kv_heads=2, head_dim=8, page_size=4,
                   query_lens=[6], seq_lens=[10], extra_pages=1)
    slots = b.slot_mapping.copy()
    slots[2] = -1
    kc, vc = kv_write(b.k_cache, b.v_cache, b.k_new, b.v_new, slots, 4)
    changed = np.argwhere((kc != b.k_cache).any(axis=(1, 3)))  # (page, head) pairs
    written = set()
    for t, sl in enumerate(slots):
        if sl >= 0:
            written.add(int(sl))
            assert (kc[sl // 4, :, sl % 4] == b.k_new[t]).all()
            assert (vc[sl // 4, :, sl % 4] == b.v_new[t]).all()
    # every slot outside the written set is untouched
    for page in range(b.num_blocks):
        for off in range(4):
            if page * 4 + off not in written:
                assert (kc[page, :, off] == b.k_cache[page, :, off]).all()
                assert (vc[page, :, off] == b.v_cache[page, :, off]).all()
    skipped = int(b.slot_mapping[2])
    assert (kc[skipped // 4, :, skipped % 4] == SENTINEL_K).all()
    assert (vc[skipped // 4, :, skipped % 4] == SENTINEL_V).all()
    assert len(changed) > 0
