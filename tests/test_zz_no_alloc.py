"""cpa_kv_write_attention_static, the entry point that allocates nothing
(its workspace is a static device array): the same results as
cpa_kv_write_attention with a caller workspace, bit for bit (output and
both caches), on calls in a row with different plans, the later ones
smaller; and its host-side refusals."""
import ctypes

import numpy as np
import pytest

from chunked_prefill_attention_slot_amd.inputs import llama3_8b_chunk, make_batch, small_parity


@pytest.fixture(scope="module")
def cpa():
    from chunked_prefill_attention_slot_amd import binding
    return binding


def test_static_refuses_oversized_plan_and_null_pointers(cpa):
    """Checked on the host before any GPU work (runs without a GPU)."""
    d = cpa.layer_desc(40, 40, 128, 128, num_blocks=5000, max_blocks_per_seq=64)
    # 64 decode rows of 8192 keys in 64-key splits: 64*40*128 partial rows of
    # 128 bf16 values, 84 MB of workspace
    p = cpa.cpa_plan_create(d, [1] * 64, [8192] * 64, {"decode_split_keys": 64})
    assert p.workspace_bytes > cpa.STATIC_SCRATCH_BYTES
    fake = ctypes.c_void_p(256)
    st = cpa._lib.cpa_kv_write_attention_static(p.handle, *([fake] * 8), None)
    assert st == cpa.CPA_ERR_WORKSPACE
    assert "static scratch" in cpa.cpa_last_error()
    assert cpa._lib.cpa_kv_write_attention_static(None, *([fake] * 8), None) == \
        cpa.CPA_ERR_INVALID_ARG
    small = cpa.cpa_plan_create(d, [4], [10])
    for hole in range(8):
        args = [fake] * 8
        args[hole] = None
        st = cpa._lib.cpa_kv_write_attention_static(small.handle, *args, None)
        assert st == cpa.CPA_ERR_INVALID_ARG, hole
        assert "NULL" in cpa.cpa_last_error()


@pytest.mark.gpu
def test_static_equals_workspace_call(cpa):
    torch = pytest.importorskip("torch")
    from tests import gpu_helpers as H
    cases = [
        ("llama3_8b_H4096", llama3_8b_chunk(4096), {0: [0, 1, 255, 511]}),    # split tiles
        ("small_parity", small_parity(), None),                              # smaller plan
        ("ragged_p16", make_batch(21, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                                  query_lens=[70, 1, 33, 5], seq_lens=[300, 90, 33, 200],
                                  extra_pages=4), None),                     # decode row, splits
        ("small_parity_again", small_parity(), None),                        # same shape again
    ]
    for name, b, rows in cases:
        print(f"[case] static scratch {name}: q_lens {list(b.query_lens)} "
              f"seq_lens {list(b.seq_lens)}", flush=True)
        ref = H.DeviceBatch(b)
        ref.kv_write_attention()
        got = H.DeviceBatch(b)
        assert got.plan.workspace_bytes <= cpa.STATIC_SCRATCH_BYTES
        cpa.cpa_kv_write_attention_static(got.plan, got.q, got.k_new, got.v_new,
                                          got.slot_mapping, got.k_cache, got.v_cache,
                                          got.block_table, got.out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.out.cpu().numpy(), ref.out.cpu().numpy())
        np.testing.assert_array_equal(H.from_dev_u16(got.k_cache), H.from_dev_u16(ref.k_cache))
        np.testing.assert_array_equal(H.from_dev_u16(got.v_cache), H.from_dev_u16(ref.v_cache))
        H.compare(got.out_f64(), H.oracle_out(b, rows=rows), f"static {name}")
        # the same plan again: the array already holds it, no upload
        got.out.fill_(-7777)
        cpa.cpa_kv_write_attention_static(got.plan, got.q, got.k_new, got.v_new,
                                          got.slot_mapping, got.k_cache, got.v_cache,
                                          got.block_table, got.out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.out.cpu().numpy(), ref.out.cpu().numpy())
