"""GPU: the fused KV write + attention call (cpa_kv_write_attention) against
the two separate calls, bit for bit (output and both caches), and against
the fp64 oracle. Every test prints its case before touching the GPU."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# Cache rows one fused prefill thread writes at most, and its threads per
# work item (the library's own constants, restated to predict its choice).
WRITES_PER_THREAD = 4
THREADS_PER_ITEM = 512

CASES = {
    # the bench's step: one Llama-3-8B chunk at each H of the sweep (fused)
    "llama3_8b_H0": dict(llama3_hist=0),
    "llama3_8b_H4096": dict(llama3_hist=4096, rows={0: [0, 1, 63, 64, 255, 256, 400, 511]}),
    "llama3_8b_H8192": dict(llama3_hist=8192, rows={0: [0, 64, 300, 511]}),
    "llama3_8b_H12288": dict(llama3_hist=12288, rows={0: [0, 1, 255, 511]}),
    # split tiles with fp32 output (fp32 partials)
    "llama3_8b_H4096_f32": dict(llama3_hist=4096, out_dtype=1, rows={0: [0, 2, 200, 511]}),
    # GQA 8/2, 16-token pages; prefixes 230 and 195 are not multiples of a
    # wave's 8 rows, so waves straddle the first new key; a decode row and a
    # fresh sequence beside them
    "ragged_p16": dict(seed=21, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                       query_lens=[70, 1, 33, 5], seq_lens=[300, 90, 33, 200], extra_pages=4),
    "ragged_p16_f32": dict(seed=22, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                           query_lens=[70, 1, 33, 5], seq_lens=[300, 90, 33, 200],
                           extra_pages=4, out_dtype=1),
    # d = 64, MHA, a long chunk over a short prefix
    "d64": dict(seed=23, num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=16,
                query_lens=[64, 100], seq_lens=[256, 100], extra_pages=2),
    # the largest page (1024 keys) with GQA 32/8 and a prefix inside a page
    "p1024": dict(seed=26, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=1024,
                  query_lens=[300], seq_lens=[2500], extra_pages=1,
                  rows={0: [0, 1, 100, 255, 256, 299]}),
    # d = 64 with GQA 8/2, 32-token pages, prefixes 1 and 61
    "d64_gqa": dict(seed=27, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32,
                    query_lens=[90, 3], seq_lens=[91, 64], extra_pages=2),
    # decode rows only: no prefill items, the write kernel runs first
    "decode_only": dict(seed=24, num_q_heads=8, num_kv_heads=8, head_dim=128, page_size=128,
                        query_lens=[1, 1, 1], seq_lens=[500, 33, 1000]),
    # MHA with 40 heads, tiles left unsplit: more new rows than the 80
    # prefill items' threads take, the write kernel runs first
    "mha40_unfused": dict(seed=25, num_q_heads=40, num_kv_heads=40, head_dim=128,
                          page_size=128, query_lens=[512], seq_lens=[600],
                          rows={0: [0, 5, 88, 300, 511]}, options={"prefill_split": 1}),
    # GQA 16 at d = 128: decode rows the decode kernel does not take and a
    # 6-token chunk, every item at most 96 rows, so the launch takes the
    # instance whose waves without rows skip their work
    "gqa16_small_items": dict(seed=28, num_q_heads=64, num_kv_heads=4, head_dim=128,
                              page_size=64, query_lens=[1, 1, 6], seq_lens=[700, 4100, 300],
                              extra_pages=2),
    # the same batch with the planner's own splits: enough items to take
    # the writes in the prefill kernel
    "mha40_split": dict(seed=25, num_q_heads=40, num_kv_heads=40, head_dim=128,
                        page_size=128, query_lens=[512], seq_lens=[600],
                        rows={0: [0, 5, 88, 300, 511]}),
}


def build(case):
    from chunked_prefill_attention_slot_amd.inputs import llama3_8b_chunk, make_batch
    c = dict(case)
    c.pop("rows", None)
    c.pop("out_dtype", None)
    c.pop("options", None)
    if "llama3_hist" in c:
        return llama3_8b_chunk(c["llama3_hist"])
    seed = c.pop("seed")
    return make_batch(seed, **c)


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_separate(name):
    from tests import gpu_helpers as H
    case = CASES[name]
    b = build(case)
    od = case.get("out_dtype", 0)
    print(f"[case] fused {name}: q_lens {list(b.query_lens)} seq_lens {list(b.seq_lens)}",
          flush=True)
    opts = case.get("options")
    sep = H.DeviceBatch(b, out_dtype=od, options=opts)
    sep.run()
    fus = H.DeviceBatch(b, out_dtype=od, options=opts)
    fus.kv_write_attention()
    torch.cuda.synchronize()
    info = fus.plan.info()
    chunks = b.num_tokens * b.num_kv_heads * (b.head_dim // 8)
    fused = info["num_prefill_items"] > 0 and \
        chunks <= info["num_prefill_items"] * THREADS_PER_ITEM * WRITES_PER_THREAD
    print(f"[fused] {name}: prefill items {info['num_prefill_items']}, "
          f"{'fused' if fused else 'write kernel first'}", flush=True)
    if name in ("decode_only", "mha40_unfused"):
        assert not fused
    else:
        assert fused
    np.testing.assert_array_equal(fus.out.cpu().numpy(), sep.out.cpu().numpy())
    np.testing.assert_array_equal(H.from_dev_u16(fus.k_cache), H.from_dev_u16(sep.k_cache))
    np.testing.assert_array_equal(H.from_dev_u16(fus.v_cache), H.from_dev_u16(sep.v_cache))
    ref = H.oracle_out(b, rows=case.get("rows"))
    H.compare(fus.out_f64(), ref, f"fused {name}")


def test_fused_repeated_calls():
    """Two batches of the same shape through one DeviceBatch in turn: the
    second call's output and cache come from its own inputs only."""
    from tests import gpu_helpers as H
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
              query_lens=[70, 33], seq_lens=[300, 33], extra_pages=2)
    b1, b2 = make_batch(31, **kw), make_batch(32, **kw)
    print("[case] fused repeated calls", flush=True)
    db = H.DeviceBatch(b1)
    db.kv_write_attention()
    torch.cuda.synchronize()
    H.compare(db.out_f64(), H.oracle_out(b1), "fused call 1")
    for name in ("q", "k_new", "v_new", "k_cache", "v_cache"):
        getattr(db, name).copy_(H.to_dev_u16(getattr(b2, name)))
    for name in ("slot_mapping", "block_table"):   # other pages, same lengths
        getattr(db, name).copy_(H.to_dev_i32(getattr(b2, name)))
    db.kv_write_attention()
    torch.cuda.synchronize()
    H.compare(db.out_f64(), H.oracle_out(b2), "fused call 2")
