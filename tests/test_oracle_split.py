"""Pins of oracle/split.py (the two-micro-batch split of the Ascend
dual-stream article, section 3.1): worked cases computed by hand from the
section's rules, an exhaustive search over all boundaries, the threshold
edges, and the invariant that attention over the two micro-batches equals
attention over the whole batch (the oracle's attention is per sequence)."""
import numpy as np

from oracle import split as sp
from oracle.attention import paged_attention


def test_simple_split_by_hand():
    # 16 decode rows then two 512-token chunks: batch_size // 2 = 9
    ql = [1] * 16 + [512, 512]
    assert sp.simple_split(ql) == (9, 9)
    assert sp.simple_split([7, 5]) == (1, 7)
    assert sp.simple_split([5]) is None
    assert sp.simple_split([]) is None


def test_balanced_split_by_hand():
    ql = [1] * 16 + [512, 512]          # total 1040, aim 520
    # boundary after the 17th sequence holds 528 tokens: |528-520| = 8
    assert sp.balanced_split(ql, 0.5, 1) == (17, 528)
    # the simple split (9 vs 1031 tokens) is what the balanced method avoids
    assert sp.balanced_split([1] * 16 + [512, 512], 0.01, 1) is None     # 528 vs 512: 3.1% > 1%
    assert sp.balanced_split([1] * 16 + [512, 512], 0.05, 513) is None   # 512 < 513
    assert sp.balanced_split([1] * 16 + [512, 512], 0.05, 512) == (17, 528)
    # tie between two boundaries: the smaller one
    assert sp.balanced_split([2, 2, 2, 2], 1.0, 1) == (2, 4)
    assert sp.balanced_split([3, 2, 3], 1.0, 1) == (1, 3)   # aim 4: |3-4| = |5-4|, take k=1


def test_balanced_split_matches_exhaustive_search():
    rng = np.random.default_rng(0)
    for _ in range(300):
        S = int(rng.integers(2, 12))
        ql = [int(v) for v in rng.integers(0, 600, S)]
        total = sum(ql)
        cands = [(abs(sum(ql[:k]) - total // 2), k) for k in range(1, S)]
        k = min(cands)[1]
        tsp = sum(ql[:k])
        n1, n2 = tsp, total - tsp
        ok = min(n1, n2) > 0 and abs(n1 - n2) / min(n1, n2) <= 0.3 and min(n1, n2) >= 16
        assert sp.balanced_split(ql, 0.3, 16) == ((k, tsp) if ok else None)


def test_split_metadata_concatenates_back():
    rng = np.random.default_rng(1)
    meta = {"query_lens": np.array([1, 1, 300, 4]), "seq_lens": np.array([50, 90, 700, 4]),
            "block_table": rng.integers(0, 99, (4, 6)), "slot_mapping": rng.integers(0, 999, 306),
            "q": rng.normal(size=(306, 2, 8)), "page_size": 16}
    pre, post = sp.split_metadata(meta, 2, 2)
    for key in ("query_lens", "seq_lens", "block_table", "slot_mapping", "q"):
        assert np.array_equal(np.concatenate([pre[key], post[key]]), meta[key])
    assert (pre["num_tokens"], post["num_tokens"]) == (2, 304)
    assert pre["page_size"] == post["page_size"] == 16


def test_attention_over_micro_batches_equals_whole():
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    ql, sl = [1, 1, 40, 1, 23], [30, 17, 70, 9, 23]
    b = make_batch(7, num_q_heads=4, num_kv_heads=2, head_dim=16, page_size=16,
                   query_lens=ql, seq_lens=sl)
    whole = paged_attention(b.q, b.k_cache, b.v_cache, b.block_table, ql, sl, 2, 16)
    for k, tsp in [sp.balanced_split(ql, 10.0, 1), sp.simple_split(ql)]:
        meta = {"q": b.q, "query_lens": np.array(ql), "seq_lens": np.array(sl),
                "block_table": b.block_table}
        pre, post = sp.split_metadata(meta, k, tsp)
        o1 = paged_attention(pre["q"], b.k_cache, b.v_cache, pre["block_table"],
                             pre["query_lens"], pre["seq_lens"], 2, 16)
        o2 = paged_attention(post["q"], b.k_cache, b.v_cache, post["block_table"],
                             post["query_lens"], post["seq_lens"], 2, 16)
        assert np.array_equal(np.concatenate([o1, o2]), whole)
