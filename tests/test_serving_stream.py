"""The multi-step request stream (inputs.ServingStream) under the oracle's
token-budget batch former, KV write and attention: prefilling each prompt
chunk by chunk over several steps into one paged cache, then decoding a
token per step, gives every token the output that one causal pass over the
request's whole logical sequence gives it (the defining property of chunked
prefill in the vLLM chunked-prefill article, section 3.2.1: a chunk's
queries attend over the cached prefix plus their own causal part). This
pins the stream's pages, slots and block table, and the step bookkeeping,
against a computation that uses no paging at all."""
import math

import numpy as np
import pytest

from chunked_prefill_attention_slot_amd.inputs import SENTINEL_K, SENTINEL_V, ServingStream
from oracle import scheduler as S
from oracle.attention import causal_chunk_attention, paged_attention, widen_bf16
from oracle.kv_cache import kv_write


def drive(stream, sched, budget_check):
    kc, vc = stream.initial_caches()
    per_req = {}                                  # rid -> lists of (q, k, v, out) rows by position
    while not sched.finished():
        batch = sched.form()
        st = stream.step(batch)
        assert st.num_tokens <= budget_check
        kc, vc = kv_write(kc, vc, st.k_new, st.v_new, st.slot_mapping, stream.page_size)
        out = paged_attention(st.q, kc, vc, st.block_table, st.query_lens, st.seq_lens,
                              stream.num_kv_heads, stream.page_size)
        t0 = 0
        for rid, q, n in batch:
            rows = per_req.setdefault(rid, [])
            assert len(rows) == n - q                 # positions arrive in order
            for i in range(q):
                rows.append((st.q[t0 + i], st.k_new[t0 + i], st.v_new[t0 + i], out[t0 + i]))
            t0 += q
        sched.commit()
    return kc, vc, per_req


@pytest.mark.parametrize("kind,budget", [(S.RULE_FIXED, 48), (S.RULE_PROGRESSIVE, 64)])
def test_chunked_steps_equal_one_causal_pass(kind, budget):
    reqs = [(70, 3, 0), (9, 2, 0), (40, 0, 1), (33, 4, 3)]
    hq, hkv, d, P = 4, 2, 16, 8
    stream = ServingStream(11, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=P,
                           requests=reqs, extra_pages=3)
    sched = S.Scheduler(budget, S.Rule(kind, fixed=16, sizes=(32, 16, 8)))
    for p, m, a in reqs:
        sched.add(p, m, a)
    kc, vc, per_req = drive(stream, sched, budget)
    g = hq // hkv
    for rid, (p, m, _) in enumerate(reqs):
        rows = per_req[rid]
        assert len(rows) == p + m
        q = widen_bf16(np.stack([r[0] for r in rows]))
        k = widen_bf16(np.stack([r[1] for r in rows]))
        v = widen_bf16(np.stack([r[2] for r in rows]))
        got = np.stack([r[3] for r in rows])
        for h in range(hq):
            ref = causal_chunk_attention(q[:, h], k[:, h // g], v[:, h // g], 0, 1 / math.sqrt(d))
            np.testing.assert_allclose(got[:, h], ref, rtol=1e-12, atol=1e-12)
    # every slot a request owns below its final length was written; the rest
    # of the pool still holds the sentinels
    written = np.zeros(kc.shape[0] * P, dtype=bool)
    for rid, (p, m, _) in enumerate(reqs):
        pg = stream.pages[rid]
        pos = np.arange(p + m)
        written[pg[pos // P] * P + pos % P] = True
    flat_k = kc.transpose(0, 2, 1, 3).reshape(-1, hkv * d)
    flat_v = vc.transpose(0, 2, 1, 3).reshape(-1, hkv * d)
    assert (flat_k[~written] == SENTINEL_K).all() and (flat_v[~written] == SENTINEL_V).all()
    assert not (flat_k[written] == SENTINEL_K).all(axis=1).any()


def test_stream_layout():
    st = ServingStream(3, num_q_heads=2, num_kv_heads=1, head_dim=8, page_size=4,
                       requests=[(10, 2, 0), (3, 0, 0)], extra_pages=1)
    assert st.num_blocks == 3 + 1 + 1 and st.max_blocks_per_seq == 3
    allp = np.concatenate(st.pages).tolist()
    assert len(set(allp)) == len(allp) == 4                  # disjoint pages from the pool
    x = st.step([(0, 1, 12), (1, 3, 3)])
    pg0, pg1 = st.pages
    assert x.slot_mapping.tolist() == [pg0[2] * 4 + 3, pg1[0] * 4, pg1[0] * 4 + 1, pg1[0] * 4 + 2]
    assert x.block_table.tolist() == [list(pg0), [pg1[0], -1, -1]]
    assert x.q.shape == (4, 2, 8) and x.k_new.shape == (4, 1, 8)
    with pytest.raises(ValueError):
        st.step([(1, 1, 5)])                   # request 1 owns one page of 4 slots
    empty = st.step([])
    assert empty.num_tokens == 0 and empty.block_table.shape == (0, 3)
