"""GPU: a prompt prefilled in predictor-chosen chunks, each chunk one fused
KV write + attention call at its own prefix, gives the same output as one
causal pass over the whole prompt (the oracle's definition), and the same
caches bit for bit; the chunk sizes are the oracle's schedule for the same
coefficients (dynamic chunked pipeline parallel design, runtime phase:
solve f(L+x) - f(L) = T, then align and cap)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("shape,prompt,align", [
    (dict(num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=16), 2500, 16),
    (dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128), 1800, 128),
])
def test_predictor_walk_equals_one_shot(shape, prompt, align):
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    from oracle import predictor as opred
    from oracle.kv_cache import kv_write
    from tests import gpu_helpers as H

    a, b = 1e-6, 1e-3                     # fixed coefficients (ms per token^2, per token)
    base = 512
    cfg = cpa.predictor_cfg(base_chunk_size=base, align=align, min_chunk=64, max_chunk=base)
    T = cpa.cpa_predictor_target(cfg, a, b)
    chunks, L = [], 0
    while L < prompt:
        ch, _ = cpa.cpa_predictor_next_chunk(cfg, a, b, T, L, prompt - L)
        assert ch > 0
        chunks.append((L, ch))
        L += ch
    ocfg = opred.PredictorConfig(base_chunk_size=base, align=align, min_chunk=64, max_chunk=base)
    want = [(l, c) for l, c, _ in opred.schedule(ocfg, a, b, opred.target(a, b, base), prompt)]
    assert chunks == want
    assert len(chunks) >= 3 and len({c for _, c in chunks}) >= 2

    b_ = make_batch(12, query_lens=[prompt], seq_lens=[prompt], **shape)
    print(f"[case] predictor walk {shape} prompt {prompt}: chunks {[c for _, c in chunks]}",
          flush=True)
    db = H.DeviceBatch(b_)
    keep = []
    for L, c in chunks:
        plan = cpa.cpa_plan_create(db.desc, [c], [L + c])
        ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
        cpa.cpa_plan_upload(plan, ws)
        sl = slice(L, L + c)
        cpa.cpa_kv_write_attention(plan, db.q[sl], db.k_new[sl], db.v_new[sl],
                                   db.slot_mapping[sl], db.k_cache, db.v_cache, db.block_table,
                                   db.out[sl], ws)
        keep.append((plan, ws))
    torch.cuda.synchronize()
    kc, vc = kv_write(b_.k_cache, b_.v_cache, b_.k_new, b_.v_new, b_.slot_mapping, b_.page_size)
    np.testing.assert_array_equal(H.from_dev_u16(db.k_cache), kc)
    np.testing.assert_array_equal(H.from_dev_u16(db.v_cache), vc)
    # every row of the first and last chunk, and rows around each boundary
    rows = set(range(chunks[0][1])) | set(range(chunks[-1][0], prompt))
    for L, _ in chunks[1:]:
        rows |= {L - 1, L, L + 1}
    ref = H.oracle_out(b_, rows={0: sorted(rows)})
    H.compare(db.out_f64(), ref, f"predictor walk {shape['head_dim']} {prompt}")
