"""GPU parity: libcpa's HIP path against the fp64 oracle, element by element,
through the C ABI. Every test prints its case before touching the GPU."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def H():
    from tests import gpu_helpers
    return gpu_helpers


def banner(msg):
    print(f"[case] {msg}", flush=True)


def make(**kw):
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    return make_batch(**kw)


# ---- KV write ------------------------------------------------------------

@pytest.mark.parametrize("case", [
    dict(seed=1, num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=16,
         query_lens=[64], seq_lens=[256]),
    dict(seed=2, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128,
         query_lens=[512], seq_lens=[4608], extra_pages=8),
    dict(seed=3, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
         query_lens=[1, 7, 0, 33], seq_lens=[50, 7, 3, 100], extra_pages=3),
])
def test_kv_write_bit_exact(H, case):
    from oracle.kv_cache import kv_write
    b = make(**case)
    sm = b.slot_mapping.copy()
    ref_sm = sm.copy()
    if b.num_tokens > 3:
        sm[2] = ref_sm[2] = -1           # a padding token: skipped
        sm[1] = b.num_blocks * b.page_size + 5   # outside the cache: not written
        ref_sm[1] = -1
        b.slot_mapping = sm
    banner(f"kv_write {case}")
    db = H.DeviceBatch(b)
    db.kv_write()
    torch.cuda.synchronize()
    kc, vc = kv_write(b.k_cache, b.v_cache, b.k_new, b.v_new, ref_sm, b.page_size)
    np.testing.assert_array_equal(H.from_dev_u16(db.k_cache), kc)
    np.testing.assert_array_equal(H.from_dev_u16(db.v_cache), vc)


# ---- attention, full comparison at sizes the oracle finishes quickly ------

def run_and_compare(H, b, label, out_dtype=0, options=None, rows=None):
    banner(label)
    db = H.DeviceBatch(b, out_dtype=out_dtype, options=options)
    db.run()
    ref = H.oracle_out(b, rows=rows)
    H.compare(db.out_f64(), ref, label)
    return db


@pytest.mark.parametrize("out_dtype", [0, 1])
def test_small_single_sequence(H, out_dtype):
    """4/4 heads, d=64, H=192 cached in 16-token pages (permuted), C=64."""
    from chunked_prefill_attention_slot_amd.inputs import small_parity
    run_and_compare(H, small_parity(), f"small d64 H192 C64 out={out_dtype}", out_dtype)


SHAPES = [
    # hq, hkv, d, P, query_lens, seq_lens
    (8, 8, 128, 16, [200], [200]),                    # H=0, two row tiles, ragged
    (32, 8, 128, 128, [300], [1300]),                 # GQA 4, page 128
    (64, 8, 128, 128, [130], [2178]),                 # GQA 8
    (16, 1, 64, 32, [45], [333]),                     # MQA 16, d=64
    (4, 2, 64, 16, [1, 1, 77, 1, 5], [90, 1, 200, 513, 5]),   # decode + prefill mix
    (40, 40, 128, 128, [1] * 4 + [129], [700, 129, 2000, 4100, 1000]),
    (12, 4, 128, 64, [3, 0, 2], [3, 9, 300]),         # tiny chunks, empty row
    (32, 2, 128, 16, [1, 1], [100, 1000]),            # decode GQA 16 -> MFMA kernel
    (48, 8, 128, 32, [1, 70, 1], [64, 300, 2000]),    # GQA 6: two heads per tile
    (128, 1, 64, 16, [1, 3, 40], [500, 3, 900]),      # GQA 128: two queries per tile
    (256, 1, 64, 16, [2, 1], [40, 700]),              # GQA 256: one query per tile
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(i) for i in range(len(SHAPES))])
def test_random_shapes(H, shape):
    hq, hkv, d, P, ql, sl = shape
    b = make(seed=sum(sl) % 1000, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
             page_size=P, query_lens=ql, seq_lens=sl, extra_pages=2)
    run_and_compare(H, b, f"shape {shape}")


def _sweep_cases(n=24, seed=2024):
    """Seeded random batches: GQA ratio, head size, page size, a mix of
    decode rows, prefill chunks and empty rows over random prefixes, and a
    random plan option (forced prefill splits, decode split size, split
    floor, a small item target) and output precision."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 16, 32]))
        while hkv * g > 64:
            hkv //= 2
        d = int(rng.choice([64, 128]))
        P = int(rng.choice([16, 32, 64, 128, 256]))
        ql, sl = [], []
        for _ in range(int(rng.integers(1, 6))):
            kind = rng.choice(["decode", "prefill", "prefill", "empty"])
            q = {"decode": 1, "empty": 0}.get(kind) or int(rng.integers(2, 300))
            h = int(rng.integers(0, 1500)) if rng.random() < 0.8 else 0
            ql.append(q)
            sl.append(max(q + h, 1))
        opt = [None, {"prefill_split": int(rng.integers(2, 9))},
               {"decode_split_keys": 64 * int(rng.integers(1, 9))},
               {"min_split_keys": 64 * int(rng.integers(1, 5))},
               {"target_items": int(rng.integers(8, 64))}][int(rng.integers(0, 5))]
        cases.append((i, hkv * g, hkv, d, P, ql, sl, opt, int(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: str(c[0]))
def test_seeded_sweep(H, case):
    i, hq, hkv, d, P, ql, sl, opt, out_dtype = case
    if sum(ql) == 0:
        ql[0], sl[0] = 1, max(sl[0], 1)
    b = make(seed=100 + i, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=P,
             query_lens=ql, seq_lens=sl, extra_pages=2)
    run_and_compare(H, b, f"sweep {case}", out_dtype=out_dtype, options=opt)


@pytest.mark.parametrize("shift", [(0.0, 0.0), (2.5, 2.5), (2.5, -2.5)])
def test_large_scores(H, shift):
    """Q and K moved by offsets (a, b): every score gains ~d*a*b*scale
    (about +-100 in log2 units at 2.5), which leaves the softmax nearly flat
    but puts all scores far outside [-64, 64], so rows take a nonzero
    reference at their first visible key; split and unsplit items alike."""
    from chunked_prefill_attention_slot_amd.inputs import f32_to_bf16_bits
    b = make(seed=12, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128,
             query_lens=[300, 70], seq_lens=[3000, 70], extra_pages=1)

    def moved(bits, c):
        x = (bits.astype(np.uint32) << 16).view(np.float32)
        return f32_to_bf16_bits(x / 4 + c)

    b.q = moved(b.q, shift[0])
    b.k_new, b.k_cache = moved(b.k_new, shift[1]), moved(b.k_cache, shift[1])
    label = f"large scores shift {shift}"
    banner(label)
    ref = H.oracle_out(b)
    for opts in (None, {"prefill_split": 1}):
        db = H.DeviceBatch(b, out_dtype=1, options=opts)
        db.run()
        H.compare(db.out_f64(), ref, f"{label} {opts}")


def test_all_rows_empty(H):
    """A batch whose every chunk is empty: each entry point succeeds without
    touching the caches or launching work."""
    b = make(seed=15, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
             query_lens=[0, 0], seq_lens=[5, 300], extra_pages=1)
    banner("all rows empty")
    db = H.DeviceBatch(b)
    assert db.plan.info()["num_tokens"] == 0
    db.run()
    db.kv_write_attention()
    torch.cuda.synchronize()
    assert db.out.numel() == 0
    np.testing.assert_array_equal(H.from_dev_u16(db.k_cache), b.k_cache)
    np.testing.assert_array_equal(H.from_dev_u16(db.v_cache), b.v_cache)


@pytest.mark.parametrize("shape", [
    # hq, hkv, d, P, query_lens, seq_lens (prefixes end inside pages; decode
    # rows of the decode kernel and of the MFMA kernel; an empty row)
    (32, 8, 128, 128, [300, 1, 1, 0], [1000, 77, 3000, 5]),
    (16, 1, 64, 16, [45, 1], [333, 100]),
    (8, 8, 64, 64, [1, 130], [65, 130]),
])
def test_nan_in_unused_slots(H, shape):
    """Every cache slot that no sequence position maps to holds a NaN bit
    pattern: keys past a range and the tail of a page must never reach a
    product (0 * NaN would poison the row)."""
    hq, hkv, d, P, ql, sl = shape
    b = make(seed=41, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=P,
             query_lens=ql, seq_lens=sl, extra_pages=3)
    used = np.zeros(b.num_blocks * P, dtype=bool)
    for s_, n in enumerate(sl):
        pos = np.arange(n)
        used[b.block_table[s_, pos // P].astype(np.int64) * P + pos % P] = True
    nan_bits = np.uint16(0x7FC0)
    for cache in (b.k_cache, b.v_cache):
        flat = cache.transpose(0, 2, 1, 3).reshape(b.num_blocks * P, hkv, d)
        flat[~used] = nan_bits
        cache[...] = flat.reshape(b.num_blocks, P, hkv, d).transpose(0, 2, 1, 3)
    assert np.isnan((b.k_cache.astype(np.uint32) << 16).view(np.float32)).any()
    for opts in (None, {"prefill_split": 1}):
        db = run_and_compare(H, b, f"NaN in unused slots {shape} {opts}", options=opts)
        assert np.isfinite(db.out_f64()).all()


@pytest.mark.parametrize("shape", [
    (32, 8, 128, 128, [300, 1], [1800, 700]),     # prefill chunk, decode row (decode kernel)
    (16, 1, 64, 16, [40, 1], [400, 300]),         # MQA: decode row through the MFMA kernel
])
def test_pages_outside_the_cache_read_as_zero(H, shape):
    """Block-table entries of cached (prefix) pages set outside [0,
    num_blocks): the kernels' bounds checks read those keys as zero K and V
    rows (score 0, still in the softmax) instead of touching memory. The
    oracle sees the same batch with those entries pointing at an all-zero
    page; fused and separate calls alike."""
    from tests.gpu_helpers import DeviceBatch
    hq, hkv, d, P, ql, sl = shape
    b = make(seed=43, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=P,
             query_lens=ql, seq_lens=sl, extra_pages=2)
    bad = [b.num_blocks + 3, -2, 1 << 30]
    ref_bt = b.block_table.copy()
    k = 0
    for s_, (q, n) in enumerate(zip(ql, sl)):
        for pg in range(0, (n - q) // P, 3):          # whole pages of the prefix only
            b.block_table[s_, pg] = bad[k % 3]
            ref_bt[s_, pg] = b.num_blocks              # the appended zero page
            k += 1
    assert k > 0
    import copy
    r = copy.copy(b)
    zero = np.zeros((1,) + b.k_cache.shape[1:], dtype=b.k_cache.dtype)
    r.k_cache = np.concatenate([b.k_cache, zero])
    r.v_cache = np.concatenate([b.v_cache, zero])
    r.block_table = ref_bt
    ref = H.oracle_out(r)
    banner(f"pages outside the cache {shape}")
    db = DeviceBatch(b)
    db.run()
    H.compare(db.out_f64(), ref, f"pages outside the cache {shape} separate")
    db2 = DeviceBatch(b)
    db2.kv_write_attention()
    torch.cuda.synchronize()
    H.compare(db2.out_f64(), ref, f"pages outside the cache {shape} fused")


def test_page_cap_split(H):
    """Maximum item size: one sequence of 40000 keys in 16-key pages (2500
    block-table entries, over the 2047 one item stages), splitting turned
    off, so only the cap splits the tile; every row compared."""
    b = make(seed=14, num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=16,
             query_lens=[64], seq_lens=[40000], extra_pages=3)
    db = run_and_compare(H, b, "page cap split H=39936 C=64 P=16",
                         options={"prefill_split": 1})
    assert db.plan.info()["num_prefill_items"] == 2


def test_forced_splits_agree(H):
    b = make(seed=7, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128,
             query_lens=[256], seq_lens=[3000], extra_pages=1)
    outs = []
    for split in (1, 3, 4, 5, 7, 9, 17):
        db = run_and_compare(H, b, f"split {split}", options={"prefill_split": split})
        outs.append(db.out_f64())
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 1e-2


@pytest.mark.parametrize("out_dtype", [0, 1])
def test_many_splits_per_tile(H, out_dtype):
    """Tiles split more than 8 ways take the combine whose threads (2, 4 or
    8 per row) share the splits of a row: a 64-token chunk over an 8000-key
    prefix at the 4-head d = 64 shape (63 splits per row tile), decode rows
    cut into 64-key splits
    (up to 141, several batches per thread), and one plan with both kinds
    (a 70-way prefill tile beside decode rows of 1-3 splits: two combine
    launches, one per kind), and 12- and 24-way splits. Every row against
    the oracle, bf16 and fp32."""
    b = make(seed=21, num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=16,
             query_lens=[64], seq_lens=[8064])
    db = run_and_compare(H, b, f"63-way split d64 out={out_dtype}", out_dtype)
    info = db.plan.info()
    assert info["num_combine_items"] == 4 and info["num_prefill_items"] >= 4 * 60
    b = make(seed=22, num_q_heads=8, num_kv_heads=8, head_dim=128, page_size=128,
             query_lens=[1, 1, 1], seq_lens=[9000, 700, 4100])
    run_and_compare(H, b, f"decode split 64 (141 splits) out={out_dtype}", out_dtype,
                    options={"decode_split_keys": 64})
    b = make(seed=23, num_q_heads=8, num_kv_heads=8, head_dim=128, page_size=128,
             query_lens=[1, 1, 40], seq_lens=[1300, 129, 5000])
    run_and_compare(H, b, f"mixed: 70-way prefill tile + decode rows out={out_dtype}", out_dtype,
                    options={"prefill_split": 70})
    b = make(seed=24, num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=16,
             query_lens=[100], seq_lens=[3000])
    for split in (12, 24):          # 2 and 4 threads per row in the combine
        run_and_compare(H, b, f"{split}-way split d64 out={out_dtype}", out_dtype,
                        options={"prefill_split": split})


def test_decode_split_sizes_agree(H):
    b = make(seed=8, num_q_heads=8, num_kv_heads=8, head_dim=128, page_size=128,
             query_lens=[1, 1, 1], seq_lens=[5000, 129, 2048])
    for dsk in (128, 512, 8192):
        run_and_compare(H, b, f"decode split {dsk}", options={"decode_split_keys": dsk})


def test_page_permutation_is_bitwise(H):
    b = make(seed=9, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
             query_lens=[70, 1], seq_lens=[300, 90], extra_pages=5)
    banner("page permutation")
    db = H.DeviceBatch(b)
    db.run()
    first = db.out.clone()
    perm = np.random.default_rng(0).permutation(b.num_blocks)
    b.k_cache = np.empty_like(b.k_cache); b.k_cache[perm] = H.from_dev_u16(db.k_cache)
    b.v_cache = np.empty_like(b.v_cache); b.v_cache[perm] = H.from_dev_u16(db.v_cache)
    b.block_table = np.where(b.block_table >= 0, perm[np.maximum(b.block_table, 0)], -1)
    b.slot_mapping[:] = -1          # caches already hold every token
    db2 = H.DeviceBatch(b)
    db2.run()
    assert torch.equal(first, db2.out)


def test_constant_v_returns_v(H):
    b = make(seed=10, num_q_heads=8, num_kv_heads=4, head_dim=64, page_size=16,
             query_lens=[100, 1], seq_lens=[150, 300], extra_pages=1)
    one = np.uint16(0x3F80)
    b.v_cache[...] = one
    b.v_new[...] = one
    banner("constant V")
    db = H.DeviceBatch(b, out_dtype=1)
    db.run()
    # The prefill kernel divides the bf16-rounded weights that multiply V by
    # the sum of the unrounded fp32 weights, so a constant V comes back
    # scaled by a ratio within 1 +- 2^-8 (the unit roundoff of bf16 bounds
    # each weight's relative rounding error); the decode kernel is exact to
    # fp32 rounding.
    err = np.abs(db.out_f64() - 1.0)
    assert err.max() <= 2.0 ** -8 + 1e-5
    assert err[100:].max() <= 1e-5      # the decode row


def test_bound_calls_match(H):
    """binding.bind_kv_write / bind_attention (arguments marshalled once)
    launch the same work as the per-call entry points: bitwise equal."""
    b = make(seed=13, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
             query_lens=[40, 1], seq_lens=[300, 90], extra_pages=1)
    banner("bound calls")
    db = H.DeviceBatch(b)
    db.run()
    first = db.out.clone()
    db.out.fill_(0)
    kv_write, attention = db.bound()
    for _ in range(2):
        kv_write()
        attention()
    torch.cuda.synchronize()
    assert torch.equal(first, db.out)


def test_attention_requires_upload(H):
    from chunked_prefill_attention_slot_amd import binding as cpa
    b = make(seed=11, num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=16,
             query_lens=[8], seq_lens=[8])
    banner("attention without upload")
    db = H.DeviceBatch(b)
    other = cpa.cpa_plan_create(db.desc, [4], [8])
    cpa.cpa_plan_upload(other, db.workspace)      # replaces db.plan in the workspace
    with pytest.raises(cpa.CpaError) as e:
        db.attention()
    assert e.value.status == cpa.CPA_ERR_WORKSPACE


# ---- full-size workloads, checked on sampled rows ---------------------------

def sample_rows(ql, k, seed):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, ql - 1, ql // 2, min(ql - 1, 31), min(ql - 1, 32)}
    return sorted(fixed | set(int(x) for x in rng.integers(0, ql, k)))


@pytest.mark.parametrize("hist", [0, 4096, 8192, 12288])
def test_llama3_8b_chunk512(H, hist):
    """32 q / 8 kv heads, d=128, page 128, C=512 at prefix H (launch
    configuration of the bench)."""
    from chunked_prefill_attention_slot_amd.inputs import llama3_8b_chunk
    b = llama3_8b_chunk(hist)
    run_and_compare(H, b, f"llama3-8b C512 H{hist}", rows={0: sample_rows(512, 24, hist)})


def test_llama13b_mixed_batch(H):
    """16 decode rows (seq_len U[1024, 8192]) + 2 prefill chunks of 512 at
    H=2048 and 6144; 40/40 heads, d=128, page 128."""
    from chunked_prefill_attention_slot_amd.inputs import mixed_llama13b
    b = mixed_llama13b()
    rows = {s: [0] for s in range(16)}
    rows[16] = sample_rows(512, 12, 1)
    rows[17] = sample_rows(512, 12, 2)
    run_and_compare(H, b, "llama13b mixed", rows=rows)


def _run_micro_batches(H, b, label, mode, rows=None):
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.device import MicroBatchPair
    split = cpa.cpa_split_point(b.query_lens, mode, 0.5, 1)
    assert split is not None
    banner(f"{label}: micro-batches at {split}")
    whole = H.DeviceBatch(b)
    whole.run()
    db = H.DeviceBatch(b)
    db.kv_write()
    pair = MicroBatchPair(db, *split)
    pair.attention()
    torch.cuda.synchronize()
    got = db.out_f64()
    ref = H.oracle_out(b, rows=rows)
    H.compare(got, ref, label)
    # and the two halves agree with the one-call output on every row
    H.compare(got, whole.out_f64(), label + " vs one call")
    return split


def test_micro_batch_split_small(H):
    """Decode rows then prefill chunks (the chunked-prefill article's token
    budget order), split in two by the balanced rule of the dual-stream
    article and run on two streams."""
    from chunked_prefill_attention_slot_amd import binding as cpa
    b = make(seed=31, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
             query_lens=[1, 1, 1, 1, 90, 70], seq_lens=[300, 17, 129, 64, 200, 70], extra_pages=4)
    split = _run_micro_batches(H, b, "micro-batches balanced", cpa.CPA_SPLIT_BALANCED)
    assert split == (5, 94)
    _run_micro_batches(H, b, "micro-batches simple", cpa.CPA_SPLIT_SIMPLE)


def test_micro_batch_split_llama13b(H):
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.inputs import mixed_llama13b
    b = mixed_llama13b()
    rows = {s: [0] for s in range(16)}
    rows[16] = sample_rows(512, 8, 3)
    rows[17] = sample_rows(512, 8, 4)
    split = _run_micro_batches(H, b, "llama13b micro-batches", cpa.CPA_SPLIT_BALANCED, rows=rows)
    assert split == (17, 528)


@pytest.mark.parametrize("hist", [0, 30720])
def test_long_context_chunk2048(H, hist):
    """64 q / 8 kv heads, d=128, C=2048 at prefix H (max_model_len 32768)."""
    from chunked_prefill_attention_slot_amd.inputs import long_context_chunk
    b = long_context_chunk(hist)
    run_and_compare(H, b, f"70b-like C2048 H{hist}", rows={0: sample_rows(2048, 12, hist)})


@pytest.mark.parametrize("shape", [
    dict(num_q_heads=8, num_kv_heads=8, head_dim=128, page_size=16),     # decode kernel, G = 1
    dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128),   # decode kernel, G = 4
    dict(num_q_heads=32, num_kv_heads=2, head_dim=64, page_size=32),     # G = 16: MFMA kernel
])
def test_decode_row_equals_last_prefill_row(H, shape):
    """The last row of a prefill chunk and a decode row (query_len 1) over
    the same sequence see the same keys with the same query: the two paths
    (for G <= 8 two different kernels) agree within the tolerance, and each
    matches the oracle."""
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    n, C = 3000, 200
    b = make_batch(61, query_lens=[C], seq_lens=[n], extra_pages=2, **shape)
    print(f"[case] decode row vs last prefill row {shape}", flush=True)
    db = H.DeviceBatch(b)
    db.run()                                  # KV write then prefill attention
    plan = cpa.cpa_plan_create(db.desc, [1], [n])
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    cpa.cpa_plan_upload(plan, ws)
    q1 = db.q[C - 1:C].contiguous()
    out1 = torch.full_like(db.out[:1], -7777)
    cpa.cpa_attention(plan, q1, db.k_cache, db.v_cache, db.block_table, out1, ws)
    torch.cuda.synchronize()
    widen = lambda t: (t.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    pre, dec = widen(db.out[C - 1]), widen(out1[0])
    err = np.abs(pre.astype(np.float64) - dec)
    print(f"[parity] decode row vs prefill row: max_abs={err.max():.3e}", flush=True)
    assert err.max() <= H.MAX_ABS
    ref = H.oracle_out(b, rows={0: [C - 1]})
    H.compare(db.out_f64(), ref, "prefill last row")
    got = np.full_like(ref, np.nan)
    got[C - 1] = dec
    H.compare(got, ref, "decode row")
