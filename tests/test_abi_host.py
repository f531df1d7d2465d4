"""Host-side tests of libcpa (no GPU): the library loads and exports every
symbol include/cpa.h declares; the C++ predictor returns the oracle's chunk
sizes bit for bit; the planner and validator accept and reject what cpa.h
says they do."""
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="session")
def cpa():
    from chunked_prefill_attention_slot_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    from chunked_prefill_attention_slot_amd import binding
    return binding


def header_functions():
    text = open(os.path.join(ROOT, "include", "cpa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cpa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(cpa):
    declared = header_functions()
    assert len(declared) >= 13
    assert set(declared) == set(cpa.EXPORTS)
    for name in declared:
        assert hasattr(cpa._lib, name), name
    assert "gfx950" in cpa.cpa_version()


# ---- predictor: C++ vs oracle ------------------------------------------

def test_profile_sizes_match_oracle(cpa):
    from oracle.predictor import profile_sizes
    for base, n, lo in [(2048, 64, 32), (4096, 64, 1), (1000, 7, 3), (513, 64, 17)]:
        assert cpa.cpa_predictor_profile_sizes(base, n, lo) == profile_sizes(base, n, lo)


def test_profile_sizes_distinct_or_refused(cpa):
    """n sizes from base down to lo are distinct exactly when base - lo >=
    n - 1; fewer tokens than that are refused rather than repeated."""
    s = cpa.cpa_predictor_profile_sizes(100, 65, 36)      # spacing exactly 1
    assert s == list(range(100, 35, -1))
    s = cpa.cpa_predictor_profile_sizes(101, 41, 20)      # spacing 2.025
    assert len(set(s)) == 41 and s[0] == 101 and s[-1] == 20
    for base, n, lo in ((100, 66, 36), (40, 64, 32), (2048, 2, 2048)):
        with pytest.raises(cpa.CpaError):
            cpa.cpa_predictor_profile_sizes(base, n, lo)


def test_target_bit_exact(cpa):
    from oracle.predictor import target
    cfg = cpa.predictor_cfg()
    rng = np.random.default_rng(1)
    for _ in range(200):
        a, b = float(rng.uniform(-1e-6, 1e-5)), float(rng.uniform(-1e-3, 1e-2))
        assert cpa.cpa_predictor_target(cfg, a, b) == target(a, b, 2048)


@pytest.mark.parametrize("align,smooth", [(128, 1.0), (16, 1.0), (128, 0.7), (1, 0.25)])
def test_next_chunk_bit_exact_over_grid(cpa, align, smooth):
    from oracle.predictor import PredictorConfig, next_chunk, target
    ocfg = PredictorConfig(align=align, smooth_factor=smooth)
    ccfg = cpa.predictor_cfg(align=align, smooth_factor=smooth)
    rng = np.random.default_rng(align)
    coefs = [(a, b) for a in (1e-8, 1e-7, 3.3e-7, 1e-6, 1e-5) for b in (0.0, 1e-4, 7.7e-4, 1e-2)]
    coefs += [(0.0, 1e-3), (-1e-7, 1e-3), (-1e-7, -1.0), (float("nan"), 1e-3),
              (1e-6, float("inf")), (1.234e-7, 7.77e-4)]
    for a, b in coefs:
        T = target(a, b, 2048) if math.isfinite(a) and math.isfinite(b) else 3.0
        Ls = list(range(0, 32768, 97)) + [int(x) for x in rng.integers(0, 40000, 50)]
        for L in Ls:
            rem = int(rng.integers(0, 40000))
            got = cpa.cpa_predictor_next_chunk(ccfg, a, b, T, L, rem)
            exp = next_chunk(ocfg, a, b, T, L, rem)
            assert got[0] == exp[0], (a, b, L, rem)
            assert (got[1] == exp[1]) or (math.isnan(got[1]) and math.isnan(exp[1]))


def test_walk_matches_oracle(cpa):
    from oracle.predictor import PredictorConfig, schedule, target
    a, b = 1e-6, 1e-3
    T = target(a, b, 2048)
    walk = schedule(PredictorConfig(), a, b, T, 32768)
    cfg = cpa.predictor_cfg()
    L = 0
    for (Lo, co, xo) in walk:
        assert L == Lo
        c, x = cpa.cpa_predictor_next_chunk(cfg, a, b, T, L, 32768 - L)
        assert c == co and x == xo
        L += c
    assert L == 32768


def test_fit_matches_oracle(cpa):
    from oracle.predictor import fit_quadratic, profile_sizes
    l = np.array(profile_sizes(2048), dtype=float)
    rng = np.random.default_rng(5)
    for trial in range(20):
        a, b, c = 10 ** rng.uniform(-8, -5), 10 ** rng.uniform(-4, -2), rng.uniform(0.01, 1)
        t = a * l * l + b * l + c
        if trial % 2:
            t = t + rng.normal(0, 0.01 * c, l.size)
        got = cpa.cpa_predictor_fit(l, t)
        exp = fit_quadratic(l, t)
        for g, e in zip(got, exp):
            assert abs(g - e) <= 1e-9 * max(abs(e), 1e-300) + 1e-12 * float(np.abs(t).max())


def test_fit_rejects_degenerate(cpa):
    with pytest.raises(cpa.CpaError) as e:
        cpa.cpa_predictor_fit([1.0, 2.0], [1.0, 2.0])
    assert e.value.status == cpa.CPA_ERR_INVALID_ARG
    with pytest.raises(cpa.CpaError) as e:
        cpa.cpa_predictor_fit([5.0, 5.0, 5.0, 5.0], [1.0, 2.0, 3.0, 4.0])
    assert e.value.status == cpa.CPA_ERR_NUMERIC
    with pytest.raises(cpa.CpaError) as e:
        cpa.cpa_predictor_fit([1.0, 2.0, float("nan")], [1.0, 2.0, 3.0])
    assert e.value.status == cpa.CPA_ERR_NUMERIC


# ---- planner and validator -------------------------------------------------

def desc(cpa, **kw):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128,
                num_blocks=200, max_blocks_per_seq=128)
    base.update(kw)
    return cpa.layer_desc(**base)


def test_plan_rejects_bad_shapes(cpa):
    cases = [
        (dict(head_dim=96), cpa.CPA_ERR_UNSUPPORTED),
        (dict(num_q_heads=30, num_kv_heads=8), cpa.CPA_ERR_INVALID_ARG),
        (dict(page_size=100), cpa.CPA_ERR_UNSUPPORTED),
        (dict(page_size=8), cpa.CPA_ERR_UNSUPPORTED),
        (dict(scale=float("nan")), cpa.CPA_ERR_NUMERIC),
        (dict(out_dtype=7), cpa.CPA_ERR_INVALID_ARG),
    ]
    for kw, status in cases:
        with pytest.raises(cpa.CpaError) as e:
            cpa.cpa_plan_create(desc(cpa, **kw), [4], [10])
        assert e.value.status == status, kw
        assert cpa.cpa_last_error()


def test_plan_rejects_bad_lengths(cpa):
    d = desc(cpa)
    for ql, sl in [([5], [4]), ([-1], [4]), ([1], [128 * 128 + 1])]:
        with pytest.raises(cpa.CpaError) as e:
            cpa.cpa_plan_create(d, ql, sl)
        assert e.value.status == cpa.CPA_ERR_INVALID_ARG


def test_plan_counts_and_pairs(cpa):
    d = desc(cpa)
    for H in (0, 4096, 12288):
        p = cpa.cpa_plan_create(d, [512], [H + 512])
        info = p.info()
        assert info["num_tokens"] == 512
        assert info["visible_pairs"] == 32 * (512 * H + 512 * 513 // 2)
        # GQA 4 packs 4 heads x 64 queries per 256-row tile: 8 kv heads x 8 tiles
        tiles = 8 * 8
        assert info["num_prefill_items"] >= tiles
        assert info["num_decode_items"] == 0
        if info["num_combine_items"]:
            assert info["num_partial_rows"] > 0
    p = cpa.cpa_plan_create(d, [512], [12800], {"prefill_split": 1})
    assert p.info()["num_combine_items"] == 0
    assert p.info()["num_prefill_items"] == 64


def test_plan_splits_short_ranges_only_when_it_pays(cpa):
    """Tiles too few to fill the CUs are split into pieces as short as one
    64-key tile, but only when that shortens the longest item by more than
    the combine launch costs (two tiles; four for d = 64 items of at most 64
    rows, whose tiles cost about half)."""
    d = desc(cpa)
    # Llama-3-8B chunk at H = 0: 64 tiles of 64 + 64t keys; 128-key pieces
    # (2 tiles, down from 8) give 8 * (1+1+2+2+3+3+4+4) = 160 items.
    info = cpa.cpa_plan_create(d, [512], [512]).info()
    assert info["num_prefill_items"] == 160
    assert info["num_combine_items"] == 48          # every tile longer than 128 keys
    assert info["num_partial_rows"] == 256 * 8 * (2 + 2 + 3 + 3 + 4 + 4)
    tiny = desc(cpa, num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=16,
                num_blocks=4096, max_blocks_per_seq=2100)
    # 128 and 192 keys: at most 3 tiles, splitting saves 2 or less -> no split
    for n in (32, 128, 192):
        info = cpa.cpa_plan_create(tiny, [n], [n]).info()
        assert info["num_prefill_items"] == 4 and info["num_combine_items"] == 0, n
    # 256 keys: 4 tiles -> 1 tile saves 3 -> split into 16 one-tile items
    info = cpa.cpa_plan_create(tiny, [256], [256]).info()
    assert info["num_prefill_items"] == 16 and info["num_combine_items"] == 4
    # a forced floor keeps the split even where the rule would drop it
    info = cpa.cpa_plan_create(tiny, [128], [128], {"min_split_keys": 64}).info()
    assert info["num_prefill_items"] == 8 and info["num_combine_items"] == 4
    # never more items than CUs from splitting alone
    for n in (512, 1024, 1536, 2048):
        assert cpa.cpa_plan_create(tiny, [n], [n]).info()["num_prefill_items"] <= 256
    with pytest.raises(cpa.CpaError):
        cpa.cpa_plan_create(tiny, [128], [128], {"min_split_keys": 100})
    # d = 64 items of at most 64 rows (six of eight waves idle) need twice
    # the saving: 4 or 5 tiles stay whole, 6 tiles split; 128 rows and the
    # d = 128 kernel keep the two-tile rule
    for c, h, items in ((64, 192, 4), (64, 256, 4), (32, 224, 4), (64, 320, 24), (128, 128, 16)):
        assert cpa.cpa_plan_create(tiny, [c], [c + h]).info()["num_prefill_items"] == items, (c, h)
    d128 = desc(cpa, num_q_heads=4, num_kv_heads=4, head_dim=128, page_size=16,
                num_blocks=4096, max_blocks_per_seq=2100)
    assert cpa.cpa_plan_create(d128, [64], [256]).info()["num_prefill_items"] == 16


def test_plan_refuses_oversized_plans(cpa):
    """Decode rows split into one-key ranges would need billions of work
    items and partial rows: refused, not wrapped around in 32 bits."""
    d = desc(cpa, num_q_heads=40, num_kv_heads=40, num_blocks=40000, max_blocks_per_seq=256)
    with pytest.raises(cpa.CpaError) as e:
        cpa.cpa_plan_create(d, [1] * 64, [32768] * 64, {"decode_split_keys": 1})
    assert e.value.status == cpa.CPA_ERR_UNSUPPORTED and "too large" in cpa.cpa_last_error()
    # the same batch with the default split (2048 keys here) is fine
    assert cpa.cpa_plan_create(d, [1] * 64, [32768] * 64).info()["num_decode_items"] == \
        64 * 40 * 16


def test_default_decode_split_fills_the_cus(cpa):
    """Without decode_split_keys the planner takes the largest split of 2048,
    1024, 512 keys that gives at least 4 decode items per CU (256 CUs), else
    256; an explicit value is used as given."""
    d = desc(cpa, num_q_heads=40, num_kv_heads=40, num_blocks=40000, max_blocks_per_seq=256)
    def items(ql, sl, opts=None):
        return cpa.cpa_plan_create(d, ql, sl, opts).info()["num_decode_items"]
    n = [1024 + 457 * i for i in range(16)]           # 16 rows, 1024 .. 7879 keys
    per = lambda k: sum((x + k - 1) // k for x in n) * 40
    assert per(2048) >= 1024 and items([1] * 16, n) == per(2048)
    # 2 rows of 4096 keys: 2048 -> 160 items, 1024 -> 320, 512 -> 640, so 256
    assert items([1, 1], [4096, 4096]) == 2 * 40 * 16
    # 6 rows of 3000 keys: 1024 gives 720, 512 gives 1440 (>= 1024)
    assert items([1] * 6, [3000] * 6) == 6 * 40 * 6
    assert items([1] * 16, n, {"decode_split_keys": 512}) == per(512)


def test_plan_page_cap_splits(cpa):
    """A tile whose key range spans more block-table entries than one
    prefill item stages in LDS (2047) is split even when splitting is
    turned off; every piece stays within the cap."""
    d = desc(cpa, num_q_heads=1, num_kv_heads=1, head_dim=64, page_size=16,
             num_blocks=3000, max_blocks_per_seq=2600)
    n = 40000                                  # 2500 pages of 16 keys
    p = cpa.cpa_plan_create(d, [64], [n], {"prefill_split": 1})
    info = p.info()
    assert info["num_prefill_items"] == 2      # 32704 keys per piece at most
    assert info["num_combine_items"] == 1
    assert info["num_partial_rows"] == 2 * 64
    p = cpa.cpa_plan_create(d, [64], [32000], {"prefill_split": 1})
    assert p.info()["num_prefill_items"] == 1  # 2000 pages: within the cap


def test_plan_mixed_batch(cpa):
    d = desc(cpa, num_q_heads=40, num_kv_heads=40, num_blocks=1200, max_blocks_per_seq=64)
    ql = [1] * 3 + [512, 0]
    sl = [1024, 5000, 8192, 2560, 77]
    p = cpa.cpa_plan_create(d, ql, sl, {"decode_split_keys": 512})
    info = p.info()
    assert info["num_tokens"] == 515
    exp_dec = 40 * sum((n + 511) // 512 for n in sl[:3])
    assert info["num_decode_items"] == exp_dec
    assert info["num_prefill_items"] >= 40 * 2
    pairs = sum(40 * (q * (n - q) + q * (q + 1) // 2) for q, n in zip(ql, sl))
    assert info["visible_pairs"] == pairs


def test_validate_metadata(cpa):
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    b = make_batch(3, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                   query_lens=[5, 1], seq_lens=[40, 17], extra_pages=2)
    d = cpa.layer_desc(4, 2, 64, 16, b.num_blocks, b.max_blocks_per_seq)
    cpa.cpa_validate_metadata(d, b.slot_mapping, b.block_table, b.query_lens, b.seq_lens)
    sm = b.slot_mapping.copy()
    sm[1] = sm[0]
    with pytest.raises(cpa.CpaError, match="repeats"):
        cpa.cpa_validate_metadata(d, sm)
    sm[1] = b.num_blocks * 16
    with pytest.raises(cpa.CpaError, match="outside"):
        cpa.cpa_validate_metadata(d, sm)
    bt = b.block_table.copy()
    bt[0, 1] = b.num_blocks
    with pytest.raises(cpa.CpaError, match="block_table"):
        cpa.cpa_validate_metadata(d, None, bt, b.query_lens, b.seq_lens)


# ---- online calibration: C++ vs oracle ----------------------------------------

def test_calib_features_match_oracle(cpa):
    from oracle.calibration import features
    rng = np.random.default_rng(2)
    for _ in range(50):
        n = int(rng.integers(0, 20))
        C = rng.integers(-3, 4096, n)
        H = rng.integers(0, 1 << 20, n)
        assert cpa.cpa_calib_features(C, H) == features(C, H)


def test_calib_one_chunk_size_is_refused_unless_seeded(cpa):
    """Records of a single prompt whose chunks all have one size C leave
    C*(C+H) and C+H proportional: every refit is refused and no model ever
    exists. A window seeded with the startup profile's runs (H = 0, sizes
    2048 .. 32) takes the same records and keeps a model."""
    import bench
    from oracle.predictor import profile_sizes
    recs = [(cpa.cpa_calib_features([1280], [1280 * i]), 0.015 + 1e-6 * i) for i in range(12)]
    bare = cpa.Calib(min_points=5, window=30)
    for i, (f, m) in enumerate(recs):
        if i < 4:
            assert bare.record(f, m) is False        # fewer than min_points: no fit yet
        else:
            with pytest.raises(cpa.CpaError):
                bare.record(f, m)
    with pytest.raises(cpa.CpaError):
        bare.model()
    sizes = profile_sizes(2048, 64, 32)
    seeded = cpa.Calib(min_points=5, window=30)
    bench.seed_calibration(seeded, sizes, [1e-9 * l * l + 2e-6 * l + 0.012 for l in sizes])
    for f, m in recs:
        assert seeded.record(f, m) is True
    seeded.model()


def test_calib_seeded_with_profile_is_the_profile_quadratic(cpa):
    """At H = 0 the two-variable model is the one-variable quadratic
    (features [l*l, l, 1]), so a window seeded with the profile holds the 30
    largest sizes and fits the same coefficients as the one-variable least
    squares over them: the library's fit and the oracle's."""
    import bench
    from oracle.predictor import fit_quadratic, profile_sizes
    sizes = profile_sizes(2048, 64, 32)
    rng = np.random.default_rng(11)
    ms = [2e-8 * l * l + 3e-6 * l + 0.012 + float(rng.normal(0, 2e-4)) for l in sizes]
    calib = cpa.Calib(min_points=5, window=30)
    bench.seed_calibration(calib, sizes, ms)
    got = calib.model()
    top = sorted(zip(sizes, ms))[-30:]
    assert top[0][0] == 1120 and top[-1][0] == 2048
    tl, tm = [l for l, _ in top], [m for _, m in top]
    for exp in (fit_quadratic(tl, tm), cpa.cpa_predictor_fit(tl, tm)):
        for g, e in zip(got, exp):
            assert abs(g - e) <= 1e-7 * abs(e), (got, exp)


def test_calib_fit_matches_oracle(cpa):
    from oracle.calibration import features, fit
    rng = np.random.default_rng(8)
    for trial in range(10):
        feats, ms = [], []
        for _ in range(int(rng.integers(5, 31))):
            N = int(rng.integers(1, 6))
            C = rng.integers(16, 2048, N)
            H = rng.integers(0, 30000, N)
            f = features(C, H)
            feats.append(f)
            ms.append(3e-8 * f[0] + 2e-4 * f[1] + 0.03 * f[2] + rng.normal(0, 1e-3))
        got = cpa.cpa_calib_fit(feats, ms)
        exp = fit(feats, ms)
        for g, e in zip(got, exp):
            assert abs(g - e) <= 1e-9 * max(abs(e), 1e-300) + 1e-12 * max(abs(v) for v in ms)


@pytest.mark.parametrize("align,smooth", [(128, 1.0), (16, 1.0), (128, 0.6)])
def test_calib_next_chunk_bit_exact(cpa, align, smooth):
    from oracle.calibration import next_chunk, target
    from oracle.predictor import PredictorConfig
    ocfg = PredictorConfig(align=align, smooth_factor=smooth)
    ccfg = cpa.predictor_cfg(align=align, smooth_factor=smooth)
    rng = np.random.default_rng(align + int(smooth * 10))
    models = [(a, b, c) for a in (1e-9, 1e-8, 1.3e-7, 1e-6) for b in (0.0, 1e-4, 7.7e-4)
              for c in (0.0, 0.05, 1.0)]
    models += [(0.0, 1e-3, 0.1), (-1e-8, 1e-3, 0.1), (-1e-8, -1e-3, 0.1), (float("nan"), 1e-3, 0.1),
               (1e-7, float("inf"), 0.1)]
    for a, b, c in models:
        finite = all(map(np.isfinite, (a, b, c)))
        T = target(a, b, c, 2048) if finite else 2.0
        if finite:
            assert cpa.cpa_calib_target(ccfg, a, b, c) == T
        for H in list(range(0, 32768, 331)) + [int(v) for v in rng.integers(0, 40000, 40)]:
            rem = int(rng.integers(0, 40000))
            got = cpa.cpa_calib_next_chunk(ccfg, a, b, c, T, H, rem)
            exp = next_chunk(ocfg, a, b, c, T, H, rem)
            assert got[0] == exp[0], (a, b, c, H, rem)
            assert got[1] == exp[1] or (np.isnan(got[1]) and np.isnan(exp[1]))


def test_calib_window_matches_oracle(cpa):
    from oracle.calibration import Calibrator, features
    rng = np.random.default_rng(13)
    ref = Calibrator(min_points=5, window=12)
    h = cpa.Calib(min_points=5, window=12)
    with pytest.raises(cpa.CpaError):
        h.model()
    for i in range(40):
        C = rng.integers(16, 2048, 2)
        H = rng.integers(0, 20000, 2)
        f = features(C, H)
        ms = (1e-8 if i < 20 else 4e-8) * f[0] + 1e-4 * f[1] + 0.02 * f[2] + rng.normal(0, 1e-4)
        assert h.record(f, ms) == ref.record(f, ms)
        if ref.coef is not None:
            for g, e in zip(h.model(), ref.coef):
                assert abs(g - e) <= 1e-9 * abs(e) + 1e-15


def test_calib_rejects_bad_arguments(cpa):
    with pytest.raises(cpa.CpaError) as e:
        cpa.Calib(min_points=2, window=30)
    assert e.value.status == cpa.CPA_ERR_INVALID_ARG
    with pytest.raises(cpa.CpaError) as e:
        cpa.cpa_calib_fit([[1.0, 2.0, 1.0]] * 4, [1.0, 2.0, 3.0, 4.0])
    assert e.value.status == cpa.CPA_ERR_NUMERIC
    with pytest.raises(cpa.CpaError) as e:
        cpa.cpa_calib_features([5], [-1])
    assert e.value.status == cpa.CPA_ERR_INVALID_ARG


def test_calib_rank_deficient_window(cpa):
    from oracle.calibration import Calibrator, features
    feats = [features([1024], [h]) for h in range(0, 10240, 1024)]
    ms = [1e-7 * f[0] + 1e-3 * f[1] + 0.1 for f in feats]
    with pytest.raises(cpa.CpaError) as e:
        cpa.cpa_calib_fit(feats, ms)
    assert e.value.status == cpa.CPA_ERR_NUMERIC
    h, ref = cpa.Calib(min_points=5, window=5), Calibrator(min_points=5, window=5)
    for i, (f, m) in enumerate(zip(feats, ms)):
        if i < 4:                      # fewer than min_points: no fit attempted
            assert h.record(f, m) is False
        else:                          # the fit is refused, no model yet
            with pytest.raises(cpa.CpaError) as e:
                h.record(f, m)
            assert e.value.status == cpa.CPA_ERR_NUMERIC
        assert ref.record(f, m) is False
    with pytest.raises(cpa.CpaError):
        h.model()


# ---- two-micro-batch split: C++ vs oracle --------------------------------------

def test_split_point_matches_oracle(cpa):
    from oracle.split import balanced_split, simple_split
    rng = np.random.default_rng(21)
    cases = [[1] * 16 + [512, 512], [5], [], [0, 0], [3, 2, 3], [2, 2, 2, 2]]
    cases += [[int(v) for v in rng.integers(0, 700, int(rng.integers(1, 15)))] for _ in range(300)]
    for ql in cases:
        assert cpa.cpa_split_point(ql, cpa.CPA_SPLIT_SIMPLE) == simple_split(ql)
        for bt, lt in [(0.5, 1), (0.05, 100), (3.0, 0), (0.0, 1)]:
            assert cpa.cpa_split_point(ql, cpa.CPA_SPLIT_BALANCED, bt, lt) == balanced_split(ql, bt, lt), (ql, bt, lt)


def test_split_point_rejects_bad_arguments(cpa):
    for args in [([1, -2], 0, 0.5, 1), ([1, 2], 7, 0.5, 1), ([1, 2], 1, float("nan"), 1)]:
        with pytest.raises(cpa.CpaError) as e:
            cpa.cpa_split_point(*args)
        assert e.value.status == cpa.CPA_ERR_INVALID_ARG


# ---- token-budget batch former: C++ vs oracle ----------------------------------

def _both_schedulers(cpa, budget, kind, seed):
    from oracle import predictor as P
    from oracle import scheduler as S
    a, b, c = 1.1e-7, 7e-4, 0.05
    ocfg = P.PredictorConfig(align=16)
    if kind == S.RULE_CALIBRATED:
        from oracle.calibration import target as t2
        T = t2(a, b, c, 2048)
    else:
        T = P.target(a, b, 2048)
    rule = S.Rule(kind, fixed=384, sizes=(2048, 1024, 512), cfg=ocfg, a=a, b=b, c=c, T=T)
    cc = cpa.sched_cfg(budget, kind, fixed_chunk=384, sizes=(2048, 1024, 512),
                       pred=cpa.predictor_cfg(align=16), a=a, b=b, c=c, T=T)
    return S.Scheduler(budget, rule), cpa.Sched(cc)


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
@pytest.mark.parametrize("seed", range(4))
def test_scheduler_matches_oracle(cpa, kind, seed):
    rng = np.random.default_rng(100 * kind + seed)
    budget = int(rng.choice([128, 512, 2048]))
    ref, got = _both_schedulers(cpa, budget, kind, seed)
    for _ in range(int(rng.integers(1, 16))):
        p, m, t = int(rng.integers(1, 9000)), int(rng.integers(0, 40)), int(rng.integers(0, 50))
        assert ref.add(p, m, t) == got.add(p, m, t)
    steps = 0
    while not ref.finished():
        assert got.form() == ref.form()
        ref.commit()
        got.commit()
        steps += 1
        assert got.status() == (ref.finished(), steps)
    assert got.status()[0]


def test_scheduler_capacity_and_protocol(cpa):
    s = cpa.Sched(cpa.sched_cfg(1 << 20, cpa.CPA_RULE_FIXED, fixed_chunk=1 << 20))
    for p in (5, 6, 7):
        s.add(p, 1)
    with pytest.raises(cpa.CpaError):
        s.form(capacity=2)                       # three sequences do not fit
    assert s.form(capacity=3) == [(0, 5, 5), (1, 6, 6), (2, 7, 7)]
    with pytest.raises(cpa.CpaError):
        s.form()                                 # commit first
    s.commit()
    assert s.form() == [(0, 1, 6), (1, 1, 7), (2, 1, 8)]
    s.commit()
    assert s.status() == (True, 2)
    with pytest.raises(cpa.CpaError):
        cpa.Sched(cpa.sched_cfg(0))
    with pytest.raises(cpa.CpaError):
        cpa.Sched(cpa.sched_cfg(64, cpa.CPA_RULE_PROGRESSIVE, sizes=()))


def test_fused_call_rejects_null_pointers(cpa):
    """cpa_kv_write_attention checks its pointers on the host before any GPU
    work: a NULL plan or a NULL new-row pointer is CPA_ERR_INVALID_ARG (the
    other pointers are never dereferenced on the host)."""
    import ctypes
    fake = ctypes.c_void_p(256)
    p = cpa.cpa_plan_create(desc(cpa), [4], [10])
    lib = cpa._lib
    assert lib.cpa_kv_write_attention(None, fake, fake, fake, fake, fake, fake, fake, fake,
                                      fake, 1 << 20, None) == cpa.CPA_ERR_INVALID_ARG
    for hole in range(3):          # k_new, v_new, slot_mapping
        args = [fake, fake, fake]
        args[hole] = None
        st = lib.cpa_kv_write_attention(p.handle, fake, *args, fake, fake, fake, fake, fake,
                                        1 << 20, None)
        assert st == cpa.CPA_ERR_INVALID_ARG, hole
        assert "NULL" in cpa.cpa_last_error()
    p.destroy()


def test_host_entry_points_from_many_threads(cpa):
    """Plans, their info, refusals (with per-thread messages) and predictor
    calls from eight host threads at once give the single-thread results."""
    import threading
    desc = cpa.layer_desc(32, 8, 128, 128, 200, 104)
    bad = cpa.layer_desc(32, 8, 96, 128, 200, 104)
    want = cpa.cpa_plan_create(desc, [512, 1, 40], [12800, 700, 300]).info()
    cfg = cpa.predictor_cfg(align=128)
    want_chunk = cpa.cpa_predictor_next_chunk(cfg, 2e-9, 5e-6, 0.0125, 4096, 30000)
    errors = []

    def work(seed):
        try:
            for i in range(200):
                p = cpa.cpa_plan_create(desc, [512, 1, 40], [12800, 700, 300])
                assert p.info() == want
                p.destroy()
                with pytest.raises(cpa.CpaError) as e:
                    cpa.cpa_plan_create(bad, [512], [12800])
                assert "head_dim" in str(e.value)
                assert cpa.cpa_predictor_next_chunk(cfg, 2e-9, 5e-6, 0.0125, 4096,
                                                    30000) == want_chunk
        except Exception as ex:  # reported below, on the main thread
            errors.append(repr(ex))

    threads = [threading.Thread(target=work, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
