"""Host-side pieces of bench.py (no GPU): the FLOP count of a chunk, the
code digest that keys the committed counter summary, and the refusal of
more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_flops_chunk_matches_visible_pairs():
    """The FLOP count 4*Hq*d*C*(H + C/2) charges 2*d FLOP per product for
    C*H + C^2/2 pairs per head; counting the visible (query, key) pairs by
    brute force gives C*H + C(C+1)/2, i.e. C/2 pairs more (each query's own
    key). Both are pinned here."""
    hq, d, c, h = 3, 8, 6, 5
    pairs = sum(h + i + 1 for i in range(c)) * hq       # query i sees keys 0..H+i
    assert pairs == hq * (c * h + c * (c + 1) // 2)
    assert bench.flops_chunk(hq, d, c, h) == 4 * d * (pairs - hq * c / 2)


def test_code_digest_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("/* header */\nint f(int x) {\n    return x + 1;\n}  // end\n")
    c.write_text("int f(int x) {\n  return x + 2;  // one\n}\n")
    assert bench.kernel_source_digest(a) == bench.kernel_source_digest(b)
    assert bench.kernel_source_digest(a) != bench.kernel_source_digest(c)
    # several files: order and content both count
    assert bench.kernel_source_digest(a, c) != bench.kernel_source_digest(c, a)
    assert bench.kernel_source_digest(a, c) == bench.kernel_source_digest(b, c)


def test_traffic_digest_covers_planner_and_layouts():
    names = [os.path.basename(p) for p in bench.TRAFFIC_SOURCES]
    assert names == ["prefill_attn.hip", "api.cpp", "cpa_internal.h"]
    assert all(os.path.exists(p) for p in bench.TRAFFIC_SOURCES)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_online_walk_needs_the_seed_on_a_latency_floor():
    """A synthetic chunk latency shaped like the 4-head d = 64 workload: a
    per-call cost that saturates with the chunk size (so the profile at
    H = 0 is concave and its quadratic fit has a < 0) plus a cost per
    (query, key) pair and per prefix key. Unseeded, the online walk repeats
    the profile model's one chunk size and every refit is refused; seeded
    with the profile's runs, it has a model from the first chunk, the chunks
    shrink as the prefix grows, and the chunk latencies spread less."""
    import math
    import numpy as np
    from chunked_prefill_attention_slot_amd import binding as cpa
    from oracle.predictor import profile_sizes

    def lat(C, H):    # ms
        return 0.0065 + 0.0105 * (1.0 - math.exp(-C / 400.0)) + 1.0e-9 * C * H + 3e-7 * H

    sizes = profile_sizes(2048, 64, 32)
    ms = [lat(l, 0) for l in sizes]
    fit = cpa.cpa_predictor_fit(sizes, ms)
    assert fit[0] < 0                              # concave profile: degenerate model
    cfg = cpa.predictor_cfg(align=128)
    bare = cpa.Calib(min_points=5, window=30)
    rows, refused = bench.online_walk(bare, cfg, fit, 32768, lat)
    chunks = [ch for _, ch, _, _ in rows]
    # one size throughout (the last chunk is the remainder); every refit
    # from the fifth record on is refused but the one the remainder allows
    assert len(set(chunks[:-1])) == 1 and refused >= len(rows) - 5
    seeded = cpa.Calib(min_points=5, window=30)
    bench.seed_calibration(seeded, sizes, ms)
    rows2, refused2 = bench.online_walk(seeded, cfg, fit, 32768, lat)
    chunks2 = [ch for _, ch, _, _ in rows2]
    assert refused2 < len(rows2) // 2
    assert len(set(chunks2)) >= 4 and max(chunks2[-10:]) < chunks2[0]
    cv = lambda v: float(np.std(v) / np.mean(v))
    assert cv([m for _, _, m, _ in rows2]) < cv([m for _, _, m, _ in rows])
