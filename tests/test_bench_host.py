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
