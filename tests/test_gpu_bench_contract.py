"""bench.py's output line as its contract fixes it: a short run (headline
and small legs, no CPU baseline) in a child process, its last stdout line
parsed and checked field by field. The child's first import of torch can
take a minute or two on a fresh machine, hence the longer time limit."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(400)
def test_bench_json_line():
    print("[case] bench.py --legs small --steps 3 --warmup 1 --no-cpu", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--legs", "small",
                        "--steps", "3", "--warmup", "1", "--no-cpu"],
                       capture_output=True, text=True, timeout=360, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["metric"].startswith("chunked-prefill attn TFLOP/s")
    assert d["unit"] == "TFLOP/s" and d["n_gpus"] == 1
    assert d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert "workload" in d["config"] and d["config"]["hist"] == [0, 4096, 8192, 12288]
    rl = d["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 2500.0
    assert rl["achieved"] > 0 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-9
    assert rl["traffic"] is None or rl["traffic"] > rl["algorithmic_bytes_per_launch"] * 0.5
    # value is the whole step's FLOP over the step time
    flop = sum(4 * 32 * 128 * 512 * (h + 256) for h in d["config"]["hist"])
    assert abs(d["value"] - flop / (d["ms_per_step"] * 1e-3) / 1e12) < 1e-6 * d["value"]
    assert len(d["per_H"]) == 4 and all(p["call_us_mean"] > 0 for p in d["per_H"])
    assert d["small"]["us_median"] > 0
