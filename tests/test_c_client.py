"""The C ABI from C: tests/c_client/cpa_client.c is compiled with gcc as
C11 against include/cpa.h, linked to the built libcpa.so and run. It calls
host entry points only (plans, predictor, split point), so no GPU is
needed."""
import os
import shutil
import subprocess

import pytest

from chunked_prefill_attention_slot_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists(B.LIB),
                    reason="gcc or the built library is missing")
def test_c_client(tmp_path):
    exe = str(tmp_path / "cpa_client")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{B.INCLUDE}", f"-I{B.ROCM}/include", os.path.join(HERE, "c_client", "cpa_client.c"),
           "-o", exe, f"-L{B.PKG}", "-lcpa", f"-Wl,-rpath,{B.PKG}", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("done"), r.stdout + r.stderr
    assert "FAIL" not in r.stdout
    assert r.stdout.count("ok ") == 14
