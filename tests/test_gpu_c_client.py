"""The fused call from a plain C program on the GPU: tests/c_client/
cpa_gpu_client.c (libcpa and the HIP runtime only, no Python or torch in
its process) runs cpa_kv_write_attention on seeded inputs written here;
its output is compared with the oracle and its caches bit for bit."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from chunked_prefill_attention_slot_amd import build as B

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def build_client(tmp_path):
    exe = str(tmp_path / "cpa_gpu_client")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{B.INCLUDE}", f"-I{B.ROCM}/include",
           os.path.join(HERE, "c_client", "cpa_gpu_client.c"), "-o", exe,
           f"-L{B.PKG}", "-lcpa", f"-L{B.ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{B.PKG}", f"-Wl,-rpath,{B.ROCM}/lib", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
@pytest.mark.parametrize("shape", [
    # hq, hkv, d, P, query_lens, seq_lens
    (8, 2, 128, 16, [1, 70, 0, 33], [50, 300, 3, 100]),
    (4, 4, 64, 16, [64], [256]),
])
def test_c_gpu_client(tmp_path, shape):
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    from tests import gpu_helpers as H
    from oracle.kv_cache import kv_write
    hq, hkv, d, P, ql, sl = shape
    b = make_batch(seed=31, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=P,
                   query_lens=ql, seq_lens=sl, extra_pages=3)
    exe = build_client(tmp_path)
    inp, outp = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    T = int(b.num_tokens)
    with open(inp, "wb") as f:
        np.array([hq, hkv, d, P, b.num_blocks, b.max_blocks_per_seq, len(ql), T],
                 dtype=np.int32).tofile(f)
        for arr, dt in ((b.query_lens, np.int32), (b.seq_lens, np.int32),
                        (b.block_table, np.int32), (b.slot_mapping, np.int32),
                        (b.q, np.uint16), (b.k_new, np.uint16), (b.v_new, np.uint16),
                        (b.k_cache, np.uint16), (b.v_cache, np.uint16)):
            np.ascontiguousarray(np.asarray(arr, dtype=dt)).tofile(f)
    print(f"[case] C client {shape}", flush=True)
    r = subprocess.run([exe, inp, outp], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "done", r.stdout + r.stderr
    raw = np.fromfile(outp, dtype=np.uint16)
    n_q, n_c = T * hq * d, b.k_cache.size
    assert raw.size == n_q + 2 * n_c
    out = raw[:n_q].reshape(T, hq, d)
    kc, vc = raw[n_q:n_q + n_c].reshape(b.k_cache.shape), raw[n_q + n_c:].reshape(b.v_cache.shape)
    ref_kc, ref_vc = kv_write(b.k_cache, b.v_cache, b.k_new, b.v_new, b.slot_mapping, P)
    np.testing.assert_array_equal(kc, ref_kc)
    np.testing.assert_array_equal(vc, ref_vc)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    H.compare(got, H.oracle_out(b), f"C client {shape}")
