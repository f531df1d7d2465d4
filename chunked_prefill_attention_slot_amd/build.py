"""Builds libcpa.so (gfx950 kernels + host runtime) in-tree with hipcc.

    python -m chunked_prefill_attention_slot_amd.build

Every call recompiles every source. Objects go to _build/ next to this
file; the library lands beside this file as libcpa.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcpa.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only; packed fp32 ops disabled (the device pass
# accepts the feature; the host pass warns that it does not know it).
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-ffp-contract=fast"]
# Host-only C++: the predictor must round exactly as written.
HOST_FLAGS = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
              "-ffp-contract=off", "-fno-fast-math"]


def _sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    return r.returncode, " ".join(cmd), out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = _sources()
    cmds = []
    objs = []
    for f in hip:
        o = os.path.join(BUILD, f + ".o")
        objs.append(o)
        cmds.append([HIPCC, *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
    for f in cpp:
        o = os.path.join(BUILD, f + ".o")
        objs.append(o)
        cmds.append([CLANG, *COMMON, *HOST_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, 16))) as ex:
        results = list(ex.map(_run, cmds))
    failed = [r for r in results if r[0] != 0]
    for rc, cmd, out in results:
        if verbose or rc != 0:
            print(cmd)
            if out.strip():
                print(out)
    if failed:
        raise RuntimeError(f"libcpa build failed ({len(failed)} of {len(cmds)} sources)")
    tmp = LIB + ".tmp"
    rc, cmd, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
                         "-o", tmp, *objs])
    if verbose or rc != 0:
        print(cmd)
        print(out)
    if rc != 0:
        raise RuntimeError("libcpa link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
