"""Build libcpattn.so in-tree with hipcc for gfx950.

Usage: ``python -m context_attention_long_amd.build`` (or ``build()``).
Every call compiles from source; the objects go to ``_build/`` and the
library to ``context_attention_long_amd/libcpattn.so``.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcpattn.so")

SOURCES = ["plan.cpp", "api.cpp", "merge.hip", "decode_gqa.hip", "decode_mla.hip", "prefill.hip", "prefill_mla.hip", "cache_write.hip",
           "sparse_mla.hip", "topk.hip", "noalloc.hip"]

ARCH = "gfx950"
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-function"]
# Packed-FP32 VALU forms are kept out of the generated code on purpose.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-flush-denormals-to-zero"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libcpattn)")


def _compile(src, verbose):
    hipcc = _hipcc()
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc, "-c", path, "-o", obj] + COMMON + DEVICE
    else:
        cmd = [hipcc, "-c", "-x", "c++", path, "-o", obj] + COMMON + ["-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{msg}")
    if verbose and msg:
        print(msg, flush=True)
    return obj


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-o", tmp] + objs + ["--offload-arch=" + ARCH, "-fPIC"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libcpattn.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
