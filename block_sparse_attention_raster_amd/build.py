"""Builds libvsa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and the
benchmark's two probes: read bandwidth per cache level (cache_probe) and the
issue, LDS and synthetic-step rates that bound the attention step
(step_probe).

    python -m block_sparse_attention_raster_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvsa.so")
PROBE = os.path.join(PKG, "cache_probe")   # read-bandwidth probe of the benchmark
STEP_PROBE = os.path.join(PKG, "step_probe")   # issue / LDS / synthetic-step probe of the benchmark
BUILD_DIR = os.path.join(PKG, "_build")

HIP_SOURCES = ["api.hip", "pool.hip", "select.hip", "attend.hip"]
HOST_SOURCES = ["plan.cpp"]
ARCH = "gfx950"
# Packed fp32 instructions are kept out of generated code; the host pass
# warns that it does not know the feature, which is harmless.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libvsa.so next to this file. Always
    recompiles. Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, s + ".o")
        jobs.append([hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", obj])
    for s in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, s + ".o")
        jobs.append(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(_run, jobs))
    if verbose:
        for r in results:
            sys.stdout.write(r.stdout + r.stderr)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    probe_flags = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
                   "-packed-fp32-ops"]
    for src, out in (("cache_probe.hip", PROBE), ("step_probe.hip", STEP_PROBE)):
        _run([hipcc, *probe_flags, os.path.join(CSRC, src), "-o", out + ".tmp"])
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
