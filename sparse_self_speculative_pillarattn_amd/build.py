"""Build libspa.so and libspa_probe.so (HIP, gfx950) in-tree with hipcc.

    python -m sparse_self_speculative_pillarattn_amd.build

Every HIP translation unit is compiled with packed-FP32 instruction selection
turned off (-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass of
hipcc warns that it does not know the feature, which is harmless.
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
LIB = os.path.join(PKG, "libspa.so")
SOURCES = ["api.cpp", "kernels.hip", "sched.cpp", "kvcache.cpp"]
# the bandwidth probe of include/spa_probe.h: a library of its own
PROBE_LIB = os.path.join(PKG, "libspa_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = os.environ.get("SPA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(LIB)
        print(PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
