"""Build libe2m1lut.so in-tree with hipcc for gfx950.

    python -m gemm_e2m1_lut_amd.build        # or: from gemm_e2m1_lut_amd.build import build

Every .hip source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into gemm_e2m1_lut_amd/libe2m1lut.so. The platform
probe (probe/platform_probe.hip: an empty kernel and plain HBM streams, which
the benchmark runs as reference points) is built beside it into
probe/libe2m1probe.so; the library never loads it. Each call recompiles
everything.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libe2m1lut.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
PROBE_SRC = os.path.join(PKG, "probe", "platform_probe.hip")
PROBE_LIB = os.path.join(PKG, "probe", "libe2m1probe.so")

# Target: gfx950 with XNACK off, the MI355X default. Compiled for XNACK off, a
# load's destination registers may overlap its address (no replay to
# protect), which measured 2-5 % faster on the batch-4 GEMV and the prefill
# GEMM than code that serves either mode. The library does not load on a
# device running with XNACK on: set E2M1_OFFLOAD_ARCH=gfx950 (either mode) or
# gfx950:xnack+ and rebuild for one.
ARCH = "gfx950"
OFFLOAD = [f"--offload-arch={os.environ.get('E2M1_OFFLOAD_ARCH', ARCH + ':xnack-')}"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are disabled for every kernel: the compiler forms them
# from ordinary float code, and some of their forms are not trusted here.
# Kernel arguments are preloaded into SGPRs (gfx950 kernarg preload; the
# compiler keeps a fallback prologue for launches without it), so a wave's
# first loads do not wait for an argument load: about 2 % off the batch-1
# and batch-4 GEMV launches, bit-identical results.
HIPFLAGS = [
    *OFFLOAD, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", INCLUDE, "-I", CSRC,
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd: list[str]) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("command failed:\n  " + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    warnings = [ln for ln in res.stderr.splitlines() if ln.strip() and noise not in ln]
    if warnings:
        sys.stderr.write("\n".join(warnings) + "\n")


def build(jobs: int | None = None) -> str:
    """Compile every source, link the shared library and the probe; returns the library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources() + [PROBE_SRC]
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC, *HIPFLAGS, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    for path, linked in ((LIB_PATH, objs[:-1]), (PROBE_LIB, objs[-1:])):
        tmp = path + ".tmp"
        _run([HIPCC, *OFFLOAD, "-shared", "-fPIC", "-o", tmp, *linked])
        os.replace(tmp, path)
    return LIB_PATH


def clean() -> None:
    shutil.rmtree(BUILD_DIR, ignore_errors=True)
    for path in (LIB_PATH, PROBE_LIB):
        if os.path.exists(path):
            os.remove(path)


if __name__ == "__main__":
    print(build())
