"""Builds libselscan.so in-tree with hipcc for gfx950.

    python -m selective_state_space_25_amd.build

Each source compiles to its own object (in parallel), then one shared
library is linked next to this file.  All device code is compiled with
packed-FP32 instructions disabled.

The build fails when a kernel needs scratch memory (register spills): a
kernel with spill slots, even in a branch that never runs, is launched as a
scratch user, which has cost ~30% of a whole launch here.  Set
SELSCAN_ALLOW_SCRATCH=1 to build anyway.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libselscan.so")
ABI_BENCH = os.path.join(HERE, "abi_bench")   # host cost of the decode entry points, timed from C++
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["selscan.cpp", "timing.cpp", "m1_scan.hip", "m2_scan.hip", "m2_ssd.hip", "step.hip", "conv1d.hip", "m1_bwd.hip", "m2_bwd.hip", "noalloc.hip"]
ARCH = os.environ.get("SELSCAN_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libselscan)")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def scratch_users(remarks: str) -> list[tuple[str, int]]:
    """(kernel, bytes per lane) for every kernel whose resource-usage remarks
    report scratch memory."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    device = src.endswith(".hip")
    cmd = [hipcc()] + flags() + (["-Rpass-analysis=kernel-resource-usage"] if device else []) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [l for l in r.stderr.splitlines() if noise not in l]
    # the remarks and the source lines they quote stay out of the log
    err = "\n".join(l for l in lines if "kernel-resource-usage" not in l and not re.match(r"\s*\d*\s*\|", l))
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    spills = scratch_users("\n".join(lines)) if device else []
    if spills and os.environ.get("SELSCAN_ALLOW_SCRATCH", "0") != "1":
        raise RuntimeError(f"{src}: kernels use scratch memory (register spills): "
                           + ", ".join(f"{k} {b} B/lane" for k, b in spills))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(tmp, LIB)
    # the native decode timing harness, linked against the library beside it
    tmp = ABI_BENCH + ".tmp"
    cmd = [hipcc(), "-O2", "-std=c++17", "-I", INCLUDE, os.path.join(CSRC, "abi_bench.cpp"), "-o", tmp,
           "-L", HERE, "-lselscan", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building abi_bench failed:\n" + r.stderr)
    os.replace(tmp, ABI_BENCH)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
