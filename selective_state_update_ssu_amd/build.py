"""Compile the HIP sources into the in-tree shared library `_lib/libssu_amd.so`.

Every translation unit is compiled for gfx950 only, in parallel, then linked into
one shared library that exports the C ABI of include/ssu.h and include/ssd.h. Packed-fp32 VALU
instructions are disabled for the device code.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIBRARY = os.path.join(LIB_DIR, "libssu_amd.so")
# Streaming reference kernels used by the benchmark only (bandwidth ceilings and
# counter calibration); not part of the SSU library.
STREAM_LIBRARY = os.path.join(LIB_DIR, "libssu_stream.so")
STREAM_SOURCES = ["stream_ceiling.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["ssu_api.hip", "ssu_kernels_f32.hip", "ssu_kernels_f16.hip", "ssu_kernels_bf16.hip",
           "ring_trackers.hip", "ssd_api.hip", "ssd_kernels_bf16.hip", "ssd_kernels_f16.hip"]
CXXFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the device-only target feature; that note is noise.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if noise not in l and "warning generated" not in l
                    and "warnings generated" not in l and l.strip())
    return msg


def build(verbose: bool = False) -> str:
    """Compile every source and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        msg = _run([HIPCC, *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj, msg

    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES + STREAM_SOURCES))
    for obj, msg in results:
        if msg and verbose:
            print(msg, file=sys.stderr)
    objs = dict(zip(SOURCES + STREAM_SOURCES, (o for o, _ in results)))
    for lib, srcs in ((LIBRARY, SOURCES), (STREAM_LIBRARY, STREAM_SOURCES)):
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
              *[objs[s] for s in srcs]])
        os.replace(tmp, lib)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
