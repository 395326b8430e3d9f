"""Build libfp8mi.so (gfx950 HIP kernels + the C ABI) and libfp8mi_probe.so
(measurement kernels for bench.py) in-tree with hipcc.

    python -m fp8_scaled_quantization_scale_amd.build

Every HIP translation unit is compiled with packed FP32 ops disabled
(`-Xclang -target-feature -Xclang -packed-fp32-ops`) and FP32 divide kept
correctly rounded (hipcc's default), then linked into the shared libraries
next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfp8mi.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "quantize.hip", "history.hip", "gemm.hip"]
PROBE_LIB = os.path.join(HERE, "libfp8mi_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument",
    ]


def _compile(src: str) -> str:
    out = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + _flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def _link(objs, lib: str):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(5, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
