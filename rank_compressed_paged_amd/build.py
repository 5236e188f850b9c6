"""Build libstarkv.so in-tree with hipcc for gfx950.

    python -m rank_compressed_paged_amd.build [--jobs N] [--debug]

Each translation unit is compiled in parallel, then linked into
rank_compressed_paged_amd/libstarkv.so.  Packed-FP32 instructions are turned
off for device code (-packed-fp32-ops); the host pass warns that it does not
know the feature, which is harmless.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libstarkv.so")
SOURCES = ["api.cpp", "decode.hip", "append.hip", "prefill.hip", "util.hip", "fit.hip",
           "noalloc.hip", "generic.hip", "check.hip"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags(debug=False):
    flags = [f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", f"-I{INCLUDE}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
    flags += ["-O1", "-g"] if debug else ["-O3"]
    return flags


def _compile(src, debug):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(debug), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs=4, debug=False, verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args()
    build(a.jobs, a.debug, verbose=True)
    sys.exit(0)
