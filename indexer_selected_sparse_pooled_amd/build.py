"""Build libqsa.so (and the input generator's fill library) for gfx950.

Compiles every HIP source with hipcc, in parallel, in-tree:
  indexer_selected_sparse_pooled_amd/libqsa.so   <- csrc/*.hip
  qsa_inputs/libqsa_fill.so                      <- qsa_inputs/fill.hip
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqsa.so")
FILL_SRC = os.path.join(ROOT, "qsa_inputs", "fill.hip")
FILL_LIB = os.path.join(ROOT, "qsa_inputs", "libqsa_fill.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off (plain fp32 code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _compile(src, obj):
    return _run([HIPCC, *FLAGS, "-c", src, "-o", obj])


def build(verbose: bool = False) -> None:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = min(len(srcs) + 1, max(1, min(16, os.cpu_count() or 1)))
    fill_obj = os.path.join(BUILD, "fill.o")
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, s, o) for s, o in zip(srcs, objs)]
        futs.append(ex.submit(_compile, FILL_SRC, fill_obj))
        for f in futs:
            out = f.result()
            if verbose and out:
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    tmp = FILL_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", fill_obj, "-o", tmp])
    os.replace(tmp, FILL_LIB)


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
