"""Build libtwl.so in-tree with hipcc for gfx950.

    python -m ternary_weight_linear_block_amd.build [--jobs N] [--verbose]

Every HIP source is compiled with -O3 for gfx950 only, without fast-math
(the rotation depends on IEEE fp32 adds, correctly rounded division and
ties-to-even rint), with floating-point contraction off and packed-fp32
instruction selection disabled.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libtwl.so")
# microbenchmark kernels for the measured peaks bench.py reports (not part of
# the library's C ABI)
PEAKS_SRC = "peaks.hip"
PEAKS_LIB_PATH = os.path.join(PKG_DIR, "libtwl_peaks.so")

SOURCES = ["rotate_quant.hip", "pack.hip", "gemm_i8.hip", "gemv.hip", "reference_bf16.hip", "api.cpp"]

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-ffp-contract=off",
    # keep MFMA accumulators in arch VGPRs: the AGPR form makes LLVM reshuffle
    # loop-carried accumulators with v_accvgpr copies every iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-Wno-inline-asm",  # the GEMM names M0 as clobbered on purpose (see gemm_i8.hip)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines()
                    if "unknown target feature" not in ln and "packed-fp32-ops" not in ln
                    and ln.strip())
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if verbose and out:
        print(out)
    return obj


def _link(objs, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(path)} failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, path)


def build(jobs: int = 0, verbose: bool = False) -> str:
    """Compile every source, link libtwl.so (and the peaks microbenchmark
    library libtwl_peaks.so); returns the libtwl.so path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + [PEAKS_SRC]
    jobs = jobs or min(len(srcs), os.cpu_count() or 1, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB_PATH, verbose)
    _link(objs[len(SOURCES):], PEAKS_LIB_PATH, verbose)
    return LIB_PATH


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
