"""Build the HIP library libint8lin.so in-tree for gfx950 (hipcc, no GPU needed),
and libi8lpeaks.so, the measurement kernels of the benchmark's --peaks mode.

    python int8_quantized_linear_rowwise_amd/build.py [--jobs N]

Run as a script (or load this file by path): importing the package itself
loads the library and fails while it is missing or out of date.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libint8lin.so")
BUILD = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "quantize.hip", "gemm_fwd.hip", "gemm_bwd.hip", "gemm_wgrad.hip"]
PEAKS_SRC = "peaks.hip"
PEAKS_OUT = os.path.join(PKG, "libi8lpeaks.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("I8L_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 4, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES + [PEAKS_SRC]))
    for out, parts in ((OUT, objs[:-1]), (PEAKS_OUT, objs[-1:])):
        tmp = out + ".tmp"
        cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *parts, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, out)
        if verbose:
            print(f"built {out}")
    return OUT


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(4, os.cpu_count() or 1))
    a = ap.parse_args()
    try:
        build(a.jobs)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
