"""Build libbitlinear.so (gfx950) in-tree with hipcc.

    python bitlinear_absmean_ternarise_amd/build.py

Every HIP translation unit is compiled for --offload-arch=gfx950 with packed
FP32 instructions disabled and IEEE division/rounding kept (no fast-math), then
linked into one shared library next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libbitlinear.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["api.cpp", "pack.hip", "quant.hip", "forward.hip", "gemm_pipe.hip", "gemv.hip", "flip.hip", "backward.hip", "b1.hip"]
ARCH = "gfx950"
# Kernels whose arguments are a few pointers and scalars take them preloaded
# into SGPRs at dispatch (gfx950 kernarg preloading) instead of loading them
# from memory first: the activation quant kernels, 4.45 -> 4.20 us per call
# on the 700M layer's inputs (3B decode step at 8 tokens 32.1 -> 31.0 us);
# the tracker over the 16.4M model 10.94 -> 10.69 us.  The kernels that take
# a table of grouped entries (forwards, grouped pack) cannot preload it; the
# fused decode kernel takes its segment boundaries as leading scalars so that
# at least those arrive preloaded.
PRELOAD = {"quant.hip", "flip.hip", "pack.hip", "gemv.hip"}
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj_dir: str) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    extra = ["-mllvm", "-amdgpu-kernarg-preload-count=16"] if src in PRELOAD else []
    cmd = [hipcc()] + lang + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    obj_dir = os.path.join(LIBDIR, "_obj")
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_peaks(verbose)
    return LIB


PEAKS_SRC = os.path.join(ROOT, "bench_peaks.hip")
PEAKS_LIB = os.path.join(ROOT, "libbench_peaks.so")


def build_peaks(verbose: bool = False) -> str:
    """The benchmark's peak-bandwidth / peak-MFMA probes (not part of the library)."""
    tmp = PEAKS_LIB + ".tmp"
    cmd = [hipcc(), "-x", "hip"] + FLAGS + ["-shared", PEAKS_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for bench_peaks.hip:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PEAKS_LIB)
    if verbose:
        print(f"built {PEAKS_LIB}")
    return PEAKS_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
