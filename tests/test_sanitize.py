"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the CPU side:

* the CPU oracle (oracle/bitlinear_oracle.c), built with gcc and both
  sanitizers, driven through every function on ragged and degenerate
  shapes by tests/sanitize/oracle_driver.c;
* the library's host code (the C-ABI validation in api.cpp and the host-side
  launch planners of the kernel files), built with the sanitizers on the
  host pass only (-fno-gpu-sanitize: device code is never instrumented) and
  driven through every entry point's argument checks by
  tests/sanitize/abi_driver.cpp.  No kernel is launched: every call is
  rejected on the host, and the calls that pass validation run only where
  the HIP runtime reports no device (they must stop at the device check).

Builds are cached under tests/sanitize/_build/ by a hash of their sources.
"""

import hashlib
import os
import shutil
import subprocess

import pytest

from test_abi import _device_may_be_present

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(HERE, "_build")
CSRC = os.path.join(ROOT, "bitlinear_absmean_ternarise_amd", "csrc")
LIB_SOURCES = ["api.cpp", "pack.hip", "quant.hip", "forward.hip", "gemm_pipe.hip", "gemv.hip", "flip.hip",
               "backward.hip", "b1.hip"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _hash(paths, extra=""):
    h = hashlib.sha256(extra.encode())
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError(f"{' '.join(cmd)}\nexit {r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}")
    return r


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "2"
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan():
    srcs = [os.path.join(ROOT, "oracle", "bitlinear_oracle.c"), os.path.join(HERE, "oracle_driver.c")]
    exe = os.path.join(BUILD, f"oracle_driver_{_hash(srcs, ' '.join(SAN))}")
    if not os.path.exists(exe):
        os.makedirs(BUILD, exist_ok=True)
        _run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-static-libasan"] + SAN +
             srcs + ["-o", exe + ".tmp", "-lm"])
        os.replace(exe + ".tmp", exe)
    r = _run([exe], env=_env(), timeout=300)
    assert "clean" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_abi_host_code_under_asan_ubsan():
    hipcc = _hipcc()
    lib_srcs = [os.path.join(CSRC, s) for s in LIB_SOURCES]
    headers = [os.path.join(CSRC, "internal.h"), os.path.join(CSRC, "device.h"),
               os.path.join(ROOT, "include", "bitlinear.h")]
    drv = os.path.join(HERE, "abi_driver.cpp")
    flags = ["-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-gpu-sanitize",
             "-I", os.path.join(ROOT, "include")] + SAN
    exe = os.path.join(BUILD, f"abi_driver_{_hash(lib_srcs + headers + [drv], ' '.join(flags))}")
    if not os.path.exists(exe):
        odir = exe + "_obj"
        os.makedirs(odir, exist_ok=True)
        procs, objs = [], []
        for s in lib_srcs + [drv]:
            o = os.path.join(odir, os.path.basename(s) + ".o")
            objs.append(o)
            procs.append((s, subprocess.Popen([hipcc] + flags + ["-c", s, "-o", o], stdout=subprocess.PIPE,
                                              stderr=subprocess.PIPE, text=True)))
        for s, p in procs:
            out, err = p.communicate()
            assert p.returncode == 0, f"hipcc failed for {s}:\n{err[-4000:]}"
        _run([hipcc, "--offload-arch=gfx950", "-fsanitize=address,undefined", "-fno-gpu-sanitize"] + objs +
             ["-o", exe + ".tmp"])
        os.replace(exe + ".tmp", exe)
    env = _env()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"  # the HIP runtime keeps its allocations to exit
    args = [exe] + ([] if _device_may_be_present() else ["nodevice"])
    r = _run(args, env=env, timeout=300)
    assert "clean" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
