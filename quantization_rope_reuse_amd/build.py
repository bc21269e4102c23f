"""Build libhkv.so (HIP, gfx950) in place, next to this file.

    python -m quantization_rope_reuse_amd.build

Each source is compiled to an object under _build/ in parallel, then linked
into one shared library.  Flags: -O3 without any fast-math option, so fp32
division and square root stay correctly rounded and denormals are kept; the
packed-fp32 feature is disabled for the device code.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhkv.so")
SOURCES = ("api.hip", "quant.hip", "fetch.hip", "crc.hip", "order.hip", "streams.hip",
           "select.hip", "frames.hip", "probe.hip", "noalloc.hip",
           "staged.hip")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        jobs.append([cc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_test_kernels(verbose: bool = False) -> list:
    """Test-only HIP libraries under tests/hip/ (each built from one source
    with the library's flags and device headers); the GPU tests load them."""
    cc = hipcc()
    out = []
    tests_hip = os.path.join(ROOT, "tests", "hip")
    for src in sorted(os.listdir(tests_hip)):
        if not src.endswith(".hip"):
            continue
        lib = os.path.join(tests_hip, "lib" + os.path.splitext(src)[0] + ".so")
        _run([cc, *compile_flags(), "-shared", os.path.join(tests_hip, src), "-o", lib + ".tmp"],
             verbose)
        os.replace(lib + ".tmp", lib)
        out.append(lib)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
