"""Build libcsa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcsa.so")
BENCH_LIB = os.path.join(PKG, "libcsa_bench.so")  # measurement helper of bench.py only
SOURCES = ["api.cpp", "scorer.hip", "scorer_fp8.hip", "topk.hip", "attention.hip", "compressor.hip", "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _flags(extra_flags):
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # keep the compiler from emitting packed fp32 arithmetic
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}", *extra_flags]


def _quiet(text):
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def build_library(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source to an object (in parallel), then link libcsa.so."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *_flags(extra_flags), "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        return src, obj, " ".join(cmd), res.returncode, _quiet(res.stdout)

    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for src, obj, cmd, rc, out in results:
        if verbose:
            print(cmd, flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[r[1] for r in results], "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{_quiet(res.stdout)}")
    os.replace(tmp, LIB)
    # the benchmark's measurement helper (streaming-read kernel), a library of its own
    tmp = BENCH_LIB + ".tmp"
    cmd = [cc, *_flags(extra_flags), "-shared", os.path.join(CSRC, "bench_probe.hip"), "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on bench_probe.hip ({res.returncode}):\n{_quiet(res.stdout)}")
    os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
