"""The CPU oracle and the C ABI's host side under AddressSanitizer and
UndefinedBehaviorSanitizer.

Two small drivers (tests/sanitize/) are built with the sanitizers and run:
one calls every oracle entry point on small inputs with the degenerate cases
and its argument checks, the other calls every ABI entry point's checks and
workspace sizing over valid and invalid shapes (nothing reaches a launch).
Any heap overrun, use after free, leak, signed overflow or other undefined
behaviour on those paths ends the driver with a report and fails the test.
Only host code is instrumented: the HIP sources are compiled with each
sanitizer flag behind -Xarch_host, so their device code is built as usual.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE = os.path.join(ROOT, "oracle")
CSRC = os.path.join(ROOT, "compressed_sparse_attention_indexer_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = ["api.cpp", "scorer.hip", "scorer_fp8.hip", "topk.hip", "attention.hip", "compressor.hip", "noalloc.hip"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)} -> {r.returncode}\n{r.stdout[-6000:]}"
    return r.stdout


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", f"-I{ORACLE}",
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ORACLE, "oracle.c"),
          os.path.join(ORACLE, "compressor.c"), "-o", exe, "-lm"])
    out = _run([exe], env=ENV, timeout=300)
    assert out.strip().endswith("ok")


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    clang = "/opt/rocm/llvm/bin/clang++"
    flags = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", f"-I{INCLUDE}", f"-I{CSRC}", *HOST_SAN]
    jobs = [(os.path.join(CSRC, s), str(tmp_path / (os.path.splitext(s)[0] + ".o"))) for s in SOURCES]
    jobs.append((os.path.join(SAN, "abi_driver.cpp"), str(tmp_path / "abi_driver.o")))
    with ThreadPoolExecutor(8) as ex:
        list(ex.map(lambda j: _run([hipcc, *flags, "-c", j[0], "-o", j[1]]), jobs))
    exe = str(tmp_path / "abi_driver")
    _run([clang, "-fsanitize=address,undefined", *[o for _, o in jobs], "-o", exe, "-L/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    out = _run([exe], env=ENV, timeout=300)
    assert out.strip().endswith("ok")
