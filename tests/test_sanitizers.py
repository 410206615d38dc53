"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code (CPU).

Two programs under tests/sanitize/ are built with the sanitizers and run:
  oracle_driver  the fp64 oracle (oracle/pkv_oracle.c, gcc + OpenMP) over the
                 pages' examples, random small cases and every error path;
  host_driver    the host half of libpkv -- argument checks, partition choice,
                 workspace layout and launch planning (pkv_api.hip, compiled
                 for the host only, kernel launchers stubbed) and the block
                 manager (block_manager.cpp), including a multi-threaded run.
A sanitizer finding aborts the program, so the test only asks for a clean
exit and the programs' own "ok" line.  No GPU code is built or run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "paged_kv_cache_296_amd", "csrc")
INC = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
          "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "pkv_oracle.c"), os.path.join(SAN_DIR, "oracle_driver.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "oracle driver ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="ROCm compilers not installed")
def test_host_library_under_asan_ubsan(tmp_path):
    api_obj = str(tmp_path / "pkv_api.o")
    # host-only compilation of the entry points; each sanitizer flag applies
    # to the host pass only
    _run([HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-I", INC, "-I", CSRC,
          "-c", os.path.join(CSRC, "pkv_api.hip"), "-o", api_obj])
    exe = str(tmp_path / "host_driver")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", INC, "-I", CSRC,
          os.path.join(SAN_DIR, "host_driver.cpp"), os.path.join(CSRC, "block_manager.cpp"),
          api_obj, "-lpthread", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "host driver ok" in r.stdout
