"""Build libpkv.so (the HIP kernels and the C ABI of include/pkv.h) in-tree
for gfx950 with hipcc.  Every source compiles to its own object in parallel,
then one shared library is linked beside this file.
"""
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = ["pkv_api.hip", "decode.hip", "varlen.hip", "cache_write.hip", "block_manager.cpp",
           "stream_read.hip", "mfma_peak.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source extra flags.  decode.hip: the atomic optimizer would rewrite the
# single-lane work-ticket atomic into a wave-wide scan that consumes the
# returned value at once, stalling on it instead of letting it arrive while
# the current unit streams.
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src):
    obj = os.path.join(CSRC, "_obj", os.path.basename(src) + ".o")
    os.makedirs(os.path.dirname(obj), exist_ok=True)
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build() -> str:
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
