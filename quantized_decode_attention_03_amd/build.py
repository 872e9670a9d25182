"""Build libkvq.so in-tree with hipcc for gfx950.

    python -m quantized_decode_attention_03_amd.build [--incremental]

Every source is compiled to an object in `_build/` in parallel, then linked
into `quantized_decode_attention_03_amd/libkvq.so`.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvq.so")

SOURCES = ["kvq_host.cpp", "kvq_append.hip", "kvq_decode.hip", "kvq_measure.hip"]

# The decode kernel's work-sharing fetch is one lane's atomic whose result is
# read a whole page group later; the compiler's atomic rewrite (a wave
# reduction around the atomic) would read it at once and stall on it.
SOURCE_FLAGS = {"kvq_decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}

# Packed FP32 instructions stay off in all device code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libkvq")
    return path


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = ([hipcc()] + HIP_FLAGS + SOURCE_FLAGS.get(src, []) +
           ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stderr}")
    return obj


def _stale(src):
    """Whether src's object is older than src or any header (for --incremental)."""
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    deps += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    return max(os.path.getmtime(p) for p in deps) > os.path.getmtime(obj)


def build(verbose=True, incremental=False):
    """Compile every source (or, with incremental=True, only those whose object is out of date) and link."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    todo = [s for s in SOURCES if not incremental or _stale(s)]
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libkvq.so failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv[1:])
    sys.exit(0)
