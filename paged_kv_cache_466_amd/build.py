"""Builds libpkv.so (HIP kernels + C ABI + host pool) for gfx950 with hipcc.

Usage: ``python paged_kv_cache_466_amd/build.py`` (or ``build()``).  The
library lands in ``paged_kv_cache_466_amd/_lib/libpkv.so``.  Every call
recompiles from source.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libpkv.so")
OBJDIR = os.path.join(ROOT, "_build", "pkv")

SOURCES = ["api.hip", "cache_ops.hip", "paged_attn.hip", "query_tile.hip", "quest.hip", "host.cpp", "pool.cpp",
           "reuse.cpp"]
# the host-only sources, also built on their own under the address and
# undefined-behaviour sanitizers (build_host_sanitized)
HOST_SOURCES = ["host.cpp", "pool.cpp", "reuse.cpp"]
SAN_LIB = os.path.join(ROOT, "_build", "san", "libpkv_host_san.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# gfx950 code: no packed-fp32 instructions (see the header of paged_attn.hip);
# MFMA results in ordinary VGPRs, so that accumulators the softmax rescales
# are not copied between accumulation and vector registers every block
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-gpu-rdc", "-munsafe-fp-atomics", "-mllvm", "-amdgpu-mfma-vgpr-form=true"]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, *COMMON, *HIP_FLAGS, "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj, err


def build(verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    shutil.move(tmp, LIB)
    return LIB


def build_host_sanitized():
    """The host-only sources as one shared library built by g++ with
    -fsanitize=address,undefined (every error fatal).  No GPU code is in it;
    tests load it in a process of their own with the sanitizer runtime
    preloaded.  Returns its path."""
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", f"-I{INCLUDE}", f"-I{CSRC}",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           *[os.path.join(CSRC, s) for s in HOST_SOURCES], "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host build failed: {' '.join(cmd)}\n{r.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
