"""Build libkvq.so (HIP C++ for gfx950) in the package directory with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
# The debug build: the same sources with KVQ_DEBUG (device-resident ids, lengths and positions checked on the
# host before any launch; the KVQ_DECODE_KERNEL test hook that forces a decode kernel).
DEBUG_LIB = os.path.join(HERE, "libkvq_debug.so")
SOURCES = ["kvq_api.hip", "kvq_quantize.hip", "kvq_decode.hip", "kvq_decode_mfma.hip", "kvq_decode_rows.hip",
           "kvq_decode_kchan.hip", "kvq_decode_cascade.hip", "kvq_tiles.hip", "kvq_decode_fp8.hip"]
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libkvq")


# Per-source flags. The cascade kernel's maxima run over finite logits only: without NaNs the compiler
# drops the canonicalising moves it otherwise puts before every fmaxf of a matrix-core result.
SOURCE_FLAGS = {"kvq_decode_cascade.hip": ["-fno-honor-nans"]}


def common_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
            # packed fp32 instructions stay disabled in every kernel of this library
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False, jobs: int = 0, debug: bool = False) -> str:
    """Compile the release library (or, with debug=True, the debug library) and return its path."""
    cc = hipcc()
    bdir = os.path.join(HERE, "_build", "debug" if debug else "release")
    os.makedirs(bdir, exist_ok=True)
    lib = DEBUG_LIB if debug else LIB
    extra = ["-DKVQ_DEBUG"] if debug else []

    def compile_one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [cc] + common_flags() + SOURCE_FLAGS.get(src, []) + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")


def build_probe(verbose: bool = False) -> str:
    """The streaming-read probe the benchmark measures the decode kernels against (not part of libkvq)."""
    cc = hipcc()
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [cc] + common_flags() + ["-shared", os.path.join(CSRC, "probe", "kvq_stream_probe.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build_all(verbose: bool = False):
    return build(verbose), build(verbose, debug=True), build_probe(verbose)


if __name__ == "__main__":
    print(build_all(verbose="-v" in sys.argv))
