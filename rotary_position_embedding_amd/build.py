"""Build librope_mi355x.so in-tree.

Host-only sources (contracts, C entry points) are compiled with g++; the HIP
kernels with hipcc for gfx950, -O3, IEEE arithmetic (no fast-math, f32
denormals kept), packed-fp32 instruction selection disabled; hipcc links.

Beside the library, librope_mi355x.so.srchash records the SHA-256 of the
sources it was built from (csrc/, include/ and this file, which holds the
flags). The loader refuses a library whose record does not match the
sources as they are (`is_current`); `ensure_current` rebuilds it.

`build_sanitized()` (or `python -m rotary_position_embedding_amd.build
--sanitize`) builds a CPU-test variant in _build/sanitize/: the host code
(planner and C entry points) compiled by g++ with AddressSanitizer and
UndefinedBehaviorSanitizer, linked with the kernel objects of the ordinary
build (device code is not instrumented). Loaded into Python with the ASan
runtime preloaded and ROPE_MI355X_LIBRARY pointing at it, it serves the
CPU tests (validation, the *_check entry points); it is not for GPU runs.
"""
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librope_mi355x.so")
STAMP = LIB + ".srchash"
# plain streaming copies, the measuring stick bench.py sets beside the rotary
# kernels' rates (its own library: not part of the rotary C ABI)
STREAM_COPY_LIB = os.path.join(HERE, "libstream_copy.so")
STREAM_COPY_SOURCE = "stream_copy.hip"
SANITIZE_DIR = os.path.join(BUILD, "sanitize")
SANITIZED_LIB = os.path.join(SANITIZE_DIR, "librope_mi355x.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
ROCM_LIB = "/opt/rocm/lib"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HOST_SOURCES = ["rope_plan.cpp", "rope_abi.cpp"]
# the kernels of each storage type in translation units of their own (the
# vector kernel; the row, scalar and table kernels), so that they compile in
# parallel
HIP_SOURCES = ["rope_kernels.hip",
               "rope_kernels_f32.hip", "rope_kernels_f16.hip", "rope_kernels_bf16.hip",
               "rope_kernels_f32_row.hip", "rope_kernels_f16_row.hip", "rope_kernels_bf16_row.hip"]


def source_files():
    """Every file the library is built from, in a fixed order."""
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                   if f.endswith((".hip", ".hpp", ".cpp", ".h")))
    files += sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))
    files.append(os.path.abspath(__file__))
    return files


def source_hash() -> str:
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode())
        h.update(b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()


def _stamp_of(lib):
    return STAMP if lib is None or os.path.abspath(lib) == LIB else lib + ".srchash"


def built_hash(lib=None):
    """The source hash recorded when the library (default: the in-tree one)
    was built, or None."""
    try:
        with open(_stamp_of(lib)) as f:
            return f.read().strip()
    except OSError:
        return None


def is_current(lib=None) -> bool:
    if lib is None and not os.path.exists(STREAM_COPY_LIB):
        return False
    return os.path.exists(lib or LIB) and built_hash(lib) == source_hash()


def _write_stamp(lib, digest):
    stamp = _stamp_of(lib)
    with open(stamp + ".tmp%d" % os.getpid(), "w") as f:
        f.write(digest + "\n")
    os.replace(stamp + ".tmp%d" % os.getpid(), stamp)


def ensure_current(verbose: bool = False) -> str:
    """Build the library if it is missing or was built from other sources."""
    if not is_current():
        print("librope_mi355x.so is missing or older than its sources: building", file=sys.stderr, flush=True)
        build(verbose)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    digest = source_hash()  # of the sources as they are when the build starts
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE,
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)

    def hip_obj(src):
        obj = os.path.join(BUILD, src + ".o")
        _run([HIPCC, "--offload-arch=" + ARCH, "-std=c++17", "-O3", "-fPIC", "-Wall", "-ffp-contract=off",
              "-fno-gpu-flush-denormals-to-zero",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    jobs = max(1, min(len(HIP_SOURCES) + 1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        hip_objs = list(pool.map(hip_obj, HIP_SOURCES + [STREAM_COPY_SOURCE]))
    objs += hip_objs[:-1]
    tmp = STREAM_COPY_LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, hip_objs[-1]], verbose)
    os.replace(tmp, STREAM_COPY_LIB)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    _write_stamp(LIB, digest)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """The host code under ASan and UBSan, linked with the ordinary build's
    kernel objects (built first if they are not current)."""
    ensure_current(verbose)
    digest = source_hash()
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(SANITIZE_DIR, src + ".o")
        _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-Wall", "-Wextra"] + SANITIZE_FLAGS +
             ["-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    objs += [os.path.join(BUILD, src + ".o") for src in HIP_SOURCES]
    tmp = SANITIZED_LIB + ".tmp%d" % os.getpid()
    _run(["g++", "-shared"] + SANITIZE_FLAGS + ["-o", tmp] + objs +
         ["-L" + ROCM_LIB, "-lamdhip64", "-Wl,-rpath," + ROCM_LIB], verbose)
    os.replace(tmp, SANITIZED_LIB)
    _write_stamp(SANITIZED_LIB, digest)
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose=True))
    else:
        print(build(verbose=True))
