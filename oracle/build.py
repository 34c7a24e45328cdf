"""Compile the scalar CPU oracle (test infrastructure) into liboracle_rope.so.

gcc, -O2, strict IEEE: no fast-math and no multiply-add contraction, so the
arithmetic is exactly what the C source states. The SHA-256 of the sources
(rope_oracle.c, rope_oracle.h and this file) is recorded beside the library;
the loader refuses a library built from other sources.
"""
import hashlib
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_rope.so")
STAMP = LIB + ".srchash"
# the CPU tests' sanitizer variant (ASan + UBSan), selected with
# ROPE_ORACLE_LIBRARY; the arithmetic flags are the same
SANITIZED_LIB = os.path.join(os.path.dirname(HERE), "_build", "sanitize", "liboracle_rope.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined", "-g"]
SOURCES = [os.path.join(HERE, f) for f in ("rope_oracle.c", "rope_oracle.h")] + [os.path.abspath(__file__)]


def source_hash() -> str:
    h = hashlib.sha256()
    for path in SOURCES:
        h.update(os.path.basename(path).encode())
        h.update(b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()


def _stamp_of(lib):
    return STAMP if lib is None or os.path.abspath(lib) == LIB else lib + ".srchash"


def is_current(lib=None) -> bool:
    try:
        with open(_stamp_of(lib)) as f:
            recorded = f.read().strip()
    except OSError:
        return False
    return os.path.exists(lib or LIB) and recorded == source_hash()


def ensure_current(verbose: bool = False) -> str:
    if not is_current():
        build(verbose)
    return LIB


def build(verbose: bool = False, sanitize: bool = False) -> str:
    lib = SANITIZED_LIB if sanitize else LIB
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    src = os.path.join(HERE, "rope_oracle.c")
    digest = source_hash()
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", "-fno-strict-aliasing"] + \
          (SANITIZE_FLAGS if sanitize else []) + [src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    stamp = _stamp_of(lib)
    with open(stamp + ".tmp%d" % os.getpid(), "w") as f:
        f.write(digest + "\n")
    os.replace(stamp + ".tmp%d" % os.getpid(), stamp)
    return lib


def build_sanitized(verbose: bool = False) -> str:
    return build(verbose, sanitize=True)


if __name__ == "__main__":
    print(build(verbose=True))
