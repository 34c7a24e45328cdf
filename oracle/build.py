"""Compile the scalar CPU oracle (test infrastructure) into liboracle_rope.so.

gcc, -O2, strict IEEE: no fast-math and no multiply-add contraction, so the
arithmetic is exactly what the C source states.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_rope.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "rope_oracle.c")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", "-fno-strict-aliasing",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
