"""The CPU tests again, against builds of the host code and of the oracle
under AddressSanitizer and UndefinedBehaviorSanitizer.

The planner's shape, stride and overflow arithmetic and the C entry points
(rope_plan.cpp, rope_abi.cpp) and the oracle (rope_oracle.c) are compiled
with -fsanitize=address,undefined and no recovery; the kernels' objects are
the ordinary build's (device code is not instrumented, and no GPU is used:
the CPU tests call the *_check entry points, the validation in front of
every launch, and the oracle). The child process preloads the ASan runtime
into the uninstrumented interpreter and selects the two builds with
ROPE_MI355X_LIBRARY and ROPE_ORACLE_LIBRARY. Any sanitizer report ends the
child with an error. The planted-mistake oracles of test_oracle_mutants.py
are separate builds and are not rerun here.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD_FLAG = "ROPE_SANITIZED_CHILD"

pytestmark = pytest.mark.slow


def _asan_runtime():
    path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("the ASan runtime of g++ is not installed")
    return path


def _sanitized_env(**extra):
    preload = _asan_runtime()
    if os.environ.get("LD_PRELOAD"):
        preload += " " + os.environ["LD_PRELOAD"]   # keep what is already preloaded
    return dict(os.environ, LD_PRELOAD=preload,
                ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **extra)


PLANTED = r"""
#include <stdint.h>
#include <stdlib.h>
int64_t heap_overflow(int64_t n) {          /* reads one element past the end */
    int64_t* a = (int64_t*)malloc(n * sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) a[i] = i;
    int64_t v = a[n];
    free(a);
    return v;
}
int64_t shape_product(int64_t a, int64_t b) { return a * b; }   /* signed overflow */
"""


@pytest.mark.skipif(os.environ.get(CHILD_FLAG) == "1", reason="already the sanitized run")
@pytest.mark.parametrize("call, report", [("heap_overflow(4)", "AddressSanitizer: heap-buffer-overflow"),
                                          ("shape_product(1 << 40, 1 << 40)", "runtime error: signed integer overflow")])
def test_planted_errors_are_reported(tmp_path, call, report):
    """The same flags and runtime set-up report a planted out-of-bounds read
    and a planted signed overflow (the set-up is live, not silently off)."""
    from rotary_position_embedding_amd import build as product_build
    src = tmp_path / "planted.c"
    src.write_text(PLANTED)
    lib = tmp_path / "libplanted.so"
    subprocess.run(["gcc", "-O1", "-g", "-fPIC", "-shared"] + product_build.SANITIZE_FLAGS +
                   [str(src), "-o", str(lib)], check=True)
    name, args = call.split("(", 1)
    code = ("import ctypes; l = ctypes.CDLL(%r); f = l.%s; f.restype = ctypes.c_int64; "
            "f.argtypes = [ctypes.c_int64] * %d; print(f(%s))" % (str(lib), name, args.count(",") + 1, args[:-1]))
    r = subprocess.run([sys.executable, "-c", code], env=_sanitized_env(), capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0 and report in r.stderr, (r.returncode, r.stderr[-2000:])


@pytest.mark.skipif(os.environ.get(CHILD_FLAG) == "1", reason="already the sanitized run")
def test_cpu_suite_under_asan_and_ubsan():
    from oracle import build as oracle_build
    from rotary_position_embedding_amd import build as product_build
    lib = product_build.build_sanitized()
    olib = oracle_build.build_sanitized()
    env = _sanitized_env(ROPE_MI355X_LIBRARY=lib, ROPE_ORACLE_LIBRARY=olib, **{CHILD_FLAG: "1"})
    cmd = [sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           "--ignore=tests/test_oracle_mutants.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    out = r.stdout + r.stderr
    tail = "\n".join(out.splitlines()[-40:])
    assert r.returncode == 0, "sanitized CPU suite failed (rc %d):\n%s" % (r.returncode, tail)
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in out, "sanitizer report:\n%s" % tail
    # the child really ran against the sanitized builds
    assert " passed" in out, tail
    print(out.splitlines()[-1], flush=True)


@pytest.mark.skipif(os.environ.get(CHILD_FLAG) != "1", reason="runs in the sanitized child only")
def test_child_uses_the_sanitized_builds():
    """In the child, both libraries are the instrumented builds."""
    import oracle
    from rotary_position_embedding_amd import _lib
    assert _lib.LIB_PATH == os.path.abspath(os.environ["ROPE_MI355X_LIBRARY"])
    assert oracle.LIB_PATH == os.path.abspath(os.environ["ROPE_ORACLE_LIBRARY"])
    for path in (_lib.LIB_PATH, oracle.LIB_PATH):
        syms = subprocess.run(["nm", "-D", path], capture_output=True, text=True, check=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, path
    _lib.load()
    oracle.default()
