"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and its validation (the *_check entry points, which never touch the
GPU) enforces each clause of the ops' contracts."""
import ctypes
import os
import re
import subprocess

import pytest

import rotary_position_embedding_amd as rpe
from rotary_position_embedding_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rope_mi355x.h")

F32, F16, BF16, I64 = 1, 10, 16, 7
OK, NULL, DTYPE, RANK, SHAPE, ATTR, UNSUP, ALIAS = 0, -1, -2, -3, -4, -5, -6, -7


def header_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_parses():
    fns = header_functions()
    for name in ("rope_apply", "mrope_apply", "rope_apply_qk", "rope_inv_freq",
                 "rope_cos_sin_cache", "rope_status_string", "rope_last_error"):
        assert name in fns


def test_library_exports_every_declared_function():
    lib = _lib.load()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)
        assert name in _lib.SIGNATURES, "binding lacks %s" % name


def test_library_matches_its_sources():
    """The build records a hash of its sources beside the library; the tree
    under test is the build of the sources in it."""
    from rotary_position_embedding_amd import build
    assert build.is_current(), (build.built_hash(), build.source_hash())
    assert len(build.built_hash()) == 64


def test_stale_library_is_refused(monkeypatch):
    """A library whose recorded source hash differs from the sources is not
    loaded: the loader raises instead of running an older build."""
    from rotary_position_embedding_amd import build
    monkeypatch.setattr(build, "source_hash", lambda: "0" * 64)   # the sources moved on
    assert not build.is_current() and not build.is_current(_lib.LIB_PATH)
    monkeypatch.setattr(_lib, "_lib", None)       # as in a fresh process
    with pytest.raises(ImportError, match="other sources"):
        _lib.load()


def test_library_without_record_is_refused(tmp_path, monkeypatch):
    """A copy of the library with no recorded source hash beside it."""
    import shutil
    copy = tmp_path / "librope_mi355x.so"
    shutil.copyfile(_lib.LIB_PATH, copy)
    monkeypatch.setattr(_lib, "LIB_PATH", str(copy))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError, match="other sources"):
        _lib.load()


def test_source_edit_changes_the_hash(tmp_path, monkeypatch):
    """Any edit to a source file changes the hash, so the recorded one no
    longer matches and the suite's set-up rebuilds."""
    from rotary_position_embedding_amd import build
    extra = tmp_path / "extra.hpp"
    extra.write_text("// a\n")
    files = build.source_files() + [str(extra)]
    monkeypatch.setattr(build, "source_files", lambda: files)
    h1 = build.source_hash()
    extra.write_text("// b\n")
    assert build.source_hash() != h1
    assert not build.is_current()


def test_oracle_library_matches_its_sources():
    from oracle import build as oracle_build
    assert oracle_build.is_current()


def test_status_strings():
    lib = _lib.load()
    for code, name in _lib.STATUS.items():
        assert lib.rope_status_string(code).decode() == name
    assert lib.rope_status_string(-99).decode() == "ROPE_ERR_UNKNOWN"


# ---------------------------------------------------------------------------
# descriptors over fake, aligned, non-overlapping device addresses: validation
# never dereferences them.

class Alloc:
    def __init__(self):
        self.next = 1 << 32

    def __call__(self, dtype, shape, align=256):
        nbytes = {F32: 4, F16: 2, BF16: 2, I64: 8}.get(dtype, 4)
        for d in shape:
            nbytes *= d
        addr = self.next
        self.next += (nbytes + 2 * align) // align * align
        return rpe.tensor_spec(addr, dtype, shape)


def rope_case(rank=3, dt=F16, B=2, S=5, H=4, D=16, R=0, ids=True, M=16, interleaved=0,
              num_heads=None, **over):
    a = Alloc()
    Rf = R or D
    x = a(dt, (B, S, H * D) if rank == 3 else (B, H, S, D))
    y = a(dt, tuple(x.shape[:rank]))
    if ids:
        cos = a(dt, (M, Rf // 2))
        sin = a(dt, (M, Rf // 2))
        pid = a(I64, (B, S))
    else:
        cos = a(dt, (B, S, Rf // 2))
        sin = a(dt, (B, S, Rf // 2))
        pid = None
    kw = dict(x=x, cos_cache=cos, sin_cache=sin, position_ids=pid, y=y, interleaved=interleaved,
              num_heads=(H if rank == 3 else 0) if num_heads is None else num_heads,
              rotary_embedding_dim=R)
    kw.update(over)
    return kw


def with_policy(policy, fn, *args):
    old = rpe.set_kernel_policy(policy)
    try:
        return fn(*args)
    finally:
        rpe.set_kernel_policy(old)


def check_rope(kw):
    return rpe.rope_apply_check(kw["x"], kw["cos_cache"], kw["sin_cache"], kw["position_ids"],
                                kw["y"], interleaved=kw["interleaved"], num_heads=kw["num_heads"],
                                rotary_embedding_dim=kw["rotary_embedding_dim"])


def reshape(t, shape, dtype=None):
    return rpe.tensor_spec(t.data, dtype if dtype is not None else t.dtype, shape)


@pytest.mark.parametrize("rank,ids", [(3, True), (4, True), (3, False), (4, False)])
@pytest.mark.parametrize("dt", [F16, F32, BF16])
def test_rope_variants_accepted(rank, ids, dt):
    """One positive case per manifest variant (rank3/rank4 x cache2+ids / cache3)."""
    rc, variant = check_rope(rope_case(rank=rank, ids=ids, dt=dt))
    assert rc == OK, _lib.load().rope_last_error()
    # a decode-sized launch: the row kernel; with policy 2 the vector kernel
    kind = "/gather" if ids else "/per_token"
    assert variant == "row16" + kind
    assert with_policy(2, check_rope, rope_case(rank=rank, ids=ids, dt=dt)) == (OK, "vec16" + kind)


def test_rope_partial_interleaved_accepted():
    for il in (0, 1):
        rc, v = check_rope(rope_case(rank=4, dt=F32, D=96, R=64, interleaved=il))
        assert rc == OK and v == "row16/gather"        # 384-byte rows: the row kernel's general rows
        assert with_policy(2, check_rope, rope_case(rank=4, dt=F32, D=96, R=64, interleaved=il)) == (
            OK, "vec16/gather")


def test_rope_scalar_path_for_unaligned_shapes():
    rc, v = check_rope(rope_case(D=6))       # 6 halves: no 16-byte items
    assert rc == OK and v == "scalar/gather"
    kw = rope_case()
    kw["x"] = reshape(kw["x"], tuple(kw["x"].shape[:3]))
    kw["x"].data += 2                      # misaligned x
    rc, v = check_rope(kw)
    assert rc == OK and v == "scalar/gather"


def test_kernel_policy_forces_scalar():
    old = rpe.set_kernel_policy(1)
    try:
        rc, v = check_rope(rope_case())
        assert rc == OK and v == "scalar/gather"
    finally:
        rpe.set_kernel_policy(old)
    rc, v = check_rope(rope_case())
    assert v == "row16/gather"
    assert with_policy(2, check_rope, rope_case()) == (OK, "vec16/gather")
    assert with_policy(3, check_rope, rope_case()) == (OK, "row16/gather")
    assert rpe.set_kernel_policy(7) == 0 and rpe.set_kernel_policy(0) == 0  # out of range: automatic


def test_row_kernel_selection_rules():
    """The row kernel: decode-sized launches (<= 6 MiB of activations read,
    <= 4 MiB for M-RoPE), head rows of 16-byte chunks from 32 B to 1 KiB (rows
    of other than a power-of-two size, or split-half partners other than a
    power of two of lanes apart, not with QK-norm or M-RoPE). Policy 3 lifts
    the size rule."""
    big = dict(B=1, S=8192, H=32, D=128)                        # 64 MiB of fp16 X
    assert check_rope(rope_case(**big)) == (OK, "vec16/gather")
    assert with_policy(3, check_rope, rope_case(**big)) == (OK, "row16/gather")
    assert check_rope(rope_case(B=1, S=768, H=32, D=128)) == (OK, "row16/gather")    # 6 MiB
    assert check_rope(rope_case(B=1, S=769, H=32, D=128)) == (OK, "vec16/gather")
    m = dict(rank=4, B=1, H=32, D=128, M=64, section=(16, 24, 24))
    assert check_mrope(mrope_case(S=512, **m)) == (OK, "row16/mrope")               # 4 MiB
    assert check_mrope(mrope_case(S=513, **m)) == (OK, "vec16/mrope")
    assert check_rope(rope_case(D=96)) == (OK, "row16/gather")            # 192-byte rows
    assert check_rope(rope_case(D=128, R=96)) == (OK, "row16/gather")     # partners 6 lanes apart
    assert check_mrope(mrope_case(S=4, rank=4, B=1, H=4, D=96, M=64, section=(16, 16, 16))) == (
        OK, "vec16/mrope")                                                # no M-RoPE on general rows
    assert check_rope(rope_case(D=128, R=96, interleaved=1)) == (OK, "row16/gather")
    assert check_rope(rope_case(D=1024)) == (OK, "vec16/gather")          # 2 KiB rows
    assert check_rope(rope_case(D=8, dt=F16, interleaved=1)) == (OK, "vec16/gather")  # 16-byte rows
    assert check_rope(rope_case(D=8, dt=F32)) == (OK, "row16/gather")     # 32-byte rows
    assert check_rope(rope_case(D=64, dt=F32, R=32)) == (OK, "row16/gather")  # partial, 4 lanes apart


def test_row_kernel_at_prefill_sizes():
    """Above 6 MiB the row kernel still takes 2-byte launches whose rows the
    vector kernel's items fit poorly (a token's head rows filling at least
    1 KiB): with the rows adjacent, rows of other than a power-of-two size,
    interleaved pairs, split halves under 128 bytes, Q+K and the cache
    append; with the rows apart (rank 4), power-of-two rows with interleaved
    pairs or short halves; float32 rows of other sizes or partial split
    rotations; QK-norm in float32 or with halves other than 128 bytes. The
    vector kernel keeps the others."""
    big = dict(B=1, S=8192, H=32, D=128)
    assert check_rope(rope_case(**big)) == (OK, "vec16/gather")                         # halves of 128 B
    assert check_rope(rope_case(interleaved=1, **big)) == (OK, "row16/gather")
    assert check_rope(rope_case(dt=BF16, interleaved=1, **big)) == (OK, "row16/gather")
    assert check_rope(rope_case(R=64, **big)) == (OK, "row16/gather")                    # halves of 64 B
    assert check_rope(rope_case(B=1, S=8192, H=64, D=64)) == (OK, "row16/gather")
    assert check_rope(rope_case(ids=False, interleaved=1, **big)) == (OK, "row16/per_token")
    assert check_rope(rope_case(B=1, S=8192, H=16, D=256)) == (OK, "vec16/gather")       # halves of 256 B
    assert check_rope(rope_case(dt=F32, interleaved=1, **big)) == (OK, "vec16/gather")   # 4-byte type
    assert check_rope(rope_case(rank=4, **big)) == (OK, "vec16/gather")                 # rank 4: halves of 128 B
    assert check_rope(rope_case(rank=4, interleaved=1, **big)) == (OK, "row16/gather")   # rank 4, pow2 rows
    assert check_rope(rope_case(rank=4, B=8, S=1024, H=32, D=64)) == (OK, "row16/gather")
    assert check_rope(rope_case(rank=4, B=8, S=1024, H=32, D=96, R=64, interleaved=1)) == (
        OK, "vec16/gather")                                                              # rank 4, 192-byte rows
    assert check_rope(rope_case(B=1, S=1 << 16, H=2, D=64, interleaved=1)) == (OK, "vec16/gather")  # 256 B a token
    assert check_rope(rope_case(B=1, S=8192, H=32, D=96)) == (OK, "row16/gather")        # 192-byte rows
    assert check_rope(rope_case(B=1, S=8192, H=16, D=192)) == (OK, "row16/gather")       # 384-byte rows
    assert check_rope(rope_case(B=1, S=8192, H=8, D=320)) == (OK, "row16/gather")        # 40 of 64 lanes busy
    assert check_rope(rope_case(B=1, S=8192, H=32, D=96, dt=F32)) == (OK, "row16/gather")  # float32
    assert check_rope(rope_case(dt=F32, **big)) == (OK, "vec16/gather")
    assert check_rope(rope_case(dt=F32, R=64, **big)) == (OK, "row16/gather")           # partial rotation
    assert check_rope(rope_case(dt=F32, R=64, interleaved=1, **big)) == (OK, "vec16/gather")
    qk = dict(B=1, S=8192, H=32, Hk=8, M=8192)
    assert check_qk(qk_case(D=128, **qk)) == (OK, "row16/gather")
    assert check_qk(qk_case(D=128, table=False, **qk)) == (OK, "row16/on_the_fly")
    assert check_qk(qk_case(D=128, dt=F32, **qk)) == (OK, "vec16/gather")
    assert check_qk(qk_case(D=128, dt=F32, table=False, **qk)) == (OK, "row16/on_the_fly")
    assert check_norm(norm_case(shape=qk)) == (OK, "vec16/norm/gather")
    assert check_norm(norm_case(D=256, shape=qk)) == (OK, "row16/norm/gather")          # halves of 256 B
    assert check_norm(norm_case(D=64, shape=qk)) == (OK, "row16/norm/gather")           # halves of 64 B
    assert check_norm(norm_case(dt=F32, shape=qk)) == (OK, "row16/norm/gather")
    assert check_packed(packed_case(D=128, **qk)) == (OK, "vec16/gather")
    assert check_kv(kv_case(B=4, S=2048, Smax=4096, total=2048, H=32, Hk=8, D=128, M=8192)) == (OK, "row16/append")
    m = dict(rank=4, B=1, H=32, D=128, M=64, section=(16, 24, 24))
    assert check_mrope(mrope_case(S=8192, **m)) == (OK, "vec16/mrope")


def test_huge_launches_take_the_scalar_kernel():
    """The vector and row kernels index in 32 bits: 2^31 tokens or more go to
    the grid-stride scalar kernel (no memory is touched by a check)."""
    assert check_rope(rope_case(B=1, S=(1 << 31) - 8, H=1, D=16)) == (OK, "vec16/gather")
    assert check_rope(rope_case(B=1, S=1 << 31, H=1, D=16)) == (OK, "scalar/gather")
    assert check_rope(rope_case(B=2, S=1 << 30, H=1, D=16)) == (OK, "scalar/gather")


# Each clause of the manifest's contracts, negated -> its status.
def _neg_cases():
    cases = []

    def add(name, code, **kw):
        cases.append((name, code, kw))

    add("x_missing", NULL, x=None)
    add("cos_missing", NULL, cos_cache=None)
    add("sin_missing", NULL, sin_cache=None)
    add("y_missing", NULL, y=None)
    add("interleaved_2", ATTR, interleaved=2)
    add("interleaved_neg", ATTR, interleaved=-1)
    add("num_heads_negative", ATTR, num_heads=-1)
    add("rank3_without_num_heads", ATTR, num_heads=0)
    add("rotary_dim_negative", ATTR, rotary_embedding_dim=-2)
    add("rotary_dim_odd", ATTR, rotary_embedding_dim=3)
    return cases


@pytest.mark.parametrize("name,code,over", _neg_cases(), ids=[c[0] for c in _neg_cases()])
def test_rope_attribute_clauses(name, code, over):
    kw = rope_case()
    kw.update(over)
    rc, _ = check_rope(kw)
    assert rc == code, (name, rc, _lib.load().rope_last_error())


def test_rope_shape_clauses():
    lib = _lib.load()

    def expect(kw, code, what):
        rc, _ = check_rope(kw)
        assert rc == code, (what, rc, lib.rope_last_error())

    # dtype clauses
    kw = rope_case(); kw["x"] = reshape(kw["x"], tuple(kw["x"].shape[:3]), BF16)
    expect(kw, DTYPE, "x bf16 with f16 tables")
    kw = rope_case(dt=BF16); kw["x"] = reshape(kw["x"], tuple(kw["x"].shape[:3]), 11)  # double
    kw["y"] = reshape(kw["y"], tuple(kw["y"].shape[:3]), 11)
    expect(kw, DTYPE, "binary64 storage")
    kw = rope_case(); kw["cos_cache"] = reshape(kw["cos_cache"], (16, 8), F32)
    expect(kw, DTYPE, "cos dtype")
    kw = rope_case(); kw["y"] = reshape(kw["y"], (2, 5, 64), F32)
    expect(kw, DTYPE, "y dtype")
    kw = rope_case(); kw["position_ids"] = reshape(kw["position_ids"], (2, 5), F32)
    expect(kw, DTYPE, "ids dtype")
    # rank clauses
    kw = rope_case(); kw["x"] = reshape(kw["x"], (10, 64))
    expect(kw, RANK, "x rank 2")
    kw = rope_case(); kw["cos_cache"] = reshape(kw["cos_cache"], (1, 16, 8)); kw["sin_cache"] = reshape(kw["sin_cache"], (1, 16, 8))
    expect(kw, RANK, "3-D cache with ids")
    kw = rope_case(ids=False); kw["cos_cache"] = reshape(kw["cos_cache"], (10, 8)); kw["sin_cache"] = reshape(kw["sin_cache"], (10, 8))
    expect(kw, RANK, "2-D cache without ids")
    kw = rope_case(); kw["position_ids"] = reshape(kw["position_ids"], (10,))
    expect(kw, RANK, "ids rank 1")
    # shape clauses
    kw = rope_case(); kw["y"] = reshape(kw["y"], (2, 5, 32))
    expect(kw, SHAPE, "y shape")
    expect(rope_case(num_heads=3), SHAPE, "hidden % num_heads")
    expect(rope_case(D=6, H=4, num_heads=8), SHAPE, "odd head size via num_heads")       # 24/8 = 3
    expect(rope_case(rank=4, num_heads=3), SHAPE, "rank-4 num_heads disagrees")
    expect(rope_case(rotary_embedding_dim=18), SHAPE, "rotary dim > head size")
    kw = rope_case(); kw["cos_cache"] = reshape(kw["cos_cache"], (16, 7)); kw["sin_cache"] = reshape(kw["sin_cache"], (16, 7))
    expect(kw, SHAPE, "cache width")
    kw = rope_case(); kw["sin_cache"] = reshape(kw["sin_cache"], (15, 8))
    expect(kw, SHAPE, "sin shape != cos shape")
    kw = rope_case(); kw["position_ids"] = reshape(kw["position_ids"], (2, 4))
    expect(kw, SHAPE, "ids (B,S)")
    kw = rope_case(ids=False); kw["cos_cache"] = reshape(kw["cos_cache"], (2, 4, 8)); kw["sin_cache"] = reshape(kw["sin_cache"], (2, 4, 8))
    expect(kw, SHAPE, "3-D cache (B,S)")
    kw = rope_case(rank=4, D=7); expect(kw, SHAPE, "rank-4 odd head size")
    # NULL data of a non-empty tensor
    kw = rope_case(); kw["x"] = reshape(kw["x"], (2, 5, 64)); kw["x"].data = None
    expect(kw, NULL, "x data NULL")
    # negative dimension
    kw = rope_case(); kw["x"] = reshape(kw["x"], (2, -5, 64))
    expect(kw, SHAPE, "negative dim")


def test_rope_alias_clauses():
    kw = rope_case()
    kw["y"] = reshape(kw["x"], (2, 5, 64))          # exactly x: in place, allowed
    assert check_rope(kw)[0] == OK
    kw = rope_case()
    y = reshape(kw["x"], (2, 5, 64)); y.data += 16   # shifted: partial overlap
    kw["y"] = y
    assert check_rope(kw)[0] == ALIAS
    kw = rope_case()
    kw["y"] = reshape(kw["y"], (2, 5, 64)); kw["y"].data = kw["cos_cache"].data
    assert check_rope(kw)[0] == ALIAS
    kw = rope_case()
    kw["y"] = reshape(kw["y"], (2, 5, 64)); kw["y"].data = kw["position_ids"].data
    assert check_rope(kw)[0] == ALIAS


def test_rope_empty_tensors_accepted():
    for B, S in ((0, 5), (2, 0)):
        kw = rope_case(B=B, S=S)
        assert check_rope(kw)[0] == OK
    kw = rope_case(rank=4, H=0, num_heads=0)
    assert check_rope(kw)[0] == OK
    kw = rope_case(M=0)          # empty table: every id out of range, still valid
    kw["cos_cache"].data = None
    kw["sin_cache"].data = None
    assert check_rope(kw)[0] == OK


# ---------------------------------------------------------------------------
# MRotaryEmbedding README: Inputs and Attributes

def mrope_case(rank=4, dt=F16, B=2, S=5, H=3, D=16, R=0, M=20, section=(4, 2, 2), **over):
    a = Alloc()
    Rf = R or D
    x = a(dt, (B, S, H * D) if rank == 3 else (B, H, S, D))
    kw = dict(x=x, position_ids=a(I64, (3, B, S)), cos_cache=a(dt, (M, Rf // 2)),
              sin_cache=a(dt, (M, Rf // 2)), y=a(dt, tuple(x.shape[:rank])),
              mrope_section=section, interleaved=0, is_packed_batching=0, mrope_layout=0,
              num_heads=H if (rank == 3 or R) else 0, rotary_embedding_dim=R, scale=1.0)
    kw.update(over)
    return kw


def check_mrope(kw):
    kw = dict(kw)
    args = [kw.pop(k) for k in ("x", "position_ids", "cos_cache", "sin_cache", "y")]
    return rpe.mrope_apply_check(*args, **kw)


def test_huge_dimension_beside_a_zero_one():
    """A zero dimension admits any other dimension (the element count stays
    0): table widths far beyond any rotary dim are still shape errors."""
    lib = _lib.load()
    huge = 2 ** 62
    kw = rope_case()
    kw["cos_cache"] = reshape(kw["cos_cache"], (0, huge))
    kw["sin_cache"] = reshape(kw["sin_cache"], (0, huge))
    assert check_rope(kw)[0] == SHAPE, lib.rope_last_error()
    kw = rope_case(ids=False, B=0)
    kw["cos_cache"] = reshape(kw["cos_cache"], (0, 5, huge))
    kw["sin_cache"] = reshape(kw["sin_cache"], (0, 5, huge))
    assert check_rope(kw)[0] == SHAPE, lib.rope_last_error()
    kw = mrope_case()
    kw["cos_cache"] = reshape(kw["cos_cache"], (0, huge))
    kw["sin_cache"] = reshape(kw["sin_cache"], (0, huge))
    assert check_mrope(kw)[0] == SHAPE, lib.rope_last_error()


def test_head_counts_whose_packed_sum_overflows():
    """Packed layouts hold num_heads + 2 * kv_num_heads heads per token: head
    counts above 2^31 - 1 are attribute errors, not an overflowing sum."""
    lib = _lib.load()
    big = 2 ** 62
    assert check_packed(packed_case(num_heads=big, kv_num_heads=big))[0] == ATTR, lib.rope_last_error()
    assert check_kv(kv_case(num_heads=big, kv_num_heads=big))[0] == ATTR, lib.rope_last_error()
    assert check_kv(kv_case(packed=True, num_heads=big, kv_num_heads=big))[0] == ATTR, lib.rope_last_error()
    # the largest accepted count still plans (a rank-3 width of zero heads)
    kw = packed_case(B=0, num_heads=2 ** 31 - 1, kv_num_heads=1)
    kw["qkv"] = reshape(kw["qkv"], (0, 3, 0))
    kw["y"] = reshape(kw["y"], (0, 3, 0))
    assert check_packed(kw)[0] != ATTR, lib.rope_last_error()
    # a cache-append table width far beyond the head size, beside zero rows
    kw = kv_case()
    kw["cos_cache"] = reshape(kw["cos_cache"], (0, 2 ** 62))
    kw["sin_cache"] = reshape(kw["sin_cache"], (0, 2 ** 62))
    assert check_kv(kw)[0] == SHAPE, lib.rope_last_error()


def test_head_size_and_head_count_limits():
    """Head sizes and head counts reach the kernels as 32-bit values: above
    2^31 - 1 they are refused before any launch (legal shapes of a few GiB)."""
    lib = _lib.load()
    a = Alloc()
    x = a(F16, (1, 2 ** 31, 1, 2))  # 2^31 heads of 2 (8 GiB)
    kw = dict(x=x, cos_cache=a(F16, (4, 1)), sin_cache=a(F16, (4, 1)), position_ids=a(I64, (1, 1)),
              y=a(F16, (1, 2 ** 31, 1, 2)), interleaved=0, num_heads=0, rotary_embedding_dim=0)
    assert check_rope(kw)[0] == UNSUP, lib.rope_last_error()
    kw["x"] = a(F16, (1, 1, 2 ** 33)); kw["y"] = a(F16, (1, 1, 2 ** 33)); kw["num_heads"] = 2 ** 32
    assert check_rope(kw)[0] == UNSUP, lib.rope_last_error()
    D = 2 ** 31 + 2  # one head of 2^31 + 2 elements (4 GiB)
    kw = dict(x=a(F16, (1, 1, 1, D)), cos_cache=a(F16, (4, D // 2)), sin_cache=a(F16, (4, D // 2)),
              position_ids=a(I64, (1, 1)), y=a(F16, (1, 1, 1, D)), interleaved=0, num_heads=0,
              rotary_embedding_dim=0)
    assert check_rope(kw)[0] == UNSUP, lib.rope_last_error()
    kw["rotary_embedding_dim"] = 2; kw["cos_cache"] = a(F16, (4, 1)); kw["sin_cache"] = a(F16, (4, 1))
    assert check_rope(kw)[0] == UNSUP, lib.rope_last_error()
    # just below the limits: accepted
    x = a(F16, (1, 2 ** 31 - 1, 1, 2))
    kw = dict(x=x, cos_cache=a(F16, (4, 1)), sin_cache=a(F16, (4, 1)), position_ids=a(I64, (1, 1)),
              y=a(F16, (1, 2 ** 31 - 1, 1, 2)), interleaved=0, num_heads=0, rotary_embedding_dim=0)
    assert check_rope(kw)[0] == OK, lib.rope_last_error()


def test_mrope_accepted():
    for rank in (3, 4):
        for layout in (0, 1):
            for dt in (F16, F32):
                rc, v = check_mrope(mrope_case(rank=rank, mrope_layout=layout, dt=dt))
                assert rc == OK and v == "row16/mrope", _lib.load().rope_last_error()
                kw = mrope_case(rank=rank, mrope_layout=layout, dt=dt)
                assert with_policy(2, check_mrope, kw) == (OK, "vec16/mrope")
    # odd head size with a smaller even rotary dim: allowed, scalar kernel
    rc, v = check_mrope(mrope_case(D=9, R=8, section=(2, 1, 1)))
    assert rc == OK and v == "scalar/mrope"


def test_mrope_clauses():
    lib = _lib.load()
    cases = [
        ("ids missing", NULL, dict(position_ids=None)),
        ("section missing", NULL, dict(mrope_section=None)),
        ("packed batching", UNSUP, dict(is_packed_batching=1)),
        ("packed batching 2", ATTR, dict(is_packed_batching=2)),
        ("layout 2", ATTR, dict(mrope_layout=2)),
        ("interleaved 2", ATTR, dict(interleaved=2)),
        ("negative section", ATTR, dict(mrope_section=(5, -1, 4))),
        ("section sum", ATTR, dict(mrope_section=(4, 2, 1))),
        ("section entries whose sum overflows", ATTR, dict(mrope_section=(2 ** 63 - 1, 2 ** 63 - 1, 4))),
        ("rotary odd", ATTR, dict(rotary_embedding_dim=7)),
        ("rotary negative", ATTR, dict(rotary_embedding_dim=-2)),
        ("num_heads negative", ATTR, dict(num_heads=-1)),
        ("rank-4 rotary dim without num_heads", ATTR, dict(rotary_embedding_dim=8, num_heads=0,
                                                           mrope_section=(2, 1, 1))),
        ("rank-4 num_heads disagrees", SHAPE, dict(num_heads=2)),
    ]
    for name, code, over in cases:
        kw = mrope_case()
        kw.update(over)
        rc, _ = check_mrope(kw)
        assert rc == code, (name, rc, lib.rope_last_error())
    kw = mrope_case(rank=3, num_heads=0)
    assert check_mrope(kw)[0] == ATTR
    kw = mrope_case(rank=3); kw["num_heads"] = 5
    assert check_mrope(kw)[0] == SHAPE
    kw = mrope_case(D=9, R=0, section=(2, 1, 1))
    assert check_mrope(kw)[0] == SHAPE                  # odd head size needs a rotary dim
    kw = mrope_case(R=18, section=(5, 2, 2))
    assert check_mrope(kw)[0] == SHAPE                  # rotary dim > head size
    kw = mrope_case(); kw["position_ids"] = reshape(kw["position_ids"], (2, 5))
    assert check_mrope(kw)[0] == RANK
    kw = mrope_case(); kw["position_ids"] = reshape(kw["position_ids"], (2, 2, 5))
    assert check_mrope(kw)[0] == SHAPE
    kw = mrope_case(); kw["cos_cache"] = reshape(kw["cos_cache"], (20, 7)); kw["sin_cache"] = reshape(kw["sin_cache"], (20, 7))
    assert check_mrope(kw)[0] == SHAPE
    kw = mrope_case(); kw["cos_cache"] = reshape(kw["cos_cache"], (2, 10, 8))
    assert check_mrope(kw)[0] == RANK
    kw = mrope_case(); kw["sin_cache"] = reshape(kw["sin_cache"], (19, 8))
    assert check_mrope(kw)[0] == SHAPE
    kw = mrope_case(); kw["position_ids"] = reshape(kw["position_ids"], (3, 2, 5), F32)
    assert check_mrope(kw)[0] == DTYPE
    kw = mrope_case(D=2048, section=(1024, 0, 0))
    assert check_mrope(kw)[0] == UNSUP                  # beyond the stream table


# ---------------------------------------------------------------------------
# Q + K

def qk_case(rank=3, dt=F16, B=4, S=1, H=8, Hk=2, D=16, M=64, table=True, ids=True, **over):
    a = Alloc()
    q = a(dt, (B, S, H * D) if rank == 3 else (B, H, S, D))
    k = a(dt, (B, S, Hk * D) if rank == 3 else (B, Hk, S, D))
    kw = dict(q=q, k=k,
              cos_cache=a(dt, (M, D // 2) if ids else (B, S, D // 2)) if table else None,
              sin_cache=a(dt, (M, D // 2) if ids else (B, S, D // 2)) if table else None,
              position_ids=a(I64, (B, S)) if ids else None,
              yq=a(dt, tuple(q.shape[:rank])), yk=a(dt, tuple(k.shape[:rank])),
              interleaved=0, num_heads=H if rank == 3 else 0, kv_num_heads=Hk if rank == 3 else 0,
              rotary_embedding_dim=0, inv_freq=None if table else a(F32, (D // 2,)),
              attention_scaling=1.0)
    kw.update(over)
    return kw


def check_qk(kw):
    kw = dict(kw)
    args = [kw.pop(k) for k in ("q", "k", "cos_cache", "sin_cache", "position_ids", "yq", "yk")]
    return rpe.rope_apply_qk_check(*args, **kw)


def test_qk_accepted():
    for rank in (3, 4):
        for fam, pol in (("row16", 0), ("vec16", 2)):
            assert with_policy(pol, check_qk, qk_case(rank=rank)) == (OK, fam + "/gather")
            assert with_policy(pol, check_qk, qk_case(rank=rank, table=False)) == (OK, fam + "/on_the_fly")
            assert with_policy(pol, check_qk, qk_case(rank=rank, ids=False)) == (OK, fam + "/per_token")


def test_qk_clauses():
    lib = _lib.load()
    cases = [
        ("only cos", NULL, dict(sin_cache=None)),
        ("on the fly without inv_freq", NULL, dict(cos_cache=None, sin_cache=None)),
        ("kv heads do not divide", SHAPE, dict(kv_num_heads=3)),
        ("num_heads missing", ATTR, dict(num_heads=0)),
    ]
    for name, code, over in cases:
        kw = qk_case()
        kw.update(over)
        rc, _ = check_qk(kw)
        assert rc == code, (name, rc, lib.rope_last_error())
    kw = qk_case(table=False, ids=False)
    assert check_qk(kw)[0] == NULL                     # on the fly needs positions
    kw = qk_case(table=False); kw["inv_freq"] = reshape(kw["inv_freq"], (7,))
    assert check_qk(kw)[0] == SHAPE
    kw = qk_case(table=False); kw["inv_freq"] = reshape(kw["inv_freq"], (8,), F16)
    assert check_qk(kw)[0] == DTYPE
    kw = qk_case(); kw["k"] = reshape(kw["k"], (4, 2, 32))
    assert check_qk(kw)[0] == SHAPE                    # sequence differs
    kw = qk_case(); kw["k"] = reshape(kw["k"], (4, 1, 2, 16))
    assert check_qk(kw)[0] == RANK
    kw = qk_case(); kw["yk"] = reshape(kw["yk"], (4, 1, 32)); kw["yk"].data = kw["yq"].data
    assert check_qk(kw)[0] == ALIAS                    # outputs overlap
    kw = qk_case(); kw["yq"] = reshape(kw["q"], (4, 1, 128))
    kw["yk"] = reshape(kw["k"], (4, 1, 32))
    assert check_qk(kw)[0] == OK                       # both in place


# ---------------------------------------------------------------------------
# host copies of the slot-to-stream reading agree (product vs oracle, both
# written independently from the same reading) -- exercised via the check
# path is not possible, so compare on the only shared observable: counts.

def test_inv_freq_and_table_validation():
    lib = _lib.load()
    a = Alloc()
    inv = a(F32, (64,))
    assert lib.rope_inv_freq(ctypes.byref(reshape(inv, (64,), F16)), 1e4, None) == DTYPE
    assert lib.rope_inv_freq(ctypes.byref(reshape(inv, (8, 8))), 1e4, None) == RANK
    assert lib.rope_inv_freq(ctypes.byref(inv), -1.0, None) == ATTR
    assert lib.rope_inv_freq(None, 1e4, None) == NULL
    cos, sin = a(F16, (128, 64)), a(F16, (128, 64))
    f = lib.rope_cos_sin_cache
    assert f(ctypes.byref(inv), 1.0, ctypes.byref(reshape(cos, (128, 32))), ctypes.byref(reshape(sin, (128, 32))), None) == SHAPE
    assert f(ctypes.byref(inv), 1.0, ctypes.byref(cos), ctypes.byref(reshape(sin, (128, 64), F32)), None) == DTYPE
    assert f(ctypes.byref(inv), 1.0, ctypes.byref(cos), ctypes.byref(cos), None) == ALIAS
    assert f(ctypes.byref(inv), 1.0, ctypes.byref(reshape(cos, (8192,))), ctypes.byref(reshape(sin, (8192,))), None) == RANK


# ---------------------------------------------------------------------------
# packed [Q|K|V] (SparseAttention README, Inputs)

def packed_case(rank=3, dt=F16, B=2, S=3, H=8, Hk=2, D=16, M=64, table=True, inplace=False, **over):
    a = Alloc()
    shape = (B, S, (H + 2 * Hk) * D) if rank == 3 else (B, H + 2 * Hk, S, D)
    qkv = a(dt, shape)
    kw = dict(qkv=qkv,
              cos_cache=a(dt, (M, D // 2)) if table else None,
              sin_cache=a(dt, (M, D // 2)) if table else None,
              position_ids=a(I64, (B, S)),
              y=reshape(qkv, shape) if inplace else a(dt, shape),
              interleaved=0, num_heads=H, kv_num_heads=Hk, rotary_embedding_dim=0,
              inv_freq=None if table else a(F32, (D // 2,)), attention_scaling=1.0)
    kw.update(over)
    return kw


def check_packed(kw):
    kw = dict(kw)
    args = [kw.pop(k) for k in ("qkv", "cos_cache", "sin_cache", "position_ids", "y")]
    return rpe.rope_apply_qkv_packed_check(*args, **kw)


def test_packed_accepted():
    for rank in (3, 4):
        for table in (True, False):
            for inplace in (False, True):
                rc, v = check_packed(packed_case(rank=rank, table=table, inplace=inplace))
                assert rc == OK, _lib.load().rope_last_error()
                assert v == ("row16/gather" if table else "row16/on_the_fly")
                rc, v = with_policy(2, check_packed, packed_case(rank=rank, table=table, inplace=inplace))
                assert v == ("vec16/gather" if table else "vec16/on_the_fly")
    rc, v = check_packed(packed_case(D=6))
    assert rc == OK and v == "scalar/gather"


def test_packed_clauses():
    lib = _lib.load()
    cases = [
        ("num_heads missing", ATTR, dict(num_heads=0)),
        ("kv heads missing", ATTR, dict(kv_num_heads=0)),
        ("kv does not divide", SHAPE, dict(kv_num_heads=3)),
        ("interleaved 3", ATTR, dict(interleaved=3)),
        ("qkv missing", NULL, dict(qkv=None)),
        ("y missing", NULL, dict(y=None)),
        ("only sin", NULL, dict(cos_cache=None)),
    ]
    for name, code, over in cases:
        kw = packed_case()
        kw.update(over)
        rc, _ = check_packed(kw)
        assert rc == code, (name, rc, lib.rope_last_error())
    kw = packed_case(); kw["qkv"] = reshape(kw["qkv"], (2, 3, 190)); kw["y"] = reshape(kw["y"], (2, 3, 190))
    assert check_packed(kw)[0] == SHAPE            # width not (H + 2Hk) * D
    kw = packed_case(rank=4); kw["qkv"] = reshape(kw["qkv"], (2, 11, 3, 16)); kw["y"] = reshape(kw["y"], (2, 11, 3, 16))
    assert check_packed(kw)[0] == SHAPE            # dim 1 != H + 2Hk
    kw = packed_case(); kw["y"] = reshape(kw["y"], (2, 3, 96))
    assert check_packed(kw)[0] == SHAPE
    kw = packed_case(); y = reshape(kw["qkv"], (2, 3, 192)); y.data += 32; kw["y"] = y
    assert check_packed(kw)[0] == ALIAS            # shifted output
    kw = packed_case(table=False, position_ids=None)
    assert check_packed(kw)[0] == NULL


# ---------------------------------------------------------------------------
# RoPE on Q and K with the key/value cache append

I32 = 6


def kv_case(dt=F16, B=2, S=3, H=8, Hk=2, D=16, Smax=40, M=64, width=None, packed=False,
            inplace=False, total=20, **over):
    a = Alloc()
    width = D // 2 if width is None else width
    if packed:
        query = a(dt, (B, S, (H + 2 * Hk) * D))
        key = value = None
    else:
        query = a(dt, (B, S, H * D))
        key = a(dt, (B, S, Hk * D))
        value = a(dt, (B, S, Hk * D))
    kw = dict(query=query, key=key, value=value,
              past_key=a(dt, (B, Hk, Smax, D)), past_value=a(dt, (B, Hk, Smax, D)),
              key_total_sequence_lengths=a(I32, (B,)), total_sequence_length=total,
              cos_cache=a(dt, (M, width)), sin_cache=a(dt, (M, width)),
              q_out=reshape(query, (B, S, H * D)) if inplace else a(dt, (B, S, H * D)),
              rotary_interleaved=0, num_heads=H, kv_num_heads=Hk)
    kw.update(over)
    return kw


def check_kv(kw):
    kw = dict(kw)
    args = [kw.pop(k) for k in ("query", "key", "value", "past_key", "past_value",
                                "key_total_sequence_lengths", "total_sequence_length",
                                "cos_cache", "sin_cache", "q_out")]
    return rpe.rope_kv_append_check(*args, **kw)


def test_kv_append_accepted():
    for dt in (F16, F32, BF16):
        for packed in (False, True):
            rc, v = check_kv(kv_case(dt=dt, packed=packed))
            assert rc == OK, _lib.load().rope_last_error()
            assert v == "row16/append"
            assert with_policy(2, check_kv, kv_case(dt=dt, packed=packed)) == (OK, "vec16/append")
    for total in (3, 40):                                 # prompt; full cache
        assert check_kv(kv_case(total=total))[0] == OK
    rc, v = check_kv(kv_case(inplace=True))
    assert rc == OK and v == "row16/append"
    rc, v = check_kv(kv_case(D=6, width=3))                # 6 halves: no 16-byte items
    assert rc == OK and v == "scalar/append"
    rc, v = check_kv(kv_case(D=32, width=8))               # partial rotation
    assert rc == OK and v == "row16/append"
    rc, v = check_kv(kv_case(B=0))
    assert rc == OK


def test_kv_append_rotary_interleaved_any_value():
    """SparseAttention README, Attributes: rotary_interleaved 1 rotates
    adjacent pairs and every other value selects the NeoX half-split, so
    2, -1 and large values are accepted (unlike RotaryEmbedding's
    interleaved, which its manifest restricts to 0 and 1)."""
    lib = _lib.load()
    for value in (0, 1, 2, -1, 7, 2 ** 40):
        rc, v = check_kv(kv_case(rotary_interleaved=value))
        assert rc == OK and v == "row16/append", (value, rc, lib.rope_last_error())
        rc, v = check_kv_norm(kv_norm_case(rotary_interleaved=value))
        assert rc == OK, (value, rc, lib.rope_last_error())


def test_kv_append_clauses():
    lib = _lib.load()
    base = kv_case()
    cases = [
        ("query missing", NULL, dict(query=None)),
        ("only key", NULL, dict(value=None)),
        ("past_key missing", NULL, dict(past_key=None)),
        ("lengths missing", NULL, dict(key_total_sequence_lengths=None)),
        ("q_out missing", NULL, dict(q_out=None)),
        ("lengths int64", DTYPE, dict(key_total_sequence_lengths=reshape(base["key_total_sequence_lengths"], (2,), I64))),
        ("cache float32", DTYPE, dict(past_key=reshape(base["past_key"], (2, 2, 40, 16), F32))),
        ("query int64", DTYPE, dict(query=reshape(base["query"], (2, 3, 128), I64))),
        ("no heads", ATTR, dict(num_heads=0)),
        ("kv does not divide", SHAPE, dict(kv_num_heads=3)),
        ("query rank 4", RANK, dict(query=reshape(base["query"], (2, 3, 8, 16)))),
        ("key shape", SHAPE, dict(key=reshape(base["key"], (2, 3, 16)), value=reshape(base["value"], (2, 3, 16)))),
        ("value shape", SHAPE, dict(value=reshape(base["value"], (2, 1, 96)))),
        ("cache rank 3", RANK, dict(past_key=reshape(base["past_key"], (2, 80, 16)))),
        ("cache heads", SHAPE, dict(past_key=reshape(base["past_key"], (2, 1, 80, 16)),
                                    past_value=reshape(base["past_value"], (2, 1, 80, 16)))),
        ("value cache shape", SHAPE, dict(past_value=reshape(base["past_value"], (2, 2, 39, 16)))),
        ("lengths shape", SHAPE, dict(key_total_sequence_lengths=reshape(base["key_total_sequence_lengths"], (1,)))),
        ("table too wide", SHAPE, dict(cos_cache=reshape(base["cos_cache"], (32, 16)),
                                       sin_cache=reshape(base["sin_cache"], (32, 16)))),
        ("table rank 3", RANK, dict(cos_cache=reshape(base["cos_cache"], (1, 64, 8)))),
        ("sin shape", SHAPE, dict(sin_cache=reshape(base["sin_cache"], (32, 8)))),
        ("q_out shape", SHAPE, dict(q_out=reshape(base["q_out"], (2, 3, 64)))),
        ("total below S", SHAPE, dict(total_sequence_length=2)),
        ("total above cache", SHAPE, dict(total_sequence_length=41)),
        ("total above table", SHAPE, dict(cos_cache=reshape(base["cos_cache"], (10, 8)),
                                          sin_cache=reshape(base["sin_cache"], (10, 8)))),
        ("caches alias", ALIAS, dict(past_value=base["past_key"])),
        ("q_out in the cache", ALIAS, dict(q_out=reshape(base["past_key"], (2, 3, 128)))),
        ("cache over the key", ALIAS, dict(past_key=reshape(base["key"], (2, 2, 3, 16)),
                                           past_value=reshape(base["value"], (2, 2, 3, 16)),
                                           total_sequence_length=3)),
    ]
    for name, code, over in cases:
        kw = kv_case()
        kw.update(over)
        rc, _ = check_kv(kw)
        assert rc == code, (name, rc, lib.rope_last_error())
    # packed: q_out may not be the packed query
    kw = kv_case(packed=True)
    kw["q_out"] = reshape(kw["query"], (2, 3, 128))
    assert check_kv(kw)[0] == ALIAS
    kw = kv_case(packed=True)
    kw["query"] = reshape(kw["query"], (2, 3, 190))       # not (H + 2Hk) * D
    assert check_kv(kw)[0] == SHAPE


# ---------------------------------------------------------------------------
# QK-norm then RoPE

def norm_case(dt=F16, rank=3, D=128, table=True, shape=None, **over):
    kw = qk_case(dt=dt, rank=rank, D=D, table=table, **(shape or {}))
    a = Alloc()
    a.next = 1 << 40
    kw["q_weight"] = a(dt, (D,))
    kw["k_weight"] = a(dt, (D,))
    kw["epsilon"] = 1e-6
    kw.update(over)
    return kw


def check_norm(kw):
    kw = dict(kw)
    args = [kw.pop(k) for k in ("q", "k", "q_weight", "k_weight", "cos_cache", "sin_cache", "position_ids",
                                "yq", "yk")]
    return rpe.rope_apply_qk_norm_check(*args, **kw)


def test_qk_norm_accepted():
    for dt in (F16, BF16, F32):
        for table in (True, False):
            rc, v = check_norm(norm_case(dt=dt, table=table))
            assert rc == OK, _lib.load().rope_last_error()
            assert v == ("row16/norm/gather" if table else "row16/norm/on_the_fly")
            rc, v = with_policy(2, check_norm, norm_case(dt=dt, table=table))
            assert v == ("vec16/norm/gather" if table else "vec16/norm/on_the_fly")
    rc, v = check_norm(norm_case(dt=F32, D=96))      # 24 chunks per row: the row kernel's general rows
    assert rc == OK and v == "row16/norm/gather"
    assert with_policy(2, check_norm, norm_case(dt=F32, D=96)) == (OK, "scalar/norm/gather")  # no vector kernel
    rc, v = check_norm(norm_case(D=96, shape=dict(B=1, S=8192, H=32, Hk=8, M=8192)))  # any size
    assert rc == OK and v == "row16/norm/gather"
    rc, v = check_norm(norm_case(D=80, rank=4, shape=dict(B=1, S=8192, H=32, Hk=8, M=8192)))
    assert rc == OK and v == "row16/norm/gather"
    rc, v = check_norm(norm_case(dt=F32, D=1040 // 4 * 2, table=True))  # 2080-byte rows: neither
    assert rc == OK and v == "scalar/norm/gather"
    rc, v = check_norm(norm_case(rank=4))
    assert rc == OK and v == "row16/norm/gather"
    assert with_policy(2, check_norm, norm_case(rank=4)) == (OK, "vec16/norm/gather")
    rc, v = check_norm(norm_case(epsilon=0.0))
    assert rc == OK


def test_qk_norm_clauses():
    lib = _lib.load()
    base = norm_case()
    cases = [
        ("q_weight missing", NULL, dict(q_weight=None)),
        ("k_weight missing", NULL, dict(k_weight=None)),
        ("weight dtype", DTYPE, dict(q_weight=reshape(base["q_weight"], (64,), F32))),
        ("weight rank", RANK, dict(k_weight=reshape(base["k_weight"], (2, 64)))),
        ("weight length", SHAPE, dict(q_weight=reshape(base["q_weight"], (64,)))),
        ("epsilon negative", ATTR, dict(epsilon=-1e-6)),
        ("epsilon nan", ATTR, dict(epsilon=float("nan"))),
        ("epsilon inf", ATTR, dict(epsilon=float("inf"))),
        ("yq over the weight", ALIAS, dict(yq=reshape(base["q_weight"], tuple(base["yq"].shape[:3])))),
        ("q contract still applies", ATTR, dict(interleaved=2)),
    ]
    for name, code, over in cases:
        kw = norm_case()
        kw.update(over)
        rc, _ = check_norm(kw)
        assert rc == code, (name, rc, lib.rope_last_error())


def kv_norm_case(dt=F16, **over):
    kw = kv_case(dt=dt, D=128, **over)
    a = Alloc()
    a.next = 1 << 41
    kw["q_weight"] = a(dt, (128,))
    kw["k_weight"] = a(dt, (128,))
    kw["epsilon"] = 1e-6
    return kw


def check_kv_norm(kw):
    kw = dict(kw)
    args = [kw.pop(k) for k in ("query", "key", "value", "past_key", "past_value",
                                "key_total_sequence_lengths", "total_sequence_length",
                                "cos_cache", "sin_cache", "q_out", "q_weight", "k_weight")]
    return rpe.rope_kv_append_qk_norm_check(*args, **kw)


def test_kv_append_qk_norm_accepted_and_clauses():
    lib = _lib.load()
    for dt in (F16, BF16, F32):
        for packed in (False, True):
            rc, v = check_kv_norm(kv_norm_case(dt=dt, packed=packed))
            assert rc == OK, lib.rope_last_error()
            assert v == "row16/norm/append"
            assert with_policy(2, check_kv_norm, kv_norm_case(dt=dt, packed=packed)) == (OK, "vec16/norm/append")
    base = kv_norm_case()
    cases = [
        ("q_weight missing", NULL, dict(q_weight=None)),
        ("weight dtype", DTYPE, dict(k_weight=reshape(base["k_weight"], (64,), F32))),
        ("weight length", SHAPE, dict(q_weight=reshape(base["q_weight"], (64,)))),
        ("epsilon negative", ATTR, dict(epsilon=-1.0)),
        ("cache over a weight", ALIAS, dict(q_weight=reshape(base["past_key"], (128,)))),
        ("append contract still applies", SHAPE, dict(total_sequence_length=2)),
    ]
    for name, code, over in cases:
        kw = kv_norm_case()
        kw.update(over)
        rc, _ = check_kv_norm(kw)
        assert rc == code, (name, rc, lib.rope_last_error())


def test_benchmark_workloads_kernel_choice():
    """The kernel each benchmark workload runs (the planner's choice for its
    shapes): the vector kernel for the prefill steps, the row kernel for the
    decode steps."""
    assert check_rope(rope_case(B=4, S=2048, H=32, D=128, M=8192)) == (OK, "vec16/gather")            # c2
    assert check_rope(rope_case(B=4, S=2048, H=32, D=128, M=8192, dt=BF16)) == (OK, "vec16/gather")
    assert check_rope(rope_case(rank=4, dt=F32, B=8, S=1024, H=32, D=96, R=64, interleaved=1,
                                M=4096)) == (OK, "vec16/gather")                                     # c3
    assert check_mrope(mrope_case(rank=4, B=2, S=4096, H=28, D=128, M=32768,
                                  section=(16, 24, 24))) == (OK, "vec16/mrope")                      # c4
    assert check_mrope(mrope_case(rank=3, B=256, S=1, H=28, D=128, M=32768,
                                  section=(16, 24, 24))) == (OK, "row16/mrope")                      # decode
    assert check_qk(qk_case(B=256, S=1, H=32, Hk=8, D=128, M=32768)) == (OK, "row16/gather")        # c5
    assert check_qk(qk_case(B=256, S=1, H=32, Hk=8, D=128, table=False)) == (OK, "row16/on_the_fly")
    assert check_packed(packed_case(B=256, S=1, H=32, Hk=8, D=128, M=32768)) == (OK, "row16/gather")
    assert check_kv(kv_case(B=256, S=1, H=32, Hk=8, D=128, Smax=4096, M=32768, total=4096)) == (OK, "row16/append")
    assert check_norm(norm_case(table=True, shape=dict(B=4, S=2048, H=32, Hk=8, M=8192))) == \
        (OK, "vec16/norm/gather")
    assert check_norm(norm_case(table=False, shape=dict(B=256, S=1, H=32, Hk=8))) == (OK, "row16/norm/on_the_fly")
    assert check_kv_norm(kv_norm_case(B=256, S=1, H=32, Hk=8, Smax=4096, M=32768, total=4096)) == \
        (OK, "row16/norm/append")
