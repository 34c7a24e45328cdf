"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element. Tolerances are in parity.py."""
import numpy as np
import pytest
import torch

import oracle
import rotary_position_embedding_amd as rpe
from oracle_pins import angle_table, ids_in, pair_index
from parity import assert_bitwise, assert_parity, bits, compare
from gpu_io import DEV, cuda, host, one, torch_dtype, POLICIES, POLICY_IDS
from rope_inputs import BFLOAT16, EXTRA_WORKLOADS, WORKLOADS, SplitMix64, normal_tensor, with_dtype, with_layout
from rope_inputs import get as get_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _policy():
    old = rpe.set_kernel_policy(0)
    yield
    rpe.set_kernel_policy(old)


def log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------
# the five workloads at their full sizes, in the default launch configuration

def run_workload(w, onthefly=False):
    """(gpu output(s), oracle output(s), inputs) for a workload."""
    x = w.make_x()
    ids = w.make_ids()
    cos, sin = oracle.table_for(w)
    if w.op == "rope":
        want = oracle.rope_apply(x, cos, sin, ids, interleaved=w.interleaved,
                                 num_heads=w.num_heads if w.rank == 3 else 0,
                                 rotary_embedding_dim=w.rotary_embedding_dim)
        got = rpe.rope_apply(cuda(x), cuda(cos), cuda(sin), None if ids is None else cuda(ids),
                             interleaved=w.interleaved, num_heads=w.num_heads if w.rank == 3 else 0,
                             rotary_embedding_dim=w.rotary_embedding_dim)
        return host(got), want, (x, ids, cos, sin)
    if w.op == "mrope":
        want = oracle.mrope_apply(x, ids, cos, sin, w.mrope_section, w.mrope_layout,
                                  interleaved=w.interleaved, num_heads=w.num_heads,
                                  rotary_embedding_dim=w.rotary_embedding_dim, scale=w.scale)
        got = rpe.mrope_apply(cuda(x), cuda(ids), cuda(cos), cuda(sin), mrope_section=w.mrope_section,
                              mrope_layout=w.mrope_layout, interleaved=w.interleaved,
                              num_heads=w.num_heads, rotary_embedding_dim=w.rotary_embedding_dim,
                              scale=w.scale)
        return host(got), want, (x, ids, cos, sin)
    k = w.make_k()
    inv = oracle.inv_freq(w.cache_base, w.rotary_dim)
    if onthefly:
        want = oracle.rope_apply_qk(x, k, None, None, ids, num_heads=w.num_heads,
                                    kv_num_heads=w.kv_num_heads, inv_freq=inv,
                                    attention_scaling=w.scaling)
        got = rpe.rope_apply_qk(cuda(x), cuda(k), None, None, cuda(ids), num_heads=w.num_heads,
                                kv_num_heads=w.kv_num_heads, inv_freq=cuda(inv),
                                attention_scaling=w.scaling)
    else:
        want = oracle.rope_apply_qk(x, k, cos, sin, ids, num_heads=w.num_heads,
                                    kv_num_heads=w.kv_num_heads)
        got = rpe.rope_apply_qk(cuda(x), cuda(k), cuda(cos), cuda(sin), cuda(ids),
                                num_heads=w.num_heads, kv_num_heads=w.kv_num_heads)
    return (host(got[0]), host(got[1])), want, (x, k, ids)


def test_c1_rope_f32_tiny():
    w = WORKLOADS["c1_rope_f32_tiny"]
    got, want, _ = run_workload(w)
    r = assert_parity(got, want, w.name)
    log("%s %s" % (w.name, r))


def test_c2_rope_f16_prefill():
    w = WORKLOADS["c2_rope_f16_prefill"]
    got, want, _ = run_workload(w)
    r = assert_parity(got, want, w.name)
    log("%s %s" % (w.name, r))


def test_c3_rope_f32_partial_interleaved():
    w = WORKLOADS["c3_rope_f32_partial_interleaved"]
    got, want, (x, *_rest) = run_workload(w)
    r = assert_parity(got, want, w.name)
    assert_bitwise(got[..., 64:], x[..., 64:], "tail")
    log("%s %s" % (w.name, r))


@pytest.mark.parametrize("layout", [0, 1])
def test_c4_mrope_f16_prefill(layout):
    w = with_layout(WORKLOADS["c4_mrope_f16_prefill"], layout)
    got, want, (x, ids, _c, _s) = run_workload(w)
    r = assert_parity(got, want, w.name)
    # pairs whose stream id is out of range: bit copies of x
    streams = oracle.mrope_slot_streams(w.half, w.mrope_section, layout)
    sid = ids[streams]                              # (P, B, S)
    oob = (sid < 0) | (sid >= w.cache_rows)
    i, b, s = np.nonzero(oob)
    assert i.size > 0
    for j in (i, i + w.half):
        assert_bitwise(got[b, :, s, j], x[b, :, s, j], "out-of-range pairs")
    log("%s %s oob_pairs=%d" % (w.name, r, i.size))


def test_mrope_decode_full_size():
    """The M-RoPE decode step the benchmark times (mrope_f16_decode), in its
    launch configuration."""
    w = EXTRA_WORKLOADS["mrope_f16_decode"]
    got, want, _inputs = run_workload(w)
    log("%s %s" % (w.name, assert_parity(got, want, w.name)))


@pytest.mark.parametrize("onthefly", [False, True])
def test_c5_rope_qk_f16_decode(onthefly):
    w = WORKLOADS["c5_rope_qk_f16_decode"]
    (gq, gk), (wq, wk), _ = run_workload(w, onthefly)
    rq = assert_parity(gq, wq, w.name + " Q")
    rk = assert_parity(gk, wk, w.name + " K")
    log("%s onthefly=%s Q %s K %s" % (w.name, onthefly, rq, rk))


def test_c5_onthefly_equals_table_on_gpu():
    w = WORKLOADS["c5_rope_qk_f16_decode"]
    q, k, ids = cuda(w.make_x()), cuda(w.make_k()), cuda(w.make_ids())
    inv = rpe.rope_inv_freq(w.rotary_dim, w.cache_base, device=DEV)
    cos, sin = rpe.rope_cos_sin_cache(inv, w.cache_rows, torch.float16)
    a = rpe.rope_apply_qk(q, k, cos, sin, ids, num_heads=32, kv_num_heads=8)
    b = rpe.rope_apply_qk(q, k, None, None, ids, num_heads=32, kv_num_heads=8, inv_freq=inv)
    assert_bitwise(host(a[0]), host(b[0]), "Q")
    assert_bitwise(host(a[1]), host(b[1]), "K")


@pytest.mark.parametrize("name", ["c2_rope_f16_prefill_tp8", "c5_rope_qk_f16_decode_tp8",
                                  "c2_rope_f16_prefill_sp8"])
def test_parallel_shares_full_size(name):
    """One GPU's share of c2 and c5 under 8-way tensor parallelism (4 query
    heads, 1 key head) and of c2 under 8-way sequence parallelism (256
    tokens per sequence), in the launch configuration the benchmark times."""
    w = EXTRA_WORKLOADS[name]
    got, want, _ = run_workload(w)
    if w.op == "rope_qk":
        log("%s Q %s K %s" % (w.name, assert_parity(got[0], want[0], w.name + " Q"),
                              assert_parity(got[1], want[1], w.name + " K")))
    else:
        log("%s %s" % (w.name, assert_parity(got, want, w.name)))


def _resized(name, seq=None, heads=None):
    """A workload at another sequence length or head count (same seeds and
    recipe), for the launch geometries between the decode steps and the
    benchmark prefills."""
    from dataclasses import replace
    w = get_workload(name)
    xs = list(w.x_shape)
    ks = None if w.k_shape is None else list(w.k_shape)
    if seq is not None:
        xs[2 if len(xs) == 4 else 1] = seq
        if ks is not None:
            ks[2 if len(ks) == 4 else 1] = seq
    if heads is not None:
        xs[2] = heads * w.head_size
    return replace(w, x_shape=tuple(xs), k_shape=None if ks is None else tuple(ks),
                   num_heads=heads or w.num_heads, name="%s_s%s_h%s" % (name, seq, heads))


@pytest.mark.parametrize("name,seq,heads,layout,onthefly", [
    ("c4_mrope_f16_prefill", 1024, None, 0, False),    # M-RoPE, 4 heads per wave
    ("c4_mrope_f16_prefill", 1024, None, 1, False),
    ("c4_mrope_f16_prefill", 768, None, 0, False),     # M-RoPE, 2 heads per wave
    ("c2_rope_f16_prefill", None, 16, None, False),    # 4 heads per wave in batches of 4
    ("c2_rope_f16_prefill", 512, None, None, False),
    ("c3_rope_f32_partial_interleaved", 128, None, None, False),
    ("c5_rope_qk_f16_decode", 2, None, None, False),   # 5 MiB: the row kernel
    ("c5_rope_qk_f16_decode", 2, None, None, True),
    ("c2_rope_f16_prefill", None, 40, None, False),    # over one round: many waves of 2 heads
    ("c5_rope_qk_f16_decode", 32, None, None, False),
])
def test_mid_size_launches(name, seq, heads, layout, onthefly):
    """Launches between the decode steps and the benchmark prefills, and
    larger ones, in the geometries the planner gives them (fewer heads per
    wave, the row kernel up to 6 MiB, batches of 2 heads past one round of
    waves), against the oracle at full size."""
    w = _resized(name, seq, heads)
    if layout is not None:
        w = with_layout(w, layout)
    log("mid-size %s layout=%s onthefly=%s" % (w.name, layout, onthefly))
    got, want, inputs = run_workload(w, onthefly)
    if w.op == "rope_qk":
        log("%s Q %s K %s" % (w.name, assert_parity(got[0], want[0], w.name + " Q"),
                              assert_parity(got[1], want[1], w.name + " K")))
        return
    log("%s %s" % (w.name, assert_parity(got, want, w.name)))
    if w.rotary_embedding_dim:
        assert_bitwise(got[..., w.rotary_embedding_dim:], inputs[0][..., w.rotary_embedding_dim:], "tail")


def _reshaped(name, head_size=None, heads=None, interleaved=None, rotary_dim=None):
    """A rank-3 workload with another head size, head count, pairing or
    rotary_embedding_dim (same seeds and recipe)."""
    from dataclasses import replace
    w = get_workload(name)
    D = head_size or w.head_size
    H = heads or w.num_heads
    return replace(w, x_shape=(w.x_shape[0], w.x_shape[1], H * D), num_heads=H,
                   interleaved=w.interleaved if interleaved is None else interleaved,
                   rotary_embedding_dim=w.rotary_embedding_dim if rotary_dim is None else rotary_dim,
                   name="%s_d%d_h%d_il%s_r%s" % (name, D, H, interleaved, rotary_dim))


@pytest.mark.parametrize("head_size,heads,interleaved,rotary_dim,dtype", [
    (64, 64, 0, None, None),        # split halves of 64 bytes: the row kernel
    (64, 64, 1, None, None),        # interleaved pairs: the row kernel
    (128, 32, 1, None, None),
    (128, 32, 1, None, "bf16"),
    (128, 32, 0, 64, None),         # partial rotation: the row kernel, tail copied
    (128, 32, 0, 32, None),
    (256, 16, 0, None, None),       # split halves of 256 bytes: the vector kernel, batches of 2
    (96, 32, 0, None, None),        # 192-byte rows, partners 6 lanes apart: the row kernel's general rows
    (96, 32, 0, 24, None),          # 24 of 96 rotated: element-wise pairs
    (80, 32, 0, 20, "bf16"),        # 20 of 80 rotated
    (128, 32, 1, 20, None),         # interleaved, 20 rotated
    (96, 32, 1, None, None),
    (80, 32, 0, 32, None),          # 160-byte rows, rotary dim 32
    (128, 32, 0, 64, "f32"),        # float32 partial rotation: the row kernel
    (96, 32, 1, 64, "f32"),         # float32 384-byte rows
])
def test_prefill_head_shapes(head_size, heads, interleaved, rotary_dim, dtype):
    """8192-token fp16/bf16 prefills with other head sizes, pairings and
    rotary dims, each in the kernel and geometry the planner gives it,
    against the oracle at full size."""
    w = _reshaped("c2_rope_f16_prefill", head_size, heads, interleaved, rotary_dim)
    if dtype == "bf16":
        w = with_dtype(w, BFLOAT16, "bf16")
    elif dtype == "f32":
        w = with_dtype(w, np.float32, "f32")
    log("prefill head shape %s" % w.name)
    got, want, inputs = run_workload(w)
    log("%s %s" % (w.name, assert_parity(got, want, w.name)))
    if w.rotary_embedding_dim:
        rows = (w.batch, w.seq, w.num_heads, w.head_size)   # rank 3: heads side by side
        R = w.rotary_embedding_dim
        assert_bitwise(got.reshape(rows)[..., R:], inputs[0].reshape(rows)[..., R:], "tail")


@pytest.mark.parametrize("head_size,interleaved,rotary_dim", [
    (64, 0, 0),       # rank 4, split halves of 64 bytes: the row kernel
    (64, 1, 0),
    (128, 1, 0),      # rank 4, interleaved: the row kernel
    (128, 0, 64),
    (96, 1, 64),      # rank 4, 192-byte rows: the vector kernel
])
def test_prefill_rank4_head_shapes(head_size, interleaved, rotary_dim):
    """Rank-4 (8, 32, 1024, D) fp16 inputs in the kernel the planner gives
    them, against the oracle at full size, tail bitwise."""
    from dataclasses import replace
    w = with_dtype(get_workload("c3_rope_f32_partial_interleaved"), np.float16, "f16")
    xs = w.x_shape[:3] + (head_size,)
    w = replace(w, x_shape=xs, interleaved=interleaved, rotary_embedding_dim=rotary_dim,
                name="%s_d%d_il%d_r%d" % (w.name, head_size, interleaved, rotary_dim))
    log("rank-4 prefill %s" % w.name)
    got, want, inputs = run_workload(w)
    log("%s %s" % (w.name, assert_parity(got, want, w.name)))
    if rotary_dim:
        assert_bitwise(got[..., rotary_dim:], inputs[0][..., rotary_dim:], "tail")


@pytest.mark.parametrize("name", ["rope_f16_prefill_heads64", "rope_f16_prefill_neox_partial"])
def test_other_model_shapes_full_size(name):
    """The benchmark's prefills of other model shapes (64 heads of 64; 64
    heads of 96 with 24 dimensions rotated), in the launch configuration the
    benchmark times, against the oracle at full size, tails bitwise."""
    w = EXTRA_WORKLOADS[name]
    log("other model shape %s" % w.name)
    got, want, inputs = run_workload(w)
    log("%s %s" % (w.name, assert_parity(got, want, w.name)))
    if w.rotary_embedding_dim:
        rows = (w.batch, w.seq, w.num_heads, w.head_size)
        R = w.rotary_embedding_dim
        assert_bitwise(got.reshape(rows)[..., R:], inputs[0].reshape(rows)[..., R:], "tail")


def test_qk_on_the_fly_prefill_size():
    """Q+K with coefficients on the fly over 8192 tokens (the row kernel at
    prefill size), against the oracle."""
    w = _resized("c5_rope_qk_f16_decode", 32, None)
    log("Q+K on the fly %s" % w.name)
    got, want, _ = run_workload(w, onthefly=True)
    log("%s Q %s K %s" % (w.name, assert_parity(got[0], want[0], w.name + " Q"),
                          assert_parity(got[1], want[1], w.name + " K")))


# the same workloads stored in bfloat16 (same seeds and shapes)

@pytest.mark.parametrize("name,variant", [
    ("c1_rope_f32_tiny", None), ("c2_rope_f16_prefill", None), ("c3_rope_f32_partial_interleaved", None),
    ("c4_mrope_f16_prefill", 0), ("c4_mrope_f16_prefill", 1), ("c5_rope_qk_f16_decode", False),
    ("c5_rope_qk_f16_decode", True)])
def test_workloads_bf16(name, variant):
    w = with_dtype(WORKLOADS[name], BFLOAT16, "bf16")
    if w.op == "mrope":
        w = with_layout(w, variant)
    log("bf16 workload %s variant=%s" % (w.name, variant))
    got, want, inputs = run_workload(w, onthefly=bool(variant) if w.op == "rope_qk" else False)
    if w.op == "rope_qk":
        rq = assert_parity(got[0], want[0], w.name + " Q")
        rk = assert_parity(got[1], want[1], w.name + " K")
        log("%s Q %s K %s" % (w.name, rq, rk))
        return
    r = assert_parity(got, want, w.name)
    if w.rotary_embedding_dim:
        R = w.rotary_embedding_dim
        assert_bitwise(got[..., R:], inputs[0][..., R:], "tail")
    log("%s %s" % (w.name, r))


# ---------------------------------------------------------------------------
# table builders

@pytest.mark.parametrize("dt,base,R,rows,scaling", [
    (np.float16, 1e6, 128, 32768, 1.0), (np.float32, 1e4, 64, 4096, 1.0),
    (np.float16, 1e4, 8, 16, 1.0), (np.float32, 1e6, 128, 4096, 0.7), (np.float16, 5e5, 96, 1000, 1.25),
    (BFLOAT16, 1e6, 128, 32768, 1.0), (BFLOAT16, 1e4, 64, 1000, 1.25)])
def test_tables_match_oracle(dt, base, R, rows, scaling):
    inv_o = oracle.inv_freq(base, R)
    inv_g = host(rpe.rope_inv_freq(R, base, device=DEV))
    assert_bitwise(inv_g, inv_o, "inv_freq")
    cos_o, sin_o = oracle.cos_sin_cache(dt, rows, inv_o, scaling)
    cos_g, sin_g = rpe.rope_cos_sin_cache(cuda(inv_o), rows, torch_dtype(dt), scaling)
    rc = compare(host(cos_g), cos_o)
    rs = compare(host(sin_g), sin_o)
    # cos/sin of a binary32 angle rounded to binary32 by two libraries: equal
    # unless the value sits within a binary64 ulp of a rounding boundary
    assert rc["n_over_tol"] == 0 and rs["n_over_tol"] == 0
    assert rc["n_bit_diff"] + rs["n_bit_diff"] <= 2, (rc, rs)
    log("table %s base=%g R=%d rows=%d bitdiff=%d/%d" % (np.dtype(dt), base, R, rows,
                                                           rc["n_bit_diff"], rs["n_bit_diff"]))


# ---------------------------------------------------------------------------
# sweeps over shapes, both kernels, ragged tails

SHAPES = [
    # rank, dt, B, S, H, D, R, interleaved, ids, M
    (3, np.float16, 3, 37, 5, 128, 0, 0, True, 300),
    (4, np.float16, 2, 41, 3, 64, 0, 1, True, 100),
    (4, np.float32, 2, 19, 7, 96, 64, 1, True, 64),
    (4, np.float32, 3, 23, 2, 96, 64, 0, True, 64),
    (3, np.float32, 2, 33, 4, 80, 32, 0, False, 0),
    (3, np.float16, 1, 70, 3, 256, 128, 0, True, 500),
    (4, np.float16, 2, 9, 9, 80, 0, 0, False, 0),
    (3, np.float16, 5, 1, 33, 128, 0, 0, True, 1000),   # decode-like
    (4, np.float32, 1, 130, 1, 32, 0, 1, True, 140),
    (3, np.float16, 2, 13, 4, 6, 0, 0, True, 20),        # not 16-byte items
    (4, np.float16, 2, 13, 4, 18, 10, 1, True, 20),
    (3, np.float32, 2, 7, 3, 2, 0, 0, False, 0),
    (4, np.float16, 1, 17, 2, 1024, 0, 0, True, 40),     # long rows
    (3, BFLOAT16, 3, 37, 5, 128, 0, 0, True, 300),
    (4, BFLOAT16, 2, 41, 3, 64, 0, 1, True, 100),
    (4, BFLOAT16, 2, 19, 7, 96, 64, 1, True, 64),
    (3, BFLOAT16, 2, 33, 4, 80, 32, 0, False, 0),
    (3, BFLOAT16, 2, 13, 4, 6, 0, 0, True, 20),          # not 16-byte items
    # row-kernel partner distances and row sizes (policy "row" runs them there)
    (3, np.float16, 2, 11, 6, 16, 0, 0, True, 50),       # 32-byte rows: partners 1 lane apart
    (4, np.float32, 2, 9, 3, 16, 0, 0, True, 50),        # partners 2 lanes apart
    (3, np.float16, 1, 5, 3, 512, 0, 0, True, 50),       # 1 KiB rows: partners 32 lanes apart
    (3, np.float32, 1, 6, 2, 256, 128, 0, True, 50),     # 1 KiB rows, partial: 16 lanes apart
    (3, np.float16, 2, 7, 3, 128, 64, 0, True, 50),      # partial: 4 lanes apart, tail chunks
    (3, np.float16, 2, 7, 3, 128, 96, 1, True, 50),      # interleaved partial, 12 rotated chunks
    (3, BFLOAT16, 2, 11, 6, 32, 0, 0, False, 0),         # 64-byte rows, per-token table
    # pairs off the 16-byte chunks (the row kernel's element-wise instances)
    (3, np.float16, 3, 29, 7, 96, 24, 0, True, 200),     # 24 of 96 rotated: halves of 12
    (3, np.float16, 2, 17, 5, 80, 20, 0, False, 0),      # 20 of 80, per-token table
    (4, BFLOAT16, 2, 15, 3, 64, 12, 0, True, 60),        # rank 4, halves of 6
    (3, np.float16, 2, 9, 4, 128, 20, 1, True, 40),      # interleaved, 20 rotated
    (3, np.float32, 2, 11, 3, 64, 20, 0, True, 50),      # float32, halves of 10
    (3, np.float16, 2, 6, 2, 512, 40, 0, True, 60),      # 1 KiB rows, 40 rotated
]


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("case", SHAPES, ids=[str(i) for i in range(len(SHAPES))])
def test_rope_sweep(case, policy):
    rank, dt, B, S, H, D, R, il, has_ids, M = case
    rpe.set_kernel_policy(policy)
    Rf = R or D
    shape = (B, S, H * D) if rank == 3 else (B, H, S, D)
    x = normal_tensor(1000 + B * S * H + D, shape, dt)
    if has_ids:
        cos, sin = angle_table(2000 + D, M, Rf // 2, dt)
        ids = ids_in(3000 + S, (B, S), M + 3) - 1        # some -1 and some >= M
        ids[0, 0] = 0
    else:
        cos, sin = angle_table(2001 + D, B * S, Rf // 2, dt)
        cos, sin = cos.reshape(B, S, -1), sin.reshape(B, S, -1)
        ids = None
    nh = H if rank == 3 else 0
    want = oracle.rope_apply(x, cos, sin, ids, interleaved=il, num_heads=nh, rotary_embedding_dim=R)
    got = host(rpe.rope_apply(cuda(x), cuda(cos), cuda(sin), None if ids is None else cuda(ids),
                              interleaved=il, num_heads=nh, rotary_embedding_dim=R))
    assert_parity(got, want, str(case))
    xd = x if rank == 4 else x.reshape(B, S, H, D)
    gd = got if rank == 4 else got.reshape(B, S, H, D)
    assert_bitwise(gd[..., Rf:], xd[..., Rf:], "tail")
    if ids is not None:
        bad = (ids < 0) | (ids >= M)
        b, s = np.nonzero(bad)
        if rank == 4:
            assert_bitwise(got[b, :, s], x[b, :, s], "out-of-range rows")
        else:
            assert_bitwise(got[b, s], x[b, s], "out-of-range rows")


@pytest.mark.parametrize("dt", [np.float16, np.float32, BFLOAT16])
@pytest.mark.parametrize("il", [0, 1])
def test_gather_probe_bitexact(dt, il):
    B, H, S, D, M = 3, 4, 29, 128, 777
    cos, sin = angle_table(4000, M, D // 2, dt)
    ids = ids_in(4001, (B, S), M)
    j1, j2 = pair_index(il, D // 2)
    x = np.zeros((B, H, S, D), dt)
    x[..., j1] = one(dt)
    y = host(rpe.rope_apply(cuda(x), cuda(cos), cuda(sin), cuda(ids), interleaved=il))
    for h in range(H):
        assert_bitwise(y[:, h][..., j1], cos[ids], "probe cos")
        assert_bitwise(y[:, h][..., j2], sin[ids], "probe sin")


def test_in_place_and_canaries():
    B, S, H, D, M = 2, 300, 8, 128, 1024
    x = normal_tensor(5000, (B, S, H * D), np.float16)
    cos, sin = angle_table(5001, M, D // 2, np.float16)
    ids = ids_in(5002, (B, S), M)
    want = oracle.rope_apply(x, cos, sin, ids, num_heads=H)
    # in place
    xt = cuda(x)
    out = rpe.rope_apply(xt, cuda(cos), cuda(sin), cuda(ids), num_heads=H, out=xt)
    assert out.data_ptr() == xt.data_ptr()
    assert_parity(host(xt), want, "in place")
    # y inside a poisoned buffer: every element overwritten, canaries untouched
    n = x.size
    pad = 4096
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV)
    buf.view(torch.int16)[:] = 0x7e11                      # NaN with a payload
    y = buf[pad:pad + n].view(B, S, H * D)
    rpe.rope_apply(cuda(x), cuda(cos), cuda(sin), cuda(ids), num_heads=H, out=y)
    whole = bits(host(buf))
    assert (whole[:pad] == 0x7e11).all() and (whole[pad + n:] == 0x7e11).all(), "canary overwritten"
    assert_parity(host(y), want, "poisoned output")


def test_empty_inputs_launch_nothing():
    for shape, ids_shape in (((0, 4, 64), (0, 4)), ((2, 0, 64), (2, 0))):
        x = torch.empty(shape, dtype=torch.float16, device=DEV)
        cos = torch.zeros(8, 16, dtype=torch.float16, device=DEV)
        ids = torch.zeros(ids_shape, dtype=torch.int64, device=DEV)
        y = rpe.rope_apply(x, cos, cos, ids, num_heads=2)
        assert y.shape == shape


def test_empty_inputs_every_op():
    """Zero tokens: every op returns at once and touches nothing (a cache
    guard value stays)."""
    f16 = dict(dtype=torch.float16, device=DEV)
    cos = torch.zeros(8, 16, **f16)
    w = torch.ones(32, **f16)
    for B, S in ((0, 3), (2, 0)):
        q = torch.empty(B, S, 4 * 32, **f16)
        k = torch.empty(B, S, 2 * 32, **f16)
        ids = torch.zeros(B, S, dtype=torch.int64, device=DEV)
        ids3 = torch.zeros(3, B, S, dtype=torch.int64, device=DEV)
        assert rpe.mrope_apply(q, ids3, cos, cos, mrope_section=(8, 4, 4), num_heads=4).shape == q.shape
        yq, yk = rpe.rope_apply_qk(q, k, cos, cos, ids, num_heads=4, kv_num_heads=2)
        assert yq.shape == q.shape and yk.shape == k.shape
        yq, yk = rpe.rope_apply_qk_norm(q, k, w, w, cos, cos, ids, epsilon=1e-6, num_heads=4, kv_num_heads=2)
        assert yq.shape == q.shape and yk.shape == k.shape
        qkv = torch.empty(B, S, 8 * 32, **f16)
        assert rpe.rope_apply_qkv_packed(qkv, cos, cos, ids, num_heads=4, kv_num_heads=2).shape == qkv.shape
        pk = torch.full((max(B, 1), 2, 8, 32), 7.0, **f16)[:B]
        pv = pk.clone()
        lens = torch.full((B,), max(S, 1), dtype=torch.int32, device=DEV)
        out = rpe.rope_kv_append(q, k, k, pk, pv, lens, max(S, 1) if B else S, cos, cos,
                                 num_heads=4, kv_num_heads=2)
        assert out.shape == q.shape
        out = rpe.rope_kv_append_qk_norm(q, k, k, pk, pv, lens, max(S, 1) if B else S, cos, cos, w, w,
                                         epsilon=1e-6, num_heads=4, kv_num_heads=2)
        assert out.shape == q.shape
        torch.cuda.synchronize()
        assert bool((pk == 7.0).all()) and bool((pv == 7.0).all())


def test_errors_raise():
    x = torch.zeros(2, 3, 64, dtype=torch.float16, device=DEV)
    cos = torch.zeros(8, 16, dtype=torch.float16, device=DEV)
    ids = torch.zeros(2, 3, dtype=torch.int64, device=DEV)
    with pytest.raises(rpe.RopeError) as e:
        rpe.rope_apply(x, cos, cos, ids, num_heads=3)
    assert e.value.status_name == "ROPE_ERR_SHAPE"
    with pytest.raises(rpe.RopeError):
        rpe.rope_apply(x, cos.float(), cos.float(), ids, num_heads=2)
    # the cache append allocates q_out itself: a query of the wrong rank or a
    # zero head count still reaches the library, whose status names the clause
    pk = torch.zeros(2, 2, 8, 32, dtype=torch.float16, device=DEV)
    lens = torch.full((2,), 4, dtype=torch.int32, device=DEV)
    with pytest.raises(rpe.RopeError) as e:
        rpe.rope_kv_append(x.view(6, 64), None, None, pk, pk.clone(), lens, 4, cos, cos,
                           num_heads=2, kv_num_heads=2)
    assert e.value.status_name == "ROPE_ERR_RANK"
    with pytest.raises(rpe.RopeError) as e:
        rpe.rope_kv_append_qk_norm(x, None, None, pk, pk.clone(), lens, 4, cos, cos, cos[0], cos[0],
                                   epsilon=1e-6, num_heads=0, kv_num_heads=0)
    assert e.value.status_name == "ROPE_ERR_ATTRIBUTE"


# ---------------------------------------------------------------------------
# M-RoPE

MROPE = [
    # rank, dt, B, S, H, D, R, section, interleaved, scale
    (4, np.float16, 2, 45, 3, 128, 0, (16, 24, 24), 0, 1.0),
    (3, np.float16, 2, 33, 4, 128, 0, (24, 20, 20), 1, 1.0),
    (4, np.float32, 1, 50, 2, 64, 0, (10, 11, 11), 0, 2.0),
    (3, np.float32, 3, 17, 3, 96, 64, (8, 12, 12), 1, 0.5),
    (4, np.float16, 2, 20, 2, 9, 8, (2, 1, 1), 0, 1.0),      # odd head size, scalar kernel
    (4, np.float16, 2, 21, 5, 80, 48, (0, 12, 12), 0, 1.25),
    (3, np.float16, 1, 40, 2, 256, 0, (40, 44, 44), 1, 1.0),
    (4, BFLOAT16, 2, 45, 3, 128, 0, (16, 24, 24), 0, 1.0),
    (3, BFLOAT16, 2, 33, 4, 128, 0, (24, 20, 20), 1, 1.25),
    (4, BFLOAT16, 2, 20, 2, 9, 8, (2, 1, 1), 0, 1.0),
    (3, np.float16, 64, 1, 28, 128, 0, (16, 24, 24), 0, 1.0),   # decode-like
    (3, np.float16, 3, 7, 4, 128, 64, (8, 12, 12), 1, 1.5),     # partial, tail chunks, scaled
    (3, np.float32, 2, 9, 2, 256, 0, (40, 44, 44), 0, 1.0),     # 1 KiB rows
    (3, np.float32, 2, 9, 3, 32, 0, (4, 6, 6), 1, 1.0),         # 128-byte rows, interleaved
]


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("case", MROPE, ids=[str(i) for i in range(len(MROPE))])
def test_mrope_sweep(case, policy, layout):
    rank, dt, B, S, H, D, R, sec, il, scale = case
    rpe.set_kernel_policy(policy)
    Rf = R or D
    M = 97
    shape = (B, S, H * D) if rank == 3 else (B, H, S, D)
    x = normal_tensor(6000 + D + S, shape, dt)
    cos, sin = angle_table(6001 + D, M, Rf // 2, dt)
    ids = ids_in(6002 + S, (3, B, S), M + 4) - 2
    ids[:, 0, 0] = (0, 1, 2)
    ids[1, -1, -1] = 2 ** 40
    ids[2, -1, S - 2 if S > 1 else 0] = -(2 ** 40)
    want = oracle.mrope_apply(x, ids, cos, sin, sec, layout, interleaved=il, num_heads=H,
                              rotary_embedding_dim=R, scale=scale)
    got = host(rpe.mrope_apply(cuda(x), cuda(ids), cuda(cos), cuda(sin), mrope_section=sec,
                               mrope_layout=layout, interleaved=il, num_heads=H,
                               rotary_embedding_dim=R, scale=scale))
    assert_parity(got, want, str(case))
    # copies are bit-exact
    xd = x if rank == 4 else x.reshape(B, S, H, D).transpose(0, 2, 1, 3)
    gd = got if rank == 4 else got.reshape(B, S, H, D).transpose(0, 2, 1, 3)
    assert_bitwise(np.ascontiguousarray(gd[..., Rf:]), np.ascontiguousarray(xd[..., Rf:]), "tail")
    streams = oracle.mrope_slot_streams(Rf // 2, sec, layout)
    sid = ids[streams]
    oob = (sid < 0) | (sid >= M)
    i, b, s = np.nonzero(oob)
    j1, j2 = pair_index(il, Rf // 2)
    for j in (j1[i], j2[i]):
        assert_bitwise(gd[b, :, s, j], xd[b, :, s, j], "out-of-range pairs")


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("case", [(3, np.float16, 48, 1, 28, 128), (3, BFLOAT16, 8, 5, 4, 128),
                                  (4, np.float16, 2, 33, 3, 64), (3, np.float32, 16, 1, 4, 64)],
                         ids=["decode_f16", "bf16", "rank4", "decode_f32"])
def test_mrope_text_and_image_tokens(case, policy, layout):
    """Tokens whose three stream positions are equal (text) mixed with tokens
    whose streams differ (image patches), including equal positions outside
    the table (every pair kept) and a single stream out of range: the
    kernels' one-row path for equal positions against the oracle."""
    rank, dt, B, S, H, D = case
    rpe.set_kernel_policy(policy)
    M = 211
    shape = (B, S, H * D) if rank == 3 else (B, H, S, D)
    x = normal_tensor(6500 + B + S, shape, dt)
    cos, sin = angle_table(6501 + D, M, D // 2, dt)
    g = SplitMix64(6502 + B * S)
    ids = ids_in(6503 + S, (3, B, S), M)
    text = g.below(B * S, 3).reshape(B, S) != 0            # about 2/3 text tokens
    ids[1][text] = ids[0][text]
    ids[2][text] = ids[0][text]
    flat = ids.reshape(3, -1)
    flat[:, 0] = -3                                          # equal and below the table
    flat[:, -1] = M + 7                                      # equal and past the table
    if flat.shape[1] > 2:
        flat[1, 1] = 2 ** 40                                 # one stream out of range
    sec = (16, 24, 24) if D == 128 else (8, 12, 12)
    want = oracle.mrope_apply(x, ids, cos, sin, sec, layout, num_heads=H)
    got = host(rpe.mrope_apply(cuda(x), cuda(ids), cuda(cos), cuda(sin), mrope_section=sec,
                               mrope_layout=layout, num_heads=H))
    assert_parity(got, want, "%s policy %d layout %d" % (case, policy, layout))
    xd = x if rank == 4 else x.reshape(B, S, H, D).transpose(0, 2, 1, 3)
    gd = got if rank == 4 else got.reshape(B, S, H, D).transpose(0, 2, 1, 3)
    b0, s0 = np.unravel_index(0, (B, S))
    b1, s1 = np.unravel_index(B * S - 1, (B, S))
    assert_bitwise(gd[b0, :, s0], xd[b0, :, s0], "equal positions below the table")
    assert_bitwise(gd[b1, :, s1], xd[b1, :, s1], "equal positions past the table")


def test_mrope_equal_streams_equal_rope_on_gpu():
    B, H, S, D, M = 2, 6, 77, 128, 500
    x = cuda(normal_tensor(7000, (B, H, S, D), np.float16))
    cos, sin = (cuda(a) for a in angle_table(7001, M, D // 2, np.float16))
    ids = ids_in(7002, (B, S), M)
    ids3 = cuda(np.stack([ids, ids, ids]))
    a = host(rpe.rope_apply(x, cos, sin, cuda(ids)))
    for layout in (0, 1):
        b = host(rpe.mrope_apply(x, ids3, cos, sin, mrope_section=(16, 24, 24), mrope_layout=layout))
        assert_bitwise(b, a, "equal streams layout %d" % layout)


# ---------------------------------------------------------------------------
# Q + K

QK = [
    # rank, dt, B, S, H, Hk, D, R, il
    (3, np.float16, 7, 1, 8, 2, 128, 0, 0),
    (4, np.float16, 3, 17, 4, 4, 64, 0, 1),
    (3, np.float32, 2, 9, 6, 2, 96, 64, 1),
    (4, np.float32, 2, 5, 4, 1, 128, 0, 0),
    (3, np.float16, 3, 4, 4, 2, 10, 0, 0),   # scalar kernel
    (3, BFLOAT16, 7, 1, 8, 2, 128, 0, 0),
    (4, BFLOAT16, 3, 17, 4, 4, 64, 0, 1),
    (3, np.float16, 5, 3, 8, 2, 96, 24, 0),  # pairs off the 16-byte chunks
    (3, BFLOAT16, 3, 6, 4, 2, 80, 20, 1),
]


@pytest.mark.parametrize("onthefly", [False, True])
@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("case", QK, ids=[str(i) for i in range(len(QK))])
def test_qk_sweep(case, policy, onthefly):
    rank, dt, B, S, H, Hk, D, R, il = case
    rpe.set_kernel_policy(policy)
    Rf = R or D
    M = 40000
    q = normal_tensor(8000 + D, (B, S, H * D) if rank == 3 else (B, H, S, D), dt)
    k = normal_tensor(8001 + D, (B, S, Hk * D) if rank == 3 else (B, Hk, S, D), dt)
    ids = ids_in(8002, (B, S), M)
    inv = oracle.inv_freq(1e6, Rf)
    cos, sin = oracle.cos_sin_cache(dt, M, inv, 1.0)
    nh, nk = (H, Hk) if rank == 3 else (0, 0)
    if onthefly:
        want = oracle.rope_apply_qk(q, k, None, None, ids, interleaved=il, num_heads=nh, kv_num_heads=nk,
                                    rotary_embedding_dim=R, inv_freq=inv, attention_scaling=1.0)
        got = rpe.rope_apply_qk(cuda(q), cuda(k), None, None, cuda(ids), interleaved=il, num_heads=nh,
                                kv_num_heads=nk, rotary_embedding_dim=R, inv_freq=cuda(inv))
    else:
        want = oracle.rope_apply_qk(q, k, cos, sin, ids, interleaved=il, num_heads=nh, kv_num_heads=nk,
                                    rotary_embedding_dim=R)
        got = rpe.rope_apply_qk(cuda(q), cuda(k), cuda(cos), cuda(sin), cuda(ids), interleaved=il,
                                num_heads=nh, kv_num_heads=nk, rotary_embedding_dim=R)
    assert_parity(host(got[0]), want[0], "Q " + str(case))
    assert_parity(host(got[1]), want[1], "K " + str(case))


def test_qk_in_place():
    B, S, H, Hk, D = 16, 1, 8, 2, 128
    q = normal_tensor(9000, (B, S, H * D), np.float16)
    k = normal_tensor(9001, (B, S, Hk * D), np.float16)
    ids = ids_in(9002, (B, S), 4096)
    inv = oracle.inv_freq(1e6, D)
    cos, sin = oracle.cos_sin_cache(np.float16, 4096, inv)
    want = oracle.rope_apply_qk(q, k, cos, sin, ids, num_heads=H, kv_num_heads=Hk)
    qt, kt = cuda(q), cuda(k)
    rpe.rope_apply_qk(qt, kt, cuda(cos), cuda(sin), cuda(ids), num_heads=H, kv_num_heads=Hk,
                      out_q=qt, out_k=kt)
    assert_parity(host(qt), want[0], "Q in place")
    assert_parity(host(kt), want[1], "K in place")


# ---------------------------------------------------------------------------
# packed [Q|K|V]

PACKED = [
    # rank, dt, B, S, H, Hk, D, R, il
    (3, np.float16, 256, 1, 32, 8, 128, 0, 0),
    (3, np.float16, 3, 37, 8, 2, 128, 0, 1),
    (4, np.float16, 2, 29, 4, 2, 64, 0, 0),
    (3, np.float32, 2, 11, 6, 3, 96, 64, 1),
    (4, np.float32, 2, 13, 2, 1, 128, 0, 0),
    (3, np.float16, 2, 7, 4, 2, 10, 0, 0),     # scalar kernel
    (3, BFLOAT16, 256, 1, 32, 8, 128, 0, 0),
    (3, BFLOAT16, 3, 37, 8, 2, 128, 0, 1),
]


def split_packed(qkv, rank, H, Hk):
    if rank == 3:
        B, S, W = qkv.shape
        D = W // (H + 2 * Hk)
        return (np.ascontiguousarray(qkv[..., :H * D]), np.ascontiguousarray(qkv[..., H * D:(H + Hk) * D]),
                np.ascontiguousarray(qkv[..., (H + Hk) * D:]))
    return (np.ascontiguousarray(qkv[:, :H]), np.ascontiguousarray(qkv[:, H:H + Hk]),
            np.ascontiguousarray(qkv[:, H + Hk:]))


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("onthefly", [False, True])
@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("case", PACKED, ids=[str(i) for i in range(len(PACKED))])
def test_qkv_packed(case, policy, onthefly, inplace):
    rank, dt, B, S, H, Hk, D, R, il = case
    rpe.set_kernel_policy(policy)
    Rf = R or D
    M = 40000
    shape = (B, S, (H + 2 * Hk) * D) if rank == 3 else (B, H + 2 * Hk, S, D)
    qkv = normal_tensor(9100 + D + S, shape, dt)
    ids = ids_in(9101, (B, S), M)
    inv = oracle.inv_freq(1e6, Rf)
    q, k, v = split_packed(qkv, rank, H, Hk)
    nh, nk = (H, Hk) if rank == 3 else (0, 0)
    if onthefly:
        wq, wk = oracle.rope_apply_qk(q, k, None, None, ids, interleaved=il, num_heads=nh, kv_num_heads=nk,
                                      rotary_embedding_dim=R, inv_freq=inv)
        tabs = dict(cos_cache=None, sin_cache=None, inv_freq=cuda(inv))
    else:
        cos, sin = oracle.cos_sin_cache(dt, M, inv)
        wq, wk = oracle.rope_apply_qk(q, k, cos, sin, ids, interleaved=il, num_heads=nh, kv_num_heads=nk,
                                      rotary_embedding_dim=R)
        tabs = dict(cos_cache=cuda(cos), sin_cache=cuda(sin))
    xt = cuda(qkv)
    y = rpe.rope_apply_qkv_packed(xt, position_ids=cuda(ids), interleaved=il, num_heads=H, kv_num_heads=Hk,
                                  rotary_embedding_dim=R, out=xt if inplace else None, **tabs)
    gq, gk, gv = split_packed(host(y), rank, H, Hk)
    assert_parity(gq, wq, "Q " + str(case))
    assert_parity(gk, wk, "K " + str(case))
    assert_bitwise(gv, v, "V")


@pytest.mark.parametrize("onthefly", [False, True])
def test_qkv_packed_prefill_size(onthefly):
    """A packed [Q|K|V] prefill of 4 x 2048 tokens (32 + 8 + 8 heads of 128,
    fp16) in the default launch configuration: more than one round of waves,
    so the three tasks' waves run in token-group order."""
    B, S, H, Hk, D, M = 4, 2048, 32, 8, 128, 8192
    qkv = normal_tensor(9150, (B, S, (H + 2 * Hk) * D), np.float16)
    ids = ids_in(9151, (B, 1), 4096) + np.arange(S, dtype=np.int64)[None, :]
    inv = oracle.inv_freq(1e6, D)
    q, k, v = split_packed(qkv, 3, H, Hk)
    if onthefly:
        wq, wk = oracle.rope_apply_qk(q, k, None, None, ids, num_heads=H, kv_num_heads=Hk, inv_freq=inv)
        tabs = dict(cos_cache=None, sin_cache=None, inv_freq=cuda(inv))
    else:
        cos, sin = oracle.cos_sin_cache(np.float16, M, inv)
        wq, wk = oracle.rope_apply_qk(q, k, cos, sin, ids, num_heads=H, kv_num_heads=Hk)
        tabs = dict(cos_cache=cuda(cos), sin_cache=cuda(sin))
    y = rpe.rope_apply_qkv_packed(cuda(qkv), position_ids=cuda(ids), num_heads=H, kv_num_heads=Hk, **tabs)
    gq, gk, gv = split_packed(host(y), 3, H, Hk)
    log("packed prefill onthefly=%s Q %s K %s" % (onthefly, assert_parity(gq, wq, "Q"), assert_parity(gk, wk, "K")))
    assert_bitwise(gv, v, "V")


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
def test_empty_table_copies_everything(policy):
    """M = 0 rows: every id is out of range, so Y == X bit for bit (the vector
    kernel reads a substitute row and discards it)."""
    rpe.set_kernel_policy(policy)
    x = normal_tensor(9300, (2, 9, 4 * 128), np.float16)
    ids = ids_in(9301, (2, 9), 5)
    cos = torch.empty(0, 64, dtype=torch.float16, device=DEV)
    y = host(rpe.rope_apply(cuda(x), cos, cos.clone(), cuda(ids), num_heads=4))
    assert_bitwise(y, x, "empty table")
    x4 = normal_tensor(9302, (2, 4, 9, 128), np.float16)
    ids3 = ids_in(9303, (3, 2, 9), 5)
    y4 = host(rpe.mrope_apply(cuda(x4), cuda(ids3), cos, cos.clone(), mrope_section=(16, 24, 24)))
    assert_bitwise(y4, x4, "empty table, M-RoPE")


# ---------------------------------------------------------------------------
# 64-bit addressing: more than 2^31 elements (4 GiB of float16 in and out)

@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
def test_more_than_2_31_elements(policy):
    """X (1, 524291, 4096) float16 = 2^31 + 12288 elements, made on the GPU by
    torch's seeded generator (not by this library); sampled token rows, among
    them the ones past the 2^31-element and 4 GiB marks, against the oracle."""
    rpe.set_kernel_policy(policy)
    S, H, D, M = 524291, 32, 128, 8192
    gen = torch.Generator(device=DEV)
    gen.manual_seed(0x5EED)
    x = torch.randn((1, S, H * D), generator=gen, dtype=torch.float16, device=DEV)
    ids_h = ((np.arange(S, dtype=np.int64) * 7 + 3) % M).reshape(1, S)
    inv = oracle.inv_freq(1e6, D)
    cos, sin = oracle.cos_sin_cache(np.float16, M, inv)
    y = rpe.rope_apply(x, cuda(cos), cuda(sin), cuda(ids_h), num_heads=H)
    torch.cuda.synchronize()
    picks = np.unique(np.concatenate([
        [0, 1, S // 2, 524287, 524288, 524289, S - 2, S - 1],
        ids_in(0x5EEE, (64,), S)]))
    sel = torch.from_numpy(picks).to(DEV)
    xs = host(x[0].index_select(0, sel))[None]                 # (1, k, H*D)
    ys = host(y[0].index_select(0, sel))[None]
    want = oracle.rope_apply(xs, cos, sin, ids_h[:, picks], num_heads=H)
    r = assert_parity(ys, want, "rows %s" % picks[:8].tolist())
    print("2^31+ elements policy=%d rows=%d %s" % (policy, picks.size, r), flush=True)
    del x, y
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# degenerate values: signed zeros, infinities, NaN, subnormals, the largest
# finite values (rotations by unit-bounded coefficients cannot overflow a
# binary32 product, so the binary32 path and the oracle meet the same
# overflows)

def _special_values(dt):
    if np.dtype(dt) == np.float16:
        v = [0.0, -0.0, np.inf, -np.inf, np.nan, 6.0e-8, -6.0e-8, 6.1e-5, 65504.0, -65504.0, 1.0, -3.5]
        return np.array(v, np.float16)
    if np.dtype(dt) == np.float32:
        v = [0.0, -0.0, np.inf, -np.inf, np.nan, 1.4e-45, -1.4e-45, 1.2e-38, 3.4e38, -3.4e38, 1.0, -3.5]
        return np.array(v, np.float32)
    from rope_inputs import bfloat16_bits
    f = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 9.2e-41, -9.2e-41, 1.2e-38, 3.38e38, -3.38e38, 1.0, -3.5],
                 np.float32)
    bits_ = bfloat16_bits(np.where(np.isfinite(f), f, 0.0))
    bits_[2], bits_[3], bits_[4] = 0x7f80, 0xff80, 0x7fc1
    return bits_


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("dt", [np.float16, np.float32, BFLOAT16])
@pytest.mark.parametrize("il", [0, 1])
def test_special_values(dt, il, policy):
    rpe.set_kernel_policy(policy)
    B, S, H, D, M = 2, 24, 3, 64, 6
    sv = _special_values(dt)
    pick = ids_in(14000 + il, (B, S, H, D), sv.size)
    x = sv[pick]
    x = np.ascontiguousarray(x.reshape(B, S, H * D))
    th = np.array([0.0, np.pi / 2, np.pi, np.pi / 4, 1.0, 2.5])
    c = np.cos(th)[:, None] * np.ones((1, D // 2))
    s = np.sin(th)[:, None] * np.ones((1, D // 2))
    if np.dtype(dt) == BFLOAT16:
        from rope_inputs import bfloat16_bits
        cos, sin = bfloat16_bits(c.astype(np.float32)), bfloat16_bits(s.astype(np.float32))
    else:
        cos, sin = c.astype(dt), s.astype(dt)
    ids = ids_in(14002, (B, S), M)
    want = oracle.rope_apply(x, cos, sin, ids, interleaved=il, num_heads=H)
    got = host(rpe.rope_apply(cuda(x), cuda(cos), cuda(sin), cuda(ids), interleaved=il, num_heads=H))
    what = "special values dt=%s il=%d" % (np.dtype(dt).name, il)
    r = assert_parity(got, want, what)
    if np.dtype(dt) == np.float32:
        # binary32: both products exact in binary64 and one rounding there, as
        # in the oracle, so every non-NaN result (overflow to inf included)
        # has the oracle's bits
        keep = ~np.isnan(want)
        assert_bitwise(got[keep], want[keep], what + " (bits)")
    log("special values %s il=%d policy=%d %s" % (np.dtype(dt).name, il, policy, r))


def test_side_streams():
    """Calls are enqueued on the caller's current stream: two side streams run
    independent problems concurrently, and each result equals the oracle once
    its own stream is synchronised."""
    B, S, H, D, M = 2, 300, 8, 128, 1024
    inv = oracle.inv_freq(1e6, D)
    cos, sin = oracle.cos_sin_cache(np.float16, M, inv)
    cos_t, sin_t = cuda(cos), cuda(sin)
    cases = []
    for i in range(2):
        x = normal_tensor(15000 + i, (B, S, H * D), np.float16)
        ids = ids_in(15010 + i, (B, S), M)
        cases.append((x, ids, cuda(x), cuda(ids)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for (x, ids, xt, it), st in zip(cases, streams):
        with torch.cuda.stream(st):
            y = torch.empty_like(xt)
            for _ in range(20):
                rpe.rope_apply(xt, cos_t, sin_t, it, num_heads=H, out=y)
            outs.append(y)
    for (x, ids, _xt, _it), st, y in zip(cases, streams, outs):
        st.synchronize()
        want = oracle.rope_apply(x, cos, sin, ids, num_heads=H)
        assert_parity(y.cpu().numpy(), want, "side stream")


def test_hip_graph_capture_and_replay():
    """The entry points allocate nothing and never synchronise, so a decode
    step (a Q+K rotation and a cache append on its own inputs) can be
    captured in a HIP graph. Replayed several times with new inputs copied in
    eagerly between replays; every replay is checked against the oracle."""
    B, H, Hk, D, M, Smax = 32, 8, 2, 128, 4096, 64
    inv = oracle.inv_freq(1e6, D)
    cos, sin = oracle.cos_sin_cache(np.float16, M, inv)
    cos_t, sin_t = cuda(cos), cuda(sin)
    q_in = torch.empty(B, 1, H * D, dtype=torch.float16, device=DEV)
    k_in = torch.empty(B, 1, Hk * D, dtype=torch.float16, device=DEV)
    ids_t = torch.empty(B, 1, dtype=torch.int64, device=DEV)
    q2_in, k2_in, v2_in = torch.empty_like(q_in), torch.empty_like(k_in), torch.empty_like(k_in)
    lens_t = torch.empty(B, dtype=torch.int32, device=DEV)
    yq, yk, q_out = torch.empty_like(q_in), torch.empty_like(k_in), torch.empty_like(q_in)
    pk = torch.zeros(B, Hk, Smax, D, dtype=torch.float16, device=DEV)
    pv = torch.zeros_like(pk)

    def step():
        rpe.rope_apply_qk(q_in, k_in, cos_t, sin_t, ids_t, num_heads=H, kv_num_heads=Hk, out_q=yq, out_k=yk)
        rpe.rope_kv_append(q2_in, k2_in, v2_in, pk, pv, lens_t, Smax, cos_t, sin_t, num_heads=H,
                           kv_num_heads=Hk, out=q_out)

    lens_t.fill_(1)
    ids_t.zero_()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):     # warm-up outside the graph
        step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        q = normal_tensor(16000 + rep, (B, 1, H * D), np.float16)
        k = normal_tensor(16100 + rep, (B, 1, Hk * D), np.float16)
        q2 = normal_tensor(16500 + rep, (B, 1, H * D), np.float16)
        k2 = normal_tensor(16600 + rep, (B, 1, Hk * D), np.float16)
        v2 = normal_tensor(16200 + rep, (B, 1, Hk * D), np.float16)
        ids = ids_in(16300 + rep, (B, 1), M)
        lens = (ids_in(16400 + rep, (B,), Smax) + 1).astype(np.int32)
        for t, a in ((q_in, q), (k_in, k), (q2_in, q2), (k2_in, k2), (v2_in, v2), (ids_t, ids), (lens_t, lens)):
            t.copy_(cuda(a))
        pk_before, pv_before = host(pk), host(pv)
        g.replay()
        torch.cuda.synchronize()
        wq, wk = oracle.rope_apply_qk(q, k, cos, sin, ids, num_heads=H, kv_num_heads=Hk)
        assert_parity(host(yq), wq, "replay %d Q" % rep)
        assert_parity(host(yk), wk, "replay %d K" % rep)
        eq, ek, ev = oracle.rope_kv_append(q2, k2, v2, pk_before, pv_before, lens, Smax, cos, sin, H, Hk)
        assert_parity(host(q_out), eq, "replay %d q_out" % rep)
        assert_parity(host(pk), ek, "replay %d key cache" % rep)
        assert_bitwise(host(pv), ev, "replay %d value cache" % rep)
