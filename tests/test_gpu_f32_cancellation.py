"""GPU parity for float32 storage where the two products of a rotation nearly
cancel: x1*c close to x2*s (first output) or x2*c close to -x1*s (second
output), magnitudes up to 1e4.

The stated float32 bound is |gpu - oracle| <= 2e-6 * max(1, |y|). Under
cancellation |y| is tiny next to the products, so any rounding of a product
before the difference shows up at the products' scale. The kernels form both
products in binary64, where they are exact, and round the sum once to
binary64 and once to binary32 -- the oracle's own evaluation of the
definition ("ai.onnx.RotaryEmbedding" manifest, description; onnxruntime PR
#27590 review, rotate_half) -- so besides the stated bound the results are
checked bit for bit. Every op that rotates float32 data runs under all four
kernel policies (automatic, scalar, vector only, row wherever it applies).
"""
import numpy as np
import pytest
import torch

import oracle
import rotary_position_embedding_amd as rpe
from gpu_io import POLICIES, POLICY_IDS, cuda, host
from oracle_pins import angle_table, ids_in, pair_index
from parity import assert_bitwise, assert_parity
from rope_inputs import SplitMix64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _policy():
    old = rpe.set_kernel_policy(0)
    yield
    rpe.set_kernel_policy(old)


def log(msg):
    print(msg, flush=True)


def cancelling_rows(seed, c, s, D, interleaved):
    """float32 head rows (..., D) whose pairs use coefficients c, s (..., D/2
    or fewer: the first R/2 = c.shape[-1] pairs rotate, the rest is the tail).
    Pair magnitudes are log-uniform in [1e-2, 1e4]; a third of the pairs take
    x1 = rnd(x2*s/c) (the first output cancels), a third x1 = rnd(-x2*c/s) (the
    second output cancels), each then moved by 0-3 binary32 steps so the
    remaining difference varies; the rest are random. Tail elements are
    random at the same magnitudes."""
    half = c.shape[-1]
    lead = c.shape[:-1]
    n = int(np.prod(lead)) * half
    g = SplitMix64(seed)
    mag = 10.0 ** (g.uniform(n) * 6.0 - 2.0)
    x2 = g.normal(n) * mag
    x1 = g.normal(n) * mag
    kind = g.below(n, 3)
    steps = g.below(n, 4)
    cf = c.reshape(-1).astype(np.float64)
    sf = s.reshape(-1).astype(np.float64)
    x2 = x2.astype(np.float32).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        a = np.where((kind == 0) & (np.abs(cf) > 0.05), x2 * sf / cf, x1)
        a = np.where((kind == 1) & (np.abs(sf) > 0.05), -x2 * cf / sf, a)
    x1 = a.astype(np.float32)
    for k in range(1, 4):
        x1 = np.where(steps >= k, np.nextafter(x1, np.float32(np.inf)), x1)
    rows = (g.normal(int(np.prod(lead)) * D) * np.repeat(mag[::half], D)).astype(np.float32)
    rows = rows.reshape(lead + (D,))
    j1, j2 = pair_index(interleaved, half)
    rows[..., j1] = x1.reshape(lead + (half,))
    rows[..., j2] = x2.astype(np.float32).reshape(lead + (half,))
    return rows


def check(got, want, what):
    r = assert_parity(got, want, what)
    assert_bitwise(got, want, what)
    log("%s: %s" % (what, r))


# (rank, B, S, H, D, R, interleaved, table): "ids" gathers an (M, R/2) table,
# "token" is a per-token (B, S, R/2) table
ROPE_CASES = [
    (3, 2, 37, 5, 128, 0, 0, "ids"),
    (4, 2, 29, 3, 96, 64, 1, "ids"),      # partial interleaved, tail of 32
    (3, 3, 1, 32, 128, 0, 0, "ids"),      # decode-sized
    (4, 1, 50, 4, 64, 0, 0, "token"),
    (3, 2, 21, 4, 80, 48, 0, "ids"),      # partial split halves
    (3, 2, 13, 3, 6, 0, 1, "ids"),        # rows of 24 bytes: not 16-byte items
    (3, 1, 9, 2, 512, 256, 0, "ids"),     # 2 KiB rows
]


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("case", ROPE_CASES, ids=[str(i) for i in range(len(ROPE_CASES))])
def test_rope_apply_f32_cancellation(case, policy):
    rank, B, S, H, D, R, il, table = case
    rpe.set_kernel_policy(policy)
    half = (R or D) // 2
    M = 97
    if table == "ids":
        cos, sin = angle_table(21000 + D, M, half, np.float32)
        ids = ids_in(21100 + S, (B, S), M)
        c, s = cos[ids], sin[ids]                        # (B, S, half)
    else:
        cos, sin = angle_table(21001 + D, B * S, half, np.float32)
        cos, sin = cos.reshape(B, S, half), sin.reshape(B, S, half)
        ids = None
        c, s = cos, sin
    rows = cancelling_rows(21200 + D + S, np.broadcast_to(c[:, :, None], (B, S, H, half)),
                           np.broadcast_to(s[:, :, None], (B, S, H, half)), D, il)  # (B, S, H, D)
    x = rows.reshape(B, S, H * D) if rank == 3 else np.ascontiguousarray(rows.transpose(0, 2, 1, 3))
    nh = H if rank == 3 else 0
    want = oracle.rope_apply(x, cos, sin, ids, interleaved=il, num_heads=nh, rotary_embedding_dim=R)
    got = host(rpe.rope_apply(cuda(x), cuda(cos), cuda(sin), None if ids is None else cuda(ids),
                              interleaved=il, num_heads=nh, rotary_embedding_dim=R))
    check(got, want, "rope_apply f32 cancellation %s policy %d" % (case, policy))


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("onthefly", [False, True], ids=["table", "onthefly"])
@pytest.mark.parametrize("S", [1, 40])
def test_rope_apply_qk_f32_cancellation(S, onthefly, policy):
    rpe.set_kernel_policy(policy)
    B, H, Hk, D, M = 12, 8, 2, 128, 4096
    inv = oracle.inv_freq(1e6, D)
    cos, sin = oracle.cos_sin_cache(np.float32, M, inv)   # equal to the on-the-fly values
    ids = ids_in(22000 + S, (B, S), M)
    c, s = cos[ids][:, :, None], sin[ids][:, :, None]
    q = cancelling_rows(22100 + S, np.broadcast_to(c, (B, S, H, D // 2)),
                        np.broadcast_to(s, (B, S, H, D // 2)), D, 0).reshape(B, S, H * D)
    k = cancelling_rows(22200 + S, np.broadcast_to(c, (B, S, Hk, D // 2)),
                        np.broadcast_to(s, (B, S, Hk, D // 2)), D, 0).reshape(B, S, Hk * D)
    if onthefly:
        wq, wk = oracle.rope_apply_qk(q, k, None, None, ids, num_heads=H, kv_num_heads=Hk, inv_freq=inv)
        gq, gk = rpe.rope_apply_qk(cuda(q), cuda(k), None, None, cuda(ids), num_heads=H, kv_num_heads=Hk,
                                   inv_freq=cuda(inv))
    else:
        wq, wk = oracle.rope_apply_qk(q, k, cos, sin, ids, num_heads=H, kv_num_heads=Hk)
        gq, gk = rpe.rope_apply_qk(cuda(q), cuda(k), cuda(cos), cuda(sin), cuda(ids), num_heads=H,
                                   kv_num_heads=Hk)
    what = "rope_apply_qk f32 cancellation S=%d %s policy %d" % (S, "on the fly" if onthefly else "table", policy)
    check(host(gq), wq, what + " Q")
    check(host(gk), wk, what + " K")


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("S", [1, 33])
def test_mrope_f32_cancellation(S, layout, policy):
    """M-RoPE with the three streams at one position (a text token), so every
    slot takes its coefficient from the same row whatever the section map."""
    rpe.set_kernel_policy(policy)
    B, H, D, M = 2, 4, 128, 211
    cos, sin = angle_table(23000, M, D // 2, np.float32)
    p = ids_in(23001 + S, (B, S), M)
    ids = np.stack([p, p, p])
    c, s = cos[p][:, None], sin[p][:, None]                                    # (B, 1, S, half)
    x = cancelling_rows(23100 + S + layout, np.broadcast_to(c, (B, H, S, D // 2)),
                        np.broadcast_to(s, (B, H, S, D // 2)), D, 0)         # (B, H, S, D)
    want = oracle.mrope_apply(x, ids, cos, sin, (16, 24, 24), layout, num_heads=H)
    got = host(rpe.mrope_apply(cuda(x), cuda(ids), cuda(cos), cuda(sin), mrope_section=(16, 24, 24),
                               mrope_layout=layout, num_heads=H))
    check(got, want, "mrope f32 cancellation S=%d layout %d policy %d" % (S, layout, policy))


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
def test_kv_append_f32_cancellation(policy):
    """Decode with the cache append: Q to q_out and K into the key cache at
    row past + s, both rotated by that row's coefficients."""
    rpe.set_kernel_policy(policy)
    B, H, Hk, D, Smax, M = 6, 8, 2, 128, 64, 256
    cos, sin = angle_table(24000, M, D // 2, np.float32)
    lens = (ids_in(24001, (B,), Smax) + 1).astype(np.int32)
    pos = lens.astype(np.int64) - 1                                            # S = 1
    c, s = cos[pos][:, None, None], sin[pos][:, None, None]
    q = cancelling_rows(24100, np.broadcast_to(c, (B, 1, H, D // 2)),
                        np.broadcast_to(s, (B, 1, H, D // 2)), D, 0).reshape(B, 1, H * D)
    k = cancelling_rows(24200, np.broadcast_to(c, (B, 1, Hk, D // 2)),
                        np.broadcast_to(s, (B, 1, Hk, D // 2)), D, 0).reshape(B, 1, Hk * D)
    v = cancelling_rows(24300, np.broadcast_to(c, (B, 1, Hk, D // 2)),
                        np.broadcast_to(s, (B, 1, Hk, D // 2)), D, 0).reshape(B, 1, Hk * D)
    past = np.zeros((B, Hk, Smax, D), np.float32)
    wq, wk, wv = oracle.rope_kv_append(q, k, v, past, past, lens, Smax, cos, sin, H, Hk)
    pk, pv = cuda(past), cuda(past)
    gq = rpe.rope_kv_append(cuda(q), cuda(k), cuda(v), pk, pv, cuda(lens), Smax, cuda(cos), cuda(sin),
                            num_heads=H, kv_num_heads=Hk)
    what = "kv_append f32 cancellation policy %d" % policy
    check(host(gq), wq, what + " q_out")
    check(host(pk), wk, what + " key cache")
    assert_bitwise(host(pv), wv, what + " value cache")


# (rank, B, S, H, D, R): launches large enough that interleaved binary32 data
# runs two head batches per wave (the second loaded while the first stores),
# with head counts that leave the last batch partial
PIPELINED = [(3, 4, 1024, 7, 96, 64), (4, 2, 2048, 13, 128, 0), (3, 2, 1500, 11, 64, 32)]


@pytest.mark.parametrize("case", PIPELINED, ids=[str(i) for i in range(len(PIPELINED))])
def test_f32_interleaved_two_batches_per_wave(case):
    rank, B, S, H, D, R = case
    half = (R or D) // 2
    M = 509
    cos, sin = angle_table(25000 + D, M, half, np.float32)
    ids = ids_in(25100 + S, (B, S), M + 5) - 2              # a few ids outside the table
    ok = (ids >= 0) & (ids < M)
    c = np.where(ok[..., None], cos[np.clip(ids, 0, M - 1)], 1.0).astype(np.float32)
    s = np.where(ok[..., None], sin[np.clip(ids, 0, M - 1)], 0.0).astype(np.float32)
    rows = cancelling_rows(25200 + H, np.broadcast_to(c[:, :, None], (B, S, H, half)),
                           np.broadcast_to(s[:, :, None], (B, S, H, half)), D, 1)
    x = rows.reshape(B, S, H * D) if rank == 3 else np.ascontiguousarray(rows.transpose(0, 2, 1, 3))
    nh = H if rank == 3 else 0
    xt = cuda(x)
    yt = torch.empty_like(xt)
    old = rpe.set_kernel_policy(2)       # the vector kernel (the planner gives some of these the row kernel)
    try:
        launch = rpe.rope_apply_launcher(xt, cuda(cos), cuda(sin), cuda(ids), yt, interleaved=1, num_heads=nh,
                                         rotary_embedding_dim=R)
    finally:
        rpe.set_kernel_policy(old)
    assert launch.variant.startswith("vec16"), launch.variant
    launch()
    want = oracle.rope_apply(x, cos, sin, ids, interleaved=1, num_heads=nh, rotary_embedding_dim=R)
    got = host(yt)
    check(got, want, "f32 interleaved, two batches per wave %s" % (case,))
