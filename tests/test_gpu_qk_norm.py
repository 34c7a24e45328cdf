"""GPU parity for QK-norm then RoPE (through the C ABI) against the oracle,
within the tolerance parity.assert_parity_norm derives; kept pairs compare
like rotated ones (they hold the normalised values)."""
import numpy as np
import pytest

import oracle
import rotary_position_embedding_amd as rpe
from gpu_io import cuda, host, POLICIES, POLICY_IDS
from oracle_pins import angle_table, ids_in
from parity import assert_parity_norm
from rope_inputs import BFLOAT16, get, normal_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _policy():
    old = rpe.set_kernel_policy(0)
    yield
    rpe.set_kernel_policy(old)


def as_f64(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def zmax_rows(x, w, eps, rank, heads):
    """max_j |x_j w_j| / rms over each head row, shaped to broadcast over x."""
    xd = as_f64(x)
    if rank == 3:
        B, S, _ = xd.shape
        xd = xd.reshape(B, S, heads, -1)
    rms = np.sqrt((xd ** 2).mean(-1, keepdims=True) + float(np.float32(eps)))
    z = np.abs(xd * as_f64(w)) / rms
    zm = z.max(-1, keepdims=True)
    zm = np.broadcast_to(zm, xd.shape)
    return zm.reshape(x.shape)


def weights(seed, D, dt):
    """RMSNorm weights around 1 (as trained QK-norm weights are)."""
    v = 1.0 + 0.25 * normal_tensor(seed, (D,), np.float32)
    if np.dtype(dt) == BFLOAT16:
        from rope_inputs import bfloat16_bits
        return bfloat16_bits(v)
    return v.astype(dt)


NORM = [
    # rank, dt, B, S, H, Hk, D, R, il, kind
    (3, np.float16, 3, 37, 8, 2, 128, 0, 0, "gather"),
    (3, BFLOAT16, 2, 29, 4, 2, 128, 0, 0, "onthefly"),
    (4, np.float16, 2, 17, 4, 4, 64, 0, 1, "gather"),
    (3, np.float32, 2, 11, 4, 2, 64, 32, 1, "gather"),
    (3, np.float16, 2, 9, 4, 2, 128, 64, 0, "per_token"),
    (4, BFLOAT16, 1, 33, 2, 1, 256, 0, 0, "gather"),
    (3, np.float32, 2, 7, 4, 2, 96, 0, 0, "gather"),       # 384-byte rows: the row kernel's general rows
    (3, np.float16, 3, 11, 6, 3, 96, 0, 0, "gather"),      # 192-byte rows, 5 per instruction
    (3, BFLOAT16, 2, 9, 6, 2, 80, 32, 1, "onthefly"),      # 160-byte rows, partial, interleaved
    (4, np.float16, 2, 13, 4, 2, 96, 64, 0, "per_token"),  # rank 4, partners 4 lanes apart
    (3, np.float16, 2, 6, 3, 1, 192, 0, 0, "gather"),      # 384-byte rows, partners 12 lanes apart
    (3, np.float16, 2, 5, 2, 1, 10, 6, 0, "onthefly"),     # scalar kernel
    (3, np.float16, 64, 1, 32, 8, 128, 0, 0, "onthefly"),  # decode
    (3, np.float32, 2, 5, 2, 1, 256, 0, 0, "gather"),      # 1 KiB rows: the sum over 64 lanes
    (3, np.float16, 2, 9, 4, 2, 16, 0, 0, "onthefly"),     # 32-byte rows
    (3, BFLOAT16, 2, 6, 2, 2, 32, 0, 0, "per_token"),      # partners 2 lanes apart
]


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("case", NORM, ids=[str(i) for i in range(len(NORM))])
def test_qk_norm_sweep(case, policy):
    rank, dt, B, S, H, Hk, D, R, il, kind = case
    rpe.set_kernel_policy(policy)
    Rf = R or D
    M = 300
    eps = 1e-6
    q = normal_tensor(13000 + D + S, (B, S, H * D) if rank == 3 else (B, H, S, D), dt)
    k = normal_tensor(13001 + D + S, (B, S, Hk * D) if rank == 3 else (B, Hk, S, D), dt)
    wq, wk = weights(13002, D, dt), weights(13003, D, dt)
    nh, nk = (H, Hk) if rank == 3 else (0, 0)
    ids = ids_in(13004 + S, (B, S), M + 3) - 1          # some -1 and some >= M
    inv = oracle.inv_freq(1e6, Rf)
    if kind == "onthefly":
        cos = sin = None
        ids = ids_in(13005, (B, S), 40000)
        tabs = dict(cos_cache=None, sin_cache=None, inv_freq=cuda(inv))
    elif kind == "per_token":
        cos, sin = angle_table(13006, B * S, Rf // 2, dt)
        cos, sin = cos.reshape(B, S, -1), sin.reshape(B, S, -1)
        ids = None
        tabs = dict(cos_cache=cuda(cos), sin_cache=cuda(sin))
    else:
        cos, sin = angle_table(13007, M, Rf // 2, dt)
        tabs = dict(cos_cache=cuda(cos), sin_cache=cuda(sin))
    want_q, want_k = oracle.rope_apply_qk_norm(q, k, wq, wk, eps, cos, sin, ids, interleaved=il, num_heads=nh,
                                               kv_num_heads=nk, rotary_embedding_dim=R, inv_freq=inv)
    gq, gk = rpe.rope_apply_qk_norm(cuda(q), cuda(k), cuda(wq), cuda(wk), position_ids=None if ids is None
                                    else cuda(ids), epsilon=eps, interleaved=il, num_heads=nh,
                                    kv_num_heads=nk, rotary_embedding_dim=R, **tabs)
    what = "%s policy=%d" % (str(case), policy)
    rq = assert_parity_norm(host(gq), want_q, zmax_rows(q, wq, eps, rank, H), "Q " + what)
    rk = assert_parity_norm(host(gk), want_k, zmax_rows(k, wk, eps, rank, Hk), "K " + what)
    print(what, rq, rk, flush=True)


def test_qk_norm_in_place():
    B, S, H, Hk, D = 4, 9, 8, 2, 128
    q = normal_tensor(13100, (B, S, H * D), np.float16)
    k = normal_tensor(13101, (B, S, Hk * D), np.float16)
    wq, wk = weights(13102, D, np.float16), weights(13103, D, np.float16)
    ids = ids_in(13104, (B, S), 512)
    inv = oracle.inv_freq(1e6, D)
    cos, sin = oracle.cos_sin_cache(np.float16, 512, inv)
    want = oracle.rope_apply_qk_norm(q, k, wq, wk, 1e-6, cos, sin, ids, num_heads=H, kv_num_heads=Hk)
    qt, kt = cuda(q), cuda(k)
    rpe.rope_apply_qk_norm(qt, kt, cuda(wq), cuda(wk), cuda(cos), cuda(sin), cuda(ids), epsilon=1e-6,
                           num_heads=H, kv_num_heads=Hk, out_q=qt, out_k=kt)
    assert_parity_norm(host(qt), want[0], zmax_rows(q, wq, 1e-6, 3, H), "Q in place")
    assert_parity_norm(host(kt), want[1], zmax_rows(k, wk, 1e-6, 3, Hk), "K in place")


@pytest.mark.parametrize("dt,D,H,Hk", [(np.float16, 128, 32, 8), (BFLOAT16, 128, 32, 8),
                                       (np.float16, 256, 16, 8),   # halves of 256 B: the row kernel
                                       (np.float32, 128, 32, 8),   # float32: the row kernel
                                       (np.float16, 96, 32, 8),    # 192-byte rows: general rows
                                       (np.float16, 64, 32, 8),    # 128-byte rows: the row kernel
                                       (BFLOAT16, 256, 8, 4),      # 8 + 4 heads of 256
                                       (np.float16, 96, 16, 8)])   # general rows, 16 + 8 heads
def test_qk_norm_prefill_full_size(dt, D, H, Hk):
    """A Qwen3-like prefill: 4 x 2048 tokens, 32 query and 8 key heads of 128
    (or 16 and 8 of 256), positions per-sequence offset + arange into a
    (8192, D/2) table."""
    B, S, M = 4, 2048, 8192
    q = normal_tensor(13200, (B, S, H * D), dt)
    k = normal_tensor(13201, (B, S, Hk * D), dt)
    wq, wk = weights(13202, D, dt), weights(13203, D, dt)
    ids = ids_in(13204, (B, 1), 4096) + np.arange(S, dtype=np.int64)[None, :]
    inv = oracle.inv_freq(1e6, D)
    cos, sin = oracle.cos_sin_cache(dt, M, inv)
    want_q, want_k = oracle.rope_apply_qk_norm(q, k, wq, wk, 1e-6, cos, sin, ids, num_heads=H, kv_num_heads=Hk)
    gq, gk = rpe.rope_apply_qk_norm(cuda(q), cuda(k), cuda(wq), cuda(wk), cuda(cos), cuda(sin), cuda(ids),
                                    epsilon=1e-6, num_heads=H, kv_num_heads=Hk)
    rq = assert_parity_norm(host(gq), want_q, zmax_rows(q, wq, 1e-6, 3, H), "Q")
    rk = assert_parity_norm(host(gk), want_k, zmax_rows(k, wk, 1e-6, 3, Hk), "K")
    print("prefill", np.dtype(dt).name, D, rq, rk, flush=True)


def test_qk_norm_prefill_heads256_bench_size():
    """The benchmark's QK-norm prefill with heads of 256 (qk_norm_f16_prefill_heads256:
    4 x 2048 tokens, 8 query and 4 key heads) in its launch configuration."""
    w = get("qk_norm_f16_prefill_heads256")
    q, k, ids = w.make_x(), w.make_k(), w.make_ids()
    wq, wk = w.make_norm_weights()
    cos, sin = oracle.table_for(w)
    want_q, want_k = oracle.rope_apply_qk_norm(q, k, wq, wk, 1e-6, cos, sin, ids, num_heads=w.num_heads,
                                               kv_num_heads=w.kv_num_heads)
    gq, gk = rpe.rope_apply_qk_norm(cuda(q), cuda(k), cuda(wq), cuda(wk), cuda(cos), cuda(sin), cuda(ids),
                                    epsilon=1e-6, num_heads=w.num_heads, kv_num_heads=w.kv_num_heads)
    rq = assert_parity_norm(host(gq), want_q, zmax_rows(q, wq, 1e-6, 3, w.num_heads), "Q")
    rk = assert_parity_norm(host(gk), want_k, zmax_rows(k, wk, 1e-6, 3, w.kv_num_heads), "K")
    print("prefill heads of 256", rq, rk, flush=True)


def test_qk_norm_decode_full_size():
    """The decode step the benchmark times (qk_norm_f16_decode): 256 sequences
    of one token, 32 query and 8 key heads of 128, f16, ids U[0, 32768),
    coefficients on the fly, in the same launch configuration."""
    w = get("qk_norm_f16_decode")
    q, k, ids = w.make_x(), w.make_k(), w.make_ids()
    wq, wk = w.make_norm_weights()
    inv = oracle.inv_freq(w.cache_base, w.rotary_dim)
    want_q, want_k = oracle.rope_apply_qk_norm(q, k, wq, wk, 1e-6, None, None, ids, num_heads=w.num_heads,
                                               kv_num_heads=w.kv_num_heads, inv_freq=inv, attention_scaling=w.scaling)
    gq, gk = rpe.rope_apply_qk_norm(cuda(q), cuda(k), cuda(wq), cuda(wk), None, None, cuda(ids), epsilon=1e-6,
                                    num_heads=w.num_heads, kv_num_heads=w.kv_num_heads, inv_freq=cuda(inv),
                                    attention_scaling=w.scaling)
    rq = assert_parity_norm(host(gq), want_q, zmax_rows(q, wq, 1e-6, 3, w.num_heads), "Q")
    rk = assert_parity_norm(host(gk), want_k, zmax_rows(k, wk, 1e-6, 3, w.kv_num_heads), "K")
    print("decode full size", rq, rk, flush=True)
