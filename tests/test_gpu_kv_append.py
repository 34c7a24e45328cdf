"""GPU parity for RoPE on Q and K with the key/value cache append (through the
C ABI) against the oracle: q_out within the rotation tolerance (parity.py),
the caches element by element (rotated K rows within it, V rows and every
row not written bit for bit), and guard regions around the caches untouched."""
import numpy as np
import pytest
import torch

import oracle
import rotary_position_embedding_amd as rpe
from gpu_io import DEV, cuda, host, torch_dtype, POLICIES, POLICY_IDS
from oracle_pins import angle_table, ids_in
from parity import assert_bitwise, assert_parity, assert_parity_norm, bits
from rope_inputs import BFLOAT16, get, normal_tensor

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements of poison on each side of a cache


@pytest.fixture(autouse=True)
def _policy():
    old = rpe.set_kernel_policy(0)
    yield
    rpe.set_kernel_policy(old)


def guarded(arr):
    """A device copy of `arr` inside a buffer with poisoned guard regions;
    returns (view, whole buffer)."""
    dt = torch_dtype(arr.dtype)
    buf = torch.empty(arr.size + 2 * GUARD, dtype=dt, device=DEV)
    buf.view(torch.int16 if buf.element_size() == 2 else torch.int32).fill_(0x7e11)
    view = buf[GUARD:GUARD + arr.size].view(arr.shape)
    view.copy_(cuda(arr))
    return view, buf


def check_guards(buf, what):
    whole = bits(host(buf))
    assert (whole[:GUARD] == 0x7e11).all() and (whole[-GUARD:] == 0x7e11).all(), what + ": guard overwritten"


def run_case(dt, B, S, H, Hk, D, width, Smax, M, lens, total, il=0, packed=False, inplace=False, seed=0,
             gpu_il=None):
    """gpu_il: the rotary_interleaved value passed to the library, when it
    differs from the pairing `il` the oracle is asked for."""
    if packed:
        query = normal_tensor(12000 + seed, (B, S, (H + 2 * Hk) * D), dt)
        key = value = None
    else:
        query = normal_tensor(12000 + seed, (B, S, H * D), dt)
        key = normal_tensor(12001 + seed, (B, S, Hk * D), dt)
        value = normal_tensor(12002 + seed, (B, S, Hk * D), dt)
    pk = normal_tensor(12003 + seed, (B, Hk, Smax, D), dt)
    pv = normal_tensor(12004 + seed, (B, Hk, Smax, D), dt)
    cos, sin = angle_table(12005 + seed, M, width, dt)
    lens = np.asarray(lens, np.int32)
    wq, wk, wv = oracle.rope_kv_append(query, key, value, pk, pv, lens, total, cos, sin, H, Hk,
                                       interleaved=il)
    gk, bk = guarded(pk)
    gv, bv = guarded(pv)
    q_t = cuda(query)
    out = q_t if inplace else None
    got_q = rpe.rope_kv_append(q_t, None if packed else cuda(key), None if packed else cuda(value), gk, gv,
                               cuda(lens), total, cuda(cos), cuda(sin), num_heads=H, kv_num_heads=Hk,
                               rotary_interleaved=il if gpu_il is None else gpu_il, out=out)
    what = "dt=%s B=%d S=%d H=%d Hk=%d D=%d w=%d lens=%s total=%d il=%d packed=%s" % (
        np.dtype(dt).name, B, S, H, Hk, D, width, lens.tolist()[:4], total, il, packed)
    if gpu_il is not None:
        what += " rotary_interleaved=%d" % gpu_il
    assert_parity(host(got_q), wq, "q_out " + what)
    assert_parity(host(gk), wk, "present_key " + what)
    assert_bitwise(host(gv), wv, "present_value " + what)
    # rows that were not written hold their old bits
    written = np.zeros((B, Smax), bool)
    past = np.zeros(B, np.int64) if total == S else lens.astype(np.int64) - S
    for b in range(B):
        for s in range(S):
            r = past[b] + s
            if 0 <= r < Smax:
                written[b, r] = True
    keep = ~written
    hk = host(gk)
    for b in range(B):
        assert_bitwise(hk[b][:, keep[b]], pk[b][:, keep[b]], "untouched key rows " + what)
    check_guards(bk, "past_key " + what)
    check_guards(bv, "past_value " + what)
    return what


KV = [
    # dt, B, S, H, Hk, D, width, Smax, M, lens, total, il, packed
    (np.float16, 64, 1, 32, 8, 128, 64, 512, 1024, "decode", None, 0, False),
    (BFLOAT16, 3, 37, 8, 2, 128, 64, 160, 200, (37, 100, 64), 100, 0, False),
    (np.float32, 2, 45, 4, 4, 64, 32, 64, 64, (45, 20), 45, 0, False),      # prompt with padding
    (np.float16, 4, 5, 8, 2, 128, 64, 40, 40, (5, 9, 33, 40), 40, 0, True),  # packed
    (np.float16, 2, 7, 4, 2, 128, 16, 30, 50, (7, 30), 30, 1, False),       # interleaved, partial
    (BFLOAT16, 2, 3, 4, 1, 10, 5, 12, 12, (3, 11), 11, 0, False),           # scalar kernel
    (np.float32, 2, 3, 2, 2, 96, 32, 24, 30, (3, 24), 24, 1, True),
    (np.float16, 2, 3, 4, 2, 64, 16, 20, 30, (3, 11), 11, 0, False),       # partners 2 lanes apart, tail
    (np.float32, 1, 2, 2, 1, 256, 128, 8, 10, (2,), 2, 0, False),          # 1 KiB rows, prompt
    (np.float16, 3, 4, 8, 2, 80, 10, 24, 30, (4, 9, 24), 24, 0, False),     # 20 of 80 rotated: element-wise
    (BFLOAT16, 2, 3, 6, 3, 96, 10, 20, 30, (3, 11), 11, 1, True),          # interleaved 20 of 96, packed
]


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("case", KV, ids=[str(i) for i in range(len(KV))])
def test_kv_append_sweep(case, policy, inplace):
    dt, B, S, H, Hk, D, width, Smax, M, lens, total, il, packed = case
    if inplace and packed:
        pytest.skip("q_out cannot be a packed query")
    rpe.set_kernel_policy(policy)
    if lens == "decode":
        lens = ids_in(12100, (B,), Smax) + 1                 # 1..Smax, past = L - 1
        total = int(lens.max())
    print(run_case(dt, B, S, H, Hk, D, width, Smax, M, lens, total, il, packed, inplace, seed=B + S + D),
          flush=True)


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("value", [2, -1])
def test_kv_append_rotary_interleaved_other_values(value, policy):
    """SparseAttention README, Attributes: every rotary_interleaved value
    other than 1 selects the NeoX half-split, so 2 and -1 give the oracle's
    half-split result."""
    rpe.set_kernel_policy(policy)
    print(run_case(np.float16, 4, 3, 8, 2, 128, 64, 40, 50, (3, 9, 33, 40), 40, il=0, seed=91,
                   gpu_il=value), flush=True)


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
def test_kv_append_out_of_contract_lengths(policy):
    """Lengths above total_sequence_length or below S: rows outside the cache
    are skipped, positions outside the table keep their pairs, nothing
    outside the caches is written."""
    rpe.set_kernel_policy(policy)
    print(run_case(np.float16, 4, 3, 8, 2, 128, 64, 20, 20, (2, 21, 25, -7), 20, seed=77), flush=True)


def test_kv_append_decode_full_size():
    """The decode step at serving size: 256 sequences, 32 query and 8 key heads
    of 128, f16, a 512-row cache, lengths U[1, 512]; the old cache contents
    are a cheap deterministic bit pattern (values in [0, 1))."""
    B, H, Hk, D, Smax, M = 256, 32, 8, 128, 512, 32768
    lens = (ids_in(12200, (B,), Smax) + 1).astype(np.int32)
    inv = oracle.inv_freq(1e6, D)
    cos, sin = oracle.cos_sin_cache(np.float16, M, inv)
    q = normal_tensor(12201, (B, 1, H * D), np.float16)
    k = normal_tensor(12202, (B, 1, Hk * D), np.float16)
    v = normal_tensor(12203, (B, 1, Hk * D), np.float16)
    n = B * Hk * Smax * D
    pk = ((np.arange(n, dtype=np.uint64) * np.uint64(2654435761)) >> np.uint64(7) & np.uint64(0x3bff)) \
        .astype(np.uint16).view(np.float16).reshape(B, Hk, Smax, D)
    total = int(lens.max())
    wq, wk, wv = oracle.rope_kv_append(q, k, v, pk, pk, lens, total, cos, sin, H, Hk)
    gk, gv = cuda(pk), cuda(pk)
    gq = rpe.rope_kv_append(cuda(q), cuda(k), cuda(v), gk, gv, cuda(lens), total,
                            cuda(cos), cuda(sin), num_heads=H, kv_num_heads=Hk)
    r = assert_parity(host(gq), wq, "q_out")
    assert_parity(host(gk), wk, "present_key")
    assert_bitwise(host(gv), wv, "present_value")
    print("decode full size", r, flush=True)


# ---------------------------------------------------------------------------
# with QK-norm first (the decode step of a QK-norm model)

def norm_weights(seed, D, dt):
    v = 1.0 + 0.25 * normal_tensor(seed, (D,), np.float32)
    if np.dtype(dt) == BFLOAT16:
        from rope_inputs import bfloat16_bits
        return bfloat16_bits(v)
    return v.astype(dt)


def zmax(x, w, eps, heads):
    def f64(a):
        a = np.ascontiguousarray(a)
        return ((a.astype(np.uint32) << 16).view(np.float32) if a.dtype == np.uint16 else a).astype(np.float64)
    xd = f64(x)
    B, S, _ = xd.shape
    xd = xd.reshape(B, S, heads, -1)
    z = np.abs(xd * f64(w)) / np.sqrt((xd ** 2).mean(-1, keepdims=True) + float(np.float32(eps)))
    return z


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
@pytest.mark.parametrize("case", [
    # dt, B, S, H, Hk, D, width, Smax, M, total, il, packed
    (np.float16, 64, 1, 32, 8, 128, 64, 256, 512, None, 0, False),
    (BFLOAT16, 3, 9, 8, 2, 128, 32, 40, 64, 40, 1, False),
    (np.float32, 2, 5, 4, 2, 64, 32, 16, 20, 5, 0, True),
    (np.float16, 2, 3, 4, 1, 10, 3, 12, 12, 11, 0, False),    # scalar kernel
    (np.float16, 5, 2, 6, 3, 96, 48, 24, 40, 9, 0, False),    # 192-byte rows: the row kernel's general rows
    (BFLOAT16, 3, 4, 6, 2, 80, 16, 20, 30, 10, 1, True),      # 160-byte rows, interleaved, packed
], ids=["decode_f16", "chunk_bf16", "prompt_f32_packed", "odd_rows", "rows96_f16", "rows80_bf16_packed"])
def test_kv_append_qk_norm(case, policy):
    dt, B, S, H, Hk, D, width, Smax, M, total, il, packed = case
    rpe.set_kernel_policy(policy)
    eps = 1e-6
    seed = 17000 + D + S
    if total is None:
        lens = (ids_in(seed, (B,), Smax) + 1).astype(np.int32)
        total = int(lens.max())
    else:
        lens = (ids_in(seed, (B,), total - S + 1) + S).astype(np.int32)
    q = normal_tensor(seed + 1, (B, S, H * D), dt)
    k = normal_tensor(seed + 2, (B, S, Hk * D), dt)
    v = normal_tensor(seed + 3, (B, S, Hk * D), dt)
    pk = normal_tensor(seed + 4, (B, Hk, Smax, D), dt)
    pv = normal_tensor(seed + 5, (B, Hk, Smax, D), dt)
    wq, wk = norm_weights(seed + 6, D, dt), norm_weights(seed + 7, D, dt)
    cos, sin = angle_table(seed + 8, M, width, dt)
    if packed:
        qkv = np.concatenate([q, k, v], -1)
        eq, ek, ev = oracle.rope_kv_append(qkv, None, None, pk, pv, lens, total, cos, sin, H, Hk, interleaved=il,
                                           q_weight=wq, k_weight=wk, epsilon=eps)
        args = (cuda(qkv), None, None)
    else:
        eq, ek, ev = oracle.rope_kv_append(q, k, v, pk, pv, lens, total, cos, sin, H, Hk, interleaved=il,
                                           q_weight=wq, k_weight=wk, epsilon=eps)
        args = (cuda(q), cuda(k), cuda(v))
    gk, gv = cuda(pk), cuda(pv)
    gq = rpe.rope_kv_append_qk_norm(*args, gk, gv, cuda(lens), total, cuda(cos), cuda(sin), cuda(wq), cuda(wk),
                                    epsilon=eps, num_heads=H, kv_num_heads=Hk, rotary_interleaved=il)
    zq = zmax(q, wq, eps, H).max(-1, keepdims=True)
    zq = np.broadcast_to(zq, (B, S, H, D)).reshape(B, S, H * D)
    assert_parity_norm(host(gq), eq, zq, "q_out")
    # key cache: rows written get the K bound, the others must be bit-identical
    zk = zmax(k, wk, eps, Hk).max(-1)                    # (B, S, Hk)
    zmax_cache = np.zeros((B, Hk, Smax, D))
    past = np.zeros(B, np.int64) if total == S else lens.astype(np.int64) - S
    for b in range(B):
        for s in range(S):
            r = past[b] + s
            if 0 <= r < Smax:
                zmax_cache[b, :, r, :] = zk[b, s][:, None]
    assert_parity_norm(host(gk), ek, zmax_cache, "key cache")
    assert_bitwise(host(gv), ev, "value cache")


def test_kv_append_qk_norm_decode_full_size():
    """The decode step the benchmark times (qk_norm_kv_append_f16_decode) in
    its launch configuration: 256 sequences, 32 query and 8 key heads of 128,
    f16, QK-norm weights; a 512-row cache (the cache length does not change
    the launch) holding a cheap bit pattern, lengths U[1, 512]."""
    w = get("qk_norm_kv_append_f16_decode")
    B, H, Hk, D, Smax = w.batch, w.num_heads, w.kv_num_heads, w.head_size, 512
    lens = (ids_in(12300, (B,), Smax) + 1).astype(np.int32)
    inv = oracle.inv_freq(w.cache_base, D)
    cos, sin = oracle.cos_sin_cache(np.float16, w.cache_rows, inv)
    q, k, v = w.make_x(), w.make_k(), w.make_v()
    wq, wk = w.make_norm_weights()
    n = B * Hk * Smax * D
    pk = ((np.arange(n, dtype=np.uint64) * np.uint64(2654435761)) >> np.uint64(7) & np.uint64(0x3bff)) \
        .astype(np.uint16).view(np.float16).reshape(B, Hk, Smax, D)
    total = int(lens.max())
    eq, ek, ev = oracle.rope_kv_append(q, k, v, pk, pk, lens, total, cos, sin, H, Hk,
                                       q_weight=wq, k_weight=wk, epsilon=1e-6)
    gk, gv = cuda(pk), cuda(pk)
    gq = rpe.rope_kv_append_qk_norm(cuda(q), cuda(k), cuda(v), gk, gv, cuda(lens), total, cuda(cos), cuda(sin),
                                    cuda(wq), cuda(wk), epsilon=1e-6, num_heads=H, kv_num_heads=Hk)
    zq = zmax(q, wq, 1e-6, H).max(-1, keepdims=True)
    zq = np.broadcast_to(zq, (B, 1, H, D)).reshape(B, 1, H * D)
    r = assert_parity_norm(host(gq), eq, zq, "q_out")
    zk = zmax(k, wk, 1e-6, Hk).max(-1)                   # (B, 1, Hk)
    zc = np.zeros((B, Hk, Smax, D))
    for b in range(B):
        zc[b, :, lens[b] - 1, :] = zk[b, 0][:, None]
    assert_parity_norm(host(gk), ek, zc, "key cache")
    assert_bitwise(host(gv), ev, "value cache")
    print("norm decode full size", r, flush=True)


@pytest.mark.parametrize("name", ["kv_append_f16_decode", "qk_norm_kv_append_f16_decode"])
def test_kv_append_decode_bench_size(name):
    """The decode steps the benchmark times, at their exact size and launch
    configuration: 256 sequences of one new token, 32 query and 8 key heads of
    128, f16, caches of (256, 8, 4096, 128) (2 GiB each), lengths U[1, 4096],
    a (32768, 64) table. For one new token the cache append is RoPE (after
    QK-norm for the norm variant) at position L[b] - 1, stored in that cache
    row (the oracle pins tie the append to this); q_out and every written row
    are compared with the oracle, and every other cache element must still
    hold its fill value (checked on the device, the caches stay there)."""
    w = get(name)
    norm = name.startswith("qk_norm")
    B, H, Hk, D, Smax = w.batch, w.num_heads, w.kv_num_heads, w.head_size, w.extra["cache_seq"]
    q, k, v, lens = w.make_x(), w.make_k(), w.make_v(), w.make_lengths()
    total = int(lens.max())
    inv = oracle.inv_freq(w.cache_base, D)
    cos, sin = oracle.cos_sin_cache(np.float16, w.cache_rows, inv)
    pos = (lens.astype(np.int64) - 1).reshape(B, 1)
    fill_k, fill_v = 0x3c00, 0xbc00  # 1.0 and -1.0
    gk = torch.full((B, Hk, Smax, D), 1.0, dtype=torch.float16, device=DEV)
    gv = torch.full((B, Hk, Smax, D), -1.0, dtype=torch.float16, device=DEV)
    print("bench-size cache append", name, flush=True)
    if norm:
        wq, wk = w.make_norm_weights()
        eq, ek = oracle.rope_apply_qk_norm(q, k, wq, wk, 1e-6, cos, sin, pos, num_heads=H, kv_num_heads=Hk)
        gq = rpe.rope_kv_append_qk_norm(cuda(q), cuda(k), cuda(v), gk, gv, cuda(lens), total, cuda(cos),
                                        cuda(sin), cuda(wq), cuda(wk), epsilon=1e-6, num_heads=H,
                                        kv_num_heads=Hk)
    else:
        eq, ek = oracle.rope_apply_qk(q, k, cos, sin, pos, num_heads=H, kv_num_heads=Hk)
        gq = rpe.rope_kv_append(cuda(q), cuda(k), cuda(v), gk, gv, cuda(lens), total, cuda(cos), cuda(sin),
                                num_heads=H, kv_num_heads=Hk)
    torch.cuda.synchronize()
    bidx = torch.arange(B, device=DEV)
    rows = torch.from_numpy(pos[:, 0]).to(DEV)
    got_k = host(gk[bidx, :, rows, :].contiguous()).reshape(B, 1, Hk * D)
    got_v = host(gv[bidx, :, rows, :].contiguous()).reshape(B, 1, Hk * D)
    if norm:
        zq = np.broadcast_to(zmax(q, wq, 1e-6, H).max(-1, keepdims=True), (B, 1, H, D)).reshape(B, 1, H * D)
        zk = np.broadcast_to(zmax(k, wk, 1e-6, Hk).max(-1, keepdims=True), (B, 1, Hk, D)).reshape(B, 1, Hk * D)
        r = assert_parity_norm(host(gq), eq, zq, "q_out")
        assert_parity_norm(got_k, ek, zk, "written key rows")
    else:
        r = assert_parity(host(gq), eq, "q_out")
        assert_parity(got_k, ek, "written key rows")
    assert_bitwise(got_v, v, "written value rows")
    # put the fill value back into the written rows: then nothing may differ
    gk[bidx, :, rows, :] = 1.0
    gv[bidx, :, rows, :] = -1.0
    assert bool((gk.view(torch.int16) == fill_k).all()), "a key-cache row outside L[b] - 1 was written"
    assert bool((gv.view(torch.int16) == fill_v - 0x10000).all()), "a value-cache row outside L[b] - 1 was written"
    print(name, "bench size", r, flush=True)


def test_kv_append_prompt_bench_size():
    """The prompt with cache append the benchmark times, at its size and in
    its launch configuration: 4 sequences of 2048 new tokens (a prompt: each
    starts at position 0), 32 query and 8 key heads of 128, f16, caches of
    (4, 8, 4096, 128), an (8192, 64) table. q_out and the written rows 0..2047
    against the oracle (RoPE at positions 0..2047, as the pins tie the append
    to it), V rows bit for bit, and every other cache element must still hold
    its fill value."""
    w = get("kv_append_f16_prompt")
    B, S, H, Hk, D, Smax = w.batch, w.seq, w.num_heads, w.kv_num_heads, w.head_size, w.extra["cache_seq"]
    q, k, v, lens = w.make_x(), w.make_k(), w.make_v(), w.make_lengths()
    assert (lens == S).all()
    inv = oracle.inv_freq(w.cache_base, D)
    cos, sin = oracle.cos_sin_cache(np.float16, w.cache_rows, inv)
    pos = np.broadcast_to(np.arange(S, dtype=np.int64), (B, S)).copy()
    eq, ek = oracle.rope_apply_qk(q, k, cos, sin, pos, num_heads=H, kv_num_heads=Hk)
    fill_k, fill_v = 0x3c00, 0xbc00  # 1.0 and -1.0
    gk = torch.full((B, Hk, Smax, D), 1.0, dtype=torch.float16, device=DEV)
    gv = torch.full((B, Hk, Smax, D), -1.0, dtype=torch.float16, device=DEV)
    print("bench-size prompt cache append", flush=True)
    gq = rpe.rope_kv_append(cuda(q), cuda(k), cuda(v), gk, gv, cuda(lens), S, cuda(cos), cuda(sin),
                            num_heads=H, kv_num_heads=Hk)
    torch.cuda.synchronize()
    got_k = host(gk[:, :, :S, :].permute(0, 2, 1, 3).contiguous()).reshape(B, S, Hk * D)
    got_v = host(gv[:, :, :S, :].permute(0, 2, 1, 3).contiguous()).reshape(B, S, Hk * D)
    r = assert_parity(host(gq), eq, "q_out")
    assert_parity(got_k, ek, "written key rows")
    assert_bitwise(got_v, v, "written value rows")
    gk[:, :, :S, :] = 1.0
    gv[:, :, :S, :] = -1.0
    assert bool((gk.view(torch.int16) == fill_k).all()), "a key-cache row past the prompt was written"
    assert bool((gv.view(torch.int16) == fill_v - 0x10000).all()), "a value-cache row past the prompt was written"
    print("prompt bench size", r, flush=True)
