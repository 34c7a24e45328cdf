"""Randomised GPU parity: seeded random configurations of every op (shapes,
storage types, ranks, pairings, partial rotation, out-of-range ids, tables
or on the fly, in place or not, every kernel policy), each against the oracle.
Configurations come from a fixed splitmix64 stream, so a failure names a
reproducible case."""
import os

import numpy as np
import pytest
import torch

import oracle
import rotary_position_embedding_amd as rpe
from gpu_io import DEV, cuda, host
from oracle_pins import angle_table, ids_in, pair_index
from parity import assert_bitwise, assert_parity, assert_parity_norm
from rope_inputs import BFLOAT16, SplitMix64, bfloat16_bits, normal_tensor

pytestmark = pytest.mark.gpu

# seeded configurations (ROPE_FUZZ_CASES overrides the count for longer runs)
N_CASES = int(os.environ.get("ROPE_FUZZ_CASES", "1000"))


@pytest.fixture(autouse=True)
def _policy():
    old = rpe.set_kernel_policy(0)
    yield
    rpe.set_kernel_policy(old)


def pick(g, options):
    return options[int(g.below(1, len(options))[0])]


def config(i):
    g = SplitMix64(0xF022 + i)
    op = pick(g, ["rope", "mrope", "qk", "packed", "qk_norm", "kv_append", "kv_append_norm"])
    dt = pick(g, [np.float16, np.float32, BFLOAT16])
    E = 4 if np.dtype(dt) == np.float32 else 8
    D = pick(g, [2, 6, 8, 10, 16, 24, 32, 48, 64, 96, 128, 160, 256, 2 * E * 3])
    R = pick(g, [0, 0, D // 2 - (D // 2) % 2, 2 * E]) if D > 4 else 0
    if R > D or R < 0:
        R = 0
    return dict(op=op, dt=dt, D=D, R=R,
                rank=pick(g, [3, 4]), B=int(g.below(1, 4)[0]) + 1, S=int(g.below(1, 40)[0]) + 1,
                H=int(g.below(1, 9)[0]) + 1, kv_div=pick(g, [1, 2, 4]),
                il=pick(g, [0, 1]), onthefly=pick(g, [False, True]), inplace=pick(g, [False, True]),
                policy=pick(g, [0, 0, 1, 2, 3]), seed=i)


def x_like(seed, shape, dt):
    return normal_tensor(seed, shape, dt)


def weights(seed, D, dt):
    v = 1.0 + 0.25 * normal_tensor(seed, (D,), np.float32)
    return bfloat16_bits(v) if np.dtype(dt) == BFLOAT16 else v.astype(dt)


def zmax_rows(x, w, eps, rank, heads):
    a = x
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    xd = a.astype(np.float64)
    wd = w
    if wd.dtype == np.uint16:
        wd = (wd.astype(np.uint32) << 16).view(np.float32)
    if rank == 3:
        xd = xd.reshape(xd.shape[0], xd.shape[1], heads, -1)
    rms = np.sqrt((xd ** 2).mean(-1, keepdims=True) + float(np.float32(eps)))
    z = np.abs(xd * wd.astype(np.float64)) / rms
    return np.broadcast_to(z.max(-1, keepdims=True), xd.shape).reshape(x.shape)


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz(i):
    c = config(i)
    print("fuzz case", i, {k: (np.dtype(v).name if k == "dt" else v) for k, v in c.items()}, flush=True)
    rpe.set_kernel_policy(c["policy"])
    op, dt, D, R, rank, B, S, H, il = c["op"], c["dt"], c["D"], c["R"], c["rank"], c["B"], c["S"], c["H"], c["il"]
    Rf = R or D
    M = 50
    Hk = max(1, H // c["kv_div"]) if H % c["kv_div"] == 0 else H
    seed = 20000 + 10 * i
    cos, sin = angle_table(seed + 1, M, Rf // 2, dt)
    ids = ids_in(seed + 2, (B, S), M + 4) - 2            # a few ids out of range
    shape = lambda h: (B, S, h * D) if rank == 3 else (B, h, S, D)

    if op == "rope":
        x = x_like(seed, shape(H), dt)
        want = oracle.rope_apply(x, cos, sin, ids, interleaved=il, num_heads=H if rank == 3 else 0,
                                 rotary_embedding_dim=R)
        xt = cuda(x)
        got = rpe.rope_apply(xt, cuda(cos), cuda(sin), cuda(ids), interleaved=il,
                             num_heads=H if rank == 3 else 0, rotary_embedding_dim=R,
                             out=xt if c["inplace"] else None)
        assert_parity(host(got), want, "rope")
    elif op == "mrope":
        half = Rf // 2
        t = int(SplitMix64(seed + 3).below(1, half + 1)[0])
        h_ = (half - t) // 2
        sec = (t, h_, half - t - h_)
        ids3 = ids_in(seed + 4, (3, B, S), M + 4) - 2
        layout = i % 2
        x = x_like(seed, shape(H), dt)
        want = oracle.mrope_apply(x, ids3, cos, sin, sec, layout, interleaved=il, num_heads=H,
                                  rotary_embedding_dim=R)
        got = rpe.mrope_apply(cuda(x), cuda(ids3), cuda(cos), cuda(sin), mrope_section=sec, mrope_layout=layout,
                              interleaved=il, num_heads=H, rotary_embedding_dim=R)
        assert_parity(host(got), want, "mrope %s" % (sec,))
    elif op in ("qk", "qk_norm"):
        q = x_like(seed, shape(H), dt)
        k = x_like(seed + 5, shape(Hk), dt)
        nh, nk = (H, Hk) if rank == 3 else (0, 0)
        inv = oracle.inv_freq(1e4, Rf)
        ids_ok = ids_in(seed + 6, (B, S), 30000) if c["onthefly"] else ids
        tab = (None, None) if c["onthefly"] else (cos, sin)
        gtab = dict(inv_freq=cuda(inv)) if c["onthefly"] else dict(cos_cache=cuda(cos), sin_cache=cuda(sin))
        qt, kt = cuda(q), cuda(k)
        outs = dict(out_q=qt, out_k=kt) if c["inplace"] else {}
        if op == "qk":
            wq, wk = oracle.rope_apply_qk(q, k, tab[0], tab[1], ids_ok, interleaved=il, num_heads=nh,
                                          kv_num_heads=nk, rotary_embedding_dim=R, inv_freq=inv)
            gq, gk = rpe.rope_apply_qk(qt, kt, position_ids=cuda(ids_ok), interleaved=il, num_heads=nh,
                                       kv_num_heads=nk, rotary_embedding_dim=R, **gtab, **outs)
            assert_parity(host(gq), wq, "Q")
            assert_parity(host(gk), wk, "K")
        else:
            w1, w2 = weights(seed + 7, D, dt), weights(seed + 8, D, dt)
            wq, wk = oracle.rope_apply_qk_norm(q, k, w1, w2, 1e-6, tab[0], tab[1], ids_ok, interleaved=il,
                                               num_heads=nh, kv_num_heads=nk, rotary_embedding_dim=R,
                                               inv_freq=inv)
            zq, zk = zmax_rows(q, w1, 1e-6, rank, H), zmax_rows(k, w2, 1e-6, rank, Hk)
            gq, gk = rpe.rope_apply_qk_norm(qt, kt, cuda(w1), cuda(w2), position_ids=cuda(ids_ok), epsilon=1e-6,
                                            interleaved=il, num_heads=nh, kv_num_heads=nk,
                                            rotary_embedding_dim=R, **gtab, **outs)
            assert_parity_norm(host(gq), wq, zq, "Q")
            assert_parity_norm(host(gk), wk, zk, "K")
    elif op == "packed":
        Hall = H + 2 * Hk
        qkv = x_like(seed, shape(Hall), dt)
        if rank == 3:
            q, k, v = (np.ascontiguousarray(qkv[..., a * D:b * D]) for a, b in ((0, H), (H, H + Hk), (H + Hk, Hall)))
        else:
            q, k, v = (np.ascontiguousarray(qkv[:, a:b]) for a, b in ((0, H), (H, H + Hk), (H + Hk, Hall)))
        nh, nk = (H, Hk) if rank == 3 else (0, 0)
        wq, wk = oracle.rope_apply_qk(q, k, cos, sin, ids, interleaved=il, num_heads=nh, kv_num_heads=nk,
                                      rotary_embedding_dim=R)
        xt = cuda(qkv)
        y = host(rpe.rope_apply_qkv_packed(xt, cuda(cos), cuda(sin), cuda(ids), interleaved=il, num_heads=H,
                                           kv_num_heads=Hk, rotary_embedding_dim=R,
                                           out=xt if c["inplace"] else None))
        if rank == 3:
            gq, gk, gv = (y[..., a * D:b * D] for a, b in ((0, H), (H, H + Hk), (H + Hk, Hall)))
        else:
            gq, gk, gv = (y[:, a:b] for a, b in ((0, H), (H, H + Hk), (H + Hk, Hall)))
        assert_parity(np.ascontiguousarray(gq), wq, "packed Q")
        assert_parity(np.ascontiguousarray(gk), wk, "packed K")
        assert_bitwise(np.ascontiguousarray(gv), v, "packed V")
    else:  # kv_append[_norm] (rank 3 only, table width R/2 with R <= D)
        Smax = S + int(SplitMix64(seed + 9).below(1, 20)[0])
        q = x_like(seed, (B, S, H * D), dt)
        k = x_like(seed + 5, (B, S, Hk * D), dt)
        v = x_like(seed + 6, (B, S, Hk * D), dt)
        pk = x_like(seed + 7, (B, Hk, Smax, D), dt)
        pv = x_like(seed + 8, (B, Hk, Smax, D), dt)
        Mt = Smax + 2
        ct, st = angle_table(seed + 10, Mt, Rf // 2, dt)
        prompt = i % 3 == 0
        total = S if prompt else Smax
        lens = (ids_in(seed + 11, (B,), Smax - S + 1) + S).astype(np.int32)
        gk_, gv_ = cuda(pk), cuda(pv)
        qt = cuda(q)
        if op == "kv_append":
            eq, ek, ev = oracle.rope_kv_append(q, k, v, pk, pv, lens, total, ct, st, H, Hk, interleaved=il)
            gq = rpe.rope_kv_append(qt, cuda(k), cuda(v), gk_, gv_, cuda(lens), total, cuda(ct), cuda(st),
                                    num_heads=H, kv_num_heads=Hk, rotary_interleaved=il,
                                    out=qt if c["inplace"] else None)
            assert_parity(host(gq), eq, "q_out")
            assert_parity(host(gk_), ek, "key cache")
        else:
            w1, w2 = weights(seed + 12, D, dt), weights(seed + 13, D, dt)
            eq, ek, ev = oracle.rope_kv_append(q, k, v, pk, pv, lens, total, ct, st, H, Hk, interleaved=il,
                                               q_weight=w1, k_weight=w2, epsilon=1e-6)
            gq = rpe.rope_kv_append_qk_norm(qt, cuda(k), cuda(v), gk_, gv_, cuda(lens), total, cuda(ct),
                                            cuda(st), cuda(w1), cuda(w2), epsilon=1e-6, num_heads=H,
                                            kv_num_heads=Hk, rotary_interleaved=il,
                                            out=qt if c["inplace"] else None)
            assert_parity_norm(host(gq), eq, zmax_rows(q, w1, 1e-6, 3, H), "q_out")
            # every cache element against the largest normalised K value of the batch
            zk = np.max(zmax_rows(k, w2, 1e-6, 3, Hk)) if k.size else 0.0
            assert_parity_norm(host(gk_), ek, np.full(ek.shape, zk), "key cache")
        assert_bitwise(host(gv_), ev, "value cache")
