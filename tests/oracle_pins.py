"""Pins of the CPU oracle to facts outside itself.

Each pin is a function of an `oracle.Oracle` that raises AssertionError when
the oracle disagrees with something the pages or the mathematics fix: a
library routine (numpy's binary16 conversion, complex multiplication), an
arbitrary-precision evaluation (mpmath), a hand-worked fixture, an invariant
the pages state, or a brute force on tiny inputs. They run against the real
oracle (test_oracle_pins.py) and against builds with planted mistakes
(test_oracle_mutants.py), where at least one must fail.
"""
import json
import math
import os

import mpmath
import numpy as np

from rope_inputs import SplitMix64, normal_tensor, get as get_workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

mpmath.mp.prec = 200


BF16 = np.uint16   # bfloat16 arrays travel as uint16 bit patterns


def bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


def to_f64(a):
    """Values of a float32/float16/bfloat16(uint16 bits) array as float64."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def from_f64(v, dt):
    """Round float64 values to dt (bfloat16 through torch, which rounds to
    nearest-even from binary32: exact for every value used with it here)."""
    v = np.asarray(v, np.float64)
    if dt is BF16:
        import torch
        return torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return v.astype(dt)


def assert_bitwise(a, b, what):
    ba, bb = bits(a), bits(b)
    bad = np.flatnonzero(ba.reshape(-1) != bb.reshape(-1))
    assert bad.size == 0, "%s: %d elements differ bitwise, first at flat %d: %r vs %r" % (
        what, bad.size, bad[0], a.reshape(-1)[bad[0]], b.reshape(-1)[bad[0]])


def assert_value_equal(a, b, what):
    """Equal as numbers (+0 == -0), NaN == NaN."""
    a64 = to_f64(a).reshape(-1)
    b64 = to_f64(b).reshape(-1)
    ok = (a64 == b64) | (np.isnan(a64) & np.isnan(b64))
    bad = np.flatnonzero(~ok)
    assert bad.size == 0, "%s: %d elements differ, first at %d: %r vs %r" % (
        what, bad.size, bad[0], a64[bad[0]], b64[bad[0]])


def angle_table(seed, rows, half, dtype):
    """cos/sin of random angles, each rounded to dtype (independent of the oracle)."""
    th = SplitMix64(seed).uniform(rows * half).reshape(rows, half) * (2 * np.pi)
    if dtype is BF16:
        return from_f64(np.cos(th).astype(np.float32), BF16), from_f64(np.sin(th).astype(np.float32), BF16)
    return np.cos(th).astype(dtype), np.sin(th).astype(dtype)


def normal_any(seed, shape, dt):
    if dt is BF16:
        return from_f64(normal_tensor(seed, shape, np.float32), BF16)
    return normal_tensor(seed, shape, dt)


def ids_in(seed, shape, bound):
    return SplitMix64(seed).below(int(np.prod(shape)), bound).reshape(shape)


def pair_index(interleaved, half):
    i = np.arange(half)
    if interleaved:
        return 2 * i, 2 * i + 1
    return i, i + half


def to_rank4(x, num_heads):
    """(B,S,H*D) -> (B,H,S,D)"""
    B, S, hid = x.shape
    return np.ascontiguousarray(x.reshape(B, S, num_heads, hid // num_heads).transpose(0, 2, 1, 3))


def f32_of_mp(v):
    return np.float32(float(v))


# --------------------------------------------------------------------------
# binary16 conversions against numpy's (a library routine)

def pin_f16_decode_exhaustive(orc):
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in allbits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    same &= np.signbit(got) == np.signbit(ref)
    assert same.all(), "binary16 decode differs at %s" % np.flatnonzero(~same)[:5]


def pin_f16_encode_vs_numpy(orc):
    g = SplitMix64(7)
    mags = np.exp2(g.uniform(20000) * 48.0 - 30.0)          # 2^-30 .. 2^18
    signs = np.where(g.uniform(20000) < 0.5, -1.0, 1.0)
    vals = list(mags * signs)
    # every tie point between neighbouring binary16 values, and its neighbours
    h = np.arange(0, 0x7c00, 97, dtype=np.uint32).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2
    vals += list(mid) + list(np.nextafter(mid, 0)) + list(np.nextafter(mid, 1e9))
    vals += [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -24, 2.0 ** -25,
             3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25, float("inf"), -float("inf")]
    vals = np.array(vals)
    with np.errstate(over="ignore"):  # values past the binary16 range become inf on purpose
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.f64_to_f16(float(v)) for v in vals], np.uint16)
    bad = np.flatnonzero(ref != got)
    assert bad.size == 0, "binary16 encode differs for %r" % vals[bad[:5]]
    assert np.isnan(np.uint16(orc.f64_to_f16(float("nan"))).view(np.float16))


def pin_bf16_decode_exhaustive(orc):
    import torch
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16_to_f64(int(b)) for b in allbits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    same &= np.signbit(got) == np.signbit(ref)
    assert same.all(), "bfloat16 decode differs at %s" % np.flatnonzero(~same)[:5]


def _bf16_exact_rne(v):
    """bfloat16 bits of v by exact rational arithmetic (independent check)."""
    from fractions import Fraction
    import math
    if v == 0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    if a >= Fraction(2 ** 128) - Fraction(2 ** 119):
        return sign | 0x7f80
    E = max(-126, math.floor(math.log2(abs(v))))
    while E > -126 and Fraction(2) ** E > a:   # guard the float log2
        E -= 1
    while E > -126 and Fraction(2) ** (E + 1) <= a:
        E += 1
    q = Fraction(2) ** (E - 7)
    n, rem = divmod(a, q)
    n = int(n)
    if rem > q / 2 or (rem == q / 2 and n % 2 == 1):
        n += 1
    r = n * q
    if r < Fraction(2) ** -126:
        return sign | n
    E2 = E + 1 if r >= Fraction(2) ** (E + 1) else E
    frac = int(r / Fraction(2) ** (E2 - 7)) - 128
    return sign | ((E2 + 127) << 7) | frac


def rne_bf16(v):
    """bfloat16 bits of each float64 value by the exact rational rule."""
    v = np.asarray(v, np.float64)
    return np.vectorize(_bf16_exact_rne, otypes=[np.uint16])(v).reshape(v.shape)


def round_to(v, dt):
    """float64 values rounded once to dt (nearest-even)."""
    return rne_bf16(v) if dt is BF16 else np.asarray(v, np.float64).astype(dt)


def pin_bf16_encode(orc):
    import torch
    # every tie point between neighbouring bfloat16 values (exact in binary32)
    # and its binary32 neighbours, against torch's nearest-even conversion
    h = np.arange(0, 0x7f80, 61, dtype=np.uint32)
    lo = ((h << 16).view(np.float32)).astype(np.float64)
    hi = (((h + 1) << 16).view(np.float32)).astype(np.float64)
    mid32 = ((lo + hi) / 2).astype(np.float32)
    vals32 = np.concatenate([mid32, np.nextafter(mid32, np.float32(0)), np.nextafter(mid32, np.float32(1e30)),
                             -mid32, np.float32([0.0, 1e-40, 3.3e38, 3.4e38, 1.17e-38])])
    ref = torch.from_numpy(vals32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f64_to_bf16(float(v)) for v in vals32], np.uint16)
    bad = np.flatnonzero(ref != got)
    assert bad.size == 0, "bfloat16 encode differs for %r" % vals32[bad[:5]]
    # binary64 values (not binary32) against exact rational rounding
    g = SplitMix64(17)
    mags = np.exp2(g.uniform(3000) * 280.0 - 140.0)
    signs = np.where(g.uniform(3000) < 0.5, -1.0, 1.0)
    for v in mags * signs:
        assert orc.f64_to_bf16(float(v)) == _bf16_exact_rne(float(v)), v


# --------------------------------------------------------------------------
# hand-worked cases (tests/golden/hand_rotations.json)

def pin_hand_worked(orc):
    with open(os.path.join(GOLDEN, "hand_rotations.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        for dt, key in ((np.float32, "f32"), (np.float16, "f16"), (BF16, "bf16")):
            x = from_f64(case["x"], dt).reshape(1, 1, 1, 4)
            c = from_f64(case["cos"], dt)
            s = from_f64(case["sin"], dt)
            for il, pk in ((0, "half_split"), (1, "interleaved")):
                want = from_f64(case["expected"][pk][key], dt)
                # per-token (B,S,R/2) table, no ids
                y = orc.rope_apply(x, c.reshape(1, 1, 2), s.reshape(1, 1, 2), interleaved=il)
                assert_value_equal(y.reshape(-1), want, "%s %s %s" % (case["name"], key, pk))
                # gathered (M,R/2) table, id 2 of 3 rows
                ct = np.stack([from_f64(np.zeros(2), dt), from_f64(np.ones(2), dt), c])
                st = np.stack([from_f64(np.ones(2), dt), from_f64(np.zeros(2), dt), s])
                y = orc.rope_apply(x, ct, st, np.array([[2]]), interleaved=il)
                assert_value_equal(y.reshape(-1), want, "%s %s %s ids" % (case["name"], key, pk))


# --------------------------------------------------------------------------
# the rotation against two independent formulations

def pin_complex_multiplication(orc):
    """Pair (x1, x2) as x1 + i*x2 times c + i*s (numpy complex128), rounded once
    (bfloat16: rounded by the exact rational rule)."""
    for dt in (np.float32, np.float16, BF16):
        for il in (0, 1):
            for rank in (3, 4):
                B, S, H, D, M = 2, 5, 3, 12, 17
                x = normal_any(11, (B, H, S, D), dt)
                cos, sin = angle_table(12, M, D // 2, dt)
                ids = ids_in(13, (B, S), M)
                j1, j2 = pair_index(il, D // 2)
                z = to_f64(x[..., j1]) + 1j * to_f64(x[..., j2])
                w = to_f64(cos[ids]) + 1j * to_f64(sin[ids])
                prod = z * w[:, None, :, :]
                want = np.empty_like(x)
                want[..., j1] = round_to(prod.real, dt)
                want[..., j2] = round_to(prod.imag, dt)
                if rank == 4:
                    y = orc.rope_apply(x, cos, sin, ids, interleaved=il)
                else:
                    x3 = np.ascontiguousarray(x.transpose(0, 2, 1, 3)).reshape(B, S, H * D)
                    y = to_rank4(orc.rope_apply(x3, cos, sin, ids, interleaved=il, num_heads=H), H)
                assert_bitwise(y, want, "complex form dt=%s il=%d rank=%d" % (np.dtype(dt).name, il, rank))


def pin_rotate_half_form(orc):
    """q*cat(c,c) + rotate_half(q)*cat(s,s), rotate_half(q) = cat(-q2, q1), on the
    leading R elements, the rest concatenated back unchanged (partial rotation)."""
    for dt in (np.float32, np.float16, BF16):
        for D, R in ((16, 16), (16, 8), (10, 4)):
            B, H, S, M = 2, 2, 7, 9
            x = normal_any(21, (B, H, S, D), dt)
            cos, sin = angle_table(22, M, R // 2, dt)
            ids = ids_in(23, (B, S), M)
            q = to_f64(x)
            q_rot = q[..., :R]
            C = to_f64(np.concatenate([cos[ids], cos[ids]], -1))[:, None]
            Sn = to_f64(np.concatenate([sin[ids], sin[ids]], -1))[:, None]
            rot_half = np.concatenate([-q_rot[..., R // 2:], q_rot[..., :R // 2]], -1)
            emb = round_to(q_rot * C + rot_half * Sn, dt)
            want = np.concatenate([emb, x[..., R:]], -1)
            y = orc.rope_apply(x, cos, sin, ids, rotary_embedding_dim=R if R != D else 0)
            assert_bitwise(y, want, "rotate_half form dt=%s D=%d R=%d" % (np.dtype(dt).name, D, R))
            assert_bitwise(y[..., R:], x[..., R:], "pass-through")


# --------------------------------------------------------------------------
# invariants

def pin_identity(orc):
    for dt in (np.float32, np.float16, BF16):
        x = normal_any(31, (2, 3, 4, 8), dt)
        ones = from_f64(np.ones((5, 4)), dt)
        zeros = from_f64(np.zeros((5, 4)), dt)
        for il in (0, 1):
            y = orc.rope_apply(x, ones, zeros, ids_in(32, (2, 4), 5), interleaved=il)
            assert_value_equal(y, x, "identity")


def pin_norm_preserved(orc):
    for dt, rel in ((np.float32, 4 * 2.0 ** -24), (np.float16, 4 * 2.0 ** -11), (BF16, 4 * 2.0 ** -8)):
        for il in (0, 1):
            x = normal_any(41, (2, 4, 6, 16), dt)
            cos, sin = angle_table(42, 11, 8, dt)
            # the rounded table has c^2 + s^2 != 1: compare against the exact product
            ids = ids_in(43, (2, 6), 11)
            y = to_f64(orc.rope_apply(x, cos, sin, ids, interleaved=il))
            j1, j2 = pair_index(il, 8)
            xd = to_f64(x)
            c = to_f64(cos[ids])[:, None]
            s = to_f64(sin[ids])[:, None]
            n_in = (xd[..., j1] ** 2 + xd[..., j2] ** 2) * (c ** 2 + s ** 2)
            n_out = y[..., j1] ** 2 + y[..., j2] ** 2
            err = np.abs(n_out - n_in) / np.maximum(n_in, 1e-3)
            assert err.max() <= rel * 2, "norm not preserved: %g" % err.max()


def pin_inverse(orc):
    x = normal_tensor(51, (2, 3, 5, 8), np.float32)
    cos, sin = angle_table(52, 7, 4, np.float32)
    ids = ids_in(53, (2, 5), 7)
    for il in (0, 1):
        y = orc.rope_apply(x, cos, sin, ids, interleaved=il)
        back = orc.rope_apply(y, cos, -sin, ids, interleaved=il)
        err = np.abs(back.astype(np.float64) - x.astype(np.float64))
        # two rotations by a rounded unit vector: |c^2+s^2-1| <= 2^-23 plus 2 roundings
        assert err.max() <= 4 * 2.0 ** -24 * max(1.0, np.abs(x).max()) * 4, err.max()


def pin_tail_bitwise(orc):
    for dt, nan in ((np.float32, np.uint32(0x7fa00123)), (np.float16, np.uint16(0x7e55)),
                    (BF16, np.uint16(0x7fa1))):
        x = normal_any(61, (2, 2, 3, 10), dt)
        raw = bits(x).copy()
        raw[..., 6] = nan                                  # NaN payload in the tail
        raw[..., 7] = 0x80000000 if dt == np.float32 else 0x8000   # -0
        x = raw.view(dt)
        cos, sin = angle_table(62, 4, 3, dt)
        for il in (0, 1):
            y = orc.rope_apply(x, cos, sin, ids_in(63, (2, 3), 4), interleaved=il,
                               rotary_embedding_dim=6)
            assert_bitwise(y[..., 6:], x[..., 6:], "tail")


def pin_pairing_permutation(orc):
    """interleaved(P x) == P half_split(x), P: j -> 2j, R/2 + j -> 2j + 1 on [0,R)."""
    for dt in (np.float32, np.float16, BF16):
        D, R = 12, 8
        x = normal_any(71, (2, 3, 4, D), dt)
        cos, sin = angle_table(72, 6, R // 2, dt)
        ids = ids_in(73, (2, 4), 6)
        perm = np.arange(D)
        perm[:R] = np.concatenate([np.arange(R // 2), np.arange(R // 2, R)]).reshape(2, -1).T.reshape(-1)
        # perm[2j] = j, perm[2j+1] = R/2 + j
        xp = np.ascontiguousarray(x[..., perm])
        a = orc.rope_apply(xp, cos, sin, ids, interleaved=1, rotary_embedding_dim=R)
        b = orc.rope_apply(x, cos, sin, ids, interleaved=0, rotary_embedding_dim=R)
        assert_bitwise(a, np.ascontiguousarray(b[..., perm]), "pairing permutation")


def pin_rank_transpose(orc):
    for dt in (np.float32, np.float16, BF16):
        B, S, H, D = 3, 5, 4, 8
        x3 = normal_any(81, (B, S, H * D), dt)
        cos, sin = angle_table(82, 9, D // 2, dt)
        ids = ids_in(83, (B, S), 9)
        for il in (0, 1):
            y3 = orc.rope_apply(x3, cos, sin, ids, interleaved=il, num_heads=H)
            y4 = orc.rope_apply(to_rank4(x3, H), cos, sin, ids, interleaved=il)
            assert_bitwise(to_rank4(y3, H), y4, "rank 3 vs rank 4")


def pin_gather_probe(orc):
    """Every pair (1, 0) -> the pair becomes (c, s) of the gathered row."""
    for dt in (np.float32, np.float16, BF16):
        B, H, S, D, M = 2, 3, 6, 8, 13
        cos, sin = angle_table(91, M, D // 2, dt)
        ids = ids_in(92, (B, S), M)
        ids[0, 0] = 0
        ids[1, 2] = M - 1
        for il in (0, 1):
            j1, j2 = pair_index(il, D // 2)
            x = np.zeros((B, H, S, D), dt)
            x[..., j1] = from_f64(1.0, dt)
            y = orc.rope_apply(x, cos, sin, ids, interleaved=il)
            for h in range(H):
                assert_bitwise(y[:, h][..., j1], cos[ids], "probe cos")
                assert_bitwise(y[:, h][..., j2], sin[ids], "probe sin")


def pin_per_token_table(orc):
    """No ids with table T3[b][s] = T2[ids[b][s]] equals the gathered call."""
    for dt in (np.float32, np.float16, BF16):
        for rank in (3, 4):
            B, S, H, D, M = 3, 4, 2, 8, 7
            x = normal_any(101, (B, H, S, D) if rank == 4 else (B, S, H * D), dt)
            cos, sin = angle_table(102, M, D // 2, dt)
            ids = ids_in(103, (B, S), M)
            ids[0, 0] = 0
            nh = 0 if rank == 4 else H
            a = orc.rope_apply(x, cos, sin, ids, num_heads=nh)
            b = orc.rope_apply(x, np.ascontiguousarray(cos[ids]), np.ascontiguousarray(sin[ids]),
                               num_heads=nh)
            assert_bitwise(a, b, "per-token table rank %d" % rank)


def pin_out_of_range_ids(orc):
    """Reading taken: an id outside [0, M) passes the whole row through."""
    for dt in (np.float32, np.float16, BF16):
        B, H, S, D, M = 2, 2, 6, 8, 5
        x = normal_any(111, (B, H, S, D), dt)
        cos, sin = angle_table(112, M, D // 2, dt)
        ids = ids_in(113, (B, S), M)
        ids[0, 1] = -1
        ids[1, 3] = M
        ids[1, 4] = 2 ** 40
        ids[0, 0] = 0
        y = orc.rope_apply(x, cos, sin, ids)
        for b, s in ((0, 1), (1, 3), (1, 4)):
            assert_bitwise(y[b, :, s], x[b, :, s], "out-of-range row")
        assert not np.array_equal(bits(y[0, :, 0]), bits(x[0, :, 0]))


def pin_empty(orc):
    for shape in ((0, 2, 3, 8), (2, 2, 0, 8), (2, 0, 3, 8)):
        x = np.zeros(shape, np.float32)
        y = orc.rope_apply(x, np.zeros((3, 4), np.float32), np.zeros((3, 4), np.float32),
                           np.zeros((shape[0], shape[2]), np.int64))
        assert y.shape == shape


# --------------------------------------------------------------------------
# tables against arbitrary precision (the cache spot check of the ORT review:
# positions 0, 1, 7, 100, 1000 against cos(pos * inv_freq) * scaling)

def _mp_inv_freq(base, R):
    return [f32_of_mp(mpmath.power(mpmath.mpf(base), mpmath.mpf(-2 * i) / R)) for i in range(R // 2)]


def pin_inv_freq(orc):
    for base, R in ((1e6, 128), (1e4, 64), (1e4, 8), (5e5, 96), (1e4, 2)):
        want = np.array(_mp_inv_freq(base, R), np.float32)
        got = orc.inv_freq(base, R)
        assert_bitwise(got, want, "inv_freq base=%g R=%d" % (base, R))


def pin_cache_spot_rows(orc):
    rows = (0, 1, 7, 100, 1000)
    for dt, base, R, scaling in ((np.float16, 1e6, 128, 1.0), (np.float32, 1e6, 128, 1.0),
                                 (np.float32, 1e4, 64, 1.0), (np.float16, 1e4, 64, 1.25),
                                 (np.float32, 1e6, 128, 0.7), (BF16, 1e6, 128, 1.0), (BF16, 1e4, 64, 1.25)):
        inv = np.array(_mp_inv_freq(base, R), np.float32)
        cos, sin = orc.cos_sin_cache(dt, 1001, inv, scaling)
        assert cos.shape == (1001, R // 2)
        sc = np.float32(scaling)
        for p in rows:
            for i in range(R // 2):
                th = np.float32(np.float64(np.float32(p)) * np.float64(inv[i]))
                c = f32_of_mp(mpmath.cos(mpmath.mpf(float(th))))
                s = f32_of_mp(mpmath.sin(mpmath.mpf(float(th))))
                c = from_f64(np.float32(np.float64(c) * np.float64(sc)), dt)
                s = from_f64(np.float32(np.float64(s) * np.float64(sc)), dt)
                assert bits(np.array([cos[p, i]]))[0] == bits(np.array([c]))[0], (dt, p, i, cos[p, i], c)
                assert bits(np.array([sin[p, i]]))[0] == bits(np.array([s]))[0], (dt, p, i, sin[p, i], s)
        if scaling == 1.0:
            assert (to_f64(cos[0]) == 1).all() and (bits(sin[0]) == 0).all()


def pin_c1_against_real_math(orc):
    """The toy workload: every output against cos/sin(s * 10000^(-2i/8)) evaluated
    in arbitrary precision, once with the table's binary32 roundings reproduced
    (bit-exact) and once in exact real arithmetic (1e-5 relative)."""
    w = get_workload("c1_rope_f32_tiny")
    x = w.make_x()
    inv = orc.inv_freq(10000.0, 8)
    cos, sin = orc.cos_sin_cache(np.float32, 16, inv)
    y = orc.rope_apply(x, cos.reshape(1, 16, 4), sin.reshape(1, 16, 4))
    inv_mp = _mp_inv_freq(10000.0, 8)
    for h in range(2):
        for s in range(16):
            for i in range(4):
                x1 = mpmath.mpf(float(x[0, h, s, i]))
                x2 = mpmath.mpf(float(x[0, h, s, i + 4]))
                th = np.float32(np.float64(np.float32(s)) * np.float64(inv_mp[i]))
                c = mpmath.mpf(float(f32_of_mp(mpmath.cos(mpmath.mpf(float(th))))))
                sn = mpmath.mpf(float(f32_of_mp(mpmath.sin(mpmath.mpf(float(th))))))
                assert y[0, h, s, i] == f32_of_mp(x1 * c - x2 * sn), (h, s, i)
                assert y[0, h, s, i + 4] == f32_of_mp(x2 * c + x1 * sn), (h, s, i)
                thr = s * mpmath.power(10000, mpmath.mpf(-2 * i) / 8)
                r1 = x1 * mpmath.cos(thr) - x2 * mpmath.sin(thr)
                r2 = x2 * mpmath.cos(thr) + x1 * mpmath.sin(thr)
                assert abs(float(r1) - float(y[0, h, s, i])) <= 1e-5 * max(1.0, abs(float(r1)))
                assert abs(float(r2) - float(y[0, h, s, i + 4])) <= 1e-5 * max(1.0, abs(float(r2)))


def _rne_f32_of_fraction(q):
    """The binary32 value nearest to the rational q (ties to the even
    significand): one rounding, from the exact value."""
    from fractions import Fraction
    f = np.float32(float(q))                      # within one binary32 step of the answer
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - q), int(np.float32(v).view(np.uint32)) & 1))


def pin_f32_cancellation_exact(orc):
    """binary32 data where the two products of a pair nearly cancel
    (x1 = rnd(x2*s/c) or x1 = rnd(-x2*c/s), magnitudes up to 1e4): every
    output equals the exact x1*c - x2*s (x2*c + x1*s), formed in rational
    arithmetic and rounded once to binary32. A product rounded to binary32
    before the difference misses it in many of these outputs (checked, so
    the pin is known to see that mistake)."""
    from fractions import Fraction
    B, H, S, D = 1, 3, 12, 8
    half = D // 2
    cos, sin = angle_table(4243, S, half, np.float32)
    g = SplitMix64(4244)
    n = B * H * S * half
    mag = 10.0 ** (g.uniform(n) * 6.0 - 2.0)
    x2 = (g.normal(n) * mag).astype(np.float32).astype(np.float64).reshape(B, H, S, half)
    x1 = (g.normal(n) * mag).reshape(B, H, S, half)
    kind = g.below(n, 3).reshape(B, H, S, half)
    c = cos.astype(np.float64)[None, None]
    sn = sin.astype(np.float64)[None, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        x1 = np.where((kind == 0) & (np.abs(c) > 0.05), x2 * sn / c, x1)
        x1 = np.where((kind == 1) & (np.abs(sn) > 0.05), -x2 * c / sn, x1)
    x = np.zeros((B, H, S, D), np.float32)
    x[..., :half] = x1.astype(np.float32)
    x[..., half:] = x2.astype(np.float32)
    y = orc.rope_apply(x, cos.reshape(1, S, half), sin.reshape(1, S, half))
    misses = 0
    for h in range(H):
        for si in range(S):
            for i in range(half):
                a1, a2 = Fraction(float(x[0, h, si, i])), Fraction(float(x[0, h, si, i + half]))
                cc, ss = Fraction(float(cos[si, i])), Fraction(float(sin[si, i]))
                for j, exact, rounded in ((i, a1 * cc - a2 * ss, float(a1 * cc) - float(np.float32(float(a2 * ss)))),
                                          (i + half, a2 * cc + a1 * ss, float(a2 * cc) + float(np.float32(float(a1 * ss))))):
                    want = _rne_f32_of_fraction(exact)
                    assert bits(np.float32(y[0, h, si, j])) == bits(want), (h, si, j, y[0, h, si, j], want)
                    misses += np.float32(rounded) != want
    assert misses >= n // 10, "the inputs do not separate the two arithmetics (%d)" % misses


# --------------------------------------------------------------------------
# M-RoPE

def _stride3_rule(half, section):
    """The stride-3 slot rule of the interleaved multimodal models: slot i -> h if
    i % 3 == 1 and i < 3*sec_h, -> w if i % 3 == 2 and i < 3*sec_w, else t."""
    out = []
    for i in range(half):
        if i % 3 == 1 and i < 3 * section[1]:
            out.append(1)
        elif i % 3 == 2 and i < 3 * section[2]:
            out.append(2)
        else:
            out.append(0)
    return out


def pin_mrope_section_maps(orc):
    for half in range(1, 41):
        for t in range(half + 1):
            for h in range(half + 1 - t):
                w = half - t - h
                sec = (t, h, w)
                m0 = list(orc.mrope_slot_streams(half, sec, 0))
                assert m0 == [0] * t + [1] * h + [2] * w, (sec, m0)
                m1 = list(orc.mrope_slot_streams(half, sec, 1))
                assert [m1.count(k) for k in range(3)] == list(sec), (sec, m1)
                lo = min(sec)
                assert m1[:3 * lo] == [0, 1, 2] * lo, (sec, m1)
                if h == w and h <= t:
                    assert m1 == _stride3_rule(half, sec), (sec, m1)
    assert list(orc.mrope_slot_streams(64, (24, 20, 20), 1)) == _stride3_rule(64, (24, 20, 20))
    for bad in ((1, 1, 1), (-1, 3, 2), (5, 0, 0)):
        try:
            orc.mrope_slot_streams(4, bad, 0)
        except ValueError:
            continue
        raise AssertionError("section %s accepted" % (bad,))


def pin_mrope_equal_streams(orc):
    """Text-only tokens (all streams equal) reduce M-RoPE to RotaryEmbedding."""
    for dt in (np.float32, np.float16, BF16):
        for rank, D, R in ((4, 16, 0), (3, 16, 8), (4, 9, 8), (3, 10, 6)):
            for il in (0, 1):
                B, S, H, M = 2, 5, 3, 11
                Rf = R or D
                shape = (B, H, S, D) if rank == 4 else (B, S, H * D)
                x = normal_any(121, shape, dt)
                cos, sin = angle_table(122, M, Rf // 2, dt)
                ids = ids_in(123, (B, S), M)
                ids3 = np.stack([ids, ids, ids])
                sec = (Rf // 2 - 2 * (Rf // 6), Rf // 6, Rf // 6)
                want = orc.rope_apply(x, cos, sin, ids, interleaved=il, num_heads=H if rank == 3 else 0,
                                      rotary_embedding_dim=R)
                for layout in (0, 1):
                    y = orc.mrope_apply(x, ids3, cos, sin, sec, layout, interleaved=il,
                                        num_heads=H, rotary_embedding_dim=R)
                    assert_bitwise(y, want, "equal streams rank=%d D=%d R=%d il=%d layout=%d"
                                   % (rank, D, R, il, layout))


def _mrope_probe(orc, dt, section, layout, expect_map):
    B, H, S, D, M = 2, 2, 7, 2 * sum(section), 50
    half = D // 2
    cos, sin = angle_table(131, M, half, dt)
    ids = ids_in(132, (3, B, S), M)
    ids[:, 0, 0] = (0, 1, 2)
    for il in (0, 1):
        j1, j2 = pair_index(il, half)
        x = np.zeros((B, H, S, D), dt)
        x[..., j1] = from_f64(1.0, dt)
        y = orc.mrope_apply(x, ids, cos, sin, section, layout, interleaved=il, num_heads=H)
        for b in range(B):
            for s in range(S):
                for i in range(half):
                    p = ids[expect_map[i], b, s]
                    got = y[b, :, s]
                    assert (bits(got[:, j1[i]]) == bits(np.array([cos[p, i]]))[0]).all(), (section, layout, b, s, i)
                    assert (bits(got[:, j2[i]]) == bits(np.array([sin[p, i]]))[0]).all(), (section, layout, b, s, i)


def pin_mrope_stream_gather(orc):
    """Probe X = (1, 0) per pair: slot i of token (b,s) must hold the table row of
    its own stream. Maps written here independently: sections in order for
    layout 0, the stride-3 rule for layout 1 (agrees with the reading taken
    when sec_h == sec_w <= sec_t)."""
    for dt in (np.float32, np.float16, BF16):
        for sec in ((2, 1, 1), (16, 24, 24), (3, 0, 5), (24, 20, 20), (4, 2, 2)):
            half = sum(sec)
            _mrope_probe(orc, dt, sec, 0, [0] * sec[0] + [1] * sec[1] + [2] * sec[2])
            if sec[1] == sec[2] <= sec[0]:
                _mrope_probe(orc, dt, sec, 1, _stride3_rule(half, sec))


def pin_mrope_out_of_range(orc):
    for dt in (np.float32, np.float16, BF16):
        for layout in (0, 1):
            B, H, S, D, M = 2, 3, 9, 16, 20
            sec = (4, 2, 2)
            x = normal_any(141, (B, H, S, D), dt)
            cos, sin = angle_table(142, M, D // 2, dt)
            ids = ids_in(143, (3, B, S), M)
            bad = ids.copy()
            bad[0, 0, 1] = -5
            bad[1, 0, 2] = M
            bad[2, 1, 3] = 2 ** 33
            bad[1, 1, 4] = -(2 ** 40)
            bad[:, 1, 5] = -1
            oob = (bad < 0) | (bad >= M)
            y = orc.mrope_apply(x, bad, cos, sin, sec, layout, num_heads=H)
            ref = orc.mrope_apply(x, ids, cos, sin, sec, layout, num_heads=H)
            m = list(orc.mrope_slot_streams(D // 2, sec, layout))
            for b in range(B):
                for s in range(S):
                    for i in range(D // 2):
                        src = x if oob[m[i], b, s] else ref
                        for j in (i, i + D // 2):
                            assert bits(y[b, :, s, j:j + 1]).tolist() == bits(src[b, :, s, j:j + 1]).tolist(), \
                                (layout, b, s, i)


def pin_mrope_scale(orc):
    """scale = 2 (exact) equals scale 1 with a doubled table; scale 0.5 likewise."""
    for dt in (np.float32, np.float16, BF16):
        B, H, S, D, M = 2, 2, 6, 12, 9
        sec = (2, 2, 2)
        x = normal_any(151, (B, H, S, D), dt)
        cos, sin = angle_table(152, M, D // 2, dt)
        ids = ids_in(153, (3, B, S), M)
        for layout in (0, 1):
            for sc in (2.0, 0.5):
                a = orc.mrope_apply(x, ids, cos, sin, sec, layout, num_heads=H, scale=sc)
                b = orc.mrope_apply(x, ids, round_to(to_f64(cos) * sc, dt), round_to(to_f64(sin) * sc, dt), sec,
                                    layout, num_heads=H, scale=1.0)
                assert_bitwise(a, b, "scale %g" % sc)


def pin_mrope_tiny_brute_force(orc):
    """The README's usage example shapes: x [2,2,16] with 2 heads (D=8), ids
    [3,2,2], cos/sin [2,4], mrope_section [2,1,1]; every output against a
    complex-multiplication brute force with the slot rows picked by hand."""
    maps = {0: [0, 0, 1, 2], 1: [0, 1, 2, 0]}
    for dt in (np.float32, np.float16, BF16):
        x = normal_any(161, (2, 2, 16), dt)
        cos, sin = angle_table(162, 2, 4, dt)
        ids = ids_in(163, (3, 2, 2), 4) - 1          # values -1..2 with rows 0..1 valid
        for layout in (0, 1):
            for il in (0, 1):
                y = orc.mrope_apply(x, ids, cos, sin, (2, 1, 1), layout, interleaved=il, num_heads=2)
                j1, j2 = pair_index(il, 4)
                for b in range(2):
                    for s in range(2):
                        for h in range(2):
                            row = x[b, s, 8 * h:8 * h + 8]
                            out = y[b, s, 8 * h:8 * h + 8]
                            for i in range(4):
                                p = ids[maps[layout][i], b, s]
                                pair_in = (row[j1[i]], row[j2[i]])
                                pair_out = (out[j1[i]], out[j2[i]])
                                if p < 0 or p >= 2:
                                    assert bits(np.array(pair_out)).tolist() == bits(np.array(pair_in)).tolist()
                                    continue
                                z = complex(*to_f64(np.array(pair_in))) * \
                                    complex(*to_f64(np.array([cos[p, i], sin[p, i]])))
                                want = round_to(np.array([z.real, z.imag]), dt)
                                assert bits(np.array(pair_out)).tolist() == bits(want).tolist(), \
                                    (layout, il, b, s, h, i)


# --------------------------------------------------------------------------
# Q+K and on-the-fly

def pin_qk_is_two_applies(orc):
    for dt in (np.float32, np.float16, BF16):
        for rank in (3, 4):
            B, S, H, Hk, D, M = 3, 2, 4, 2, 8, 10
            q = normal_any(171, (B, H, S, D) if rank == 4 else (B, S, H * D), dt)
            k = normal_any(172, (B, Hk, S, D) if rank == 4 else (B, S, Hk * D), dt)
            cos, sin = angle_table(173, M, D // 2, dt)
            ids = ids_in(174, (B, S), M)
            yq, yk = orc.rope_apply_qk(q, k, cos, sin, ids, num_heads=H, kv_num_heads=Hk)
            assert_bitwise(yq, orc.rope_apply(q, cos, sin, ids, num_heads=H if rank == 3 else 0), "Q")
            assert_bitwise(yk, orc.rope_apply(k, cos, sin, ids, num_heads=Hk if rank == 3 else 0), "K")


def pin_onthefly_equals_table(orc):
    for dt in (np.float32, np.float16, BF16):
        for sc in (1.0, 1.25):
            B, S, H, Hk, D, M = 4, 3, 4, 2, 16, 40000
            inv = orc.inv_freq(1e6, D)
            cos, sin = orc.cos_sin_cache(dt, M, inv, sc)
            q = normal_any(181, (B, S, H * D), dt)
            k = normal_any(182, (B, S, Hk * D), dt)
            ids = ids_in(183, (B, S), M)
            ids[0, 0] = 0
            ids[1, 1] = M - 1
            a = orc.rope_apply_qk(q, k, None, None, ids, num_heads=H, kv_num_heads=Hk,
                                  inv_freq=inv, attention_scaling=sc)
            b = orc.rope_apply_qk(q, k, cos, sin, ids, num_heads=H, kv_num_heads=Hk)
            assert_bitwise(a[0], b[0], "on-the-fly Q")
            assert_bitwise(a[1], b[1], "on-the-fly K")
            for p in (0, 1, 7, 100, 1000, M - 1):
                c, s = orc.onthefly_row(dt, p, inv, sc)
                assert_bitwise(c, cos[p], "row %d cos" % p)
                assert_bitwise(s, sin[p], "row %d sin" % p)


# --------------------------------------------------------------------------
# RoPE on Q and K with the key/value cache append (SparseAttention README)

def _kv_positions(B, S, lens, total):
    """past + s per token: 0-based in the prompt (total == S), else L[b] - S."""
    past = np.zeros(B, np.int64) if total == S else lens.astype(np.int64) - S
    return past[:, None] + np.arange(S, dtype=np.int64)[None, :]


def _kv_expected(orc, q, k, v, pk, pv, lens, total, cos, sin, H, Hk, il):
    """Expected outputs assembled with numpy scatters around the pinned
    RotaryEmbedding oracle (rank 3, gathered rows = the token positions)."""
    B, S, _ = q.shape
    D = pk.shape[3]
    Smax = pk.shape[2]
    pos = _kv_positions(B, S, lens, total)
    R = 2 * cos.shape[1]
    q_out = orc.rope_apply(q, cos, sin, pos, interleaved=il, num_heads=H, rotary_embedding_dim=R if R != D else 0)
    k_rot = orc.rope_apply(k, cos, sin, pos, interleaved=il, num_heads=Hk, rotary_embedding_dim=R if R != D else 0)
    ek, ev = pk.copy(), pv.copy()
    for b in range(B):
        for s in range(S):
            r = pos[b, s]
            if 0 <= r < Smax:
                ek[b, :, r, :] = k_rot[b, s].reshape(Hk, D)
                ev[b, :, r, :] = v[b, s].reshape(Hk, D)
    return q_out, ek, ev


def pin_kv_append_probe(orc):
    """Hand-checkable: every Q and K pair (1, 0) becomes (c, s) of table row
    past + s, V lands unchanged in the same cache row, every other row keeps
    its old value. Decode (total > S) and prompt (total == S)."""
    for dt in (np.float32, np.float16, BF16):
        B, S, H, Hk, D, Smax, M = 2, 2, 2, 1, 8, 7, 9
        cos, sin = angle_table(201, M, D // 2, dt)
        j1, j2 = pair_index(0, D // 2)
        q = np.zeros((B, S, H, D), dt)
        q[..., j1] = from_f64(1.0, dt)
        k = np.zeros((B, S, Hk, D), dt)
        k[..., j1] = from_f64(1.0, dt)
        v = normal_any(202, (B, S, Hk * D), dt)
        old = normal_any(203, (B, Hk, Smax, D), dt)
        for lens, total, rows in (((3, 6), 6, ((1, 2), (4, 5))), ((2, 2), 2, ((0, 1), (0, 1)))):
            qo, ko, vo = orc.rope_kv_append(q.reshape(B, S, -1), k.reshape(B, S, -1), v, old, old,
                                            np.array(lens, np.int32), total, cos, sin, H, Hk)
            for b in range(B):
                for s in range(S):
                    r = rows[b][s]
                    for h in range(H):
                        assert_bitwise(qo[b, s, h * D:(h + 1) * D][j1], cos[r], "q cos")
                        assert_bitwise(qo[b, s, h * D:(h + 1) * D][j2], sin[r], "q sin")
                    assert_bitwise(ko[b, 0, r][j1], cos[r], "k cos")
                    assert_bitwise(ko[b, 0, r][j2], sin[r], "k sin")
                    assert_bitwise(vo[b, 0, r], v[b, s], "v row")
                untouched = [i for i in range(Smax) if i not in rows[b]]
                assert_bitwise(ko[b, :, untouched], old[b, :, untouched], "k other rows")
                assert_bitwise(vo[b, :, untouched], old[b, :, untouched], "v other rows")


def pin_kv_append_equals_rope_and_scatter(orc):
    for dt in (np.float32, np.float16, BF16):
        for il in (0, 1):
            for D, half in ((16, 8), (16, 4), (12, 2)):
                B, S, H, Hk, Smax, M = 3, 4, 4, 2, 13, 20
                q = normal_any(211, (B, S, H * D), dt)
                k = normal_any(212, (B, S, Hk * D), dt)
                v = normal_any(213, (B, S, Hk * D), dt)
                pk = normal_any(214, (B, Hk, Smax, D), dt)
                pv = normal_any(215, (B, Hk, Smax, D), dt)
                cos, sin = angle_table(216, M, half, dt)
                for lens, total in (((4, 9, 13), 13), ((4, 4, 4), 4), ((1, 3, 4), 4), ((5, 6, 7), 9)):
                    lens = np.array(lens, np.int32)
                    got = orc.rope_kv_append(q, k, v, pk, pv, lens, total, cos, sin, H, Hk, interleaved=il)
                    want = _kv_expected(orc, q, k, v, pk, pv, lens, total, cos, sin, H, Hk, il)
                    for g, w, what in zip(got, want, ("q_out", "present_key", "present_value")):
                        assert_bitwise(g, w, "%s dt=%s il=%d D=%d lens=%s" % (what, np.dtype(dt).name, il, D,
                                                                           lens.tolist()))


def pin_kv_append_packed_equals_split(orc):
    for dt in (np.float16, BF16):
        B, S, H, Hk, D, Smax, M = 2, 3, 4, 2, 16, 9, 12
        qkv = normal_any(221, (B, S, (H + 2 * Hk) * D), dt)
        q = np.ascontiguousarray(qkv[..., :H * D])
        k = np.ascontiguousarray(qkv[..., H * D:(H + Hk) * D])
        v = np.ascontiguousarray(qkv[..., (H + Hk) * D:])
        pk = normal_any(222, (B, Hk, Smax, D), dt)
        cos, sin = angle_table(223, M, D // 2, dt)
        lens = np.array([5, 9], np.int32)
        a = orc.rope_kv_append(qkv, None, None, pk, pk, lens, 9, cos, sin, H, Hk)
        b = orc.rope_kv_append(q, k, v, pk, pk, lens, 9, cos, sin, H, Hk)
        for x, y in zip(a, b):
            assert_bitwise(x, y, "packed vs split")


def pin_kv_append_out_of_contract(orc):
    """Rows outside the cache are not written; positions outside the table
    keep their pairs (Q and K) -- the rule used for every gathered id."""
    dt = np.float32
    B, S, H, Hk, D, Smax, M = 3, 2, 2, 1, 8, 6, 5
    q = normal_any(231, (B, S, H * D), dt)
    k = normal_any(232, (B, S, Hk * D), dt)
    v = normal_any(233, (B, S, Hk * D), dt)
    pk = normal_any(234, (B, Hk, Smax, D), dt)
    cos, sin = angle_table(235, M, D // 2, dt)
    lens = np.array([7, 1, 6], np.int32)      # past 5 (rows 5, 6), past -1 (rows -1, 0), past 4 (rows 4, 5)
    qo, ko, vo = orc.rope_kv_append(q, k, v, pk, pk, lens, 6, cos, sin, H, Hk)
    assert_bitwise(qo[0, 0], q[0, 0], "position 5 >= M keeps Q")
    assert_bitwise(qo[1, 0], q[1, 0], "position -1 keeps Q")
    assert_bitwise(ko[0, 0, 5], k[0, 0], "row 5 holds K unrotated (position >= M)")
    assert_bitwise(vo[0, 0, 5], v[0, 0], "row 5 holds V")
    assert_bitwise(ko[1, 0, 0], orc.rope_apply(k, cos, sin, np.zeros((B, S), np.int64), num_heads=1)[1, 1],
                   "row 0 of batch 1 holds K at position 0")
    rest = [r for r in range(Smax) if r != 0]
    assert_bitwise(ko[1, 0, rest], pk[1, 0, rest], "batch 1: row -1 not written")
    assert_bitwise(ko[2, 0, :4], pk[2, 0, :4], "batch 2: rows below the past untouched")


def pin_kv_append_with_qk_norm(orc):
    """With QK-norm weights the append equals QK-norm + RoPE of Q and K at the
    positions past + s (oracle_rope_apply_qk_norm, pinned below), K scattered
    into the key cache, V copied unnormalised; packed input alike."""
    for dt in (np.float16, BF16, np.float32):
        for il in (0, 1):
            B, S, H, Hk, D, Smax, M = 3, 2, 4, 2, 16, 11, 14
            q = normal_any(291, (B, S, H * D), dt)
            k = normal_any(292, (B, S, Hk * D), dt)
            v = normal_any(293, (B, S, Hk * D), dt)
            pk = normal_any(294, (B, Hk, Smax, D), dt)
            wq = normal_any(295, (D,), dt)
            wk = normal_any(296, (D,), dt)
            cos, sin = angle_table(297, M, 6, dt)           # R = 12 < D: a normalised tail
            lens = np.array([2, 9, 11], np.int32)
            for total in (11, 2):
                got = orc.rope_kv_append(q, k, v, pk, pk, lens, total, cos, sin, H, Hk, interleaved=il,
                                         q_weight=wq, k_weight=wk, epsilon=1e-6)
                pos = _kv_positions(B, S, lens, total)
                eq, ek_rot = orc.rope_apply_qk_norm(q, k, wq, wk, 1e-6, cos, sin, pos, interleaved=il,
                                                    num_heads=H, kv_num_heads=Hk, rotary_embedding_dim=12)
                ek, ev = pk.copy(), pk.copy()
                for b in range(B):
                    for s_ in range(S):
                        ek[b, :, pos[b, s_], :] = ek_rot[b, s_].reshape(Hk, D)
                        ev[b, :, pos[b, s_], :] = v[b, s_].reshape(Hk, D)
                for g, w, what in zip(got, (eq, ek, ev), ("q_out", "key cache", "value cache")):
                    assert_bitwise(g, w, "norm append %s dt=%s il=%d total=%d" % (what, np.dtype(dt).name,
                                                                                  il, total))
            qkv = np.concatenate([q, k, v], -1)
            a = orc.rope_kv_append(qkv, None, None, pk, pk, lens, 11, cos, sin, H, Hk, interleaved=il,
                                   q_weight=wq, k_weight=wk, epsilon=1e-6)
            b_ = orc.rope_kv_append(q, k, v, pk, pk, lens, 11, cos, sin, H, Hk, interleaved=il,
                                    q_weight=wq, k_weight=wk, epsilon=1e-6)
            for x, y in zip(a, b_):
                assert_bitwise(x, y, "packed norm append")


# --------------------------------------------------------------------------
# QK-norm (RMSNorm over the head row) then RoPE

def pin_qk_norm_hand_worked(orc):
    """D = 4, x = (2, 2, 2, 2): mean of squares 4. epsilon 0: 1/rms = 1/2, so
    with weights w = (1, 4, 0.5, 2), z_j = 2 * w_j / 2 = w_j.
    Quarter turn (c, s) = (0, 1) on both slots:
    half-split pairs (z0, z2) = (1, 0.5) -> (-0.5, 1), (z1, z3) = (4, 2) -> (-2, 4),
    so y = (-0.5, -2, 1, 4); interleaved (z0, z1) = (1, 4) -> (-4, 1),
    (z2, z3) = (0.5, 2) -> (-2, 0.5), so y = (-4, 1, -2, 0.5).
    epsilon 12: 1/sqrt(4 + 12) = 1/4, z = w/2, y halves. Exact in every type."""
    for dt in (np.float32, np.float16, BF16):
        x = from_f64([2.0, 2.0, 2.0, 2.0], dt).reshape(1, 1, 1, 4)
        w = from_f64([1.0, 4.0, 0.5, 2.0], dt)
        c = from_f64([[0.0, 0.0]], dt)
        sn = from_f64([[1.0, 1.0]], dt)
        ids = np.zeros((1, 1), np.int64)
        for eps, f in ((0.0, 1.0), (12.0, 0.5)):
            for il, want in ((0, [-0.5, -2.0, 1.0, 4.0]), (1, [-4.0, 1.0, -2.0, 0.5])):
                yq, yk = orc.rope_apply_qk_norm(x, x, w, w, eps, c, sn, ids, interleaved=il)
                assert_bitwise(yq.reshape(-1), from_f64(np.array(want) * f, dt), "qk-norm eps=%g il=%d" % (eps, il))
                assert_bitwise(yk.reshape(-1), from_f64(np.array(want) * f, dt), "qk-norm K")


def pin_qk_norm_constant_magnitude_rows(orc):
    """Rows with |x_j| = a for all j, unit weights, epsilon 0: z = sign(x), so
    the result is RotaryEmbedding of the +-1 row (the mean, not the sum, of
    the squares; the square root)."""
    for dt in (np.float32, np.float16, BF16):
        for D, R in ((16, 16), (12, 8)):
            B, S, H, M = 2, 3, 2, 7
            sign = np.where(SplitMix64(241).uniform(B * S * H * D) < 0.5, -1.0, 1.0).reshape(B, H, S, D)
            a = np.exp2(np.floor(SplitMix64(242).uniform(B * H * S) * 10 - 5)).reshape(B, H, S, 1)
            x = from_f64(sign * a, dt)
            ones = from_f64(np.ones(D), dt)
            cos, sin = angle_table(243, M, R // 2, dt)
            ids = ids_in(244, (B, S), M)
            rd = R if R != D else 0
            yq, _ = orc.rope_apply_qk_norm(x, x, ones, ones, 0.0, cos, sin, ids, rotary_embedding_dim=rd)
            want = orc.rope_apply(from_f64(sign, dt), cos, sin, ids, rotary_embedding_dim=rd)
            assert_bitwise(yq, want, "constant-magnitude rows dt=%s D=%d" % (np.dtype(dt).name, D))


def pin_qk_norm_scale_invariant(orc):
    """epsilon 0: scaling a row by 2^k changes nothing, bit for bit."""
    for dt in (np.float32, np.float16, BF16):
        x = normal_any(251, (2, 3, 4, 16), dt)
        w = normal_any(252, (16,), dt)
        cos, sin = angle_table(253, 9, 8, dt)
        ids = ids_in(254, (2, 4), 9)
        a, _ = orc.rope_apply_qk_norm(x, x, w, w, 0.0, cos, sin, ids)
        for k in (-3, 2):
            xs = from_f64(to_f64(x) * 2.0 ** k, dt)
            b, _ = orc.rope_apply_qk_norm(xs, xs, w, w, 0.0, cos, sin, ids)
            assert_bitwise(a, b, "scale 2^%d" % k)


def pin_qk_norm_unit_rows(orc):
    """Unit weights, epsilon 0, a table of rotations: every output row has
    sum of squares D (the normalised row has mean square 1 and the rotation
    keeps the pair norms), within the roundings."""
    for dt, rel in ((np.float32, 2.0 ** -20), (np.float16, 2.0 ** -8), (BF16, 2.0 ** -5)):
        B, S, H, D, M = 2, 5, 3, 32, 11
        x = normal_any(261, (B, H, S, D), dt)
        ones = from_f64(np.ones(D), dt)
        th = SplitMix64(262).uniform(M * D // 2).reshape(M, D // 2) * 2 * np.pi
        cos, sin = from_f64(np.cos(th).astype(np.float32), dt), from_f64(np.sin(th).astype(np.float32), dt)
        ids = ids_in(263, (B, S), M)
        for il in (0, 1):
            y, _ = orc.rope_apply_qk_norm(x, x, ones, ones, 0.0, cos, sin, ids, interleaved=il)
            ssq = (to_f64(y) ** 2).sum(-1)
            assert np.abs(ssq / D - 1).max() < rel, np.abs(ssq / D - 1).max()


def pin_qk_norm_kept_pairs_and_tail(orc):
    """An out-of-range id keeps the pairs: the row is normalised and not
    rotated, which equals a table row (1, 0); the tail is normalised too."""
    for dt in (np.float32, np.float16, BF16):
        B, S, H, D, R, M = 2, 4, 2, 16, 8, 6
        x = normal_any(271, (B, S, H * D), dt)
        w = normal_any(272, (D,), dt)
        cos, sin = angle_table(273, M, R // 2, dt)
        ids = ids_in(274, (B, S), M)
        ids[0, 1] = -1
        ids[1, 2] = M
        ident_c = np.concatenate([cos, from_f64(np.ones((1, R // 2)), dt)])
        ident_s = np.concatenate([sin, from_f64(np.zeros((1, R // 2)), dt)])
        ids_ident = ids.copy()
        ids_ident[0, 1] = M
        ids_ident[1, 2] = M
        a, _ = orc.rope_apply_qk_norm(x, x, w, w, 1e-6, cos, sin, ids, num_heads=H, kv_num_heads=H,
                                      rotary_embedding_dim=R)
        b, _ = orc.rope_apply_qk_norm(x, x, w, w, 1e-6, ident_c, ident_s, ids_ident, num_heads=H,
                                      kv_num_heads=H, rotary_embedding_dim=R)
        assert_bitwise(a, b, "kept pairs = identity row")
        # tail: same as the tail of a full-width identity rotation
        c_full = from_f64(np.ones((M, D // 2)), dt)
        s_full = from_f64(np.zeros((M, D // 2)), dt)
        full, _ = orc.rope_apply_qk_norm(x, x, w, w, 1e-6, c_full, s_full, ids_in(275, (B, S), M),
                                         num_heads=H, kv_num_heads=H)
        assert_bitwise(a.reshape(B, S, H, D)[..., R:], full.reshape(B, S, H, D)[..., R:], "normalised tail")


def pin_qk_norm_weights_per_projection(orc):
    """Q uses q_weight and K uses k_weight: K's result equals the Q result of
    a call whose Q is K and whose q_weight is k_weight."""
    dt = np.float16
    q = normal_any(281, (2, 3, 4 * 16), dt)
    k = normal_any(282, (2, 3, 2 * 16), dt)
    wq = normal_any(283, (16,), dt)
    wk = normal_any(284, (16,), dt)
    inv = orc.inv_freq(1e4, 16)
    ids = ids_in(285, (2, 3), 100)
    for tables in (True, False):
        cos, sin = orc.cos_sin_cache(dt, 100, inv) if tables else (None, None)
        _, yk = orc.rope_apply_qk_norm(q, k, wq, wk, 1e-6, cos, sin, ids, num_heads=4, kv_num_heads=2,
                                       inv_freq=inv)
        yq2, _ = orc.rope_apply_qk_norm(k, k, wk, wq, 1e-6, cos, sin, ids, num_heads=2, kv_num_heads=2,
                                        inv_freq=inv)
        assert_bitwise(yk, yq2, "k_weight routing")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
