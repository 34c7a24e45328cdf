"""Seeded synthetic-input generators shared by the oracle side and the GPU side.

Holds none of the rotary-embedding arithmetic: only random numbers and the
structure of the workloads' inputs. Each generator is written from its
published definition:

* splitmix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; the 64-bit finaliser constants are the published
  ones): state advances by the golden-ratio increment, output is the mixed
  state.
* Standard normal by the Box-Muller transform (Box & Muller 1958) in binary64
  from two uniform draws u1, u2 in [0, 1): r = sqrt(-2 ln(1 - u1)),
  angle 2 pi u2; both outputs are used.
* Integers uniform on [0, n) by Lemire's multiply-shift ("Fast random integer
  generation in an interval", ACM TOMACS 2019), without the rejection step:
  floor(z * n / 2^64) for a 64-bit draw z.
"""
import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


class SplitMix64:
    """Counter-style splitmix64: draw k (k = 0, 1, ...) mixes seed + (k+1)*golden."""

    def __init__(self, seed: int):
        self.seed = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
        self.counter = 0

    def next_u64(self, n: int) -> np.ndarray:
        out = np.empty(n, np.uint64)
        with np.errstate(over="ignore"):
            for lo in range(0, n, _CHUNK):
                hi = min(n, lo + _CHUNK)
                k = np.arange(self.counter + lo + 1, self.counter + hi + 1, dtype=np.uint64)
                z = self.seed + k * _GOLDEN
                z = (z ^ (z >> np.uint64(30))) * _M1
                z = (z ^ (z >> np.uint64(27))) * _M2
                out[lo:hi] = z ^ (z >> np.uint64(31))
        self.counter += n
        return out

    def uniform(self, n: int) -> np.ndarray:
        """n doubles in [0, 1): the top 53 bits of each draw times 2^-53."""
        return (self.next_u64(n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)

    def normal(self, n: int) -> np.ndarray:
        """n standard normal doubles by Box-Muller."""
        m = (n + 1) // 2
        out = np.empty(2 * m, np.float64)
        for lo in range(0, m, _CHUNK):
            hi = min(m, lo + _CHUNK)
            u = self.uniform(2 * (hi - lo))
            u1, u2 = u[0::2], u[1::2]
            r = np.sqrt(-2.0 * np.log1p(-u1))
            a = 2.0 * np.pi * u2
            out[2 * lo:2 * hi:2] = r * np.cos(a)
            out[2 * lo + 1:2 * hi:2] = r * np.sin(a)
        return out[:n]

    def below(self, n: int, bound: int) -> np.ndarray:
        """n integers uniform on [0, bound), bound < 2^32 (vectorised)."""
        if not 0 < bound < (1 << 32):
            raise ValueError("bound must be in (0, 2^32)")
        z = self.next_u64(n)
        b = np.uint64(bound)
        zh = z >> np.uint64(32)
        zl = z & np.uint64(0xFFFFFFFF)
        # floor(z*b / 2^64) with z = zh*2^32 + zl, evaluated without overflow
        with np.errstate(over="ignore"):
            t = zh * b + ((zl * b) >> np.uint64(32))
        return (t >> np.uint64(32)).astype(np.int64)

    def below_big(self, bound: int) -> int:
        """One integer uniform on [0, bound) for any bound < 2^64."""
        z = int(self.next_u64(1)[0])
        return (z * bound) >> 64


BFLOAT16 = np.uint16
"""bfloat16 tensors are carried as uint16 arrays of their bit patterns."""


def bfloat16_bits(v) -> np.ndarray:
    """bfloat16 bit patterns of binary32 values, nearest-even (finite inputs):
    add 0x7fff plus the lowest kept bit, then keep the upper 16 bits."""
    u = np.ascontiguousarray(np.asarray(v, np.float32)).view(np.uint32).astype(np.uint64)
    return ((u + np.uint64(0x7fff) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)


def normal_tensor(seed: int, shape, dtype) -> np.ndarray:
    """N(0,1) values rounded to `dtype` (numpy's round-to-nearest-even; for
    bfloat16 through binary32, then nearest-even to 8 significant bits)."""
    n = int(np.prod(shape))
    v = SplitMix64(seed).normal(n)
    if np.dtype(dtype) == BFLOAT16:
        return bfloat16_bits(v.astype(np.float32)).reshape(shape)
    return v.astype(dtype).reshape(shape)


def uniform_ints(seed: int, shape, bound: int) -> np.ndarray:
    n = int(np.prod(shape))
    return SplitMix64(seed).below(n, bound).reshape(shape)


def sample_without_replacement(gen: SplitMix64, population: int, k: int):
    """k distinct indices of range(population): partial Fisher-Yates."""
    pool = {}
    out = []
    for i in range(k):
        j = i + int(gen.below(1, population - i)[0])
        vi, vj = pool.get(i, i), pool.get(j, j)
        pool[i], pool[j] = vj, vi
        out.append(vj)
    return out
