"""Scalar CPU oracle for rotary position embedding apply -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product library (rotary_position_embedding_amd)
never imports it, and this package never imports the product.

Thin numpy wrappers around liboracle_rope.so (rope_oracle.c). float16 arrays
travel as numpy float16 and bfloat16 arrays as numpy uint16 bit patterns
(bit patterns pass through untouched). The functions
and their parity status are documented in rope_oracle.h.

`Oracle(path)` binds the wrappers to one build of the C file; the module-level
functions use the default build. Tests also bind planted-mistake builds to
check that the pins catch them.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ROPE_ORACLE_LIBRARY selects another build of the same C file (the
# sanitizer build of the CPU tests); by default the in-tree one
LIB_PATH = os.path.abspath(os.environ.get("ROPE_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle_rope.so"))
SOURCE_PATH = os.path.join(_HERE, "rope_oracle.c")

F32 = 1
F16 = 10
BF16 = 16
# bfloat16 arrays travel as numpy uint16 bit patterns
_DTYPE_CODE = {np.dtype(np.float32): F32, np.dtype(np.float16): F16, np.dtype(np.uint16): BF16}


def _ptr(a):
    return None if a is None else a.ctypes.data


def _code(dtype):
    try:
        return _DTYPE_CODE[np.dtype(dtype)]
    except KeyError:
        raise TypeError("oracle supports float32, float16 and bfloat16 (uint16 bits), got %s" % dtype)


def _dense(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != np.dtype(dtype):
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def _dims(x, num_heads):
    """(rank, B, S, H, D) of X; rank 3 needs the head count."""
    if x.ndim == 4:
        B, H, S, D = x.shape
        return 4, B, S, H, D
    if x.ndim == 3:
        B, S, hidden = x.shape
        if not num_heads or hidden % num_heads:
            raise ValueError("rank-3 X needs num_heads dividing hidden")
        return 3, B, S, num_heads, hidden // num_heads
    raise ValueError("X must be rank 3 or 4")


class Oracle:
    def __init__(self, lib_path=LIB_PATH):
        if not os.path.exists(lib_path):
            raise RuntimeError("oracle library not built: %s (run python -m oracle.build)" % lib_path)
        if os.path.abspath(lib_path) == LIB_PATH:
            from . import build as _build
            if not _build.is_current(lib_path):
                raise RuntimeError("oracle library %s was built from other sources "
                                   "(run python -m oracle.build)" % lib_path)
        lib = ctypes.CDLL(lib_path)
        i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
        sig = {
            "oracle_f16_to_f64": ([ctypes.c_uint16], ctypes.c_double),
            "oracle_f64_to_f16": ([ctypes.c_double], ctypes.c_uint16),
            "oracle_bf16_to_f64": ([ctypes.c_uint16], ctypes.c_double),
            "oracle_f64_to_bf16": ([ctypes.c_double], ctypes.c_uint16),
            "oracle_inv_freq": ([ctypes.c_double, i64, vp], None),
            "oracle_cos_sin_cache": ([i32, i64, i64, vp, f32, vp, vp], None),
            "oracle_rope_apply": ([i32, i32, i64, i64, i64, i64, i64, i64,
                                   vp, vp, vp, vp, vp, i64], None),
            "oracle_mrope_slot_streams": ([i64, vp, i64, vp], i32),
            "oracle_mrope_apply": ([i32, i32, i64, i64, i64, i64, i64, i64,
                                    vp, vp, vp, vp, vp, i64, vp, i64, f32], None),
            "oracle_onthefly_row": ([i32, i64, vp, i64, f32, vp, vp], None),
            "oracle_rope_apply_qk": ([i32, i32, i64, i64, i64, i64, i64, i64, i64,
                                      vp, vp, vp, vp, vp, vp, vp, i64, vp, f32], None),
            "oracle_rope_kv_append": ([i32, i64, i64, i64, i64, i64, i64, i64,
                                       vp, vp, vp, vp, i64, vp, vp, i64, vp, vp, i64, vp,
                                       vp, vp, f32], None),
            "oracle_rope_apply_qk_norm": ([i32, i32, i64, i64, i64, i64, i64, i64, i64,
                                           vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, i64, vp, f32], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        self.lib = lib
        self.path = lib_path

    # -- scalar helpers ------------------------------------------------------
    def f16_to_f64(self, bits: int) -> float:
        return self.lib.oracle_f16_to_f64(bits)

    def f64_to_f16(self, v: float) -> int:
        return self.lib.oracle_f64_to_f16(v)

    def bf16_to_f64(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_f64(bits)

    def f64_to_bf16(self, v: float) -> int:
        return self.lib.oracle_f64_to_bf16(v)

    # -- coefficient tables --------------------------------------------------
    def inv_freq(self, base: float, rotary_dim: int) -> np.ndarray:
        out = np.zeros(max(rotary_dim // 2, 1), np.float32)
        self.lib.oracle_inv_freq(float(base), rotary_dim, _ptr(out))
        return out[:rotary_dim // 2]

    def cos_sin_cache(self, dtype, rows: int, inv_freq_arr, scaling: float = 1.0):
        inv = _dense(inv_freq_arr, np.float32)
        half = inv.shape[0]
        cos = np.zeros((rows, half), dtype)
        sin = np.zeros((rows, half), dtype)
        self.lib.oracle_cos_sin_cache(_code(dtype), rows, half, _ptr(inv), scaling,
                                      _ptr(cos), _ptr(sin))
        return cos, sin

    def onthefly_row(self, dtype, position: int, inv_freq_arr, scaling: float = 1.0):
        inv = _dense(inv_freq_arr, np.float32)
        half = inv.shape[0]
        c = np.zeros(half, dtype)
        s = np.zeros(half, dtype)
        self.lib.oracle_onthefly_row(_code(dtype), position, _ptr(inv), half, scaling,
                                     _ptr(c), _ptr(s))
        return c, s

    # -- the three operations ------------------------------------------------
    def rope_apply(self, x, cos, sin, position_ids=None, interleaved=0, num_heads=0,
                   rotary_embedding_dim=0):
        """RotaryEmbedding. cos/sin: (M, R/2) with ids, (B, S, R/2) without."""
        x = _dense(x)
        cos = _dense(cos, x.dtype)
        sin = _dense(sin, x.dtype)
        ids = _dense(position_ids, np.int64)
        rank, B, S, H, D = _dims(x, num_heads)
        R = rotary_embedding_dim or D
        M = cos.shape[0] if ids is not None else 0
        y = np.zeros_like(x)
        self.lib.oracle_rope_apply(_code(x.dtype), rank, B, S, H, D, R, interleaved,
                                   _ptr(x), _ptr(y), _ptr(cos), _ptr(sin), _ptr(ids), M)
        return y

    def mrope_slot_streams(self, half: int, section, layout: int) -> np.ndarray:
        sec = np.asarray(section, np.int64)
        out = np.zeros(max(half, 1), np.int8)
        rc = self.lib.oracle_mrope_slot_streams(half, _ptr(sec), layout, _ptr(out))
        if rc != 0:
            raise ValueError("mrope_section must be 3 non-negative ints summing to %d" % half)
        return out[:half]

    def mrope_apply(self, x, position_ids, cos, sin, mrope_section, mrope_layout=0,
                    interleaved=0, num_heads=0, rotary_embedding_dim=0, scale=1.0):
        """MRotaryEmbedding. position_ids (3, B, S); cos/sin (M, R/2)."""
        x = _dense(x)
        cos = _dense(cos, x.dtype)
        sin = _dense(sin, x.dtype)
        ids = _dense(position_ids, np.int64)
        rank, B, S, H, D = _dims(x, num_heads if x.ndim == 3 else None)
        R = rotary_embedding_dim or D
        sec = np.asarray(mrope_section, np.int64)
        if sec.shape != (3,) or sec.min() < 0 or sec.sum() != R // 2:
            raise ValueError("bad mrope_section")
        if ids.shape != (3, B, S):
            raise ValueError("position_ids must be (3, B, S)")
        y = np.zeros_like(x)
        self.lib.oracle_mrope_apply(_code(x.dtype), rank, B, S, H, D, R, interleaved,
                                    _ptr(x), _ptr(y), _ptr(cos), _ptr(sin), _ptr(ids),
                                    cos.shape[0], _ptr(sec), mrope_layout, scale)
        return y

    def rope_apply_qk(self, q, k, cos=None, sin=None, position_ids=None, interleaved=0,
                      num_heads=0, kv_num_heads=0, rotary_embedding_dim=0,
                      inv_freq=None, attention_scaling=1.0):
        """Q and K rotated with shared coefficients; cos=None selects on-the-fly."""
        q = _dense(q)
        k = _dense(k, q.dtype)
        ids = _dense(position_ids, np.int64)
        rank, B, S, H, D = _dims(q, num_heads)
        rk, Bk, Sk, Hk, Dk = _dims(k, kv_num_heads)
        if (rk, Bk, Sk, Dk) != (rank, B, S, D):
            raise ValueError("Q and K disagree on rank, batch, sequence or head size")
        R = rotary_embedding_dim or D
        inv = None
        if cos is None:
            inv = _dense(inv_freq, np.float32)
            if ids is None or inv is None:
                raise ValueError("on-the-fly needs position_ids and inv_freq")
            M = 0
        else:
            cos = _dense(cos, q.dtype)
            sin = _dense(sin, q.dtype)
            M = cos.shape[0] if ids is not None else 0
        yq = np.zeros_like(q)
        yk = np.zeros_like(k)
        self.lib.oracle_rope_apply_qk(_code(q.dtype), rank, B, S, H, Hk, D, R, interleaved,
                                      _ptr(q), _ptr(k), _ptr(yq), _ptr(yk), _ptr(cos),
                                      _ptr(sin), _ptr(ids), M, _ptr(inv), attention_scaling)
        return yq, yk

    def rope_apply_qk_norm(self, q, k, q_weight, k_weight, epsilon, cos=None, sin=None,
                           position_ids=None, interleaved=0, num_heads=0, kv_num_heads=0,
                           rotary_embedding_dim=0, inv_freq=None, attention_scaling=1.0):
        """RMSNorm of every Q and K head row (weights (D,), epsilon), then the
        rotation of rope_apply_qk; cos=None selects on-the-fly."""
        q = _dense(q)
        k = _dense(k, q.dtype)
        qw = _dense(q_weight, q.dtype)
        kw = _dense(k_weight, q.dtype)
        ids = _dense(position_ids, np.int64)
        rank, B, S, H, D = _dims(q, num_heads)
        rk, Bk, Sk, Hk, Dk = _dims(k, kv_num_heads)
        if (rk, Bk, Sk, Dk) != (rank, B, S, D) or qw.shape != (D,) or kw.shape != (D,):
            raise ValueError("Q, K and the weights disagree")
        R = rotary_embedding_dim or D
        inv = None
        if cos is None:
            inv = _dense(inv_freq, np.float32)
            if ids is None or inv is None:
                raise ValueError("on-the-fly needs position_ids and inv_freq")
            M = 0
        else:
            cos = _dense(cos, q.dtype)
            sin = _dense(sin, q.dtype)
            M = cos.shape[0] if ids is not None else 0
        yq = np.zeros_like(q)
        yk = np.zeros_like(k)
        self.lib.oracle_rope_apply_qk_norm(_code(q.dtype), rank, B, S, H, Hk, D, R, interleaved,
                                           _ptr(q), _ptr(k), _ptr(qw), _ptr(kw), float(epsilon),
                                           _ptr(yq), _ptr(yk), _ptr(cos), _ptr(sin), _ptr(ids), M,
                                           _ptr(inv), attention_scaling)
        return yq, yk

    def rope_kv_append(self, query, key, value, past_key, past_value, key_total_sequence_lengths,
                       total_sequence_length, cos, sin, num_heads, kv_num_heads, interleaved=0,
                       q_weight=None, k_weight=None, epsilon=0.0):
        """RoPE on Q and K and the key/value cache append. query (B,S,H*D), or
        packed [Q|K|V] when key and value are None; past_key/past_value
        (B,Hk,Smax,D) are copied and the updated copies returned with q_out:
        (q_out, present_key, present_value). With q_weight and k_weight ((D,)),
        Q and K are RMS-normalised first (QK-norm)."""
        query = _dense(query)
        packed = key is None
        if packed != (value is None):
            raise ValueError("key and value are both given or both None")
        key = _dense(key, query.dtype)
        value = _dense(value, query.dtype)
        lens = _dense(key_total_sequence_lengths, np.int32)
        cos = _dense(cos, query.dtype)
        sin = _dense(sin, query.dtype)
        pk = np.array(past_key, copy=True, order="C")
        pv = np.array(past_value, copy=True, order="C")
        B, S, W = query.shape
        Hall = num_heads + (2 * kv_num_heads if packed else 0)
        D = W // Hall
        Bc, Hk, Smax, Dc = pk.shape
        if (Bc, Hk, Dc) != (B, kv_num_heads, D) or pv.shape != pk.shape:
            raise ValueError("cache shape disagrees with the inputs")
        R = 2 * cos.shape[1]
        qwt = _dense(q_weight, query.dtype)
        kwt = _dense(k_weight, query.dtype)
        if (qwt is None) != (kwt is None):
            raise ValueError("q_weight and k_weight are both given or both None")
        q_out = np.zeros((B, S, num_heads * D), query.dtype)
        self.lib.oracle_rope_kv_append(_code(query.dtype), B, S, num_heads, kv_num_heads, D, R, interleaved,
                                       _ptr(query), _ptr(key), _ptr(value), _ptr(lens),
                                       int(total_sequence_length), _ptr(cos), _ptr(sin), cos.shape[0],
                                       _ptr(pk), _ptr(pv), Smax, _ptr(q_out), _ptr(qwt), _ptr(kwt),
                                       float(epsilon))
        return q_out, pk, pv


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def f16_to_f64(bits):
    return default().f16_to_f64(bits)


def f64_to_f16(v):
    return default().f64_to_f16(v)


def bf16_to_f64(bits):
    return default().bf16_to_f64(bits)


def f64_to_bf16(v):
    return default().f64_to_bf16(v)


def inv_freq(base, rotary_dim):
    return default().inv_freq(base, rotary_dim)


def cos_sin_cache(dtype, rows, inv_freq_arr, scaling=1.0):
    return default().cos_sin_cache(dtype, rows, inv_freq_arr, scaling)


def onthefly_row(dtype, position, inv_freq_arr, scaling=1.0):
    return default().onthefly_row(dtype, position, inv_freq_arr, scaling)


def rope_apply(*a, **kw):
    return default().rope_apply(*a, **kw)


def mrope_slot_streams(half, section, layout):
    return default().mrope_slot_streams(half, section, layout)


def mrope_apply(*a, **kw):
    return default().mrope_apply(*a, **kw)


def rope_apply_qk(*a, **kw):
    return default().rope_apply_qk(*a, **kw)


def rope_kv_append(*a, **kw):
    return default().rope_kv_append(*a, **kw)


def rope_apply_qk_norm(*a, **kw):
    return default().rope_apply_qk_norm(*a, **kw)


def table_for(workload, dtype=None):
    """cos/sin tables for a workload (rope_inputs.Workload), built by the oracle.

    Gathered workloads get the (M, R/2) table; the per-token case gets the
    (B, S, R/2) table with rows for positions 0..S-1 in every batch."""
    dt = dtype or workload.dtype
    inv = inv_freq(workload.cache_base, workload.rotary_dim)
    pos = workload.cache_positions()
    cos, sin = cos_sin_cache(dt, len(pos), inv, workload.scaling)
    if not workload.has_ids and workload.op != "mrope":
        cos = np.ascontiguousarray(np.broadcast_to(cos, (workload.batch,) + cos.shape))
        sin = np.ascontiguousarray(np.broadcast_to(sin, (workload.batch,) + sin.shape))
    return cos, sin
