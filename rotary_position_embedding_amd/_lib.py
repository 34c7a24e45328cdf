"""ctypes view of librope_mi355x.so (declared in include/rope_mi355x.h).

Loading fails loudly if the library has not been built, or was built from
other sources than the ones beside it: there is no other implementation
behind these names.
"""
import ctypes
import os

from . import build as _build

HERE = os.path.dirname(os.path.abspath(__file__))
# ROPE_MI355X_LIBRARY selects another build of the same sources (the
# sanitizer build of the CPU tests); by default the in-tree library
LIB_PATH = os.path.abspath(os.environ.get("ROPE_MI355X_LIBRARY") or os.path.join(HERE, "librope_mi355x.so"))

ROPE_FLOAT = 1
ROPE_INT32 = 6
ROPE_INT64 = 7
ROPE_FLOAT16 = 10
ROPE_BFLOAT16 = 16

STATUS = {
    0: "ROPE_OK", -1: "ROPE_ERR_NULL", -2: "ROPE_ERR_DTYPE", -3: "ROPE_ERR_RANK",
    -4: "ROPE_ERR_SHAPE", -5: "ROPE_ERR_ATTRIBUTE", -6: "ROPE_ERR_UNSUPPORTED",
    -7: "ROPE_ERR_ALIAS", -8: "ROPE_ERR_LAUNCH",
}

# Every function declared in the header: name -> (argtypes, restype).
# rope_tensor* arguments are passed as c_void_p to allow NULL.


class RopeTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("shape", ctypes.c_int64 * 4)]


_vp, _i64, _f32, _f64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_int
_ccp = ctypes.POINTER(ctypes.c_char_p)

SIGNATURES = {
    "rope_status_string": ([_int], ctypes.c_char_p),
    "rope_last_error": ([], ctypes.c_char_p),
    "rope_apply": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp], _int),
    "mrope_apply": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _f32, _vp], _int),
    "rope_apply_qk": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _f32, _vp], _int),
    "rope_inv_freq": ([_vp, _f64, _vp], _int),
    "rope_cos_sin_cache": ([_vp, _f32, _vp, _vp, _vp], _int),
    "rope_apply_check": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _ccp], _int),
    "mrope_apply_check": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _f32, _ccp], _int),
    "rope_apply_qk_check": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _f32, _ccp], _int),
    "rope_set_kernel_policy": ([_int], _int),
    "rope_apply_qkv_packed": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _f32, _vp], _int),
    "rope_apply_qkv_packed_check": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _f32, _ccp], _int),
    "rope_apply_qk_norm": ([_vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _f32, _vp], _int),
    "rope_apply_qk_norm_check": ([_vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _f32, _ccp], _int),
    "rope_kv_append_qk_norm": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _f32,
                                _i64, _i64, _i64, _vp], _int),
    "rope_kv_append_qk_norm_check": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _f32,
                                      _i64, _i64, _i64, _ccp], _int),
    "rope_kv_append": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _vp], _int),
    "rope_kv_append_check": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _ccp], _int),
}

_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "librope_mi355x.so is not built (%s); run python -m rotary_position_embedding_amd.build -- "
            "there is no fallback implementation" % LIB_PATH)
    if not _build.is_current(LIB_PATH):
        raise ImportError(
            "%s was built from other sources (recorded %s, sources now %s); "
            "rebuild it with python -m rotary_position_embedding_amd.build" % (LIB_PATH, _build.built_hash(LIB_PATH),
                                                         _build.source_hash()))
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def desc(data_ptr: int, dtype_code: int, shape) -> RopeTensor:
    t = RopeTensor()
    t.data = data_ptr
    t.dtype = dtype_code
    t.rank = len(shape)
    for i, d in enumerate(shape):
        t.shape[i] = int(d)
    return t


def ref(t):
    """Pointer to a RopeTensor, or None."""
    return None if t is None else ctypes.addressof(t)
