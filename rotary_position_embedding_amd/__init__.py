"""Rotary position embedding for AMD Instinct MI355X (gfx950).

Python face of librope_mi355x.so. Each function here only marshals torch
tensors into the C ABI (include/rope_mi355x.h): device pointers, shapes,
element types and the current HIP stream. Every step of the computation runs
in the library's HIP kernels; nothing falls back to torch or the CPU.

    rope_apply      ONNX RotaryEmbedding
    mrope_apply     com.microsoft.MRotaryEmbedding
    rope_apply_qk   Q and K rotated with shared coefficients (table or on the fly)
    rope_apply_qkv_packed  the same on a packed [Q|K|V] activation
    rope_inv_freq   frequency vector base^(-2i/R)
    rope_cos_sin_cache  cos/sin tables from inv_freq
"""
import ctypes

import torch

from . import _lib
from ._lib import ROPE_BFLOAT16, ROPE_FLOAT, ROPE_FLOAT16, ROPE_INT32, ROPE_INT64

__all__ = ["RopeError", "rope_apply", "mrope_apply", "rope_apply_qk", "rope_inv_freq",
           "rope_cos_sin_cache", "rope_apply_check", "mrope_apply_check",
           "rope_apply_qk_check", "set_kernel_policy", "library_path", "Launcher",
           "rope_apply_launcher", "mrope_apply_launcher", "rope_apply_qk_launcher",
           "rope_apply_qkv_packed", "rope_apply_qkv_packed_check", "rope_apply_qkv_packed_launcher",
           "rope_kv_append", "rope_kv_append_check", "rope_kv_append_launcher",
           "rope_apply_qk_norm", "rope_apply_qk_norm_check", "rope_apply_qk_norm_launcher",
           "rope_kv_append_qk_norm", "rope_kv_append_qk_norm_check", "rope_kv_append_qk_norm_launcher"]

_DTYPE = {torch.float32: ROPE_FLOAT, torch.float16: ROPE_FLOAT16, torch.int64: ROPE_INT64,
          torch.bfloat16: ROPE_BFLOAT16, torch.int32: ROPE_INT32}

library_path = _lib.LIB_PATH


class RopeError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.status_name = _lib.STATUS.get(status, "ROPE_ERR_UNKNOWN")
        super().__init__("%s: %s" % (self.status_name, message))


def _check(rc):
    if rc != 0:
        msg = _lib.load().rope_last_error().decode(errors="replace")
        raise RopeError(rc, msg)


def _desc(t, device=None):
    """rope_tensor for a dense tensor; None stays None (absent input)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor, got %r" % type(t))
    if not t.is_contiguous():
        raise ValueError("tensors must be dense row-major (contiguous)")
    if device is not None and t.device != device:
        raise ValueError("all tensors must be on %s, got %s" % (device, t.device))
    return _lib.desc(t.data_ptr(), _DTYPE.get(t.dtype, 0), tuple(t.shape))


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _device_of(x):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("inputs must be GPU tensors")
    return x.device


class _on_device:
    """Make `device` current for the call if it is not already."""

    def __init__(self, device):
        self.device = device
        self.prev = None

    def __enter__(self):
        cur = torch.cuda.current_device()
        if cur != self.device.index:
            self.prev = cur
            torch.cuda.set_device(self.device)

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)


# ---------------------------------------------------------------------------

def rope_apply(x, cos_cache, sin_cache, position_ids=None, *, interleaved=0, num_heads=0,
               rotary_embedding_dim=0, out=None):
    """ONNX RotaryEmbedding. Returns y (a new tensor, or `out`; out may be x)."""
    dev = _device_of(x)
    y = torch.empty_like(x) if out is None else out
    dx, dc, ds, di, dy = (_desc(t, dev) for t in (x, cos_cache, sin_cache, position_ids, y))
    with _on_device(dev):
        _check(_lib.load().rope_apply(_lib.ref(dx), _lib.ref(dc), _lib.ref(ds), _lib.ref(di),
                                      _lib.ref(dy), interleaved, num_heads, rotary_embedding_dim,
                                      _stream(dev)))
    return y


def mrope_apply(x, position_ids, cos_cache, sin_cache, *, mrope_section, interleaved=0,
                is_packed_batching=0, mrope_layout=0, num_heads=0, rotary_embedding_dim=0,
                scale=1.0, out=None):
    """com.microsoft.MRotaryEmbedding. position_ids: (3, B, S) int64."""
    dev = _device_of(x)
    y = torch.empty_like(x) if out is None else out
    dx, di, dc, ds, dy = (_desc(t, dev) for t in (x, position_ids, cos_cache, sin_cache, y))
    sec = (ctypes.c_int64 * 3)(*[int(v) for v in mrope_section]) if mrope_section is not None else None
    with _on_device(dev):
        _check(_lib.load().mrope_apply(_lib.ref(dx), _lib.ref(di), _lib.ref(dc), _lib.ref(ds),
                                       _lib.ref(dy), interleaved, is_packed_batching, mrope_layout,
                                       sec, num_heads, rotary_embedding_dim, scale, _stream(dev)))
    return y


def rope_apply_qk(q, k, cos_cache=None, sin_cache=None, position_ids=None, *, interleaved=0,
                  num_heads=0, kv_num_heads=0, rotary_embedding_dim=0, inv_freq=None,
                  attention_scaling=1.0, out_q=None, out_k=None):
    """Q and K with the same coefficients, one launch. cos_cache=sin_cache=None
    computes the coefficients on the fly from inv_freq and position_ids."""
    dev = _device_of(q)
    yq = torch.empty_like(q) if out_q is None else out_q
    yk = torch.empty_like(k) if out_k is None else out_k
    ds = [_desc(t, dev) for t in (q, k, cos_cache, sin_cache, position_ids, yq, yk, inv_freq)]
    with _on_device(dev):
        _check(_lib.load().rope_apply_qk(*[_lib.ref(d) for d in ds[:7]], interleaved, num_heads,
                                         kv_num_heads, rotary_embedding_dim, _lib.ref(ds[7]),
                                         attention_scaling, _stream(dev)))
    return yq, yk


def rope_apply_qkv_packed(qkv, cos_cache=None, sin_cache=None, position_ids=None, *,
                          interleaved=0, num_heads=0, kv_num_heads=0, rotary_embedding_dim=0,
                          inv_freq=None, attention_scaling=1.0, out=None):
    """Packed [Q|K|V] (rank 3 (B, S, (H+2Hk)*D) or rank 4 (B, H+2Hk, S, D)):
    query and key heads rotated, value heads copied; out may be qkv (in place)."""
    dev = _device_of(qkv)
    y = torch.empty_like(qkv) if out is None else out
    ds = [_desc(t, dev) for t in (qkv, cos_cache, sin_cache, position_ids, y, inv_freq)]
    with _on_device(dev):
        _check(_lib.load().rope_apply_qkv_packed(*[_lib.ref(d) for d in ds[:5]], interleaved,
                                                 num_heads, kv_num_heads, rotary_embedding_dim,
                                                 _lib.ref(ds[5]), attention_scaling, _stream(dev)))
    return y


def rope_apply_qkv_packed_check(qkv, cos_cache, sin_cache, position_ids, y, *, interleaved=0,
                                num_heads=0, kv_num_heads=0, rotary_embedding_dim=0,
                                inv_freq=None, attention_scaling=1.0):
    v = _variant_out()
    rc = _lib.load().rope_apply_qkv_packed_check(_lib.ref(qkv), _lib.ref(cos_cache),
                                                 _lib.ref(sin_cache), _lib.ref(position_ids),
                                                 _lib.ref(y), interleaved, num_heads, kv_num_heads,
                                                 rotary_embedding_dim, _lib.ref(inv_freq),
                                                 attention_scaling, ctypes.byref(v))
    return rc, (v.value.decode() if rc == 0 and v.value else None)


def rope_apply_qkv_packed_launcher(qkv, cos_cache, sin_cache, position_ids, out, *, interleaved=0,
                                   num_heads=0, kv_num_heads=0, rotary_embedding_dim=0,
                                   inv_freq=None, attention_scaling=1.0):
    dev = _device_of(qkv)
    ds = [_desc(t, dev) for t in (qkv, cos_cache, sin_cache, position_ids, out, inv_freq)]
    rc, variant = rope_apply_qkv_packed_check(*ds[:5], interleaved=interleaved, num_heads=num_heads,
                                        kv_num_heads=kv_num_heads,
                                        rotary_embedding_dim=rotary_embedding_dim,
                                        inv_freq=ds[5], attention_scaling=attention_scaling)
    _check(rc)
    args = [_lib.ref(d) for d in ds[:5]] + [interleaved, num_heads, kv_num_heads, rotary_embedding_dim,
                                            _lib.ref(ds[5]), attention_scaling, _stream(dev)]
    return Launcher(_lib.load().rope_apply_qkv_packed, args,
                    (ds, qkv, cos_cache, sin_cache, position_ids, out, inv_freq), variant)


def rope_apply_qk_norm(q, k, q_weight, k_weight, cos_cache=None, sin_cache=None, position_ids=None, *,
                       epsilon, interleaved=0, num_heads=0, kv_num_heads=0, rotary_embedding_dim=0,
                       inv_freq=None, attention_scaling=1.0, out_q=None, out_k=None):
    """RMSNorm of every Q and K head row (weights (D,), epsilon) then the
    rotation of rope_apply_qk, in one pass. Returns (yq, yk)."""
    dev = _device_of(q)
    yq = torch.empty_like(q) if out_q is None else out_q
    yk = torch.empty_like(k) if out_k is None else out_k
    ds = [_desc(t, dev) for t in (q, k, q_weight, k_weight, cos_cache, sin_cache, position_ids, yq, yk,
                                  inv_freq)]
    with _on_device(dev):
        _check(_lib.load().rope_apply_qk_norm(
            _lib.ref(ds[0]), _lib.ref(ds[1]), _lib.ref(ds[2]), _lib.ref(ds[3]), float(epsilon),
            *[_lib.ref(d) for d in ds[4:9]], interleaved, num_heads, kv_num_heads, rotary_embedding_dim,
            _lib.ref(ds[9]), attention_scaling, _stream(dev)))
    return yq, yk


def rope_apply_qk_norm_check(q, k, q_weight, k_weight, cos_cache, sin_cache, position_ids, yq, yk, *,
                             epsilon, interleaved=0, num_heads=0, kv_num_heads=0, rotary_embedding_dim=0,
                             inv_freq=None, attention_scaling=1.0):
    v = _variant_out()
    rc = _lib.load().rope_apply_qk_norm_check(
        _lib.ref(q), _lib.ref(k), _lib.ref(q_weight), _lib.ref(k_weight), float(epsilon),
        _lib.ref(cos_cache), _lib.ref(sin_cache), _lib.ref(position_ids), _lib.ref(yq), _lib.ref(yk),
        interleaved, num_heads, kv_num_heads, rotary_embedding_dim, _lib.ref(inv_freq), attention_scaling,
        ctypes.byref(v))
    return rc, (v.value.decode() if rc == 0 and v.value else None)


def rope_apply_qk_norm_launcher(q, k, q_weight, k_weight, cos_cache, sin_cache, position_ids, out_q, out_k,
                                *, epsilon, interleaved=0, num_heads=0, kv_num_heads=0,
                                rotary_embedding_dim=0, inv_freq=None, attention_scaling=1.0):
    dev = _device_of(q)
    ds = [_desc(t, dev) for t in (q, k, q_weight, k_weight, cos_cache, sin_cache, position_ids, out_q, out_k,
                                  inv_freq)]
    rc, variant = rope_apply_qk_norm_check(*ds[:9], epsilon=epsilon, interleaved=interleaved, num_heads=num_heads,
                                     kv_num_heads=kv_num_heads, rotary_embedding_dim=rotary_embedding_dim,
                                     inv_freq=ds[9], attention_scaling=attention_scaling)
    _check(rc)
    args = [_lib.ref(ds[0]), _lib.ref(ds[1]), _lib.ref(ds[2]), _lib.ref(ds[3]), float(epsilon)] + \
        [_lib.ref(d) for d in ds[4:9]] + [interleaved, num_heads, kv_num_heads, rotary_embedding_dim,
                                          _lib.ref(ds[9]), attention_scaling, _stream(dev)]
    return Launcher(_lib.load().rope_apply_qk_norm, args,
                    (ds, q, k, q_weight, k_weight, cos_cache, sin_cache, position_ids, out_q, out_k, inv_freq),
                    variant)


def rope_kv_append(query, key, value, past_key, past_value, key_total_sequence_lengths,
                   total_sequence_length, cos_cache, sin_cache, *, num_heads, kv_num_heads,
                   rotary_interleaved=0, out=None):
    """RoPE on Q and K with K and V appended to the caches in place (the
    SparseAttention rotary inputs). key = value = None: query is packed
    [Q|K|V]. Returns q_out ((B, S, H*D): a new tensor, or `out`, which may be
    an unpacked query); past_key and past_value are updated in place."""
    dev = _device_of(query)
    out = _q_out_for(query, key, num_heads, kv_num_heads) if out is None else out
    ds = [_desc(t, dev) for t in (query, key, value, past_key, past_value, key_total_sequence_lengths,
                                  cos_cache, sin_cache, out)]
    with _on_device(dev):
        _check(_lib.load().rope_kv_append(*[_lib.ref(d) for d in ds[:6]], int(total_sequence_length),
                                          *[_lib.ref(d) for d in ds[6:]], rotary_interleaved, num_heads,
                                          kv_num_heads, _stream(dev)))
    return out


def rope_kv_append_check(query, key, value, past_key, past_value, key_total_sequence_lengths,
                         total_sequence_length, cos_cache, sin_cache, q_out, *, num_heads,
                         kv_num_heads, rotary_interleaved=0):
    v = _variant_out()
    refs = [_lib.ref(d) for d in (query, key, value, past_key, past_value, key_total_sequence_lengths)]
    rc = _lib.load().rope_kv_append_check(*refs, int(total_sequence_length), _lib.ref(cos_cache),
                                          _lib.ref(sin_cache), _lib.ref(q_out), rotary_interleaved,
                                          num_heads, kv_num_heads, ctypes.byref(v))
    return rc, (v.value.decode() if rc == 0 and v.value else None)


def rope_kv_append_launcher(query, key, value, past_key, past_value, key_total_sequence_lengths,
                            total_sequence_length, cos_cache, sin_cache, out, *, num_heads,
                            kv_num_heads, rotary_interleaved=0):
    dev = _device_of(query)
    ds = [_desc(t, dev) for t in (query, key, value, past_key, past_value, key_total_sequence_lengths,
                                  cos_cache, sin_cache, out)]
    rc, variant = rope_kv_append_check(*ds[:6], total_sequence_length, *ds[6:], num_heads=num_heads,
                                 kv_num_heads=kv_num_heads, rotary_interleaved=rotary_interleaved)
    _check(rc)
    args = [_lib.ref(d) for d in ds[:6]] + [int(total_sequence_length)] + [_lib.ref(d) for d in ds[6:]] + \
        [rotary_interleaved, num_heads, kv_num_heads, _stream(dev)]
    return Launcher(_lib.load().rope_kv_append, args,
                    (ds, query, key, value, past_key, past_value, key_total_sequence_lengths, cos_cache,
                     sin_cache, out), variant)


def _q_out_for(query, key, num_heads, kv_num_heads):
    """q_out of (B, S, num_heads * head_size); shapes the library will refuse
    get an empty placeholder, so that its status names the failing clause."""
    groups = num_heads + (2 * kv_num_heads if key is None else 0)
    if query.dim() != 3 or groups < 1:
        return torch.empty(0, dtype=query.dtype, device=query.device)
    B, S, width = query.shape
    return torch.empty(B, S, width // groups * num_heads, dtype=query.dtype, device=query.device)


def rope_kv_append_qk_norm(query, key, value, past_key, past_value, key_total_sequence_lengths,
                           total_sequence_length, cos_cache, sin_cache, q_weight, k_weight, *, epsilon,
                           num_heads, kv_num_heads, rotary_interleaved=0, out=None):
    """rope_kv_append with Q and K RMS-normalised first (QK-norm weights (D,),
    epsilon); V copied as it is. Returns q_out; the caches are updated in place."""
    dev = _device_of(query)
    out = _q_out_for(query, key, num_heads, kv_num_heads) if out is None else out
    ds = [_desc(t, dev) for t in (query, key, value, past_key, past_value, key_total_sequence_lengths,
                                  cos_cache, sin_cache, out, q_weight, k_weight)]
    with _on_device(dev):
        _check(_lib.load().rope_kv_append_qk_norm(
            *[_lib.ref(d) for d in ds[:6]], int(total_sequence_length), *[_lib.ref(d) for d in ds[6:11]],
            float(epsilon), rotary_interleaved, num_heads, kv_num_heads, _stream(dev)))
    return out


def rope_kv_append_qk_norm_check(query, key, value, past_key, past_value, key_total_sequence_lengths,
                                 total_sequence_length, cos_cache, sin_cache, q_out, q_weight, k_weight, *,
                                 epsilon, num_heads, kv_num_heads, rotary_interleaved=0):
    v = _variant_out()
    refs = [_lib.ref(d) for d in (query, key, value, past_key, past_value, key_total_sequence_lengths)]
    rc = _lib.load().rope_kv_append_qk_norm_check(
        *refs, int(total_sequence_length), _lib.ref(cos_cache), _lib.ref(sin_cache), _lib.ref(q_out),
        _lib.ref(q_weight), _lib.ref(k_weight), float(epsilon), rotary_interleaved, num_heads, kv_num_heads,
        ctypes.byref(v))
    return rc, (v.value.decode() if rc == 0 and v.value else None)


def rope_kv_append_qk_norm_launcher(query, key, value, past_key, past_value, key_total_sequence_lengths,
                                    total_sequence_length, cos_cache, sin_cache, out, q_weight, k_weight, *,
                                    epsilon, num_heads, kv_num_heads, rotary_interleaved=0):
    dev = _device_of(query)
    ds = [_desc(t, dev) for t in (query, key, value, past_key, past_value, key_total_sequence_lengths,
                                  cos_cache, sin_cache, out, q_weight, k_weight)]
    rc, variant = rope_kv_append_qk_norm_check(*ds[:6], total_sequence_length, *ds[6:], epsilon=epsilon,
                                         num_heads=num_heads, kv_num_heads=kv_num_heads,
                                         rotary_interleaved=rotary_interleaved)
    _check(rc)
    args = [_lib.ref(d) for d in ds[:6]] + [int(total_sequence_length)] + [_lib.ref(d) for d in ds[6:11]] + \
        [float(epsilon), rotary_interleaved, num_heads, kv_num_heads, _stream(dev)]
    return Launcher(_lib.load().rope_kv_append_qk_norm, args,
                    (ds, query, key, value, past_key, past_value, key_total_sequence_lengths, cos_cache,
                     sin_cache, out, q_weight, k_weight), variant)


def rope_inv_freq(rotary_dim, base, device="cuda", out=None):
    """float32 (rotary_dim/2,) with inv_freq[i] = base^(-2i/rotary_dim)."""
    if out is None:
        out = torch.empty(rotary_dim // 2, dtype=torch.float32, device=device)
    dev = _device_of(out)
    d = _desc(out, dev)
    with _on_device(dev):
        _check(_lib.load().rope_inv_freq(_lib.ref(d), float(base), _stream(dev)))
    return out


def rope_cos_sin_cache(inv_freq, rows, dtype=torch.float16, scaling=1.0, out=None):
    """(rows, R/2) cos and sin tables of `dtype` for positions 0..rows-1."""
    dev = _device_of(inv_freq)
    if out is None:
        cos = torch.empty(rows, inv_freq.shape[0], dtype=dtype, device=dev)
        sin = torch.empty(rows, inv_freq.shape[0], dtype=dtype, device=dev)
    else:
        cos, sin = out
    di, dc, ds = (_desc(t, dev) for t in (inv_freq, cos, sin))
    with _on_device(dev):
        _check(_lib.load().rope_cos_sin_cache(_lib.ref(di), scaling, _lib.ref(dc), _lib.ref(ds),
                                              _stream(dev)))
    return cos, sin


# ---------------------------------------------------------------------------
# validation only (no GPU needed): status code and the kernel variant chosen

def _variant_out():
    return ctypes.c_char_p()


def rope_apply_check(x, cos_cache, sin_cache, position_ids=None, y=None, *, interleaved=0,
                     num_heads=0, rotary_embedding_dim=0):
    """(status, variant) for tensors given as rope_tensor-like objects (see
    tensor_spec); raises nothing."""
    v = _variant_out()
    rc = _lib.load().rope_apply_check(_lib.ref(x), _lib.ref(cos_cache), _lib.ref(sin_cache),
                                      _lib.ref(position_ids), _lib.ref(y), interleaved, num_heads,
                                      rotary_embedding_dim, ctypes.byref(v))
    return rc, (v.value.decode() if rc == 0 and v.value else None)


def mrope_apply_check(x, position_ids, cos_cache, sin_cache, y, *, mrope_section, interleaved=0,
                      is_packed_batching=0, mrope_layout=0, num_heads=0, rotary_embedding_dim=0,
                      scale=1.0):
    v = _variant_out()
    sec = (ctypes.c_int64 * 3)(*[int(s) for s in mrope_section]) if mrope_section is not None else None
    rc = _lib.load().mrope_apply_check(_lib.ref(x), _lib.ref(position_ids), _lib.ref(cos_cache),
                                       _lib.ref(sin_cache), _lib.ref(y), interleaved,
                                       is_packed_batching, mrope_layout, sec, num_heads,
                                       rotary_embedding_dim, scale, ctypes.byref(v))
    return rc, (v.value.decode() if rc == 0 and v.value else None)


def rope_apply_qk_check(q, k, cos_cache, sin_cache, position_ids, yq, yk, *, interleaved=0,
                        num_heads=0, kv_num_heads=0, rotary_embedding_dim=0, inv_freq=None,
                        attention_scaling=1.0):
    v = _variant_out()
    rc = _lib.load().rope_apply_qk_check(_lib.ref(q), _lib.ref(k), _lib.ref(cos_cache),
                                         _lib.ref(sin_cache), _lib.ref(position_ids), _lib.ref(yq),
                                         _lib.ref(yk), interleaved, num_heads, kv_num_heads,
                                         rotary_embedding_dim, _lib.ref(inv_freq),
                                         attention_scaling, ctypes.byref(v))
    return rc, (v.value.decode() if rc == 0 and v.value else None)


def tensor_spec(data_ptr, dtype_code, shape):
    """A rope_tensor descriptor from a raw address (for validation-only calls)."""
    return _lib.desc(data_ptr, dtype_code, shape)


def describe(t):
    """rope_tensor descriptor of a torch tensor (for the *_check functions)."""
    return _desc(t)


def set_kernel_policy(policy):
    """0: automatic, 1: the scalar kernel always, 2: the vector kernel wherever
    it applies (never the row kernel), 3: the row kernel wherever its shape
    rules allow, at any size. Returns the old policy."""
    return _lib.load().rope_set_kernel_policy(int(policy))


# ---------------------------------------------------------------------------
# pre-marshalled launches: descriptors and stream fixed once, each call is a
# single C call (for tight loops; the tensors must stay alive and unchanged
# in shape, address and stream)

class Launcher:
    """Zero-argument callable that re-issues one C-ABI call. `variant` names
    the kernel the call runs (as the *_check functions report it, e.g.
    "vec16/gather"), fixed when the launcher is made."""

    def __init__(self, fn, args, keep, variant=None):
        self._fn = fn
        self._args = args
        self._keep = keep      # descriptors and tensors referenced by args
        self.variant = variant

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _check(rc)


def rope_apply_launcher(x, cos_cache, sin_cache, position_ids, out, *, interleaved=0,
                        num_heads=0, rotary_embedding_dim=0):
    dev = _device_of(x)
    ds = [_desc(t, dev) for t in (x, cos_cache, sin_cache, position_ids, out)]
    rc, variant = rope_apply_check(*ds, interleaved=interleaved, num_heads=num_heads,
                             rotary_embedding_dim=rotary_embedding_dim)
    _check(rc)
    args = [_lib.ref(d) for d in ds] + [interleaved, num_heads, rotary_embedding_dim, _stream(dev)]
    return Launcher(_lib.load().rope_apply, args, (ds, x, cos_cache, sin_cache, position_ids, out), variant)


def mrope_apply_launcher(x, position_ids, cos_cache, sin_cache, out, *, mrope_section, interleaved=0,
                         is_packed_batching=0, mrope_layout=0, num_heads=0, rotary_embedding_dim=0,
                         scale=1.0):
    dev = _device_of(x)
    ds = [_desc(t, dev) for t in (x, position_ids, cos_cache, sin_cache, out)]
    sec = (ctypes.c_int64 * 3)(*[int(v) for v in mrope_section])
    rc, variant = mrope_apply_check(*ds, mrope_section=mrope_section, interleaved=interleaved,
                              is_packed_batching=is_packed_batching, mrope_layout=mrope_layout,
                              num_heads=num_heads, rotary_embedding_dim=rotary_embedding_dim,
                              scale=scale)
    _check(rc)
    args = [_lib.ref(d) for d in ds] + [interleaved, is_packed_batching, mrope_layout, sec, num_heads,
                                        rotary_embedding_dim, scale, _stream(dev)]
    return Launcher(_lib.load().mrope_apply, args, (ds, sec, x, position_ids, cos_cache, sin_cache, out),
                    variant)


def rope_apply_qk_launcher(q, k, cos_cache, sin_cache, position_ids, out_q, out_k, *, interleaved=0,
                           num_heads=0, kv_num_heads=0, rotary_embedding_dim=0, inv_freq=None,
                           attention_scaling=1.0):
    dev = _device_of(q)
    ds = [_desc(t, dev) for t in (q, k, cos_cache, sin_cache, position_ids, out_q, out_k, inv_freq)]
    rc, variant = rope_apply_qk_check(*ds[:7], interleaved=interleaved, num_heads=num_heads,
                                kv_num_heads=kv_num_heads, rotary_embedding_dim=rotary_embedding_dim,
                                inv_freq=ds[7], attention_scaling=attention_scaling)
    _check(rc)
    args = [_lib.ref(d) for d in ds[:7]] + [interleaved, num_heads, kv_num_heads, rotary_embedding_dim,
                                            _lib.ref(ds[7]), attention_scaling, _stream(dev)]
    return Launcher(_lib.load().rope_apply_qk, args,
                    (ds, q, k, cos_cache, sin_cache, position_ids, out_q, out_k, inv_freq), variant)
