"""ctypes/numpy front end of the CPU oracle.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. The GPU library never calls it and
has no fallback to it.

Inputs are numpy arrays on the host: bf16 data as ``uint16`` bit patterns,
fp32 as ``float32``. Every function returns freshly allocated numpy arrays and
raises ``OracleError`` on a nonzero status.
"""
import ctypes
import os

import numpy as np

from . import build as _build

FMT_E4M3 = 1
FMT_E2M1 = 2
FMT_E5M2 = 3
FMT_E5M6 = 4
OUT_BF16 = 1
OUT_F32 = 2
SF_ROUND_POW2 = 1
SF_COL_MAJOR = 2
SF_PACKED_UE8M0 = 4
_FMT_NAMES = {"e4m3": FMT_E4M3, "e2m1": FMT_E2M1, "e5m2": FMT_E5M2, "e5m6": FMT_E5M6}

_lib = None


class OracleError(RuntimeError):
    pass


def fmt_id(fmt):
    if isinstance(fmt, str):
        return _FMT_NAMES[fmt.lower()]
    return int(fmt)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _build.is_current():
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
    vp = ctypes.c_void_p
    sig = {
        "oracle_version": ([], i32),
        "oracle_decode": ([i32, ctypes.c_uint8], f32),
        "oracle_encode": ([i32, f32], ctypes.c_uint8),
        "oracle_encode_array": ([i32, vp, i64, vp], None),
        "oracle_decode_array": ([i32, vp, i64, vp], None),
        "oracle_decode16": ([i32, ctypes.c_uint16], f32),
        "oracle_encode16": ([i32, f32], ctypes.c_uint16),
        "oracle_encode_array16": ([i32, vp, i64, vp], None),
        "oracle_decode_array16": ([i32, vp, i64, vp], None),
        "oracle_exp_array": ([vp, i64, vp], None),
        "oracle_format_max": ([i32], f32),
        "oracle_default_floor": ([i32], f32),
        "oracle_scale": ([i32, f32, f32, vp, vp], i32),
        "oracle_per_token": ([vp, i64, i64, i32, i32, f32, vp, vp], i32),
        "oracle_per_token_f32": ([vp, i64, i64, i32, i32, f32, vp, vp], i32),
        "oracle_swiglu_per_token": ([vp, i64, i64, vp, i32, i32, f32, vp, vp], i32),
        "oracle_swiglu_values": ([vp, i64, i64, vp, vp], i32),
        "oracle_per_block": ([vp, i64, i64, i32, i32, f32, vp, vp], i32),
        "oracle_per_channel_T": ([vp, i64, i64, i32, i32, f32, vp, vp], i32),
        "oracle_dequant_per_token": ([vp, vp, i64, i64, i32, i32, vp], i32),
        "oracle_cast_back": ([vp, vp, i64, i64, i32, i32, i32, vp], i32),
        "oracle_f32_to_bf16": ([f32], ctypes.c_uint16),
        "oracle_per_token_sf": ([vp, i64, i64, i32, i32, f32, i32, vp, vp], i32),
        "oracle_swiglu_per_token_sf": ([vp, i64, i64, vp, i32, i32, f32, i32, vp, vp], i32),
        "oracle_swiglu_values_ex": ([vp, i64, i64, vp, f32, vp, vp], i32),
        "oracle_swiglu_per_token_ex": ([vp, i64, i64, vp, i32, i32, f32, i32, f32, vp, vp, vp],
                                       i32),
        "oracle_swiglu_backward_values": ([vp, vp, i64, i64, vp, f32, vp], i32),
        "oracle_swiglu_backward_per_token": ([vp, vp, i64, i64, vp, i32, i32, f32, f32, vp, vp],
                                             i32),
        "oracle_swiglu_per_channel_T": ([vp, i64, i64, vp, i32, i32, f32, f32, vp, vp], i32),
        "oracle_per_channel": ([vp, i64, i64, i32, i32, f32, vp, vp], i32),
        "oracle_per_block_sf": ([vp, i64, i64, i32, i32, f32, i32, vp, vp], i32),
        "oracle_per_channel_sf": ([vp, i64, i64, i32, i32, f32, i32, vp, vp], i32),
        "oracle_per_channel_T_sf": ([vp, i64, i64, i32, i32, f32, i32, vp, vp], i32),
        "oracle_swiglu_per_channel_T_sf": ([vp, i64, i64, vp, i32, i32, f32, i32, f32, vp, vp],
                                           i32),
        "oracle_swiglu_backward_per_token_sf": ([vp, vp, i64, i64, vp, i32, i32, f32, i32, f32,
                                                 vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle status {rc}")


def _u16(x):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("bf16 input must be given as uint16 bit patterns")
    return x


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _code_shape(fmt, rows, cols):
    if fmt == FMT_E2M1:
        return (rows, cols // 2)
    if fmt == FMT_E5M6:
        return (rows, cols // 2 * 3)
    return (rows, cols)


def exp_f32(x):
    """e^x rounded to the nearest fp32 value, for fp32 x (SiLU's exponential)."""
    x = _f32(x)
    out = np.empty_like(x)
    _load().oracle_exp_array(_ptr(x), x.size, _ptr(out))
    return out


def format_max(fmt):
    return _load().oracle_format_max(fmt_id(fmt))


def default_floor(fmt):
    return _load().oracle_default_floor(fmt_id(fmt))


def encode(fmt, y):
    """fp32 values -> codes (uint8; uint16 for E5M6)."""
    f = fmt_id(fmt)
    y = _f32(y)
    if f == FMT_E5M6:
        out = np.empty(y.shape, np.uint16)
        _load().oracle_encode_array16(f, _ptr(y), y.size, _ptr(out))
        return out
    out = np.empty(y.shape, np.uint8)
    _load().oracle_encode_array(f, _ptr(y), y.size, _ptr(out))
    return out


def decode(fmt, codes):
    f = fmt_id(fmt)
    if f == FMT_E5M6:
        codes = np.ascontiguousarray(codes, dtype=np.uint16)
        out = np.empty(codes.shape, np.float32)
        _load().oracle_decode_array16(f, _ptr(codes), codes.size, _ptr(out))
        return out
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float32)
    _load().oracle_decode_array(f, _ptr(codes), codes.size, _ptr(out))
    return out


def unpack_e5m6(q):
    """Packed E5M6 rows (three bytes per column pair, little-endian bit
    stream) -> uint16 codes, one per column."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    t = q.reshape(q.shape[:-1] + (q.shape[-1] // 3, 3)).astype(np.uint16)
    out = np.empty(q.shape[:-1] + (q.shape[-1] // 3 * 2,), np.uint16)
    out[..., 0::2] = t[..., 0] | ((t[..., 1] & 0xF) << 8)
    out[..., 1::2] = (t[..., 1] >> 4) | (t[..., 2] << 4)
    return out


def scale(fmt, amax, clamp_min=0.0):
    sf = np.zeros(1, np.float32)
    inv = np.zeros(1, np.float32)
    _check(_load().oracle_scale(fmt_id(fmt), float(amax), float(clamp_min), _ptr(sf), _ptr(inv)),
           "scale")
    return sf[0], inv[0]


def per_token(x, fmt="e4m3", group=128, clamp_min=0.0):
    f = fmt_id(fmt)
    x = _u16(x)
    rows, cols = x.shape
    q = np.zeros(_code_shape(f, rows, cols), np.uint8)
    sf = np.zeros((rows, cols // group if group > 0 else 0), np.float32)
    _check(_load().oracle_per_token(_ptr(x), rows, cols, f, group, clamp_min, _ptr(q), _ptr(sf)),
           "per_token")
    return q, sf


def per_token_f32(x, fmt="e4m3", group=128, clamp_min=0.0):
    f = fmt_id(fmt)
    x = _f32(x)
    rows, cols = x.shape
    q = np.zeros(_code_shape(f, rows, cols), np.uint8)
    sf = np.zeros((rows, cols // group if group > 0 else 0), np.float32)
    _check(_load().oracle_per_token_f32(_ptr(x), rows, cols, f, group, clamp_min, _ptr(q),
                                        _ptr(sf)), "per_token_f32")
    return q, sf


def e2m1(x, group=32, clamp_min=0.0):
    return per_token(x, FMT_E2M1, group, clamp_min)


def swiglu_values(h, w=None):
    h = _u16(h)
    rows, two_n = h.shape
    cols = two_n // 2
    w = None if w is None else _f32(w)
    v = np.zeros((rows, cols), np.float32)
    _check(_load().oracle_swiglu_values(_ptr(h), rows, cols, _ptr(w), _ptr(v)), "swiglu_values")
    return v


def swiglu_per_token(h, w=None, fmt="e4m3", group=128, clamp_min=0.0):
    f = fmt_id(fmt)
    h = _u16(h)
    rows, two_n = h.shape
    cols = two_n // 2
    w = None if w is None else _f32(w)
    q = np.zeros(_code_shape(f, rows, cols), np.uint8)
    sf = np.zeros((rows, cols // group if group > 0 else 0), np.float32)
    _check(_load().oracle_swiglu_per_token(_ptr(h), rows, cols, _ptr(w), f, group, clamp_min,
                                           _ptr(q), _ptr(sf)), "swiglu_per_token")
    return q, sf


def per_block(x, fmt="e4m3", block=128, clamp_min=0.0):
    f = fmt_id(fmt)
    x = _u16(x)
    rows, cols = x.shape
    q = np.zeros(_code_shape(f, rows, cols), np.uint8)
    sf = np.zeros((rows // block, cols // block), np.float32)
    _check(_load().oracle_per_block(_ptr(x), rows, cols, f, block, clamp_min, _ptr(q), _ptr(sf)),
           "per_block")
    return q, sf


def per_channel_T(x, fmt="e4m3", group=128, clamp_min=0.0):
    f = fmt_id(fmt)
    x = _u16(x)
    rows, cols = x.shape
    qT = np.zeros(_code_shape(f, cols, rows), np.uint8)
    sf = np.zeros((cols, rows // group), np.float32)
    _check(_load().oracle_per_channel_T(_ptr(x), rows, cols, f, group, clamp_min, _ptr(qT),
                                        _ptr(sf)), "per_channel_T")
    return qT, sf


def dequant_per_token(q, sf, cols, fmt="e4m3", group=128):
    f = fmt_id(fmt)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sf = _f32(sf)
    rows = q.shape[0]
    out = np.zeros((rows, cols), np.float32)
    _check(_load().oracle_dequant_per_token(_ptr(q), _ptr(sf), rows, cols, f, group, _ptr(out)),
           "dequant_per_token")
    return out


def cast_back(q, sf, cols, fmt="e4m3", group=128, out_dtype="bf16"):
    """Per-token codes + scales -> bf16 (uint16 bit patterns) or fp32."""
    f = fmt_id(fmt)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sf = _f32(sf)
    rows = q.shape[0]
    od = OUT_BF16 if out_dtype == "bf16" else OUT_F32
    out = np.zeros((rows, cols), np.uint16 if od == OUT_BF16 else np.float32)
    _check(_load().oracle_cast_back(_ptr(q), _ptr(sf), rows, cols, f, group, od, _ptr(out)),
           "cast_back")
    return out


def f32_to_bf16(x):
    """fp32 values -> bf16 bit patterns (uint16), round to nearest even."""
    x = _f32(x)
    lib = _load()
    return np.array([lib.oracle_f32_to_bf16(float(v)) for v in x.ravel()],
                    np.uint16).reshape(x.shape)


def sf_shape(rows, cols, group, sf_flags):
    """Shape and dtype of the scale tensor for a layout."""
    groups = cols // group
    rows_pad = (rows + 3) // 4 * 4
    if sf_flags & SF_PACKED_UE8M0:
        shape = (groups // 4, rows_pad) if sf_flags & SF_COL_MAJOR else (rows, groups // 4)
        return shape, np.uint32
    shape = (groups, rows_pad) if sf_flags & SF_COL_MAJOR else (rows, groups)
    return shape, np.float32


def per_token_sf(x, fmt="e4m3", group=128, clamp_min=0.0, sf_flags=0, sf_fill=0):
    """Per-token cast with a scale-factor layout; unwritten padding keeps
    sf_fill."""
    f = fmt_id(fmt)
    x = _u16(x)
    rows, cols = x.shape
    q = np.zeros(_code_shape(f, rows, cols), np.uint8)
    shape, dt = sf_shape(rows, cols, group, sf_flags)
    sf = np.full(shape, sf_fill, dt)
    _check(_load().oracle_per_token_sf(_ptr(x), rows, cols, f, group, clamp_min, sf_flags, _ptr(q),
                                       _ptr(sf)), "per_token_sf")
    return q, sf


def swiglu_per_token_sf(h, w=None, fmt="e4m3", group=128, clamp_min=0.0, sf_flags=0, sf_fill=0):
    f = fmt_id(fmt)
    h = _u16(h)
    rows, two_n = h.shape
    cols = two_n // 2
    w = None if w is None else _f32(w)
    q = np.zeros(_code_shape(f, rows, cols), np.uint8)
    shape, dt = sf_shape(rows, cols, group, sf_flags)
    sf = np.full(shape, sf_fill, dt)
    _check(_load().oracle_swiglu_per_token_sf(_ptr(h), rows, cols, _ptr(w), f, group, clamp_min,
                                              sf_flags, _ptr(q), _ptr(sf)), "swiglu_per_token_sf")
    return q, sf


def swiglu_values_ex(h, w=None, swiglu_clamp=0.0):
    """SwiGLU values with the clamp; returns (v, number of clamped values)."""
    h = _u16(h)
    rows, two_n = h.shape
    cols = two_n // 2
    w = None if w is None else _f32(w)
    v = np.zeros((rows, cols), np.float32)
    count = np.zeros(1, np.uint64)
    _check(_load().oracle_swiglu_values_ex(_ptr(h), rows, cols, _ptr(w), swiglu_clamp, _ptr(v),
                                           _ptr(count)), "swiglu_values_ex")
    return v, int(count[0])


def swiglu_per_token_ex(h, w=None, fmt="e4m3", group=128, clamp_min=0.0, sf_flags=0,
                        swiglu_clamp=0.0, sf_fill=0):
    """Clamped SwiGLU + per-token cast; returns (q, sf, clamp count)."""
    f = fmt_id(fmt)
    h = _u16(h)
    rows, two_n = h.shape
    cols = two_n // 2
    w = None if w is None else _f32(w)
    q = np.zeros(_code_shape(f, rows, cols), np.uint8)
    shape, dt = sf_shape(rows, cols, group, sf_flags)
    sf = np.full(shape, sf_fill, dt)
    count = np.zeros(1, np.uint64)
    _check(_load().oracle_swiglu_per_token_ex(_ptr(h), rows, cols, _ptr(w), f, group, clamp_min,
                                              sf_flags, swiglu_clamp, _ptr(q), _ptr(sf),
                                              _ptr(count)), "swiglu_per_token_ex")
    return q, sf, int(count[0])


def swiglu_backward_values(h, dv, w=None, swiglu_clamp=0.0):
    """[dg | du] fp32 [rows, 2*cols] for the gradient dv [rows, cols] (bf16 bits)."""
    h = _u16(h)
    dv = _u16(dv)
    rows, two_n = h.shape
    cols = two_n // 2
    w = None if w is None else _f32(w)
    out = np.zeros((rows, two_n), np.float32)
    _check(_load().oracle_swiglu_backward_values(_ptr(h), _ptr(dv), rows, cols, _ptr(w),
                                                 swiglu_clamp, _ptr(out)),
           "swiglu_backward_values")
    return out


def swiglu_backward_per_token(h, dv, w=None, fmt="e4m3", group=128, clamp_min=0.0,
                              swiglu_clamp=0.0):
    f = fmt_id(fmt)
    h = _u16(h)
    dv = _u16(dv)
    rows, two_n = h.shape
    cols = two_n // 2
    w = None if w is None else _f32(w)
    q = np.zeros(_code_shape(f, rows, two_n), np.uint8)
    sf = np.zeros((rows, two_n // group if group > 0 else 0), np.float32)
    _check(_load().oracle_swiglu_backward_per_token(_ptr(h), _ptr(dv), rows, cols, _ptr(w), f,
                                                    group, clamp_min, swiglu_clamp, _ptr(q),
                                                    _ptr(sf)), "swiglu_backward_per_token")
    return q, sf


def swiglu_per_channel_T(h, w=None, fmt="e4m3", group=128, clamp_min=0.0, swiglu_clamp=0.0):
    f = fmt_id(fmt)
    h = _u16(h)
    rows, two_n = h.shape
    cols = two_n // 2
    w = None if w is None else _f32(w)
    qT = np.zeros(_code_shape(f, cols, rows), np.uint8)
    sf = np.zeros((cols, rows // group if group > 0 else 0), np.float32)
    _check(_load().oracle_swiglu_per_channel_T(_ptr(h), rows, cols, _ptr(w), f, group, clamp_min,
                                               swiglu_clamp, _ptr(qT), _ptr(sf)),
           "swiglu_per_channel_T")
    return qT, sf


def per_channel(x, fmt="e4m3", group=128, clamp_min=0.0):
    """Per-channel cast in the input layout: q [rows, cols], sf [rows/group, cols]."""
    f = fmt_id(fmt)
    x = _u16(x)
    rows, cols = x.shape
    q = np.zeros(_code_shape(f, rows, cols), np.uint8)
    sf = np.zeros((rows // group if group > 0 else 0, cols), np.float32)
    _check(_load().oracle_per_channel(_ptr(x), rows, cols, f, group, clamp_min, _ptr(q), _ptr(sf)),
           "per_channel")
    return q, sf


def per_block_sf(x, fmt="e4m3", block=128, clamp_min=0.0, sf_flags=0):
    """Per-block cast with round_sf (SF_ROUND_POW2, the one option it takes)."""
    f = fmt_id(fmt)
    x = _u16(x)
    rows, cols = x.shape
    q = np.zeros(_code_shape(f, rows, cols), np.uint8)
    sf = np.zeros((rows // block, cols // block) if block > 0 else (0, 0), np.float32)
    _check(_load().oracle_per_block_sf(_ptr(x), rows, cols, f, block, clamp_min, sf_flags, _ptr(q),
                                       _ptr(sf)), "per_block_sf")
    return q, sf


def per_channel_sf(x, fmt="e4m3", group=128, clamp_min=0.0, sf_flags=0):
    """Per-channel cast in the input layout with round_sf (SF_ROUND_POW2 only)."""
    f = fmt_id(fmt)
    x = _u16(x)
    rows, cols = x.shape
    q = np.zeros(_code_shape(f, rows, cols), np.uint8)
    sf = np.zeros((rows // group if group > 0 else 0, cols), np.float32)
    _check(_load().oracle_per_channel_sf(_ptr(x), rows, cols, f, group, clamp_min, sf_flags,
                                         _ptr(q), _ptr(sf)), "per_channel_sf")
    return q, sf


def per_channel_T_sf(x, fmt="e4m3", group=128, clamp_min=0.0, sf_flags=0, sf_fill=0):
    """Transposed per-channel cast with a scale layout: the per-token layout
    of x^T (rows = the channels, groups = the token groups)."""
    f = fmt_id(fmt)
    x = _u16(x)
    rows, cols = x.shape
    qT = np.zeros(_code_shape(f, cols, rows), np.uint8)
    shape, dt = sf_shape(cols, rows, group, sf_flags)
    sf = np.full(shape, sf_fill, dt)
    _check(_load().oracle_per_channel_T_sf(_ptr(x), rows, cols, f, group, clamp_min, sf_flags,
                                           _ptr(qT), _ptr(sf)), "per_channel_T_sf")
    return qT, sf


def swiglu_per_channel_T_sf(h, w=None, fmt="e4m3", group=128, clamp_min=0.0, sf_flags=0,
                            swiglu_clamp=0.0, sf_fill=0):
    f = fmt_id(fmt)
    h = _u16(h)
    rows, two_n = h.shape
    cols = two_n // 2
    w = None if w is None else _f32(w)
    qT = np.zeros(_code_shape(f, cols, rows), np.uint8)
    shape, dt = sf_shape(cols, rows, group, sf_flags)
    sf = np.full(shape, sf_fill, dt)
    _check(_load().oracle_swiglu_per_channel_T_sf(_ptr(h), rows, cols, _ptr(w), f, group,
                                                  clamp_min, sf_flags, swiglu_clamp, _ptr(qT),
                                                  _ptr(sf)), "swiglu_per_channel_T_sf")
    return qT, sf


def swiglu_backward_per_token_sf(h, dv, w=None, fmt="e4m3", group=128, clamp_min=0.0,
                                 sf_flags=0, swiglu_clamp=0.0, sf_fill=0):
    """SwiGLU backward + per-token cast of [dg | du] with a scale layout over
    rows of 2*cols values."""
    f = fmt_id(fmt)
    h = _u16(h)
    dv = _u16(dv)
    rows, two_n = h.shape
    cols = two_n // 2
    w = None if w is None else _f32(w)
    q = np.zeros(_code_shape(f, rows, two_n), np.uint8)
    shape, dt = sf_shape(rows, two_n, group, sf_flags)
    sf = np.full(shape, sf_fill, dt)
    _check(_load().oracle_swiglu_backward_per_token_sf(_ptr(h), _ptr(dv), rows, cols, _ptr(w), f,
                                                       group, clamp_min, sf_flags, swiglu_clamp,
                                                       _ptr(q), _ptr(sf)),
           "swiglu_backward_per_token_sf")
    return q, sf
