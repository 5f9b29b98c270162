"""Loading of libqcast.so and the ctypes signatures of its C ABI.

The library must have been built in-tree (``python -m
precision_quantization_amd.build``) from the sources beside it:
a missing or stale library is an error, never a fallback.
"""
import ctypes

from . import build as _build

QCAST_OK = 0
FMT_E4M3 = 1
FMT_E2M1 = 2
FMT_E5M2 = 3
FMT_E5M6 = 4
OUT_BF16 = 1
OUT_F32 = 2
SF_ROUND_POW2 = 1
SF_COL_MAJOR = 2
SF_PACKED_UE8M0 = 4
_FMT = {"e4m3": FMT_E4M3, "e2m1": FMT_E2M1, "e5m2": FMT_E5M2, "e5m6": FMT_E5M6}

_lib = None


class QcastError(RuntimeError):
    """A nonzero qcast_status, or a library that is missing or stale."""

    def __init__(self, status, what):
        self.status = status
        super().__init__(what)


def fmt_id(fmt):
    if isinstance(fmt, str):
        try:
            return _FMT[fmt.lower()]
        except KeyError:
            raise QcastError(4, f"unknown format {fmt!r}") from None
    return int(fmt)


def load():
    """The loaded library (built from the current sources), or QcastError."""
    global _lib
    if _lib is not None:
        return _lib
    import os
    if not os.path.exists(_build.LIB):
        raise QcastError(-1, f"{_build.LIB} is not built; run python -m precision_quantization_amd.build")
    if not _build.is_current():
        raise QcastError(-1, f"{_build.LIB} was built from other sources; rebuild it")
    lib = ctypes.CDLL(_build.LIB)
    i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    sig = {
        "qcast_per_token": [vp, i64, i64, i32, i32, f32, vp, vp, vp],
        "qcast_e2m1": [vp, i64, i64, i32, f32, vp, vp, vp],
        "qcast_swiglu_per_token": [vp, i64, i64, vp, i32, i32, f32, vp, vp, vp],
        "qcast_per_block": [vp, i64, i64, i32, i32, f32, vp, vp, vp],
        "qcast_per_channel_T": [vp, i64, i64, i32, i32, f32, vp, vp, vp],
        "qcast_cast_back": [vp, vp, i64, i64, i32, i32, i32, vp, vp],
        "qcast_per_token_sf": [vp, i64, i64, i32, i32, f32, i32, vp, vp, vp],
        "qcast_swiglu_per_token_sf": [vp, i64, i64, vp, i32, i32, f32, i32, vp, vp, vp],
        "qcast_swiglu_per_token_ex": [vp, i64, i64, vp, i32, i32, f32, i32, f32, vp, vp, vp,
                                      vp, vp],
        "qcast_swiglu_backward_per_token": [vp, vp, i64, i64, vp, i32, i32, f32, f32, vp, vp,
                                            vp],
        "qcast_swiglu_per_channel_T": [vp, i64, i64, vp, i32, i32, f32, f32, vp, vp, vp, vp,
                                       vp],
        "qcast_per_channel": [vp, i64, i64, i32, i32, f32, vp, vp, vp],
        "qcast_swiglu_per_token_noalloc": [vp, i64, i64, vp, i32, i32, f32, i32, f32, vp, vp,
                                           vp, vp],
        "qcast_per_block_sf": [vp, i64, i64, i32, i32, f32, i32, vp, vp, vp],
        "qcast_per_channel_sf": [vp, i64, i64, i32, i32, f32, i32, vp, vp, vp],
        "qcast_per_channel_T_sf": [vp, i64, i64, i32, i32, f32, i32, vp, vp, vp],
        "qcast_swiglu_per_channel_T_sf": [vp, i64, i64, vp, i32, i32, f32, i32, f32, vp, vp, vp,
                                          vp, vp],
        "qcast_swiglu_backward_per_token_sf": [vp, vp, i64, i64, vp, i32, i32, f32, i32, f32, vp,
                                               vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = i32
    lib.qcast_status_str.argtypes = [i32]
    lib.qcast_status_str.restype = ctypes.c_char_p
    lib.qcast_abi_version.argtypes = []
    lib.qcast_abi_version.restype = i32
    lib.qcast_bench_copy.argtypes = [vp, vp, i64, vp]
    lib.qcast_bench_copy.restype = i32
    lib.qcast_bench_check_scale.argtypes = [i32, ctypes.c_uint32, ctypes.c_uint32, vp, vp]
    lib.qcast_bench_check_scale.restype = i32
    lib.qcast_bench_time_next.argtypes = [vp, vp]
    lib.qcast_bench_time_next.restype = i32
    lib.qcast_bench_per_channel_T_traffic.argtypes = [vp, i64, i64, vp, vp]
    lib.qcast_bench_per_channel_T_traffic.restype = i32
    lib.qcast_set_num_cus.argtypes = [i32]
    lib.qcast_set_num_cus.restype = None
    _lib = lib
    return lib


def check(status, what):
    if status != QCAST_OK:
        msg = load().qcast_status_str(status).decode()
        raise QcastError(status, f"{what}: {msg} (status {status})")


EXPORTS = ["qcast_per_token", "qcast_e2m1", "qcast_swiglu_per_token", "qcast_per_block",
           "qcast_per_channel_T", "qcast_cast_back", "qcast_per_token_sf",
           "qcast_swiglu_per_token_sf", "qcast_swiglu_per_token_ex",
           "qcast_swiglu_backward_per_token", "qcast_swiglu_per_channel_T", "qcast_per_channel",
           "qcast_swiglu_per_token_noalloc", "qcast_per_block_sf", "qcast_per_channel_sf",
           "qcast_per_channel_T_sf", "qcast_swiglu_per_channel_T_sf",
           "qcast_swiglu_backward_per_token_sf", "qcast_status_str", "qcast_abi_version", "qcast_set_num_cus",
           "qcast_bench_copy", "qcast_bench_check_scale", "qcast_bench_time_next",
           "qcast_bench_per_channel_T_traffic"]
