"""The C ABI without a GPU: the library loads, exports every function that
include/qcast.h declares, and rejects bad arguments before any HIP call.

No test here passes a pointer that a kernel could dereference: rejected calls
return before launching, and the one call that would get past validation is
made only on a host without a GPU (it must then report QCAST_ERR_DEVICE).
"""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT, gpu_available

HEADERS = [os.path.join(ROOT, "include", h) for h in ("qcast.h", "qcast_bench.h")]

(OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_FORMAT, ERR_GROUP, ERR_LAUNCH, ERR_DEVICE,
 ERR_VALUE) = range(9)
E4M3, E2M1, E5M2 = 1, 2, 3
A16 = 0x10000          # aligned, never dereferenced (rejected before use)
MIS = 0x10008          # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    from precision_quantization_amd import _lib
    return _lib.load()


def declared_functions():
    names = []
    for h in HEADERS:
        names += re.findall(r"QCAST_API\s+[\w\s\*]+?\b(qcast_\w+)\s*\(", open(h).read())
    return names


def test_every_header_is_covered():
    import glob
    assert sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))) == sorted(HEADERS)


def test_header_declares_the_five_casts():
    names = declared_functions()
    for n in ["qcast_per_token", "qcast_swiglu_per_token", "qcast_per_block",
              "qcast_per_channel_T", "qcast_e2m1"]:
        assert n in names


def test_library_exports_every_declared_symbol_and_nothing_else():
    from precision_quantization_amd import build
    out = subprocess.run(["nm", "-D", "--defined-only", build.LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions())


def test_binding_names_match_the_c_entry_points():
    import precision_quantization_amd as pq
    for n in declared_functions():
        if n != "qcast_status_str":
            assert callable(getattr(pq, n)), n


def test_abi_version_and_status_strings(lib):
    assert lib.qcast_abi_version() == 5
    for s in range(9):
        assert lib.qcast_status_str(s).decode()
    assert lib.qcast_status_str(99).decode() == "unknown status"
    assert "out of range" in lib.qcast_status_str(8).decode()


def pt(lib, x=A16, rows=4, cols=256, fmt=E4M3, group=128, q=A16, sf=A16):
    return lib.qcast_per_token(x, rows, cols, fmt, group, 0.0, q, sf, None)


def test_per_token_validation(lib):
    assert pt(lib, fmt=9) == ERR_FORMAT
    assert pt(lib, group=16) == ERR_GROUP
    assert pt(lib, group=256) == ERR_GROUP
    assert pt(lib, cols=200) == ERR_SHAPE
    assert pt(lib, rows=-1) == ERR_SHAPE
    assert pt(lib, rows=2 ** 60, cols=2 ** 10) == ERR_SHAPE        # element count overflow
    assert pt(lib, x=None) == ERR_NULL
    assert pt(lib, q=None) == ERR_NULL
    assert pt(lib, sf=None) == ERR_NULL
    assert pt(lib, x=MIS) == ERR_ALIGN
    assert pt(lib, q=MIS) == ERR_ALIGN
    assert pt(lib, sf=A16 + 2) == ERR_ALIGN
    # empty inputs are valid and launch nothing, even with null pointers
    assert pt(lib, rows=0, x=None, q=None, sf=None) == OK
    assert pt(lib, cols=0, x=None, q=None, sf=None) == OK


def test_e2m1_validation(lib):
    assert lib.qcast_e2m1(A16, 4, 256, 16, 0.0, A16, A16, None) == ERR_GROUP
    assert lib.qcast_e2m1(A16, 4, 48, 32, 0.0, A16, A16, None) == ERR_SHAPE
    assert lib.qcast_e2m1(None, 4, 64, 32, 0.0, A16, A16, None) == ERR_NULL
    assert lib.qcast_e2m1(None, 0, 64, 32, 0.0, None, None, None) == OK


def test_swiglu_validation(lib):
    f = lib.qcast_swiglu_per_token
    assert f(A16, 4, 256, None, 9, 32, 0.0, A16, A16, None) == ERR_FORMAT
    assert f(A16, 4, 256, None, E4M3, 100, 0.0, A16, A16, None) == ERR_GROUP
    assert f(A16, 4, 200, None, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert f(A16, 4, 1 << 19, None, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE  # row too long
    assert f(None, 4, 256, None, E4M3, 128, 0.0, A16, A16, None) == ERR_NULL
    assert f(A16, 4, 256, A16 + 2, E4M3, 128, 0.0, A16, A16, None) == ERR_ALIGN
    assert f(None, 0, 256, None, E4M3, 128, 0.0, None, None, None) == OK


def test_per_block_validation(lib):
    f = lib.qcast_per_block
    assert f(A16, 256, 256, 9, 128, 0.0, A16, A16, None) == ERR_FORMAT
    assert f(A16, 256, 256, E4M3, 64, 0.0, A16, A16, None) == ERR_GROUP
    assert f(A16, 200, 256, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert f(A16, 256, 200, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert f(A16, 256, 256, E4M3, 128, 0.0, None, A16, None) == ERR_NULL
    assert f(A16, 256, 256, E4M3, 128, 0.0, MIS, A16, None) == ERR_ALIGN


def test_per_channel_T_validation(lib):
    f = lib.qcast_per_channel_T
    assert f(A16, 256, 64, 0, 128, 0.0, A16, A16, None) == ERR_FORMAT
    assert f(A16, 256, 64, E4M3, 64, 0.0, A16, A16, None) == ERR_GROUP
    assert f(A16, 200, 64, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert f(A16, 256, 60, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert f(A16, 256, 64, E4M3, 128, 0.0, A16, None, None) == ERR_NULL
    assert f(MIS, 256, 64, E4M3, 128, 0.0, A16, A16, None) == ERR_ALIGN


@pytest.mark.skipif(gpu_available(), reason="only meaningful on a host without a GPU")
def test_valid_call_without_a_device_reports_device_error(lib):
    assert pt(lib) == ERR_DEVICE


def test_binding_rejects_cpu_tensors():
    import torch
    import precision_quantization_amd as pq
    with pytest.raises(pq.QcastError):
        pq.qcast_per_token(torch.zeros(4, 128, dtype=torch.bfloat16))


def test_bench_copy_validation(lib):
    assert lib.qcast_bench_copy(A16, A16 + 4096, 100, None) == ERR_SHAPE
    assert lib.qcast_bench_copy(None, A16, 64, None) == ERR_NULL
    assert lib.qcast_bench_copy(MIS, A16, 64, None) == ERR_ALIGN
    assert lib.qcast_bench_copy(None, None, 0, None) == OK


def test_sf_layout_validation(lib):
    f = lib.qcast_per_token_sf
    assert f(A16, 4, 512, E4M3, 128, 0.0, 8, A16, A16, None) == ERR_FORMAT      # unknown flag
    assert f(A16, 4, 384, E4M3, 128, 0.0, 4, A16, A16, None) == ERR_SHAPE      # 3 groups, packed
    assert f(A16, 4, 512, E4M3, 128, 0.0, 7, None, A16, None) == ERR_NULL
    assert f(A16, 4, 512, E2M1, 32, 0.0, 6, A16, A16 + 2, None) == ERR_ALIGN
    g = lib.qcast_swiglu_per_token_sf
    assert g(A16, 4, 512, None, E4M3, 128, 0.0, 16, A16, A16, None) == ERR_FORMAT
    assert g(A16, 4, 384, None, E4M3, 128, 0.0, 4, A16, A16, None) == ERR_SHAPE
    assert g(A16, 4, 512, None, E2M1, 32, 0.0, 4, None, A16, None) == ERR_NULL   # E2M1 taken


def test_swiglu_ex_validation(lib):
    f = lib.qcast_swiglu_per_token_ex
    nan = float("nan")
    assert f(A16, 4, 256, None, 9, 32, 0.0, 0, 1.0, A16, A16, None, None, None) == ERR_FORMAT
    assert f(A16, 4, 256, None, E4M3, 128, 0.0, 8, 1.0, A16, A16, None, None, None) == ERR_FORMAT
    assert f(A16, 4, 256, None, E4M3, 100, 0.0, 0, 1.0, A16, A16, None, None, None) == ERR_GROUP
    assert f(A16, 4, 200, None, E4M3, 128, 0.0, 0, 1.0, A16, A16, None, None, None) == ERR_SHAPE
    assert f(A16, 4, 256, None, E4M3, 128, 0.0, 0, nan, A16, A16, None, None, None) == ERR_VALUE
    assert f(A16, 0, 256, None, E4M3, 128, 0.0, 0, nan, None, None, None, None, None) == ERR_VALUE
    assert f(None, 4, 256, None, E4M3, 128, 0.0, 0, 1.0, A16, A16, None, None, None) == ERR_NULL
    assert f(A16, 4, 256, None, E4M3, 128, 0.0, 0, 1.0, A16, A16, A16 + 4, None, None) == ERR_ALIGN
    assert f(None, 0, 256, None, E4M3, 128, 0.0, 0, 1.0, None, None, None, None, None) == OK
    # the count workspace is 128-byte aligned
    assert f(A16, 4, 256, None, E4M3, 128, 0.0, 0, 1.0, A16, A16, A16, A16 + 64, None) == ERR_ALIGN


def test_swiglu_backward_validation(lib):
    f = lib.qcast_swiglu_backward_per_token
    assert f(A16, A16, 4, 256, None, 9, 32, 0.0, 0.0, A16, A16, None) == ERR_FORMAT
    assert f(A16, A16, 4, 256, None, E4M3, 16, 0.0, 0.0, A16, A16, None) == ERR_GROUP
    assert f(A16, A16, 4, 200, None, E4M3, 128, 0.0, 0.0, A16, A16, None) == ERR_SHAPE
    assert f(A16, A16, 4, 1 << 19, None, E4M3, 128, 0.0, 0.0, A16, A16, None) == ERR_SHAPE
    assert f(A16, A16, 4, 256, None, E4M3, 128, 0.0, float("nan"), A16, A16, None) == ERR_VALUE
    assert f(A16, None, 4, 256, None, E4M3, 128, 0.0, 0.0, A16, A16, None) == ERR_NULL
    assert f(A16, MIS, 4, 256, None, E5M2, 128, 0.0, 0.0, A16, A16, None) == ERR_ALIGN
    assert f(None, None, 0, 256, None, E4M3, 128, 0.0, 0.0, None, None, None) == OK


def test_swiglu_per_channel_T_validation(lib):
    f = lib.qcast_swiglu_per_channel_T
    assert f(A16, 256, 64, None, 9, 128, 0.0, 0.0, A16, A16, None, None, None) == ERR_FORMAT
    assert f(A16, 256, 64, None, E4M3, 32, 0.0, 0.0, A16, A16, None, None, None) == ERR_GROUP
    assert f(A16, 200, 64, None, E4M3, 128, 0.0, 0.0, A16, A16, None, None, None) == ERR_SHAPE
    assert f(A16, 256, 60, None, E4M3, 128, 0.0, 0.0, A16, A16, None, None, None) == ERR_SHAPE
    assert f(A16, 256, 64, None, E4M3, 128, 0.0, float("nan"), A16, A16, None, None, None) == ERR_VALUE
    assert f(A16, 256, 64, None, E4M3, 128, 0.0, 0.0, None, A16, None, None, None) == ERR_NULL
    assert f(A16, 256, 64, A16 + 2, E4M3, 128, 0.0, 0.0, A16, A16, None, None, None) == ERR_ALIGN
    assert f(A16, 256, 64, None, E4M3, 128, 0.0, 1.0, A16, A16, A16 + 4, None, None) == ERR_ALIGN
    assert f(None, 0, 64, None, E4M3, 128, 0.0, 0.0, None, None, None, None, None) == OK
    assert f(A16, 256, 64, None, E4M3, 128, 0.0, 1.0, A16, A16, A16, A16 + 16, None) == ERR_ALIGN


def test_per_channel_validation(lib):
    f = lib.qcast_per_channel
    assert f(A16, 256, 64, 9, 128, 0.0, A16, A16, None) == ERR_FORMAT
    assert f(A16, 256, 64, E4M3, 64, 0.0, A16, A16, None) == ERR_GROUP
    assert f(A16, 200, 64, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert f(A16, 256, 60, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert f(A16, 256, 64, E4M3, 128, 0.0, A16, None, None) == ERR_NULL
    assert f(A16, 256, 64, E5M2, 128, 0.0, MIS, A16, None) == ERR_ALIGN
    assert f(None, 0, 64, E4M3, 128, 0.0, None, None, None) == OK


def test_e5m6_formats(lib):
    E5M6 = 4
    # accepted by the per-token casts and cast_back (null output is the first error)
    assert lib.qcast_per_token(A16, 4, 256, E5M6, 128, 0.0, None, A16, None) == ERR_NULL
    assert lib.qcast_per_token_sf(A16, 4, 512, E5M6, 128, 0.0, 5, None, A16, None) == ERR_NULL
    assert lib.qcast_cast_back(A16, A16, 4, 256, E5M6, 32, 1, None, None) == ERR_NULL
    assert lib.qcast_per_token(A16, 4, 256, E5M6, 16, 0.0, A16, A16, None) == ERR_GROUP
    # and by every other cast
    assert lib.qcast_swiglu_per_token(A16, 4, 256, None, E5M6, 128, 0.0, None, A16, None) == ERR_NULL
    assert lib.qcast_per_block(A16, 256, 256, E5M6, 128, 0.0, None, A16, None) == ERR_NULL
    assert lib.qcast_per_channel_T(A16, 256, 64, E5M6, 128, 0.0, None, A16, None) == ERR_NULL
    assert lib.qcast_per_channel(A16, 256, 64, E5M6, 128, 0.0, None, A16, None) == ERR_NULL
    assert lib.qcast_swiglu_backward_per_token(A16, A16, 4, 256, None, E5M6, 128, 0.0, 0.0, None,
                                               A16, None) == ERR_NULL
    assert lib.qcast_swiglu_per_channel_T(A16, 256, 64, None, E5M6, 128, 0.0, 0.0, None, A16,
                                          None, None, None) == ERR_NULL
    assert lib.qcast_e2m1(A16, 4, 256, 32, 0.0, None, A16, None) == ERR_NULL
    assert lib.qcast_bench_check_scale(E5M6, 1, 0, A16, None) == ERR_SHAPE
    assert lib.qcast_bench_check_scale(5, 1, 2, A16, None) == ERR_FORMAT


def test_shapes_past_the_32_bit_indexing_are_refused_before_any_hip_call(lib):
    big = 1 << 24                       # 128 * big = 2^31
    assert lib.qcast_per_block(A16, 128, big, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert lib.qcast_per_channel_T(A16, 128, big, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert lib.qcast_per_channel_T(A16, 1 << 25, 64, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert lib.qcast_per_channel(A16, 128, big, E4M3, 128, 0.0, A16, A16, None) == ERR_SHAPE
    assert lib.qcast_swiglu_per_channel_T(A16, 128, 1 << 23, None, E4M3, 128, 0.0, 0.0, A16, A16,
                                          None, None, None) == ERR_SHAPE
    assert lib.qcast_per_token(A16, 1 << 24, 1 << 12, E4M3, 32, 0.0, A16, A16, None) == ERR_SHAPE
    assert lib.qcast_cast_back(A16, A16, 1 << 30, 1 << 13, E4M3, 128, 1, A16, None) == ERR_SHAPE
    # the largest shapes that fit pass validation (then find no device here)
    if not gpu_available():
        assert lib.qcast_per_block(A16, 128, big - 128, E4M3, 128, 0.0, A16, A16, None) == ERR_DEVICE
        assert lib.qcast_per_channel_T(A16, 128, big - 8, E4M3, 128, 0.0, A16, A16,
                                       None) == ERR_DEVICE
        assert lib.qcast_per_channel(A16, 128, big - 8, E4M3, 128, 0.0, A16, A16, None) == ERR_DEVICE


def test_time_next_validation(lib):
    assert lib.qcast_bench_time_next(None, A16) == ERR_NULL
    assert lib.qcast_bench_time_next(A16, None) == ERR_NULL


def test_cast_back_validation(lib):
    f = lib.qcast_cast_back
    assert f(A16, A16, 4, 256, 9, 128, 1, A16, None) == ERR_FORMAT
    assert f(A16, A16, 4, 256, E4M3, 128, 3, A16, None) == ERR_FORMAT      # out dtype
    assert f(A16, A16, 4, 256, E4M3, 96, 1, A16, None) == ERR_GROUP
    assert f(A16, A16, 4, 200, E4M3, 128, 1, A16, None) == ERR_SHAPE
    assert f(None, A16, 4, 256, E5M2, 128, 2, A16, None) == ERR_NULL
    assert f(A16, A16, 4, 256, E2M1, 32, 1, MIS, None) == ERR_ALIGN
    assert f(None, None, 0, 256, E4M3, 128, 1, None, None) == OK


def test_e5m2_accepted_by_every_cast(lib):
    # past format validation, a null output is the first error
    assert lib.qcast_per_token(A16, 4, 256, E5M2, 128, 0.0, None, A16, None) == ERR_NULL
    assert lib.qcast_swiglu_per_token(A16, 4, 256, None, E5M2, 128, 0.0, None, A16, None) == ERR_NULL
    assert lib.qcast_per_block(A16, 256, 256, E5M2, 128, 0.0, None, A16, None) == ERR_NULL
    assert lib.qcast_per_channel_T(A16, 256, 64, E5M2, 128, 0.0, None, A16, None) == ERR_NULL


def test_check_scale_validation(lib):
    f = lib.qcast_bench_check_scale
    assert f(9, 1, 10, A16, None) == ERR_FORMAT
    assert f(E4M3, 10, 1, A16, None) == ERR_SHAPE
    assert f(E4M3, 1, 0x7F800000, A16, None) == ERR_SHAPE
    assert f(E4M3, 1, 10, None, None) == ERR_NULL
    assert f(E4M3, 1, 10, A16 + 2, None) == ERR_ALIGN


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from precision_quantization_amd import _lib, build
    monkeypatch.setattr(build, "LIB", str(tmp_path / "libqcast.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.QcastError):
        _lib.load()


def test_per_channel_T_traffic_validation(lib):
    f = lib.qcast_bench_per_channel_T_traffic
    assert f(A16, 200, 64, A16, None) == ERR_SHAPE          # tokens not a multiple of 128
    assert f(A16, 256, 60, A16, None) == ERR_SHAPE          # channels not a multiple of 8
    assert f(A16, 128, 1 << 24, A16, None) == ERR_SHAPE     # past the 32-bit tile offsets
    assert f(A16, -128, 64, A16, None) == ERR_SHAPE
    assert f(None, 256, 64, A16, None) == ERR_NULL
    assert f(A16, 256, 64, MIS, None) == ERR_ALIGN
    assert f(None, 0, 64, None, None) == OK


def test_non_finite_clamp_min_is_refused_by_every_cast(lib):
    nan, inf = float("nan"), float("inf")
    for c in (nan, inf):
        assert lib.qcast_per_token(A16, 4, 256, E4M3, 128, c, A16, A16, None) == ERR_VALUE
        assert lib.qcast_per_token_sf(A16, 4, 512, E4M3, 128, c, 5, A16, A16, None) == ERR_VALUE
        assert lib.qcast_e2m1(A16, 4, 256, 32, c, A16, A16, None) == ERR_VALUE
        assert lib.qcast_swiglu_per_token(A16, 4, 256, None, E4M3, 128, c, A16, A16,
                                          None) == ERR_VALUE
        assert lib.qcast_swiglu_per_token_sf(A16, 4, 256, None, E4M3, 128, c, 1, A16, A16,
                                             None) == ERR_VALUE
        assert lib.qcast_swiglu_per_token_ex(A16, 4, 256, None, E4M3, 128, c, 0, 1.0, A16, A16,
                                             None, None, None) == ERR_VALUE
        assert lib.qcast_swiglu_backward_per_token(A16, A16, 4, 256, None, E4M3, 128, c, 0.0,
                                                   A16, A16, None) == ERR_VALUE
        assert lib.qcast_swiglu_per_channel_T(A16, 256, 64, None, E4M3, 128, c, 0.0, A16, A16,
                                              None, None, None) == ERR_VALUE
        assert lib.qcast_per_block(A16, 256, 256, E4M3, 128, c, A16, A16, None) == ERR_VALUE
        assert lib.qcast_per_channel_T(A16, 256, 64, E4M3, 128, c, A16, A16, None) == ERR_VALUE
        assert lib.qcast_per_channel(A16, 256, 64, E4M3, 128, c, A16, A16, None) == ERR_VALUE
        # refused even for an empty input
        assert lib.qcast_per_token(None, 0, 256, E4M3, 128, c, None, None, None) == ERR_VALUE
    # zero and negative floors (-inf included) select the default: past this check, a null
    # output is the first error
    for c in (0.0, -1.0, -inf):
        assert lib.qcast_per_token(A16, 4, 256, E4M3, 128, c, None, A16, None) == ERR_NULL
    # the largest finite floor is accepted
    assert lib.qcast_per_token(A16, 4, 256, E4M3, 128, 3.4028235e38, None, A16, None) == ERR_NULL


def test_binding_rejects_an_odd_gate_up_width():
    import torch
    import precision_quantization_amd as pq
    h = torch.zeros(4, 513, dtype=torch.bfloat16)
    for fn in (pq.qcast_swiglu_per_token, pq.qcast_swiglu_per_token_sf,
               pq.qcast_swiglu_per_token_ex, pq.qcast_swiglu_per_channel_T):
        with pytest.raises(pq.QcastError, match="even number of columns"):
            fn(h)
    with pytest.raises(pq.QcastError, match="even number of columns"):
        pq.qcast_swiglu_backward_per_token(h, torch.zeros(4, 256, dtype=torch.bfloat16))


def test_binding_rejects_e5m6_codes_whose_width_is_not_a_multiple_of_3():
    import torch
    import precision_quantization_amd as pq
    q = torch.zeros(4, 100, dtype=torch.uint8)
    with pytest.raises(pq.QcastError, match="multiple of 3"):
        pq.qcast_cast_back(q, torch.zeros(4, 2), "e5m6", 32)


def test_swiglu_noalloc_validation(lib):
    f = lib.qcast_swiglu_per_token_noalloc
    nan = float("nan")
    assert f(A16, 4, 256, None, 9, 32, 0.0, 0, 1.0, A16, A16, A16, None) == ERR_FORMAT
    assert f(A16, 4, 256, None, E4M3, 128, 0.0, 8, 1.0, A16, A16, A16, None) == ERR_FORMAT
    assert f(A16, 4, 256, None, E4M3, 100, 0.0, 0, 1.0, A16, A16, A16, None) == ERR_GROUP
    assert f(A16, 4, 200, None, E4M3, 128, 0.0, 0, 1.0, A16, A16, A16, None) == ERR_SHAPE
    assert f(A16, 4, 256, None, E4M3, 128, 0.0, 0, nan, A16, A16, A16, None) == ERR_VALUE
    assert f(A16, 4, 256, None, E4M3, 128, nan, 0, 1.0, A16, A16, A16, None) == ERR_VALUE
    assert f(None, 4, 256, None, E4M3, 128, 0.0, 0, 1.0, A16, A16, A16, None) == ERR_NULL
    assert f(A16, 4, 256, None, E4M3, 128, 0.0, 0, 1.0, A16, A16, A16 + 4, None) == ERR_ALIGN
    assert f(A16, 4, 256, None, E4M3, 128, 0.0, 0, 1.0, MIS, A16, A16, None) == ERR_ALIGN
    assert f(None, 0, 256, None, E4M3, 128, 0.0, 0, 1.0, None, None, None, None) == OK
    if not gpu_available():
        # valid arguments reach the device lookup, which finds no GPU here
        assert f(A16, 4, 256, None, E4M3, 128, 0.0, 0, 1.0, A16, A16, A16, None) == ERR_DEVICE


def test_noalloc_scratch_size_is_declared():
    text = open(HEADERS[0]).read()
    assert "#define QCAST_NOALLOC_SCRATCH_BYTES 8192" in text
    src = open(os.path.join(ROOT, "precision_quantization_amd", "csrc", "qcast_abi.hip")).read()
    assert "static __device__ __align__(256) unsigned long long scratch[" in src
    assert "hipGetSymbolAddress" in src and "hipMalloc" not in src


def test_layouts_of_the_other_casts_validation(lib):
    nan = float("nan")
    # per-block and input-layout per-channel: round_sf only
    f = lib.qcast_per_block_sf
    for flags in (2, 4, 6, 8):
        assert f(A16, 256, 256, E4M3, 128, 0.0, flags, A16, A16, None) == ERR_FORMAT
    assert f(A16, 256, 256, E4M3, 128, 0.0, 1, None, A16, None) == ERR_NULL
    assert f(A16, 256, 256, E4M3, 128, nan, 1, A16, A16, None) == ERR_VALUE
    g = lib.qcast_per_channel_sf
    for flags in (2, 4, 6, 8):
        assert g(A16, 256, 64, E4M3, 128, 0.0, flags, A16, A16, None) == ERR_FORMAT
    assert g(A16, 256, 64, E2M1, 128, 0.0, 1, A16, None, None) == ERR_NULL
    # transposed per-channel: every layout; packed words need 4 token groups
    t = lib.qcast_per_channel_T_sf
    assert t(A16, 512, 64, E4M3, 128, 0.0, 8, A16, A16, None) == ERR_FORMAT
    assert t(A16, 384, 64, E4M3, 128, 0.0, 4, A16, A16, None) == ERR_SHAPE
    assert t(A16, 384, 64, E4M3, 128, 0.0, 3, A16, None, None) == ERR_NULL    # col-major fine
    assert t(A16, 512, 64, E4M3, 128, 0.0, 6, A16, None, None) == ERR_NULL
    assert t(A16, 512, 64, E5M2, 128, 0.0, 4, A16, A16 + 2, None) == ERR_ALIGN
    assert t(None, 0, 64, E4M3, 128, 0.0, 4, None, None, None) == OK
    u = lib.qcast_swiglu_per_channel_T_sf
    assert u(A16, 512, 64, None, E4M3, 128, 0.0, 8, 0.0, A16, A16, None, None, None) == ERR_FORMAT
    assert u(A16, 384, 64, None, E4M3, 128, 0.0, 4, 0.0, A16, A16, None, None, None) == ERR_SHAPE
    assert u(A16, 512, 64, None, E4M3, 128, 0.0, 5, nan, A16, A16, None, None, None) == ERR_VALUE
    assert u(A16, 512, 64, None, E4M3, 128, 0.0, 4, 1.0, A16, None, None, None, None) == ERR_NULL
    # backward: packed words must not straddle the dg and du halves
    b = lib.qcast_swiglu_backward_per_token_sf
    assert b(A16, A16, 4, 256, None, E4M3, 128, 0.0, 8, 0.0, A16, A16, None) == ERR_FORMAT
    assert b(A16, A16, 4, 256, None, E4M3, 128, 0.0, 4, 0.0, A16, A16, None) == ERR_SHAPE
    assert b(A16, A16, 4, 384, None, E4M3, 128, 0.0, 4, 0.0, A16, A16, None) == ERR_SHAPE
    assert b(A16, A16, 4, 512, None, E4M3, 128, 0.0, 4, 0.0, A16, None, None) == ERR_NULL
    assert b(A16, A16, 4, 256, None, E4M3, 128, 0.0, 2, 0.0, A16, None, None) == ERR_NULL
    assert b(A16, A16, 4, 256, None, E4M3, 128, nan, 2, 0.0, A16, A16, None) == ERR_VALUE
    assert b(None, None, 0, 256, None, E4M3, 128, 0.0, 2, 0.0, None, None, None) == OK
