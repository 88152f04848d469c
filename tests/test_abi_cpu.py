"""The C-ABI library on the host (no GPU needed): it loads, exports every function
include/vda.h declares, and rejects bad plan arguments before touching a device."""
import ctypes
import math

import pytest

import frame_wise_delta_vda_amd as vda
from frame_wise_delta_vda_amd import vda as binding


@pytest.fixture(scope="module")
def lib():
    return vda.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = vda.declared_functions()
    assert set(names) == {"vda_plan_create", "vda_forward", "vda_forward_stages", "vda_forward_gated",
                          "vda_backward",
                          "vda_plan_destroy",
                          "vda_plan_workspace_bytes", "vda_status_string", "vda_debug_workspace",
                          "vda_plan_enable_timing", "vda_plan_timings", "vda_forward_noalloc",
                          "vda_plan_set_scan_chunk", "vda_plan_get_scan_chunk", "vda_plan_set_timed_stages"}
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in vda.STATUS.items():
        assert vda.vda_status_string(code) == name
    assert vda.vda_status_string(99) == "VDA_ERROR_UNKNOWN"


def _create(lib, *args):
    h = ctypes.c_void_p(12345)
    st = lib.vda_plan_create(*args[:7], ctypes.c_float(args[7]), args[8], ctypes.byref(h))
    return st, h.value


@pytest.mark.parametrize("args,expected", [
    ((1, 1, 1, 1, 48, 32, 0, 1.0, 1), binding.VDA_ERROR_NOT_SUPPORTED),     # d not supported
    ((1, 1, 1, 1, 32, 256, 0, 1.0, 1), binding.VDA_ERROR_NOT_SUPPORTED),    # dv not supported
    ((1, 1, 1, 1, 32, 32, 0, 1.0, 7), binding.VDA_ERROR_NOT_SUPPORTED),     # dtype
    ((-1, 1, 1, 1, 32, 32, 0, 1.0, 1), binding.VDA_ERROR_INVALID_VALUE),
    ((1, 1, -2, 1, 32, 32, 0, 1.0, 1), binding.VDA_ERROR_INVALID_VALUE),
    ((1, 1, 1, 1, 32, 32, -1, 1.0, 1), binding.VDA_ERROR_INVALID_VALUE),
    ((1, 1, 1, 1, 32, 32, 0, 0.0, 1), binding.VDA_ERROR_INVALID_VALUE),     # lambda == 0
    ((1, 1, 1, 1, 32, 32, 0, -1.0, 1), binding.VDA_ERROR_INVALID_VALUE),
    ((1, 1, 1, 1, 32, 32, 0, math.nan, 1), binding.VDA_ERROR_INVALID_VALUE),
    ((1, 1, 1, 1, 32, 32, 0, math.inf, 1), binding.VDA_ERROR_INVALID_VALUE),
    ((2**40, 2**40, 1, 1, 32, 32, 0, 1.0, 1), binding.VDA_ERROR_INVALID_VALUE),  # overflow
    ((1, 1, 1, 2**24, 32, 32, 0, 1.0, 1), binding.VDA_ERROR_NOT_SUPPORTED),  # frame too long
    ((1, 1, 1, 1, 32, 32, 2**24, 1.0, 1), binding.VDA_ERROR_NOT_SUPPORTED),  # text too long
])
def test_plan_create_rejects_bad_arguments(lib, args, expected):
    st, h = _create(lib, *args)
    assert st == expected
    assert h is None  # *plan_out cleared on error


def test_null_handles(lib):
    assert lib.vda_plan_create(1, 1, 1, 1, 32, 32, 0, ctypes.c_float(1.0), 1, None) == \
        binding.VDA_ERROR_INVALID_VALUE
    assert lib.vda_plan_destroy(None) == binding.VDA_SUCCESS
    assert lib.vda_plan_workspace_bytes(None) == 0
    assert lib.vda_forward(None, *([None] * 7)) == binding.VDA_ERROR_INVALID_VALUE
    assert lib.vda_forward_stages(None, 7, *([None] * 7)) == binding.VDA_ERROR_INVALID_VALUE
    assert lib.vda_forward_gated(None, *([None] * 10)) == binding.VDA_ERROR_INVALID_VALUE
    assert lib.vda_backward(None, *([None] * 12)) == binding.VDA_ERROR_INVALID_VALUE
    p = ctypes.c_void_p()
    assert lib.vda_debug_workspace(None, ctypes.byref(p), None, None, None) == \
        binding.VDA_ERROR_INVALID_VALUE
    assert lib.vda_plan_enable_timing(None, 4) == binding.VDA_ERROR_INVALID_VALUE
    assert lib.vda_plan_set_scan_chunk(None, 8) == binding.VDA_ERROR_INVALID_VALUE
    c = ctypes.c_int64()
    assert lib.vda_plan_get_scan_chunk(None, ctypes.byref(c)) == binding.VDA_ERROR_INVALID_VALUE
    assert lib.vda_plan_set_timed_stages(None, 4) == binding.VDA_ERROR_INVALID_VALUE
    calls = ctypes.c_int()
    assert lib.vda_plan_timings(None, ctypes.byref(calls), None, None, None) == \
        binding.VDA_ERROR_INVALID_VALUE


def test_binding_raises_vda_error(lib):
    with pytest.raises(vda.VdaError) as e:
        vda.vda_plan_create(1, 1, 1, 1, 40, 32, 0, 1.0, "bf16")
    assert e.value.status == binding.VDA_ERROR_NOT_SUPPORTED


def test_noalloc_rejects_bad_and_oversized_problems_before_any_device_call(lib):
    # argument errors are those of vda_plan_create; a workspace above the fixed scratch is
    # TOO_LARGE; none of these touches a device, so they hold on a host with no GPU
    f = lib.vda_forward_noalloc
    nul = [None] * 7
    assert f(1, 1, 1, 1, 48, 32, 0, ctypes.c_float(1.0), 1, *nul) == binding.VDA_ERROR_NOT_SUPPORTED
    assert f(1, 1, 1, 1, 32, 32, 0, ctypes.c_float(0.0), 1, *nul) == binding.VDA_ERROR_INVALID_VALUE
    assert f(-1, 1, 1, 1, 32, 32, 0, ctypes.c_float(1.0), 1, *nul) == binding.VDA_ERROR_INVALID_VALUE
    assert f(2**40, 2**40, 1, 1, 32, 32, 0, ctypes.c_float(1.0), 1, *nul) == binding.VDA_ERROR_INVALID_VALUE
    # four heads of the 768p shape (bf16, d = dv = 128, 90 frames): 4 x 17.8 MB > 64 MiB
    assert f(1, 4, 90, 4032, 128, 128, 256, ctypes.c_float(1.0), 1, *nul) == binding.VDA_ERROR_TOO_LARGE
    # no output element: nothing to do, no pointer read
    assert f(1, 4, 0, 4032, 128, 128, 256, ctypes.c_float(1.0), 1, *nul) == binding.VDA_SUCCESS
    assert vda.vda_status_string(binding.VDA_ERROR_TOO_LARGE) == "VDA_ERROR_TOO_LARGE"
