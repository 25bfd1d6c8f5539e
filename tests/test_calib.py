"""The benchmark's measurement library (libpkv_calib.so) loads, exports what
include/pkv_calib.h declares, and rejects bad arguments before touching a
GPU.  (No compute: there is no GPU here.)"""
import ctypes
import os
import re

from paged_kv_cache_prepare_amd import _build

HEADER = os.path.join(os.path.dirname(_build.HERE), "include", "pkv_calib.h")


def _lib():
    if not os.path.exists(_build.CALIB_LIB_PATH):
        _build.build()
    lib = ctypes.CDLL(_build.CALIB_LIB_PATH)
    P = ctypes.c_void_p
    lib.pkv_calib_clock.argtypes = [P, ctypes.c_int64, P]
    lib.pkv_calib_read_runs.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, P, P]
    return lib


def test_exports_every_declared_symbol():
    names = re.findall(r"^int (pkv_calib_\w+)\(", open(HEADER).read(), re.M)
    assert sorted(names) == ["pkv_calib_clock", "pkv_calib_read_runs"]
    lib = _lib()
    for n in names:
        assert hasattr(lib, n), n


def test_rejects_bad_arguments():
    lib = _lib()
    buf = ctypes.create_string_buffer(64)
    p = ctypes.cast(buf, ctypes.c_void_p)
    assert lib.pkv_calib_clock(None, 100, None) == 1
    assert lib.pkv_calib_clock(p, 0, None) == 1
    assert lib.pkv_calib_clock(p, 10**9 + 1, None) == 1
    assert lib.pkv_calib_read_runs(None, p, 1, 4, p, None) == 1
    assert lib.pkv_calib_read_runs(p, p, 0, 4, p, None) == 1
    assert lib.pkv_calib_read_runs(p, p, 1, 0, p, None) == 1
    assert lib.pkv_calib_read_runs(p, p, 1, 5, p, None) == 1
    assert lib.pkv_calib_read_runs(p, p, 1, 3, p, None) == 1
