"""The C ABI library on the CPU: it loads, exports what include/mhc.h declares, and rejects
bad sizes and null handles before any device call. No compute runs here."""

import ctypes
import os
import subprocess

import pytest

from mhc_hyper_connection_02_amd import binding

LIB = binding.LIB_PATH

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmhc_amd.so not built")


def test_header_declares_the_entry_points():
    names = binding.header_functions()
    for want in ("mhc_create", "mhc_destroy", "mhc_reset", "mhc_set_option", "mhc_boundary",
                 "mhc_residual_only", "mhc_finalize", "mhc_collapse_mean", "mhc_pre_coeffs",
                 "mhc_status_string", "mhc_get_errors", "mhc_first", "mhc_collapse_norm",
                 "mhc_pre_coeffs_deferred", "mhc_pre_coeffs_flush"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = binding.load_library()
    for name in binding.header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(binding.header_functions()) <= exported


def test_binding_signatures_cover_the_header():
    assert set(binding.header_functions()) == set(binding._SIGS)


def test_status_strings():
    lib = binding.load_library()
    for code in range(8):
        s = lib.mhc_status_string(code).decode()
        assert s.startswith("MHC")
    assert "unknown" in lib.mhc_status_string(99).decode()


def test_create_rejects_bad_sizes_before_any_device_call():
    lib = binding.load_library()
    h = ctypes.c_void_p(123)
    cases = [
        ((0, 4, 32, 8, 8, 0), 2), ((7, 4, 32, 8, 8, 0), 2), ((7168, 4, 0, 8, 8, 0), 2),
        ((7168, 4, 70000, 8, 8, 0), 2), ((7168, 4, 32, 0, 8, 0), 2), ((7168, 4, 32, 65, 8, 0), 2),
        ((7168, 4, 32, 8, 0, 0), 2), ((7168, 4, 32, 8, 8, -1), 2), ((7168, 2, 32, 8, 8, 0), 5),
        ((65544, 4, 32, 8, 8, 0), 2),
    ]
    for args, want in cases:
        assert lib.mhc_create(*args, ctypes.byref(h)) == want, args
        assert h.value is None  # *out is cleared on failure
        h = ctypes.c_void_p(123)
    assert lib.mhc_create(7168, 4, 32, 8, 8, 0, None) == 1


def test_null_handle_is_invalid_everywhere():
    lib = binding.load_library()
    z = None
    assert lib.mhc_destroy(z) == 0
    assert lib.mhc_reset(z, z) == 1
    assert lib.mhc_set_option(z, 1, 64) == 1
    assert lib.mhc_get_errors(z, None, 0, z) == 1
    assert lib.mhc_boundary(z, z, 1, z, z, z, z, z, 0.0, 1, z, z, z, z, z) == 1
    assert lib.mhc_residual_only(z, z, 1, z, z, z, 1, z, z) == 1
    assert lib.mhc_finalize(z, z, 1, z, z, z, z, z, z, z, z, 0.0, 1, z, z, z, z, z) == 1
    assert lib.mhc_collapse_mean(z, z, 1, z, z) == 1
    assert lib.mhc_pre_coeffs(z, z, z, z, z, 0.0, 0.0, 0.0, 2.0, 20, 1, z, z, z, z) == 1
    assert lib.mhc_pre_coeffs_deferred(z, z, z, z, z, 0.0, 0.0, 0.0, 2.0, 20, 1, z, z, z, z) == 1
    assert lib.mhc_pre_coeffs_flush(z, z) == 1
    assert lib.mhc_first(z, z, z, 0.0, 1, z, z, z, z, z) == 1
    assert lib.mhc_collapse_norm(z, z, z, z, 0.0, 1, z, z, z, z) == 1
