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
                 "mhc_pre_coeffs_deferred", "mhc_pre_coeffs_flush", "mhc_boundary_coeffs",
                 "mhc_finalize_coeffs", "mhc_mxfp8_scale_bytes", "mhc_floor_boundary_traffic",
                 "mhc_floor_empty"):
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


def test_mxfp8_scale_bytes_host_only():
    """Scale-buffer sizes of both layouts (no device work): row-major rows * hidden/32;
    swizzled 128x4 rows padded to 128 and blocks to 4."""
    lib = binding.load_library()
    n = ctypes.c_uint64(0)
    cases = [((32, 7168, 0), 32 * 224), ((32, 7168, 1), 128 * 224), ((130, 1056, 1), 256 * 36),
             ((0, 1056, 1), 0), ((1, 32, 1), 128 * 4), ((128, 128, 1), 128 * 4),
             ((65536, 65536, 1), 65536 * 2048)]
    for args, want in cases:
        assert lib.mhc_mxfp8_scale_bytes(*args, ctypes.byref(n)) == 0, args
        assert n.value == want, args
    for args, code in [((4, 1000, 0), 2), ((-1, 1024, 0), 2), ((4, 0, 1), 2), ((4, 1024, 2), 2)]:
        assert lib.mhc_mxfp8_scale_bytes(*args, ctypes.byref(n)) == code, args
    assert lib.mhc_mxfp8_scale_bytes(4, 1024, 0, None) == 1


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
    assert lib.mhc_boundary_coeffs(z, z, 1, z, z, z, z, z, 0.0, 1, z, z, z, z, None, z) == 1
    assert lib.mhc_finalize_coeffs(z, z, 1, z, z, z, z, z, z, z, z, 0.0, 1, z, z, z, z, None,
                                   z) == 1


def test_coeff_args_struct_matches_the_header(tmp_path):
    """The binding's ctypes mirror of mhc_coeff_args has the C struct's size and field
    offsets (a small C program compiled against include/mhc.h prints them)."""
    fields = [f for f, _ in binding.CoeffArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text(
        '#include "mhc.h"\n#include <stddef.h>\n#include <stdio.h>\nint main(void) {\n'
        '  printf("%zu\\n", sizeof(mhc_coeff_args));\n'
        + "".join(f'  printf("%zu\\n", offsetof(mhc_coeff_args, {f}));\n' for f in fields)
        + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(binding.HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(binding.CoeffArgs)] + [getattr(binding.CoeffArgs, f).offset
                                                 for f in fields]
    assert got == want


class _StubHandle:
    """Just the sizes the binding reads; every case below fails before the library is called."""
    hidden, hc_mult, top_k = 64, 4, 8
    ptr = None


def _fused_args(rows=3, hidden=64, fn_rows=None, scale_len=3):
    import torch
    n, nc = 4, 24
    d = dict(
        x=torch.zeros((2, rows, hidden), dtype=torch.bfloat16),
        s=torch.zeros((rows, n, hidden), dtype=torch.bfloat16),
        post=torch.zeros((rows, n)), comb=torch.zeros((rows, n, n)), pre=torch.zeros((rows, n)),
        w=torch.zeros((hidden,), dtype=torch.bfloat16))
    nxt = {"fn": torch.zeros((fn_rows or n * hidden, nc), dtype=torch.bfloat16),
           "scale": torch.zeros((scale_len,)), "base": torch.zeros((nc,)), "rms_eps": 1e-6,
           "pre_eps": 1e-6, "sinkhorn_eps": 1e-6, "post_alpha": 2.0, "sinkhorn_iters": 20}
    return d, nxt


@pytest.mark.parametrize("case", ["no_pre", "fn_shape", "scale_len", "next_out_shape",
                                  "streams_hidden"])
def test_fused_binding_rejects_bad_arguments(case):
    import torch
    h = _StubHandle()
    d, nxt = _fused_args(fn_rows=8 if case == "fn_shape" else None,
                         scale_len=4 if case == "scale_len" else 3)
    pre = None if case == "no_pre" else d["pre"]
    if case == "streams_hidden":
        d["s"] = torch.zeros((3, 4, 32), dtype=torch.bfloat16)
    next_out = None
    if case == "next_out_shape":
        next_out = (torch.zeros((3, 4)), torch.zeros((3, 4)), torch.zeros((3, 16)))
    with pytest.raises(ValueError):
        binding.boundary_coeffs(h, d["x"], d["s"], d["post"], d["comb"], pre, d["w"], 1e-6, nxt,
                                next_out=next_out)


def test_floor_calls_reject_bad_sizes_before_any_device_call():
    lib = binding.load_library()
    z = None
    p = ctypes.c_void_p(256)
    # shape first (rows, tp, hidden), then null pointers, then alignment; rows == 0 is a no-op
    assert lib.mhc_floor_boundary_traffic(p, 0, p, 4, 1024, p, p, p, p, z) == 2
    assert lib.mhc_floor_boundary_traffic(p, 65, p, 4, 1024, p, p, p, p, z) == 2
    assert lib.mhc_floor_boundary_traffic(p, 8, p, -1, 1024, p, p, p, p, z) == 2
    assert lib.mhc_floor_boundary_traffic(p, 8, p, 4, 1000, p, p, p, p, z) == 2
    assert lib.mhc_floor_boundary_traffic(p, 8, p, 4, 16, p, p, p, p, z) == 2
    assert lib.mhc_floor_boundary_traffic(p, 8, p, 0, 1024, z, z, z, z, z) == 0
    assert lib.mhc_floor_boundary_traffic(z, 8, p, 4, 1024, p, p, p, p, z) == 1
    assert lib.mhc_floor_boundary_traffic(p, 8, p, 4, 1024, p, p, p, z, z) == 1
    assert lib.mhc_floor_boundary_traffic(ctypes.c_void_p(258), 8, p, 4, 1024, p, p, p, p, z) == 3
    assert lib.mhc_floor_empty(-1, 1024, z) == 2
    assert lib.mhc_floor_empty(4, 1000, z) == 2
    assert lib.mhc_floor_empty(0, 1024, z) == 0


def test_noalloc_boundary_rejects_bad_sizes_before_any_device_call():
    """mhc_boundary_noalloc validates shapes, limits and pointers before touching the device
    (these cases never reach a HIP call)."""
    lib = binding.load_library()
    z = None
    q = ctypes.c_void_p(256)
    assert lib.mhc_boundary_noalloc(7168, q, 8, q, q, q, q, q, 1e-6, 1025, q, q, q, q, 0, z) == 4
    assert lib.mhc_boundary_noalloc(16392, q, 8, q, q, q, q, q, 1e-6, 4, q, q, q, q, 0, z) == 4
    assert lib.mhc_boundary_noalloc(7168, q, 65, q, q, q, q, q, 1e-6, 4, q, q, q, q, 0, z) == 4
    assert lib.mhc_boundary_noalloc(7164, q, 8, q, q, q, q, q, 1e-6, 4, q, q, q, q, 0, z) == 2
    assert lib.mhc_boundary_noalloc(0, q, 8, q, q, q, q, q, 1e-6, 4, q, q, q, q, 0, z) == 2
    assert lib.mhc_boundary_noalloc(7168, q, 0, q, q, q, q, q, 1e-6, 4, q, q, q, q, 0, z) == 2
    assert lib.mhc_boundary_noalloc(7168, q, 8, q, q, q, q, q, 1e-6, -1, q, q, q, q, 0, z) == 2
    assert lib.mhc_boundary_noalloc(7168, z, 8, q, q, q, q, q, 1e-6, 4, q, q, q, q, 0, z) == 1
    assert lib.mhc_boundary_noalloc(7168, q, 8, z, q, q, q, q, 1e-6, 4, q, q, q, q, 0, z) == 1
    # pre without a norm weight; MXFP8 data without scales; misaligned partials
    assert lib.mhc_boundary_noalloc(7168, q, 8, q, q, q, q, z, 1e-6, 4, q, q, q, q, 0, z) == 1
    assert lib.mhc_boundary_noalloc(7168, q, 8, q, q, q, q, q, 1e-6, 4, q, q, q, z, 0, z) == 1
    assert lib.mhc_boundary_noalloc(7168, ctypes.c_void_p(258), 8, q, q, q, q, q, 1e-6, 4, q, q,
                                    q, q, 0, z) == 3
    assert lib.mhc_boundary_noalloc(7168, q, 8, q, q, q, q, q, 1e-6, 0, z, z, z, z, 0, z) == 0
