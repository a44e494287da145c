"""mhc_boundary_noalloc (the boundary for callers that cannot allocate) through the C ABI:
its outputs equal mhc_boundary's on a handle bit for bit (the same kernels, launch shape and
order of sums), and match the oracle, on two calls in a row, the second with fewer rows, a
smaller tp and another hidden size; sizes beyond its fixed scratch are rejected."""

import ctypes

import numpy as np
import pytest
import torch

from mhc_hyper_connection_02_amd import binding, synth

from gpu_helpers import (N, T, say, handle_for, gpu_boundary, oracle_boundary,
                         compare_boundary_outputs)

pytestmark = pytest.mark.gpu

_vp, _i, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float


def _lib():
    lib = binding.load_library()
    fn = lib.mhc_boundary_noalloc
    fn.argtypes = [_i, _vp, _i, _vp, _vp, _vp, _vp, _vp, _f, _i, _vp, _vp, _vp, _vp, _i, _vp]
    fn.restype = _i
    return fn


def _noalloc(d, reset=0):
    fn = _lib()
    tp, rows, hidden = d["x_partials"].shape
    t = {k: T(d[k]) for k in ("x_partials", "residual", "post", "comb", "pre", "norm_weight")}
    ro = torch.empty_like(t["residual"])
    li = torch.empty((rows, hidden), dtype=torch.bfloat16, device=ro.device)
    md = ms = None
    if d["mxfp8"]:
        md = torch.empty((rows, hidden), dtype=torch.uint8, device=ro.device)
        ms = torch.empty((rows, hidden // 32), dtype=torch.uint8, device=ro.device)
    p = lambda x: None if x is None else _vp(x.data_ptr())  # noqa: E731
    st = fn(hidden, p(t["x_partials"]), tp, p(t["residual"]), p(t["post"]), p(t["comb"]),
            p(t["pre"]), p(t["norm_weight"]), d["eps"], rows, p(ro), p(li), p(md), p(ms), reset,
            _vp(torch.cuda.current_stream().cuda_stream))
    assert st == 0, binding.load_library().mhc_status_string(st)
    torch.cuda.synchronize()
    out = {"residual": N(ro), "layer_input": N(li)}
    if md is not None:
        out["mx_data"], out["mx_scale"] = N(md), N(ms)
    return out


def test_noalloc_boundary_equals_the_handle_boundary_on_two_calls():
    cases = [("config 1: rows=32 hidden=7168 tp=8 mxfp8", synth.config(1)),
             ("rows=5 hidden=2080 tp=3", synth.boundary_inputs(41, rows=5, hidden=2080, tp=3))]
    for what, d in cases:
        say(f"case: allocation-free boundary, {what}")
        tp, rows, hidden = d["x_partials"].shape
        got = _noalloc(d)
        want = gpu_boundary(handle_for(hidden, rows, tp=tp), d)
        assert set(got) == set(want)
        for k in want:
            assert np.array_equal(got[k], want[k]), f"{what}: {k} differs from mhc_boundary's"
        compare_boundary_outputs(got, oracle_boundary(d), f"allocation-free, {what}")


def test_noalloc_residual_only_equals_the_handle_call():
    """pre = NULL: the residual-only form (no layer input, no row handoff) through the
    allocation-free entry, bit-identical to mhc_residual_only on a handle and within the
    oracle's tolerance."""
    d = synth.boundary_inputs(43, rows=9, hidden=3072, tp=8)
    say("case: allocation-free residual-only rows=9 hidden=3072 tp=8")
    fn = _lib()
    tp, rows, hidden = d["x_partials"].shape
    t = {k: T(d[k]) for k in ("x_partials", "residual", "post", "comb")}
    ro = torch.empty_like(t["residual"])
    st = fn(hidden, _vp(t["x_partials"].data_ptr()), tp, _vp(t["residual"].data_ptr()),
            _vp(t["post"].data_ptr()), _vp(t["comb"].data_ptr()), None, None, 0.0, rows,
            _vp(ro.data_ptr()), None, None, None, 0, _vp(torch.cuda.current_stream().cuda_stream))
    assert st == 0, binding.load_library().mhc_status_string(st)
    torch.cuda.synchronize()
    want = gpu_boundary(handle_for(hidden, rows, tp=tp), d, residual_only=True)
    assert np.array_equal(N(ro), want["residual"])
    compare_boundary_outputs({"residual": N(ro)}, oracle_boundary(d, residual_only=True),
                             "allocation-free residual-only")


def test_noalloc_boundary_rejects_sizes_beyond_its_scratch():
    say("case: allocation-free boundary, limits")
    fn = _lib()
    z = None
    q = _vp(256)
    s = _vp(torch.cuda.current_stream().cuda_stream)
    assert fn(7168, q, 8, q, q, q, q, q, 1e-6, 1025, q, q, q, q, 0, s) == 4  # rows > 1024
    assert fn(16392, q, 8, q, q, q, q, q, 1e-6, 4, q, q, q, q, 0, s) == 4    # hidden > 16384
    assert fn(7168, q, 65, q, q, q, q, q, 1e-6, 4, q, q, q, q, 0, s) == 4    # tp > 64
    assert fn(7164, q, 8, q, q, q, q, q, 1e-6, 4, q, q, q, q, 0, s) == 2     # hidden % 8
    assert fn(7168, z, 8, q, q, q, q, q, 1e-6, 4, q, q, q, q, 0, s) == 1     # no partials
    assert fn(7168, q, 8, q, q, q, q, q, 1e-6, 0, z, z, z, z, 0, s) == 0     # empty call
