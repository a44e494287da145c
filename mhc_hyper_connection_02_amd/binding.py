"""Thin Python binding of libmhc_amd.so (argument marshalling only).

Every function has the name of the C entry point it wraps (without the
``mhc_`` prefix) and does three things: checks that the torch tensors it was
given have the dtype, device, layout and shapes the C contract requires (the
C side sees only pointers), allocates outputs that were not passed in, and
calls the entry point on the current HIP stream. All arithmetic runs in the
library's kernels; there is no fallback. If the library is missing, the first
call raises.
"""

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmhc_amd.so")
INCLUDE = os.path.join(os.path.dirname(_PKG), "include")
HEADER = os.path.join(INCLUDE, "mhc.h")

MHC_OK = 0
MHC_OPT_BOUNDARY_BLOCK = 1
MHC_OPT_SPIN_LIMIT = 2
MHC_OPT_SCALE_LAYOUT = 3
MHC_OPT_LANE_ELEMS = 4
MHC_OPT_TILE_PLACEMENT = 5
MHC_TILE_PER_XCD = 0
MHC_TILE_SPREAD = 1
MHC_OPT_ROW_HANDOFF = 6
MHC_HANDOFF_DEVICE = 0
MHC_HANDOFF_XCD = 1
MHC_SCALE_ROW_MAJOR = 0
MHC_SCALE_SWIZZLED_128X4 = 1
_VALUE_ERRORS = {1, 2, 3, 4, 5}

_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

class CoeffArgs(ctypes.Structure):
    """``mhc_coeff_args``: a coefficient call's arguments, for the fused calls."""
    _fields_ = [("fn", _vp), ("scale", _vp), ("base", _vp), ("rms_eps", _f), ("pre_eps", _f),
                ("sinkhorn_eps", _f), ("post_alpha", _f), ("sinkhorn_iters", _i),
                ("deferred", _i), ("pre_out", _vp), ("post_out", _vp), ("comb_out", _vp)]


_SIGS = {
    "mhc_status_string": ([_i], ctypes.c_char_p),
    "mhc_create": ([_i, _i, _i, _i, _i, _i, ctypes.POINTER(_vp)], _i),
    "mhc_set_option": ([_vp, _i, _i], _i),
    "mhc_mxfp8_scale_bytes": ([_i, _i, _i, ctypes.POINTER(ctypes.c_uint64)], _i),
    "mhc_get_errors": ([_vp, ctypes.POINTER(ctypes.c_uint), _i, _vp], _i),
    "mhc_destroy": ([_vp], _i),
    "mhc_reset": ([_vp, _vp], _i),
    "mhc_boundary": ([_vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _f, _i, _vp, _vp, _vp, _vp, _vp], _i),
    "mhc_residual_only": ([_vp, _vp, _i, _vp, _vp, _vp, _i, _vp, _vp], _i),
    "mhc_finalize": ([_vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _i, _vp, _vp,
                      _vp, _vp, _vp], _i),
    "mhc_collapse_mean": ([_vp, _vp, _i, _vp, _vp], _i),
    "mhc_first": ([_vp, _vp, _vp, _f, _i, _vp, _vp, _vp, _vp, _vp], _i),
    "mhc_collapse_norm": ([_vp, _vp, _vp, _vp, _f, _i, _vp, _vp, _vp, _vp], _i),
    "mhc_pre_coeffs": ([_vp, _vp, _vp, _vp, _vp, _f, _f, _f, _f, _i, _i, _vp, _vp, _vp, _vp], _i),
    "mhc_pre_coeffs_deferred": ([_vp, _vp, _vp, _vp, _vp, _f, _f, _f, _f, _i, _i, _vp, _vp, _vp,
                                 _vp], _i),
    "mhc_pre_coeffs_flush": ([_vp, _vp], _i),
    "mhc_boundary_coeffs": ([_vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _f, _i, _vp, _vp, _vp, _vp,
                             ctypes.POINTER(CoeffArgs), _vp], _i),
    "mhc_finalize_coeffs": ([_vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _i, _vp,
                             _vp, _vp, _vp, ctypes.POINTER(CoeffArgs), _vp], _i),
    "mhc_boundary_noalloc": ([_i, _vp, _i, _vp, _vp, _vp, _vp, _vp, _f, _i, _vp, _vp, _vp, _vp,
                              _i, _vp], _i),
    # include/mhc_floor.h: measurement floors of the boundary's launch geometry
    "mhc_floor_boundary_traffic": ([_vp, _i, _vp, _i, _i, _vp, _vp, _vp, _vp, _vp], _i),
    "mhc_floor_empty": ([_i, _i, _vp], _i),
}


def header_functions(paths=None):
    """Names of the functions the headers under include/ declare."""
    if paths is None:
        paths = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))
    names = set()
    for path in paths:
        with open(path) as f:
            text = f.read()
        names.update(re.findall(r"^\s*(?:int|const char\*)\s+(mhc_\w+)\s*\(", text, re.M))
    return sorted(names)


def load_library(path=LIB_PATH):
    """Load libmhc_amd.so (after torch, so torch's HIP runtime is the one in use)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m mhc_hyper_connection_02_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


class MhcError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = load_library().mhc_status_string(status).decode()
        super().__init__(f"{where}: {msg}")


class MhcValueError(MhcError, ValueError):
    pass


def _check(status, where):
    if status != MHC_OK:
        raise (MhcValueError if status in _VALUE_ERRORS else MhcError)(status, where)


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return _vp(s.cuda_stream)


def _need(t, name, dtype, shape, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class Handle:
    """An ``mhc_create`` handle: sized by hidden, hc_mult, max_rows, max_tp and top_k on one device."""

    def __init__(self, hidden, hc_mult=4, max_rows=128, max_tp=8, top_k=8, device=None):
        lib = load_library()
        dev = torch.device("cuda", torch.cuda.current_device() if device is None else device)
        self.hidden, self.hc_mult, self.max_rows = hidden, hc_mult, max_rows
        self.max_tp, self.top_k, self.device = max_tp, top_k, dev
        self.scale_layout = MHC_SCALE_ROW_MAJOR
        h = _vp()
        with torch.cuda.device(dev):
            _check(lib.mhc_create(hidden, hc_mult, max_rows, max_tp, top_k, dev.index,
                                  ctypes.byref(h)), "mhc_create")
        self._h = h

    @property
    def ptr(self):
        if self._h is None:
            raise RuntimeError("handle is closed")
        return self._h

    def set_option(self, option, value):
        _check(load_library().mhc_set_option(self.ptr, option, value), "mhc_set_option")
        if option == MHC_OPT_SCALE_LAYOUT:
            self.scale_layout = value

    def errors(self, clear=False, stream=None):
        """Row-handoff waits that gave up (``mhc_get_errors``); waits for the stream."""
        n = ctypes.c_uint(0)
        _check(load_library().mhc_get_errors(self.ptr, ctypes.byref(n), int(bool(clear)),
                                             _stream(stream)), "mhc_get_errors")
        return n.value

    def reset(self, stream=None):
        _check(load_library().mhc_reset(self.ptr, _stream(stream)), "mhc_reset")

    def close(self):
        if getattr(self, "_h", None) is not None:
            _check(load_library().mhc_destroy(self._h), "mhc_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def mxfp8_scale_bytes(rows, hidden, layout=MHC_SCALE_ROW_MAJOR):
    """``mhc_mxfp8_scale_bytes``: bytes of an MXFP8 scale buffer in a scale layout."""
    n = ctypes.c_uint64(0)
    _check(load_library().mhc_mxfp8_scale_bytes(rows, hidden, layout, ctypes.byref(n)),
           "mhc_mxfp8_scale_bytes")
    return n.value


def _mx_outputs(h, rows, hidden, dev, mx_out):
    """The E4M3 data [rows, hidden] and the scale bytes: [rows, hidden // 32] row-major, or
    the swizzled 128x4 layout's padded byte vector (allocated zeroed, so that the padding
    the kernels leave alone reads as zero)."""
    swizzled = getattr(h, "scale_layout", MHC_SCALE_ROW_MAJOR) == MHC_SCALE_SWIZZLED_128X4
    scale_shape = ((mxfp8_scale_bytes(rows, hidden, MHC_SCALE_SWIZZLED_128X4),) if swizzled
                   else (rows, hidden // 32))
    if mx_out is None:
        alloc = torch.zeros if swizzled else torch.empty
        mx_out = (torch.empty((rows, hidden), dtype=torch.uint8, device=dev),
                  alloc(scale_shape, dtype=torch.uint8, device=dev))
    mx_data, mx_scale = mx_out
    _need(mx_data, "mx_data_out", torch.uint8, (rows, hidden), dev)
    _need(mx_scale, "mx_scale_out", torch.uint8, scale_shape, dev)
    return mx_data, mx_scale


def _mix_outputs(h, residual, pre, norm_weight, mxfp8, residual_out, layer_input_out, mx_out):
    rows, n, hidden = residual.shape
    dev = residual.device
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _need(residual_out, "residual_out", torch.bfloat16, (rows, n, hidden), dev)
    if pre is None:
        if norm_weight is not None or mxfp8 or layer_input_out is not None or mx_out is not None:
            raise ValueError("residual-only (pre=None) takes no norm weight and writes no layer input")
        return residual_out, None, None, None
    _need(pre, "pre", torch.float32, (rows, n), dev)
    _need(norm_weight, "norm_weight", torch.bfloat16, (hidden,), dev)
    if layer_input_out is None:
        layer_input_out = torch.empty((rows, hidden), dtype=torch.bfloat16, device=dev)
    _need(layer_input_out, "layer_input_out", torch.bfloat16, (rows, hidden), dev)
    mx_data = mx_scale = None
    if mxfp8:
        mx_data, mx_scale = _mx_outputs(h, rows, hidden, dev, mx_out)
    return residual_out, layer_input_out, mx_data, mx_scale


def _check_mix_inputs(h, residual, post, comb):
    if residual.dim() != 3:
        raise ValueError("residual must be [rows, hc_mult, hidden]")
    rows, n, hidden = residual.shape
    dev = residual.device
    if n != h.hc_mult or hidden != h.hidden:
        raise ValueError(f"residual {tuple(residual.shape)} does not fit the handle "
                         f"(hc_mult={h.hc_mult}, hidden={h.hidden})")
    _need(residual, "residual", torch.bfloat16, (rows, n, hidden), dev)
    _need(post, "post", torch.float32, (rows, n), dev)
    _need(comb, "comb", torch.float32, (rows, n, n), dev)
    return rows, n, hidden, dev


def _result(residual_out, layer_input_out, mx_data, mx_scale):
    out = {"residual": residual_out}
    if layer_input_out is not None:
        out["layer_input"] = layer_input_out
    if mx_data is not None:
        out["mx_data"], out["mx_scale"] = mx_data, mx_scale
    return out


def boundary(h, x_partials, residual, post, comb, pre=None, norm_weight=None, eps=0.0,
             mxfp8=False, residual_out=None, layer_input_out=None, mx_out=None, stream=None):
    """``mhc_boundary``: TP partials [tp,rows,hidden] -> dict(residual, layer_input?, mx_data?, mx_scale?)."""
    rows, n, hidden, dev = _check_mix_inputs(h, residual, post, comb)
    if x_partials.dim() != 3:
        raise ValueError("x_partials must be [tp, rows, hidden]")
    tp = x_partials.shape[0]
    _need(x_partials, "x_partials", torch.bfloat16, (tp, rows, hidden), dev)
    ro, li, md, ms = _mix_outputs(h, residual, pre, norm_weight, mxfp8, residual_out,
                                  layer_input_out, mx_out)
    st = load_library().mhc_boundary(h.ptr, _ptr(x_partials), tp, _ptr(residual), _ptr(post),
                                     _ptr(comb), _ptr(pre), _ptr(norm_weight), float(eps), rows,
                                     _ptr(ro), _ptr(li), _ptr(md), _ptr(ms), _stream(stream))
    _check(st, "mhc_boundary")
    return _result(ro, li, md, ms)


def boundary_noalloc(x_partials, residual, post, comb, pre=None, norm_weight=None, eps=0.0,
                     mxfp8=False, residual_out=None, layer_input_out=None, mx_out=None,
                     reset=False, stream=None):
    """``mhc_boundary_noalloc``: ``boundary`` without a handle (the library allocates nothing;
    outputs not passed in are allocated here by torch)."""
    if x_partials.dim() != 3 or residual.dim() != 3:
        raise ValueError("x_partials must be [tp, rows, hidden], residual [rows, 4, hidden]")
    tp, rows, hidden = x_partials.shape
    dev = residual.device
    _need(x_partials, "x_partials", torch.bfloat16, (tp, rows, hidden), dev)
    _need(residual, "residual", torch.bfloat16, (rows, 4, hidden), dev)
    _need(post, "post", torch.float32, (rows, 4), dev)
    _need(comb, "comb", torch.float32, (rows, 4, 4), dev)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _need(residual_out, "residual_out", torch.bfloat16, (rows, 4, hidden), dev)
    li = md = ms = None
    if pre is not None:
        _need(pre, "pre", torch.float32, (rows, 4), dev)
        _need(norm_weight, "norm_weight", torch.bfloat16, (hidden,), dev)
        li = layer_input_out if layer_input_out is not None else torch.empty(
            (rows, hidden), dtype=torch.bfloat16, device=dev)
        _need(li, "layer_input_out", torch.bfloat16, (rows, hidden), dev)
        if mxfp8:
            md, ms = mx_out if mx_out is not None else (
                torch.empty((rows, hidden), dtype=torch.uint8, device=dev),
                torch.empty((rows, hidden // 32), dtype=torch.uint8, device=dev))
            _need(md, "mx_data_out", torch.uint8, (rows, hidden), dev)
            _need(ms, "mx_scale_out", torch.uint8, (rows, hidden // 32), dev)
    st = load_library().mhc_boundary_noalloc(
        hidden, _ptr(x_partials), tp, _ptr(residual), _ptr(post), _ptr(comb), _ptr(pre),
        _ptr(norm_weight), float(eps), rows, _ptr(residual_out), _ptr(li), _ptr(md), _ptr(ms),
        int(bool(reset)), _stream(stream))
    _check(st, "mhc_boundary_noalloc")
    return _result(residual_out, li, md, ms)


def residual_only(h, x_partials, residual, post, comb, residual_out=None, stream=None):
    """``mhc_residual_only``: returns the new streams [rows, hc_mult, hidden]."""
    rows, n, hidden, dev = _check_mix_inputs(h, residual, post, comb)
    tp = x_partials.shape[0]
    _need(x_partials, "x_partials", torch.bfloat16, (tp, rows, hidden), dev)
    ro, _, _, _ = _mix_outputs(h, residual, None, None, False, residual_out, None, None)
    st = load_library().mhc_residual_only(h.ptr, _ptr(x_partials), tp, _ptr(residual), _ptr(post),
                                          _ptr(comb), rows, _ptr(ro), _stream(stream))
    _check(st, "mhc_residual_only")
    return ro


def finalize(h, gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx, shared_output,
             residual, post, comb, pre=None, norm_weight=None, eps=0.0, mxfp8=False,
             residual_out=None, layer_input_out=None, mx_out=None, stream=None):
    """``mhc_finalize``: the boundary on an unfinalized MoE output."""
    rows, n, hidden, dev = _check_mix_inputs(h, residual, post, comb)
    if gemm2_permuted.dim() != 2:
        raise ValueError("gemm2_permuted must be [num_permuted, hidden]")
    P = gemm2_permuted.shape[0]
    _need(gemm2_permuted, "gemm2_permuted", torch.bfloat16, (P, hidden), dev)
    _need(expert_weights, "expert_weights", torch.float32, (rows, h.top_k), dev)
    _need(expanded_idx_to_permuted_idx, "expanded_idx_to_permuted_idx", torch.int32,
          (rows * h.top_k,), dev)
    _need(shared_output, "shared_output", torch.bfloat16, (rows, hidden), dev)
    ro, li, md, ms = _mix_outputs(h, residual, pre, norm_weight, mxfp8, residual_out,
                                  layer_input_out, mx_out)
    st = load_library().mhc_finalize(h.ptr, _ptr(gemm2_permuted), P, _ptr(expert_weights),
                                     _ptr(expanded_idx_to_permuted_idx), _ptr(shared_output),
                                     _ptr(residual), _ptr(post), _ptr(comb), _ptr(pre),
                                     _ptr(norm_weight), float(eps), rows, _ptr(ro), _ptr(li),
                                     _ptr(md), _ptr(ms), _stream(stream))
    _check(st, "mhc_finalize")
    return _result(ro, li, md, ms)


def collapse_mean(h, streams, out=None, stream=None):
    """``mhc_collapse_mean``: [rows, hc_mult, hidden] -> [rows, hidden] bf16."""
    if streams.dim() != 3:
        raise ValueError("streams must be [rows, hc_mult, hidden]")
    rows, n, hidden = streams.shape
    dev = streams.device
    if n != h.hc_mult or hidden != h.hidden:
        raise ValueError("streams do not fit the handle")
    _need(streams, "streams", torch.bfloat16, (rows, n, hidden), dev)
    if out is None:
        out = torch.empty((rows, hidden), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (rows, hidden), dev)
    _check(load_library().mhc_collapse_mean(h.ptr, _ptr(streams), rows, _ptr(out), _stream(stream)),
           "mhc_collapse_mean")
    return out


def _layer_outputs(h, rows, dev, mxfp8, layer_input_out, mx_out):
    hidden = h.hidden
    if layer_input_out is None:
        layer_input_out = torch.empty((rows, hidden), dtype=torch.bfloat16, device=dev)
    _need(layer_input_out, "layer_input_out", torch.bfloat16, (rows, hidden), dev)
    mx_data = mx_scale = None
    if mxfp8:
        mx_data, mx_scale = _mx_outputs(h, rows, hidden, dev, mx_out)
    elif mx_out is not None:
        raise ValueError("mx_out given without mxfp8=True")
    return layer_input_out, mx_data, mx_scale


def first(h, x, norm_weight, eps, mxfp8=False, residual_out=None, layer_input_out=None,
          mx_out=None, stream=None):
    """``mhc_first``: embedding [rows, hidden] -> dict(residual [rows, n, hidden] (x in every
    stream), layer_input, mx_data?, mx_scale?)."""
    if x.dim() != 2 or x.shape[1] != h.hidden:
        raise ValueError(f"x must be [rows, {h.hidden}]")
    rows, dev = x.shape[0], x.device
    _need(x, "x", torch.bfloat16, (rows, h.hidden), dev)
    _need(norm_weight, "norm_weight", torch.bfloat16, (h.hidden,), dev)
    if residual_out is None:
        residual_out = torch.empty((rows, h.hc_mult, h.hidden), dtype=torch.bfloat16, device=dev)
    _need(residual_out, "residual_out", torch.bfloat16, (rows, h.hc_mult, h.hidden), dev)
    li, md, ms = _layer_outputs(h, rows, dev, mxfp8, layer_input_out, mx_out)
    st = load_library().mhc_first(h.ptr, _ptr(x), _ptr(norm_weight), float(eps), rows,
                                  _ptr(residual_out), _ptr(li), _ptr(md), _ptr(ms),
                                  _stream(stream))
    _check(st, "mhc_first")
    return _result(residual_out, li, md, ms)


def collapse_norm(h, residual, pre, norm_weight, eps, mxfp8=False, out=None, mx_out=None,
                  stream=None):
    """``mhc_collapse_norm``: streams [rows, n, hidden] and pre [rows, n] -> dict(layer_input
    [rows, hidden], mx_data?, mx_scale?)."""
    if residual.dim() != 3:
        raise ValueError("residual must be [rows, hc_mult, hidden]")
    rows, n, hidden = residual.shape
    dev = residual.device
    if n != h.hc_mult or hidden != h.hidden:
        raise ValueError("residual does not fit the handle")
    _need(residual, "residual", torch.bfloat16, (rows, n, hidden), dev)
    _need(pre, "pre", torch.float32, (rows, n), dev)
    _need(norm_weight, "norm_weight", torch.bfloat16, (hidden,), dev)
    li, md, ms = _layer_outputs(h, rows, dev, mxfp8, out, mx_out)
    st = load_library().mhc_collapse_norm(h.ptr, _ptr(residual), _ptr(pre), _ptr(norm_weight),
                                          float(eps), rows, _ptr(li), _ptr(md), _ptr(ms),
                                          _stream(stream))
    _check(st, "mhc_collapse_norm")
    res = {"layer_input": li}
    if md is not None:
        res["mx_data"], res["mx_scale"] = md, ms
    return res


def pre_coeffs(h, residual, fn, scale, base, rms_eps, pre_eps, sinkhorn_eps, post_alpha,
               sinkhorn_iters, out=None, stream=None, deferred=False):
    """``mhc_pre_coeffs``: streams [rows, n, hidden] -> (pre [rows,n], post [rows,n], comb [rows,n,n]).
    With ``deferred``, ``mhc_pre_coeffs_deferred``: the outputs are written by the boundary
    call that consumes them, or by :func:`pre_coeffs_flush`."""
    if residual.dim() != 3:
        raise ValueError("residual must be [rows, hc_mult, hidden]")
    rows, n, hidden = residual.shape
    dev = residual.device
    if n != h.hc_mult or hidden != h.hidden:
        raise ValueError("residual does not fit the handle")
    nc = 2 * n + n * n
    _need(residual, "residual", torch.bfloat16, (rows, n, hidden), dev)
    _need(fn, "fn", torch.bfloat16, (n * hidden, nc), dev)
    _need(scale, "scale", torch.float32, (3,), dev)
    _need(base, "base", torch.float32, (nc,), dev)
    if out is None:
        out = (torch.empty((rows, n), dtype=torch.float32, device=dev),
               torch.empty((rows, n), dtype=torch.float32, device=dev),
               torch.empty((rows, n, n), dtype=torch.float32, device=dev))
    pre, post, comb = out
    _need(pre, "pre_out", torch.float32, (rows, n), dev)
    _need(post, "post_out", torch.float32, (rows, n), dev)
    _need(comb, "comb_out", torch.float32, (rows, n, n), dev)
    name = "mhc_pre_coeffs_deferred" if deferred else "mhc_pre_coeffs"
    st = getattr(load_library(), name)(h.ptr, _ptr(residual), _ptr(fn), _ptr(scale), _ptr(base),
                                       float(rms_eps), float(pre_eps), float(sinkhorn_eps),
                                       float(post_alpha), int(sinkhorn_iters), rows, _ptr(pre),
                                       _ptr(post), _ptr(comb), _stream(stream))
    _check(st, name)
    return pre, post, comb


def pre_coeffs_flush(h, stream=None):
    """``mhc_pre_coeffs_flush``: complete a pending deferred coefficient call."""
    _check(load_library().mhc_pre_coeffs_flush(h.ptr, _stream(stream)), "mhc_pre_coeffs_flush")


def _coeff_args(h, rows, dev, nxt, out, deferred):
    """Check a coefficient call's arguments (a dict with fn, scale, base, rms_eps, pre_eps,
    sinkhorn_eps, post_alpha, sinkhorn_iters) and its outputs; -> (CoeffArgs, outputs)."""
    n, hidden = h.hc_mult, h.hidden
    nc = 2 * n + n * n
    _need(nxt["fn"], "fn", torch.bfloat16, (n * hidden, nc), dev)
    _need(nxt["scale"], "scale", torch.float32, (3,), dev)
    _need(nxt["base"], "base", torch.float32, (nc,), dev)
    if out is None:
        out = (torch.empty((rows, n), dtype=torch.float32, device=dev),
               torch.empty((rows, n), dtype=torch.float32, device=dev),
               torch.empty((rows, n, n), dtype=torch.float32, device=dev))
    pre, post, comb = out
    _need(pre, "next pre_out", torch.float32, (rows, n), dev)
    _need(post, "next post_out", torch.float32, (rows, n), dev)
    _need(comb, "next comb_out", torch.float32, (rows, n, n), dev)
    a = CoeffArgs(_ptr(nxt["fn"]), _ptr(nxt["scale"]), _ptr(nxt["base"]), float(nxt["rms_eps"]),
                  float(nxt["pre_eps"]), float(nxt["sinkhorn_eps"]), float(nxt["post_alpha"]),
                  int(nxt["sinkhorn_iters"]), 1 if deferred else 0, _ptr(pre), _ptr(post),
                  _ptr(comb))
    return a, out


def boundary_coeffs(h, x_partials, residual, post, comb, pre, norm_weight, eps, nxt,
                    mxfp8=False, residual_out=None, layer_input_out=None, mx_out=None,
                    next_out=None, deferred=False, stream=None):
    """``mhc_boundary_coeffs``: :func:`boundary` and then :func:`pre_coeffs` on its new streams
    with the arguments in ``nxt`` (a dict), in one kernel. Returns boundary's dict plus
    ``next`` = (pre, post, comb) of the next sublayer. ``deferred``: the next coefficients
    stay pending, as after :func:`pre_coeffs_deferred`."""
    rows, n, hidden, dev = _check_mix_inputs(h, residual, post, comb)
    if x_partials.dim() != 3:
        raise ValueError("x_partials must be [tp, rows, hidden]")
    tp = x_partials.shape[0]
    _need(x_partials, "x_partials", torch.bfloat16, (tp, rows, hidden), dev)
    if pre is None:
        raise ValueError("the fused call writes a layer input: pre is required")
    ro, li, md, ms = _mix_outputs(h, residual, pre, norm_weight, mxfp8, residual_out,
                                  layer_input_out, mx_out)
    a, nout = _coeff_args(h, rows, dev, nxt, next_out, deferred)
    st = load_library().mhc_boundary_coeffs(h.ptr, _ptr(x_partials), tp, _ptr(residual),
                                            _ptr(post), _ptr(comb), _ptr(pre),
                                            _ptr(norm_weight), float(eps), rows, _ptr(ro),
                                            _ptr(li), _ptr(md), _ptr(ms), ctypes.byref(a),
                                            _stream(stream))
    _check(st, "mhc_boundary_coeffs")
    res = _result(ro, li, md, ms)
    res["next"] = nout
    return res


def finalize_coeffs(h, gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx,
                    shared_output, residual, post, comb, pre, norm_weight, eps, nxt,
                    mxfp8=False, residual_out=None, layer_input_out=None, mx_out=None,
                    next_out=None, deferred=False, stream=None):
    """``mhc_finalize_coeffs``: :func:`finalize` and then :func:`pre_coeffs` on its new
    streams, in one kernel; returns and defers as :func:`boundary_coeffs`."""
    rows, n, hidden, dev = _check_mix_inputs(h, residual, post, comb)
    if gemm2_permuted.dim() != 2:
        raise ValueError("gemm2_permuted must be [num_permuted, hidden]")
    P = gemm2_permuted.shape[0]
    _need(gemm2_permuted, "gemm2_permuted", torch.bfloat16, (P, hidden), dev)
    _need(expert_weights, "expert_weights", torch.float32, (rows, h.top_k), dev)
    _need(expanded_idx_to_permuted_idx, "expanded_idx_to_permuted_idx", torch.int32,
          (rows * h.top_k,), dev)
    _need(shared_output, "shared_output", torch.bfloat16, (rows, hidden), dev)
    if pre is None:
        raise ValueError("the fused call writes a layer input: pre is required")
    ro, li, md, ms = _mix_outputs(h, residual, pre, norm_weight, mxfp8, residual_out,
                                  layer_input_out, mx_out)
    a, nout = _coeff_args(h, rows, dev, nxt, next_out, deferred)
    st = load_library().mhc_finalize_coeffs(h.ptr, _ptr(gemm2_permuted), P, _ptr(expert_weights),
                                            _ptr(expanded_idx_to_permuted_idx),
                                            _ptr(shared_output), _ptr(residual), _ptr(post),
                                            _ptr(comb), _ptr(pre), _ptr(norm_weight), float(eps),
                                            rows, _ptr(ro), _ptr(li), _ptr(md), _ptr(ms),
                                            ctypes.byref(a), _stream(stream))
    _check(st, "mhc_finalize_coeffs")
    res = _result(ro, li, md, ms)
    res["next"] = nout
    return res


# ---------------------------------------------------------------------------
# include/mhc_floor.h: what a kernel of the boundary's shape costs without its arithmetic
# ---------------------------------------------------------------------------

def floor_boundary_traffic(x_partials, residual, residual_out, layer_input_out, mx_data_out,
                           mx_scale_out, stream=None):
    """``mhc_floor_boundary_traffic``: the boundary's bytes moved with its geometry, no
    arithmetic (the outputs' values mean nothing)."""
    tp, rows, hidden = x_partials.shape
    dev = x_partials.device
    _need(x_partials, "x_partials", torch.bfloat16, (tp, rows, hidden), dev)
    _need(residual, "residual", torch.bfloat16, (rows, 4, hidden), dev)
    _need(residual_out, "residual_out", torch.bfloat16, (rows, 4, hidden), dev)
    _need(layer_input_out, "layer_input_out", torch.bfloat16, (rows, hidden), dev)
    _need(mx_data_out, "mx_data_out", torch.uint8, (rows, hidden), dev)
    _need(mx_scale_out, "mx_scale_out", torch.uint8, (rows, hidden // 32), dev)
    _check(load_library().mhc_floor_boundary_traffic(
        _ptr(x_partials), tp, _ptr(residual), rows, hidden, _ptr(residual_out),
        _ptr(layer_input_out), _ptr(mx_data_out), _ptr(mx_scale_out), _stream(stream)),
        "mhc_floor_boundary_traffic")


def floor_empty(rows, hidden, stream=None):
    """``mhc_floor_empty``: an empty kernel of the same grid."""
    _check(load_library().mhc_floor_empty(int(rows), int(hidden), _stream(stream)),
           "mhc_floor_empty")
