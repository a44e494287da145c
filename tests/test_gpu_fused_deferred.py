"""Deferred fused calls (mhc_coeff_args.deferred = 1): the fused boundary + coefficient kernel
leaves the next coefficients as per-chunk partial sums, and whoever consumes them (a boundary,
finalize, residual-only or fused call on the new streams, a flush, or the epilogue that any
other call enqueues first) finishes them. The partial sums are the ones the undeferred kernel
adds, and every finisher adds them in chunk order with the same epilogue, so every output must
equal the undeferred path's bit for bit; that path is held to the oracle by the fused parity
tests (one oracle check here as well)."""

import numpy as np
import pytest
import torch

import oracle
from mhc_hyper_connection_02_amd import binding, synth

from gpu_helpers import N, T, assert_f32_close, handle_for, say

pytestmark = pytest.mark.gpu


def _next_args(seed, hidden):
    d = synth.pre_inputs(seed, rows=1, hidden=hidden)
    return {"fn": T(d["fn"]), "scale": T(d["scale"]), "base": T(d["base"]),
            "rms_eps": d["rms_eps"], "pre_eps": d["pre_eps"], "sinkhorn_eps": d["sinkhorn_eps"],
            "post_alpha": d["post_alpha"], "sinkhorn_iters": d["sinkhorn_iters"]}, d


def _nan_coeffs(rows):
    return (torch.full((rows, 4), float("nan"), device="cuda"),
            torch.full((rows, 4), float("nan"), device="cuda"),
            torch.full((rows, 4, 4), float("nan"), device="cuda"))


def _producer(h, d, nxt, deferred, rows):
    """A fused boundary writing the next coefficients into NaN-filled tensors."""
    dv = {k: T(v) for k, v in d.items() if isinstance(v, np.ndarray)}
    return binding.boundary_coeffs(h, dv["x_partials"], dv["residual"], dv["post"], dv["comb"],
                                   dv["pre"], dv["norm_weight"], d["eps"], nxt, mxfp8=d["mxfp8"],
                                   next_out=_nan_coeffs(rows), deferred=deferred)


def _consume(h, kind, a, e, f, nxt2, rows):
    """The call after the producer: `kind` on its new streams with its next coefficients."""
    streams = a["residual"]
    pre, post, comb = a["next"]
    x = T(e["x_partials"])
    if kind == "boundary":
        return binding.boundary(h, x, streams, post, comb, pre, T(e["norm_weight"]), e["eps"],
                                mxfp8=e["mxfp8"])
    if kind == "finalize":
        return binding.finalize(h, T(f["gemm2_permuted"]), T(f["expert_weights"]),
                                T(f["expanded_idx_to_permuted_idx"]), T(f["shared_output"]),
                                streams, post, comb, pre, T(e["norm_weight"]), e["eps"])
    if kind == "residual_only":
        return {"residual": binding.residual_only(h, x, streams, post, comb)}
    if kind in ("fused", "fused_deferred"):
        o = binding.boundary_coeffs(h, x, streams, post, comb, pre, T(e["norm_weight"]),
                                    e["eps"], nxt2, mxfp8=e["mxfp8"], next_out=_nan_coeffs(rows),
                                    deferred=kind == "fused_deferred")
        binding.pre_coeffs_flush(h)
        p2, q2, c2 = o.pop("next")
        o.update({"next_pre": p2, "next_post": q2, "next_comb": c2})
        return o
    if kind == "flush":
        binding.pre_coeffs_flush(h)
        return {}
    if kind == "other":  # a call that does not consume them: their epilogue is enqueued first
        return {"mean": binding.collapse_mean(h, streams)}
    raise ValueError(kind)


def _run(kind, deferred, rows, hidden, tp=8):
    d = synth.boundary_inputs(300 + rows, rows=rows, hidden=hidden, tp=tp, x_sigma=0.5,
                              mxfp8=hidden % 32 == 0)
    e = synth.boundary_inputs(400 + rows, rows=rows, hidden=hidden, tp=tp, x_sigma=0.5,
                              mxfp8=hidden % 32 == 0)
    f = synth.finalize_inputs(500 + rows, rows=rows, hidden=hidden, top_k=8)
    nxt, _ = _next_args(600 + rows, hidden)
    nxt2, _ = _next_args(700 + rows, hidden)
    h = handle_for(hidden, rows, tp=tp)
    a = _producer(h, d, nxt, deferred, rows)
    o = _consume(h, kind, a, e, f, nxt2, rows)
    torch.cuda.synchronize()
    out = {"p_" + k: N(v) for k, v in a.items() if k != "next"}
    out.update({"pre": N(a["next"][0]), "post": N(a["next"][1]), "comb": N(a["next"][2])})
    out.update({"c_" + k: N(v) for k, v in o.items()})
    assert h.errors() == 0
    return out


@pytest.mark.parametrize("kind,rows,hidden", [
    ("boundary", 128, 7168), ("finalize", 64, 7168), ("residual_only", 32, 7168),
    ("fused", 128, 7168), ("fused_deferred", 96, 7168), ("flush", 128, 7168),
    ("other", 40, 4096), ("boundary", 5, 1056), ("fused", 17, 1000), ("boundary", 20, 8192),
    ("fused_deferred", 300, 7168),
])
def test_deferred_fused_equals_undeferred(kind, rows, hidden):
    say(f"case: deferred fused call consumed by {kind} rows={rows} hidden={hidden}")
    a = _run(kind, False, rows, hidden)
    b = _run(kind, True, rows, hidden)
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{kind}: {k} differs"
    for k in ("pre", "post", "comb"):
        assert not np.isnan(b[k]).any(), f"{kind}: {k} not written"


@pytest.mark.parametrize("tp", [3, 13, 16])
def test_deferred_fused_other_tp(tp):
    """Slice counts other than 8 in the deferred producer and consumer: a short batch (its
    loads past tp re-read the last slice and are dropped), a full batch and a short one,
    two full batches."""
    rows, hidden = 40, 2048
    say(f"case: deferred fused consumer tp={tp} rows={rows} hidden={hidden}")
    a = _run("fused_deferred", False, rows, hidden, tp)
    b = _run("fused_deferred", True, rows, hidden, tp)
    for k in a:
        assert np.array_equal(a[k], b[k]), f"tp {tp}: {k} differs"


def test_deferred_fused_coefficients_match_the_oracle():
    rows, hidden = 64, 7168
    say(f"case: deferred fused coefficients vs oracle rows={rows} hidden={hidden}")
    got = _run("boundary", True, rows, hidden)
    _, c = _next_args(600 + rows, hidden)
    want = oracle.pre_coeffs(got["p_residual"], c["fn"], c["scale"], c["base"], c["rms_eps"],
                             c["pre_eps"], c["sinkhorn_eps"], c["post_alpha"],
                             c["sinkhorn_iters"])
    for name, w in zip(("pre", "post", "comb"), want):
        assert_f32_close(got[name], w, f"deferred fused next {name}")


def test_deferred_fused_fallback_beyond_the_fused_rows():
    """Over 1024 rows the call runs mhc_boundary and mhc_pre_coeffs_deferred; a fused
    consumer of the same size then runs its two calls too (finishing the pending ones inside
    the boundary kernel)."""
    rows, hidden = 1030, 1024
    say(f"case: deferred fused fallback rows={rows} hidden={hidden}")
    a = _run("fused", False, rows, hidden)
    b = _run("fused", True, rows, hidden)
    for k in a:
        assert np.array_equal(a[k], b[k]), f"fallback: {k} differs"


def _chain_inputs(rows, hidden):
    d = synth.boundary_inputs(800, rows=rows, hidden=hidden, tp=8, x_sigma=0.5, mxfp8=True)
    f = synth.finalize_inputs(801, rows=rows, hidden=hidden, top_k=8)
    return (d, {k: T(v) for k, v in d.items() if isinstance(v, np.ndarray)},
            {k: T(v) for k, v in f.items() if isinstance(v, np.ndarray)},
            [_next_args(810 + i, hidden)[0] for i in range(2)])


def _chain(h, steps, deferred, inputs):
    """`steps` fused calls, each consuming the previous one's coefficients (boundary and
    finalize alternating), then a flush; returns every output. Device inputs only (the
    chain is also captured)."""
    d, dv, fv, nx = inputs
    streams, pre, post, comb = dv["residual"], dv["pre"], dv["post"], dv["comb"]
    outs = []

    def step(i, streams, pre, post, comb):
        if i % 2 == 0:
            return binding.boundary_coeffs(h, dv["x_partials"], streams, post, comb, pre,
                                           dv["norm_weight"], d["eps"], nx[i % 2], mxfp8=True,
                                           deferred=deferred)
        return binding.finalize_coeffs(h, fv["gemm2_permuted"], fv["expert_weights"],
                                       fv["expanded_idx_to_permuted_idx"], fv["shared_output"],
                                       streams, post, comb, pre, dv["norm_weight"], d["eps"],
                                       nx[i % 2], mxfp8=True, deferred=deferred)

    for i in range(steps):
        o = step(i, streams, pre, post, comb)
        streams = o["residual"]
        pre, post, comb = o["next"]
        outs += [o["residual"], o["layer_input"], o["mx_data"], o["mx_scale"]]
    binding.pre_coeffs_flush(h)
    return outs + [pre, post, comb]


def test_deferred_fused_chain_equals_undeferred():
    rows, hidden = 128, 7168
    say(f"case: chain of 6 deferred fused calls rows={rows} hidden={hidden}")
    h = handle_for(hidden, rows)
    inputs = _chain_inputs(rows, hidden)
    a = [N(t) for t in _chain(h, 6, False, inputs)]
    b = [N(t) for t in _chain(h, 6, True, inputs)]
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x, y), f"chain output {i} differs"
    assert h.errors() == 0


def test_graph_replays_of_a_deferred_fused_chain():
    """The chain captured whole (it begins and ends with nothing pending), replayed three
    times with eager calls between: every replay equals the eager run bit for bit."""
    rows, hidden = 128, 7168
    say(f"case: HIP graph replays of a deferred fused chain rows={rows} hidden={hidden}")
    h = handle_for(hidden, rows)
    inputs = _chain_inputs(rows, hidden)
    eager = [N(t) for t in _chain(h, 4, True, inputs)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _chain(h, 4, True, inputs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = _chain(h, 4, True, inputs)
    for rep in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(outs, eager)):
            assert np.array_equal(N(x), y), f"replay {rep} output {i}"
        _chain(h, 2, False, inputs)
        torch.cuda.synchronize()
    assert h.errors() == 0


def test_deferred_fused_chain_with_spread_tiles_equals_tile_per_xcd():
    """A chain of deferred fused calls gives the same bits with a tile's chunks spread over the
    XCDs as with each tile on one XCD (MHC_OPT_TILE_PLACEMENT)."""
    rows, hidden = 128, 7168
    say(f"case: chain of 6 deferred fused calls, spread vs per-XCD tiles rows={rows}")
    inputs = _chain_inputs(rows, hidden)
    out = []
    for placement in (binding.MHC_TILE_PER_XCD, binding.MHC_TILE_SPREAD):
        h = handle_for(hidden, rows)
        h.set_option(binding.MHC_OPT_TILE_PLACEMENT, placement)
        out.append([N(t) for t in _chain(h, 6, True, inputs)])
        torch.cuda.synchronize()
        assert h.errors() == 0
    for i, (x, y) in enumerate(zip(*out)):
        assert np.array_equal(x, y), f"chain output {i} differs between placements"
