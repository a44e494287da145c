"""Deferred coefficient calls (mhc_pre_coeffs_deferred): the consuming boundary finishes the
coefficients inside its kernel. Every result must equal the two-kernel path bit for bit
(same arithmetic, same order), and that path is held to the oracle by the parity tests.
"""

import numpy as np
import pytest
import torch

import oracle
from mhc_hyper_connection_02_amd import binding, synth

from gpu_helpers import N, T, assert_f32_close, handle_for, say

pytestmark = pytest.mark.gpu


def _coeff_inputs(seed, rows, hidden):
    d = synth.pre_inputs(seed, rows=rows, hidden=hidden)
    return {k: (T(v) if isinstance(v, np.ndarray) else v) for k, v in d.items()}


def _coeffs(h, streams, c, deferred, out=None):
    return binding.pre_coeffs(h, streams, c["fn"], c["scale"], c["base"], c["rms_eps"],
                              c["pre_eps"], c["sinkhorn_eps"], c["post_alpha"],
                              c["sinkhorn_iters"], out=out, deferred=deferred)


def _empty_coeffs(rows, dev="cuda"):
    return (torch.full((rows, 4), float("nan"), device=dev),
            torch.full((rows, 4), float("nan"), device=dev),
            torch.full((rows, 4, 4), float("nan"), device=dev))


def _run(kind, deferred, rows, hidden, block=None):
    """A coefficient call on the streams, then the boundary of `kind` consuming it."""
    tp = 8
    d = synth.boundary_inputs(900 + rows, rows=rows, hidden=hidden, tp=tp, mxfp8=hidden % 32 == 0)
    f = synth.finalize_inputs(950 + rows, rows=rows, hidden=hidden, top_k=8)
    c = _coeff_inputs(990 + rows, rows, hidden)
    h = handle_for(hidden, rows, tp=tp, top_k=8, block=block)
    streams = T(d["residual"])
    pre, post, comb = _coeffs(h, streams, c, deferred, out=_empty_coeffs(rows))
    mx = d["mxfp8"] and kind != "residual_only"
    if kind == "boundary":
        o = binding.boundary(h, T(d["x_partials"]), streams, post, comb, pre,
                             T(d["norm_weight"]), d["eps"], mxfp8=mx)
    elif kind == "finalize":
        o = binding.finalize(h, T(f["gemm2_permuted"]), T(f["expert_weights"]),
                             T(f["expanded_idx_to_permuted_idx"]), T(f["shared_output"]),
                             streams, post, comb, pre, T(d["norm_weight"]), d["eps"], mxfp8=mx)
    else:
        o = {"residual": binding.residual_only(h, T(d["x_partials"]), streams, post, comb)}
    torch.cuda.synchronize()
    out = {k: N(v) for k, v in o.items()}
    out.update({"pre": N(pre), "post": N(post), "comb": N(comb)})
    assert h.errors() == 0
    return out


@pytest.mark.parametrize("kind,rows,hidden,block", [
    ("boundary", 32, 7168, None), ("boundary", 128, 7168, None), ("boundary", 5, 1056, 256),
    ("boundary", 300, 4096, 128), ("finalize", 64, 7168, None), ("finalize", 3, 512, 512),
    ("residual_only", 32, 7168, None), ("residual_only", 17, 1024, None),
])
def test_deferred_equals_two_kernel_path(kind, rows, hidden, block):
    say(f"case: deferred coefficients consumed by {kind} rows={rows} hidden={hidden} "
        f"block={block}")
    a = _run(kind, False, rows, hidden, block)
    b = _run(kind, True, rows, hidden, block)
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=False), f"{kind}: {k} differs"


def test_deferred_coefficients_match_the_oracle():
    rows, hidden = 64, 7168
    say(f"case: deferred coefficients vs oracle rows={rows} hidden={hidden}")
    got = _run("boundary", True, rows, hidden)
    c = synth.pre_inputs(990 + rows, rows=rows, hidden=hidden)
    d = synth.boundary_inputs(900 + rows, rows=rows, hidden=hidden, tp=8)
    want = oracle.pre_coeffs(d["residual"], c["fn"], c["scale"], c["base"], c["rms_eps"],
                             c["pre_eps"], c["sinkhorn_eps"], c["post_alpha"], c["sinkhorn_iters"])
    for name, b in zip(("pre", "post", "comb"), want):
        assert_f32_close(got[name], b, f"deferred {name}")


def test_a_call_that_does_not_consume_flushes_first():
    """Pending coefficients, then a boundary with other post/comb buffers, a collapse and
    an explicit flush: the pending outputs are written as by the two-kernel path."""
    rows, hidden = 16, 2048
    say(f"case: deferred flush paths rows={rows} hidden={hidden}")
    d = synth.boundary_inputs(31, rows=rows, hidden=hidden, tp=2, mxfp8=True)
    c = _coeff_inputs(32, rows, hidden)
    h = handle_for(hidden, rows, tp=2)
    streams = T(d["residual"])
    want = [N(t) for t in _coeffs(h, streams, c, False)]
    # 1. a boundary on other coefficient buffers: flushes, its own results unaffected
    out = _coeffs(h, streams, c, True, out=_empty_coeffs(rows))
    o = binding.boundary(h, T(d["x_partials"]), streams, T(d["post"]), T(d["comb"]), T(d["pre"]),
                         T(d["norm_weight"]), d["eps"], mxfp8=True)
    ref = binding.boundary(h, T(d["x_partials"]), streams, T(d["post"]), T(d["comb"]),
                           T(d["pre"]), T(d["norm_weight"]), d["eps"], mxfp8=True)
    torch.cuda.synchronize()
    for k in o:
        assert np.array_equal(N(o[k]), N(ref[k])), k
    for a, b in zip(out, want):
        assert np.array_equal(N(a), b)
    # 2. a collapse call flushes
    out = _coeffs(h, streams, c, True, out=_empty_coeffs(rows))
    binding.collapse_mean(h, streams)
    torch.cuda.synchronize()
    for a, b in zip(out, want):
        assert np.array_equal(N(a), b)
    # 3. an explicit flush; then a second flush is a no-op
    out = _coeffs(h, streams, c, True, out=_empty_coeffs(rows))
    binding.pre_coeffs_flush(h)
    binding.pre_coeffs_flush(h)
    torch.cuda.synchronize()
    for a, b in zip(out, want):
        assert np.array_equal(N(a), b)
    # 4. a second deferred call flushes the first (whose partials it overwrites)
    out1 = _coeffs(h, streams, c, True, out=_empty_coeffs(rows))
    out2 = _coeffs(h, streams, c, True, out=_empty_coeffs(rows))
    binding.pre_coeffs_flush(h)
    torch.cuda.synchronize()
    for a, b, w in zip(out1, out2, want):
        assert np.array_equal(N(a), w) and np.array_equal(N(b), w)
    assert h.errors() == 0
