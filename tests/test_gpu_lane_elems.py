"""The boundary, finalize and head kernels with four or two elements per lane
(MHC_OPT_LANE_ELEMS = 4 or 2: 8- or 4-byte vectors at two or four times the threads) against
the oracle, and against the eight-elements-per-lane form: the new streams bit for bit (every element's
arithmetic is the same), the layer input within the bf16 tolerance of the oracle, and the
MXFP8 form bit-exact against the oracle's quantizer of the GPU's own layer input."""

import numpy as np
import pytest
import torch

from mhc_hyper_connection_02_amd import binding, synth

from gpu_helpers import (compare_boundary_outputs, gpu_boundary, gpu_finalize, handle_for,
                         oracle_boundary, oracle_finalize, say)

pytestmark = pytest.mark.gpu


def _handle(hidden, rows, elems, tp=8):
    h = handle_for(hidden, rows, tp=tp)
    h.set_option(binding.MHC_OPT_LANE_ELEMS, elems)
    return h


@pytest.mark.parametrize("rows,hidden,tp", [(32, 7168, 8), (64, 7168, 8), (128, 7168, 8),
                                            (5, 1056, 3), (1, 32, 1), (130, 4096, 2),
                                            (17, 1000, 8), (33, 8, 4), (300, 2048, 8)])
@pytest.mark.parametrize("elems", [4, 2])
def test_boundary_fewer_elements_per_lane(rows, hidden, tp, elems):
    mx = hidden % 32 == 0
    say(f"case: boundary lane_elems={elems} rows={rows} hidden={hidden} tp={tp} mxfp8={mx}")
    d = synth.boundary_inputs(900 + rows, rows=rows, hidden=hidden, tp=tp, x_sigma=0.5, mxfp8=mx)
    got = gpu_boundary(_handle(hidden, rows, elems, tp), d)
    ref = gpu_boundary(_handle(hidden, rows, 8, tp), d)
    compare_boundary_outputs(got, oracle_boundary(d), f"lane_elems={elems} {rows}x{hidden}")
    assert np.array_equal(got["residual"], ref["residual"]), "streams differ from 8 per lane"
    same = float(np.mean(got["layer_input"] == ref["layer_input"]))
    assert same > 0.99, f"layer input: only {same:.4f} bit-identical to 8 per lane"


@pytest.mark.parametrize("rows,hidden,top_k", [(64, 7168, 8), (3, 1056, 8), (40, 1024, 3),
                                               (9, 4096, 12)])
@pytest.mark.parametrize("elems", [4, 2])
def test_finalize_fewer_elements_per_lane(rows, hidden, top_k, elems):
    mx = hidden % 32 == 0
    say(f"case: finalize lane_elems={elems} rows={rows} hidden={hidden} top_k={top_k}")
    d = synth.finalize_inputs(950 + rows, rows=rows, hidden=hidden, top_k=top_k, mxfp8=mx)
    h4 = handle_for(hidden, rows, top_k=top_k)
    h4.set_option(binding.MHC_OPT_LANE_ELEMS, elems)
    h8 = handle_for(hidden, rows, top_k=top_k)
    got, ref = gpu_finalize(h4, d), gpu_finalize(h8, d)
    compare_boundary_outputs(got, oracle_finalize(d), f"finalize lane_elems={elems} {rows}x{hidden}")
    assert np.array_equal(got["residual"], ref["residual"]), "streams differ from 8 per lane"
    assert h4.errors() == 0


def test_lane_elems_option_values():
    h = handle_for(1024, 4)
    for bad in (0, 1, 3, 16):
        with pytest.raises(ValueError):
            h.set_option(binding.MHC_OPT_LANE_ELEMS, bad)
    for ok in (4, 2, 8):
        h.set_option(binding.MHC_OPT_LANE_ELEMS, ok)
    torch.cuda.synchronize()


@pytest.mark.parametrize("rows,hidden", [(32, 7168), (5, 1056), (128, 7168), (3, 8)])
def test_first_and_head_fewer_elements_per_lane(rows, hidden):
    import oracle
    from oracle import codecs
    from gpu_helpers import N, T, assert_bf16_close
    mx = hidden % 32 == 0
    say(f"case: first/head lane_elems=2,4,8 rows={rows} hidden={hidden} mxfp8={mx}")
    rng = np.random.default_rng(rows + hidden)
    x = codecs.f64_to_bf16_bits(rng.normal(0, 1, (rows, hidden)))
    w = codecs.f64_to_bf16_bits(rng.normal(1, 0.1, hidden))
    d = synth.boundary_inputs(rows + 7, rows=rows, hidden=hidden, tp=1, mxfp8=mx)
    for elems in (2, 4, 8):
        h = handle_for(hidden, rows)
        h.set_option(binding.MHC_OPT_LANE_ELEMS, elems)
        f = {k: N(v) for k, v in binding.first(h, T(x), T(w), 1e-6, mxfp8=mx).items()}
        hd = {k: N(v) for k, v in binding.collapse_norm(h, T(d["residual"]), T(d["pre"]),
                                                       T(d["norm_weight"]), d["eps"],
                                                       mxfp8=mx).items()}
        torch.cuda.synchronize()
        wf = oracle.first(x, w, 1e-6, mxfp8=mx)
        wh = oracle.collapse_norm(d["residual"], d["pre"], d["norm_weight"], d["eps"], mxfp8=mx)
        assert np.array_equal(f["residual"], wf["residual"]), "first: streams are x, bit for bit"
        assert_bf16_close(f["layer_input"], wf["layer_input"], f"first {elems}/lane")
        assert_bf16_close(hd["layer_input"], wh["layer_input"], f"head {elems}/lane")
        for got in (f, hd):
            if mx:
                codes, scales = codecs.mxfp8_quantize(got["layer_input"])
                assert np.array_equal(got["mx_scale"], scales)
                assert np.array_equal(got["mx_data"], codes)
        assert h.errors() == 0
        h.close()
