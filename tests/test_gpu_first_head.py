"""GPU parity of the first layer's entry (mhc_first) and the head's collapse + norm
(mhc_collapse_norm) against the oracle, on the same seeded inputs."""

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs
from mhc_hyper_connection_02_amd import binding, synth

from gpu_helpers import N, T, assert_bf16_close, handle_for, say

pytestmark = pytest.mark.gpu


def _check_layer(g, o, what):
    """Layer input within the bf16 tolerance; MXFP8 bit-exact against the oracle's quantizer
    of the GPU's own layer input."""
    assert_bf16_close(g["layer_input"], o["layer_input"], what + " layer input")
    if "mx_data" in o:
        codes, scales = codecs.mxfp8_quantize(g["layer_input"])
        assert np.array_equal(g["mx_scale"], scales), what + ": E8M0 scales"
        assert np.array_equal(g["mx_data"], codes), what + ": E4M3 codes"


def _first_inputs(seed, rows, hidden):
    rng = np.random.default_rng(seed)
    x = synth.chain_embedding(rows, hidden) if seed == 0 else \
        codecs.f64_to_bf16_bits(rng.normal(0, 1, (rows, hidden)))
    w = codecs.f64_to_bf16_bits(rng.normal(1, 0.1, hidden))
    return x, w


@pytest.mark.parametrize("rows,hidden,block", [(32, 7168, None), (128, 7168, 256), (5, 1056, 512),
                                               (1, 8, 128), (200, 4096, 128)])
def test_first_matches_oracle(rows, hidden, block):
    mx = hidden % 32 == 0
    say(f"case: first rows={rows} hidden={hidden} block={block} mxfp8={mx}")
    x, w = _first_inputs(rows, rows, hidden)
    h = handle_for(hidden, rows, block=block)
    got = {k: N(v) for k, v in binding.first(h, T(x), T(w), 1e-6, mxfp8=mx).items()}
    want = oracle.first(x, w, 1e-6, mxfp8=mx)
    assert np.array_equal(got["residual"], want["residual"]), "streams are x, bit for bit"
    _check_layer(got, want, f"first {rows}x{hidden}")
    assert h.errors() == 0


def test_first_then_coefficients_equal_the_chain_entry():
    """first() and a coefficient call on its streams: the chained step's entry."""
    rows, hidden = 16, 7168
    say(f"case: first + pre_coeffs rows={rows} hidden={hidden}")
    x, w = _first_inputs(0, rows, hidden)
    d = synth.pre_inputs(9, rows=rows, hidden=hidden)
    h = handle_for(hidden, rows)
    out = binding.first(h, T(x), T(w), 1e-6)
    got = binding.pre_coeffs(h, out["residual"], T(d["fn"]), T(d["scale"]), T(d["base"]),
                             d["rms_eps"], d["pre_eps"], d["sinkhorn_eps"], d["post_alpha"], 20)
    torch.cuda.synchronize()
    want = oracle.pre_coeffs(oracle.first(x, w, 1e-6)["residual"], d["fn"], d["scale"],
                             d["base"], d["rms_eps"], d["pre_eps"], d["sinkhorn_eps"],
                             d["post_alpha"], 20)
    for name, a, b in zip(("pre", "post", "comb"), got, want):
        a = N(a)
        assert np.all(np.abs(a - b) <= 1e-5 + 1e-5 * np.abs(b)), name


@pytest.mark.parametrize("rows,hidden,block", [(32, 7168, None), (128, 7168, 512), (7, 1056, 256),
                                               (300, 2048, 128)])
def test_collapse_norm_matches_oracle(rows, hidden, block):
    mx = hidden % 32 == 0
    say(f"case: collapse_norm rows={rows} hidden={hidden} block={block} mxfp8={mx}")
    d = synth.boundary_inputs(700 + rows, rows=rows, hidden=hidden, tp=1)
    h = handle_for(hidden, rows, block=block)
    got = {k: N(v) for k, v in binding.collapse_norm(h, T(d["residual"]), T(d["pre"]),
                                                      T(d["norm_weight"]), d["eps"],
                                                      mxfp8=mx).items()}
    want = oracle.collapse_norm(d["residual"], d["pre"], d["norm_weight"], d["eps"], mxfp8=mx)
    _check_layer(got, want, f"collapse_norm {rows}x{hidden}")
    assert h.errors() == 0


def test_collapse_norm_rounds_the_collapse_before_the_norm():
    """The row of the oracle pin, repeated over 8 elements: the GPU output is the one of the
    rounded collapse (0.75), not of the unrounded one (0.74609375)."""
    say("case: collapse_norm rounding point, hidden=8")
    pattern = np.array([1.453125, 0.90625] * 4)
    s = np.zeros((1, 4, 8))
    s[0, 0] = pattern
    s[0, 1, 0::2] = 2.0 ** -9
    s = codecs.f64_to_bf16_bits(s)
    pre = np.array([[1.0, 1.0, 0.0, 0.0]], np.float32)
    w = codecs.f64_to_bf16_bits(np.ones(8))
    h = handle_for(8, 1)
    got = codecs.bf16_bits_to_f64(N(binding.collapse_norm(h, T(s), T(pre), T(w), 0.0)["layer_input"]))
    assert np.array_equal(got, np.array([[1.203125, 0.75] * 4]))
    assert np.array_equal(got, codecs.bf16_bits_to_f64(
        oracle.collapse_norm(s, pre, w, 0.0)["layer_input"]))


def test_first_and_head_validation_on_a_device_handle():
    say("case: mhc_first / mhc_collapse_norm argument checks")
    lib = binding.load_library()
    R, H = 4, 1000  # hidden % 32 != 0: no MXFP8
    h = handle_for(H, R)
    x = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((H,), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros((R, 4, H), dtype=torch.bfloat16, device="cuda")
    li = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
    md = torch.zeros((R, H), dtype=torch.uint8, device="cuda")
    ms = torch.zeros((R, H // 32 + 1), dtype=torch.uint8, device="cuda")
    pre = torch.zeros((R, 4), dtype=torch.float32, device="cuda")
    p = binding._ptr
    # rows == 0 is an empty call, pointers unchecked
    assert lib.mhc_first(h.ptr, None, None, 0.0, 0, None, None, None, None, None) == 0
    assert lib.mhc_collapse_norm(h.ptr, None, None, None, 0.0, 0, None, None, None, None) == 0
    # missing outputs, a lone MXFP8 pointer, negative eps, too many rows, misalignment
    assert lib.mhc_first(h.ptr, p(x), p(w), 1e-6, R, p(s), None, None, None, None) == 1
    assert lib.mhc_first(h.ptr, p(x), p(w), 1e-6, R, p(s), p(li), p(md), None, None) == 1
    assert lib.mhc_first(h.ptr, p(x), p(w), -1.0, R, p(s), p(li), None, None, None) == 2
    assert lib.mhc_first(h.ptr, p(x), p(w), 1e-6, R + 1, p(s), p(li), None, None, None) == 4
    assert lib.mhc_first(h.ptr, p(x), p(w), 1e-6, R, p(s), p(li), p(md), p(ms), None) == 5
    xb = torch.zeros((R * H + 8,), dtype=torch.bfloat16, device="cuda")
    assert lib.mhc_first(h.ptr, binding._vp(xb.data_ptr() + 2), p(w), 1e-6, R, p(s), p(li),
                         None, None, None) == 3
    assert lib.mhc_collapse_norm(h.ptr, p(s), None, p(w), 1e-6, R, p(li), None, None, None) == 1
    assert lib.mhc_collapse_norm(h.ptr, p(s), p(pre), p(w), float("nan"), R, p(li), None, None,
                                 None) == 2
    assert lib.mhc_collapse_norm(h.ptr, p(s), p(pre), p(w), 1e-6, R, p(li), p(md), p(ms),
                                 None) == 5
    torch.cuda.synchronize()
