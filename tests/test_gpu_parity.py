"""GPU parity: the HIP library through its C ABI against the oracle, on the same seeded inputs.

Run on an MI355X: ``python -u -m pytest -m gpu tests -x -v --timeout 120 --timeout-method thread``.
Each test prints its case before the first GPU call.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs
from mhc_hyper_connection_02_amd import binding, synth

from gpu_helpers import (T, N, say, assert_bf16_close, assert_f32_close, handle_for,
                         with_stated_comb, gpu_boundary, oracle_boundary, gpu_finalize,
                         oracle_finalize, compare_boundary_outputs)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# The workloads at their full sizes
# ---------------------------------------------------------------------------

def test_config0_tiny_boundary():
    say("case: config 0 boundary rows=4 hidden=1024 tp=2, comb = Sinkhorn(exp N(0,1))")
    d = with_stated_comb(synth.config(0), 1000)
    h = handle_for(1024, 4, tp=2)
    g = gpu_boundary(h, d)
    o = oracle_boundary(d)
    st = compare_boundary_outputs(g, o, "config 0")
    say(f"  {st}")
    assert set(g) == {"residual", "layer_input"}


def test_config1_decode_boundary_mxfp8_and_determinism():
    say("case: config 1 boundary rows=32 hidden=7168 tp=8 mxfp8, comb = Sinkhorn(exp N(0,1))")
    d = with_stated_comb(synth.config(1), 1001)
    h = handle_for(7168, 32, tp=8)
    g = gpu_boundary(h, d)
    o = oracle_boundary(d)
    st = compare_boundary_outputs(g, o, "config 1")
    say(f"  {st}")
    g2 = gpu_boundary(h, d)
    for k in g:
        assert np.array_equal(g[k], g2[k]), f"second run differs in {k}"


def test_config1_residual_only_equals_full_streams():
    say("case: config 1 residual-only rows=32 hidden=7168 tp=8, comb = Sinkhorn(exp N(0,1))")
    d = with_stated_comb(synth.config(1), 1001)
    h = handle_for(7168, 32, tp=8)
    ro = gpu_boundary(h, d, residual_only=True)
    full = gpu_boundary(h, d)
    o = oracle_boundary(d, residual_only=True)
    assert_bf16_close(ro["residual"], o["residual"], "config 1 residual-only")
    # both run the same lane code for the streams (two elements per lane, the same slice
    # and mix order): bit-identical
    assert np.array_equal(ro["residual"], full["residual"]), "residual-only vs full streams"
    assert h.errors() == 0


def test_config2_moe_finalize_mxfp8():
    say("case: config 2 finalize rows=64 top_k=8 hidden=7168 mxfp8, comb = Sinkhorn(exp N(0,1))")
    d = with_stated_comb(synth.config(2), 1002)
    h = handle_for(7168, 64, tp=1, top_k=8)
    g = gpu_finalize(h, d)
    o = oracle_finalize(d)
    st = compare_boundary_outputs(g, o, "config 2")
    say(f"  {st}")
    ro = gpu_finalize(h, d, pre=False)
    # the same lane code for the streams (elementwise arithmetic does not depend on how many
    # elements a lane holds): bit-identical
    assert np.array_equal(ro["residual"], g["residual"]), "finalize residual-only vs full"
    assert h.errors() == 0


def test_config3_pre_coeffs():
    say("case: config 3 pre_coeffs rows=64 hidden=7168")
    d = synth.config(3)
    h = handle_for(7168, 64)
    pre, post, comb = binding.pre_coeffs(h, T(d["residual"]), T(d["fn"]), T(d["scale"]),
                                         T(d["base"]), d["rms_eps"], d["pre_eps"],
                                         d["sinkhorn_eps"], d["post_alpha"], d["sinkhorn_iters"])
    torch.cuda.synchronize()
    op, oq, oc = oracle.pre_coeffs(d["residual"], d["fn"], d["scale"], d["base"], d["rms_eps"],
                                   d["pre_eps"], d["sinkhorn_eps"], d["post_alpha"],
                                   d["sinkhorn_iters"])
    e1 = assert_f32_close(N(pre), op, "pre")
    e2 = assert_f32_close(N(post), oq, "post")
    e3 = assert_f32_close(N(comb), oc, "comb")
    say(f"  max |err| pre {e1:.2e} post {e2:.2e} comb {e3:.2e}")
    # reported, not asserted: how far rows are from summing to 1 after 20 iterations
    say(f"  comb max |rowsum-1| {np.abs(N(comb).sum(axis=2) - 1).max():.2e}")


# ---------------------------------------------------------------------------
# Tiles, ragged tails and block sizes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,hidden,tp,block", [
    (1, 512, 1, 128), (5, 1056, 3, 128), (9, 2080, 8, 256), (17, 7168, 8, 512),
    (13, 3072, 5, 256), (8, 33 * 32, 2, 512), (3, 8 * 40, 4, 128),
    # slice counts past one group of eight: a full group and a ragged one, two full
    # groups, and the largest count a handle takes
    (6, 2080, 13, 256), (4, 1024, 16, 128), (3, 1024, 64, 128), (10, 7168, 24, 512),
])
def test_boundary_ragged(rows, hidden, tp, block):
    mx = hidden % 32 == 0
    say(f"case: boundary rows={rows} hidden={hidden} tp={tp} block={block} mxfp8={mx}")
    d = synth.boundary_inputs(100 + rows, rows=rows, hidden=hidden, tp=tp, mxfp8=mx)
    h = handle_for(hidden, rows, tp=tp, block=block)
    compare_boundary_outputs(gpu_boundary(h, d), oracle_boundary(d), f"ragged {rows}x{hidden}")


@pytest.mark.parametrize("rows,hidden,tp", [
    (1, 512, 1), (5, 1056, 3), (13, 3072, 13), (3, 8 * 40, 16), (9, 2080, 8), (40, 7168, 8),
])
def test_residual_only_ragged(rows, hidden, tp):
    """The residual-only kernel (no layer input) on ragged shapes: one partly idle chunk
    (hidden 320), a ragged last chunk, ragged slice groups; its streams match the oracle and
    are bit-identical to a full call's on the same inputs."""
    say(f"case: residual-only rows={rows} hidden={hidden} tp={tp}")
    d = synth.boundary_inputs(150 + rows, rows=rows, hidden=hidden, tp=tp, mxfp8=False)
    h = handle_for(hidden, rows, tp=tp)
    ro = gpu_boundary(h, d, residual_only=True)
    assert_bf16_close(ro["residual"], oracle_boundary(d, residual_only=True)["residual"],
                      f"residual-only {rows}x{hidden}")
    full = gpu_boundary(h, d)
    assert np.array_equal(ro["residual"], full["residual"]), "residual-only vs full streams"
    assert h.errors() == 0


@pytest.mark.parametrize("rows,hidden,top_k", [(7, 1056, 3), (4, 2048, 12), (33, 7168, 8)])
def test_finalize_residual_only_ragged(rows, hidden, top_k):
    say(f"case: finalize residual-only rows={rows} hidden={hidden} top_k={top_k}")
    d = synth.finalize_inputs(250 + rows, rows=rows, hidden=hidden, top_k=top_k, mxfp8=False)
    h = handle_for(hidden, rows, tp=1, top_k=top_k)
    ro = gpu_finalize(h, d, pre=False)
    assert_bf16_close(ro["residual"], oracle_finalize(d, pre=False)["residual"],
                      f"finalize residual-only {rows}x{hidden}")
    assert np.array_equal(ro["residual"], gpu_finalize(h, d)["residual"])
    assert h.errors() == 0


@pytest.mark.parametrize("rows,hidden,top_k,block", [
    (1, 512, 1, 128), (7, 1056, 3, 256), (20, 7168, 8, 512), (4, 2048, 12, 256),
])
def test_finalize_ragged(rows, hidden, top_k, block):
    say(f"case: finalize rows={rows} hidden={hidden} top_k={top_k} block={block}")
    d = synth.finalize_inputs(200 + rows, rows=rows, hidden=hidden, top_k=top_k,
                              mxfp8=hidden % 32 == 0)
    h = handle_for(hidden, rows, tp=1, top_k=top_k, block=block)
    compare_boundary_outputs(gpu_finalize(h, d), oracle_finalize(d), f"finalize {rows}x{hidden}")


@pytest.mark.parametrize("rows,hidden,iters", [(1, 256, 20), (17, 1024, 20), (128, 7168, 20),
                                               (5, 7168, 0), (3, 96, 1)])
def test_pre_coeffs_ragged(rows, hidden, iters):
    say(f"case: pre_coeffs rows={rows} hidden={hidden} iters={iters}")
    d = synth.pre_inputs(300 + rows, rows=rows, hidden=hidden)
    h = handle_for(hidden, rows)
    got = binding.pre_coeffs(h, T(d["residual"]), T(d["fn"]), T(d["scale"]), T(d["base"]),
                             d["rms_eps"], d["pre_eps"], d["sinkhorn_eps"], d["post_alpha"], iters)
    torch.cuda.synchronize()
    want = oracle.pre_coeffs(d["residual"], d["fn"], d["scale"], d["base"], d["rms_eps"],
                             d["pre_eps"], d["sinkhorn_eps"], d["post_alpha"], iters)
    for name, a, b in zip(("pre", "post", "comb"), got, want):
        assert_f32_close(N(a), b, f"{name} rows={rows} hidden={hidden}")


# The split-K kernel of the coefficient call is compiled for 1..8 k steps per wave, picked at
# launch from the split count (about 256 workgroups over the 16-row blocks, each slice at
# most 32 steps of 32 k). These shapes reach each of the eight, with ragged row blocks and,
# where the split count does not divide the steps, a ragged last slice.
@pytest.mark.parametrize("steps_per_wave,rows,hidden", [
    (1, 1, 256), (2, 1, 10240), (3, 17, 10240), (4, 33, 8192), (5, 33, 12288),
    (6, 65, 8192), (7, 65, 10240), (8, 65, 12288)])
def test_pre_coeffs_every_split_k_width(steps_per_wave, rows, hidden):
    say(f"case: pre_coeffs rows={rows} hidden={hidden} ({steps_per_wave} k steps per wave)")
    d = synth.pre_inputs(400 + steps_per_wave, rows=rows, hidden=hidden)
    h = handle_for(hidden, rows)
    got = _pre_call(h, d)
    for name, a, b in zip(("pre", "post", "comb"), got, _pre_oracle(d)):
        assert_f32_close(a, b, f"{name} rows={rows} hidden={hidden}")


def _pre_call(h, d, iters=None):
    it = d["sinkhorn_iters"] if iters is None else iters
    got = binding.pre_coeffs(h, T(d["residual"]), T(d["fn"]), T(d["scale"]), T(d["base"]),
                             d["rms_eps"], d["pre_eps"], d["sinkhorn_eps"], d["post_alpha"], it)
    torch.cuda.synchronize()
    return [N(a) for a in got]


def _pre_oracle(d, iters=None):
    it = d["sinkhorn_iters"] if iters is None else iters
    return oracle.pre_coeffs(d["residual"], d["fn"], d["scale"], d["base"], d["rms_eps"],
                             d["pre_eps"], d["sinkhorn_eps"], d["post_alpha"], it)


def test_pre_coeffs_row_counts_change_between_calls():
    """One handle, calls whose split layouts differ (16-row tiles x k-splits: 4x64, 8x32,
    1x256, 19x8) in one scratch area; a repeated call is bit-identical."""
    say("case: pre_coeffs rows 64, 128, 5, 300, 64 on one handle, hidden=7168")
    h = handle_for(7168, 300)
    first = None
    for rows in (64, 128, 5, 300, 64):
        d = synth.pre_inputs(500 + rows, rows=rows, hidden=7168)
        d["sinkhorn_iters"] = 20
        got = _pre_call(h, d)
        for name, a, b in zip(("pre", "post", "comb"), got, _pre_oracle(d)):
            assert_f32_close(a, b, f"{name} rows={rows}")
        if rows == 64:
            if first is None:
                first = got
            else:  # the same call again: bit-identical (fixed split order)
                for a, b in zip(got, first):
                    assert np.array_equal(a, b)
    assert h.errors() == 0


@pytest.mark.parametrize("rows,hidden", [(4096, 512), (1000, 7168)])
def test_pre_coeffs_large_row_counts(rows, hidden):
    say(f"case: pre_coeffs rows={rows} hidden={hidden}")
    d = synth.pre_inputs(600 + rows, rows=rows, hidden=hidden)
    h = handle_for(hidden, rows)
    for name, a, b in zip(("pre", "post", "comb"), _pre_call(h, d, 20), _pre_oracle(d, 20)):
        assert_f32_close(a, b, f"{name} rows={rows} hidden={hidden}")
    assert h.errors() == 0


def test_block_sizes_agree():
    say("case: config 1 at block 128 / 256 / 512")
    d = synth.config(1)
    outs = []
    for block in (128, 256, 512):
        h = handle_for(7168, 32, tp=8, block=block)
        outs.append(gpu_boundary(h, d))
    for o in outs[1:]:
        assert np.array_equal(o["residual"], outs[0]["residual"])  # per-element arithmetic
        assert_bf16_close(o["layer_input"], outs[0]["layer_input"], "block layer input")


# ---------------------------------------------------------------------------
# Special cases with exact answers
# ---------------------------------------------------------------------------

def test_finalize_one_hot_gather_bit_exact():
    R, K, H = 16, 8, 7168
    say(f"case: finalize one-hot gather rows={R} top_k={K} hidden={H}")
    d = synth.finalize_inputs(7, rows=R, hidden=H, top_k=K)
    rng = np.random.default_rng(1)
    pick = rng.integers(0, K, size=R)
    w = np.zeros((R, K), np.float32)
    w[np.arange(R), pick] = 1.0
    d["expert_weights"] = w
    d["shared_output"] = np.zeros((R, H), np.uint16)
    d["comb"] = np.zeros((R, 4, 4), np.float32)
    d["post"] = np.ones((R, 4), np.float32)
    h = handle_for(H, R, tp=1, top_k=K)
    g = gpu_finalize(h, d, mxfp8=False)
    idx = d["expanded_idx_to_permuted_idx"]
    for r in range(R):
        want = d["gemm2_permuted"][idx[r * K + pick[r]]]
        for i in range(4):
            assert np.array_equal(g["residual"][r, i], want), (r, i)


def test_finalize_out_of_range_indices_are_skipped():
    R, K, H = 6, 4, 1024
    say(f"case: finalize with out-of-range indices rows={R} top_k={K}")
    d = synth.finalize_inputs(8, rows=R, hidden=H, top_k=K)
    idx = d["expanded_idx_to_permuted_idx"].copy()
    idx[[1, 6, 11]] = [-1, R * K, 1 << 30]
    d["expanded_idx_to_permuted_idx"] = idx
    h = handle_for(H, R, tp=1, top_k=K)
    compare_boundary_outputs(gpu_finalize(h, d), oracle_finalize(d), "skip indices")


def test_identity_premix_selects_stream_zero():
    R, H = 8, 2048
    say("case: comb = I, post = 0, pre = e0")
    d = synth.boundary_inputs(9, rows=R, hidden=H, tp=2, mxfp8=True)
    d["comb"] = np.broadcast_to(np.eye(4, dtype=np.float32), (R, 4, 4)).copy()
    d["post"] = np.zeros((R, 4), np.float32)
    pre = np.zeros((R, 4), np.float32)
    pre[:, 0] = 1.0
    d["pre"] = pre
    h = handle_for(H, R, tp=2)
    g = gpu_boundary(h, d)
    assert np.array_equal(g["residual"], d["residual"])
    want = oracle.rms_norm(codecs.bf16_bits_to_f64(d["residual"][:, 0]), d["norm_weight"], d["eps"])
    assert_bf16_close(g["layer_input"], want, "RMSNorm(stream 0)")


def test_in_place_streams_and_zero_layer_input():
    R, H = 4, 1024
    say("case: residual_out aliases residual; zero streams give a zero MXFP8 block")
    d = synth.boundary_inputs(10, rows=R, hidden=H, tp=2, mxfp8=True)
    d["residual"][1] = 0
    d["x_partials"][:, 1] = 0
    o = oracle_boundary(d)
    h = handle_for(H, R, tp=2)
    res = T(d["residual"])
    out = binding.boundary(h, T(d["x_partials"]), res, T(d["post"]), T(d["comb"]), T(d["pre"]),
                           T(d["norm_weight"]), d["eps"], mxfp8=True, residual_out=res)
    torch.cuda.synchronize()
    assert out["residual"].data_ptr() == res.data_ptr()
    g = {k: N(v) for k, v in out.items()}
    compare_boundary_outputs(g, o, "in place")
    assert np.all(g["mx_scale"][1] == 0) and np.all(g["mx_data"][1] == 0)
    assert np.all(g["layer_input"][1] == 0)


def test_zero_rows_is_a_noop():
    say("case: rows = 0")
    h = handle_for(1024, 4)
    lib = binding.load_library()
    assert lib.mhc_boundary(h.ptr, None, 1, None, None, None, None, None, 0.0, 0, None, None,
                            None, None, None) == 0
    assert lib.mhc_finalize(h.ptr, None, 1, None, None, None, None, None, None, None, None, 0.0, 0,
                            None, None, None, None, None) == 0
    assert lib.mhc_pre_coeffs(h.ptr, None, None, None, None, 0.0, 0.0, 0.0, 2.0, 20, 0, None,
                              None, None, None) == 0


def test_max_rows_and_tp_limits():
    say("case: rows == max_rows, tp == max_tp; and one above each (rejected, nothing launched)")
    R, H, TP = 24, 1024, 3
    d = synth.boundary_inputs(11, rows=R, hidden=H, tp=TP)
    h = handle_for(H, R, tp=TP)
    compare_boundary_outputs(gpu_boundary(h, d), oracle_boundary(d), "max rows")
    small = handle_for(H, R - 1, tp=TP)
    with pytest.raises(binding.MhcValueError):
        gpu_boundary(small, d)
    d2 = synth.boundary_inputs(12, rows=4, hidden=H, tp=TP + 1)
    with pytest.raises(binding.MhcValueError):
        gpu_boundary(handle_for(H, 4, tp=TP), d2)


def test_validation_on_a_device_handle():
    say("case: argument validation (no kernel is launched for any of these)")
    lib = binding.load_library()
    H, R = 1024, 4
    h = handle_for(H, R, tp=2)
    x = torch.zeros((2, R, H), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros((R, 4, H), dtype=torch.bfloat16, device="cuda")
    f4 = torch.zeros((R, 4), dtype=torch.float32, device="cuda")
    f16 = torch.zeros((R, 4, 4), dtype=torch.float32, device="cuda")
    w = torch.zeros((H,), dtype=torch.bfloat16, device="cuda")
    li = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
    md = torch.zeros((R, H), dtype=torch.uint8, device="cuda")
    ms = torch.zeros((R, H // 32), dtype=torch.uint8, device="cuda")
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731

    def call(**kw):
        a = dict(x=x, tp=2, s=s, post=f4, comb=f16, pre=f4, w=w, eps=1e-6, rows=R, out=s, li=li,
                 md=md, ms=ms)
        a.update(kw)
        return lib.mhc_boundary(h.ptr, p(a["x"]), a["tp"], p(a["s"]), p(a["post"]), p(a["comb"]),
                                p(a["pre"]), p(a["w"]), a["eps"], a["rows"], p(a["out"]),
                                p(a["li"]), p(a["md"]), p(a["ms"]), None)

    assert call(rows=R + 1) == 4
    assert call(tp=3) == 4
    assert call(tp=0) == 2
    assert call(rows=-1) == 2
    assert call(x=None) == 1
    assert call(pre=None) == 1             # pre missing while norm weight / layer input given
    assert call(li=None) == 1
    assert call(ms=None) == 1              # MXFP8 outputs come in pairs
    assert call(pre=None, w=None, li=None) == 1  # MXFP8 needs pre
    assert call(eps=-1.0) == 2
    assert call(eps=float("nan")) == 2
    bad = torch.zeros((2 * R * H + 8,), dtype=torch.bfloat16, device="cuda")
    assert lib.mhc_boundary(h.ptr, bad.data_ptr() + 2, 2, p(s), p(f4), p(f16), p(f4), p(w), 1e-6,
                            R, p(s), p(li), p(md), p(ms), None) == 3
    assert lib.mhc_set_option(h.ptr, binding.MHC_OPT_BOUNDARY_BLOCK, 96) == 2
    assert lib.mhc_set_option(h.ptr, 77, 64) == 1
    h2 = binding.Handle(1000, 4, max_rows=R, max_tp=2)  # hidden % 32 != 0: no MXFP8
    x2 = torch.zeros((2, R, 1000), dtype=torch.bfloat16, device="cuda")
    s2 = torch.zeros((R, 4, 1000), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((1000,), dtype=torch.bfloat16, device="cuda")
    li2 = torch.zeros((R, 1000), dtype=torch.bfloat16, device="cuda")
    assert lib.mhc_boundary(h2.ptr, p(x2), 2, p(s2), p(f4), p(f16), p(f4), p(w2), 1e-6, R, p(s2),
                            p(li2), p(md), p(ms), None) == 5
    assert lib.mhc_pre_coeffs(h.ptr, p(s), p(w), p(f4), p(f4), 1e-6, 1e-6, 1e-6, 2.0, 1001, R,
                              p(f4), p(f4), p(f16), None) == 2
    torch.cuda.synchronize()


def test_collapse_mean():
    R, H = 40, 7168
    say(f"case: collapse_mean rows={R} hidden={H}")
    d = synth.boundary_inputs(13, rows=R, hidden=H, tp=1)
    h = handle_for(H, R)
    g = N(binding.collapse_mean(h, T(d["residual"])))
    torch.cuda.synchronize()
    assert_bf16_close(g, oracle.collapse_mean(d["residual"]), "collapse mean")
    same = np.repeat(d["residual"][:, :1], 4, axis=1)
    assert np.array_equal(N(binding.collapse_mean(h, T(same))), d["residual"][:, 0])


def test_reset_then_reuse():
    say("case: mhc_reset between calls")
    d = synth.config(0)
    h = handle_for(1024, 4, tp=2)
    d3 = synth.pre_inputs(7, rows=4, hidden=1024)
    d3["sinkhorn_iters"] = 20
    a = gpu_boundary(h, d)
    pa = _pre_call(h, d3)
    h.reset()
    b = gpu_boundary(h, d)
    pb = _pre_call(h, d3)
    for k in a:
        assert np.array_equal(a[k], b[k])
    for x, y in zip(pa, pb):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# The row handoff: rounds, the error word, a bounded wait, graph replays
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,hidden,block", [(400, 7168, 128), (70, 32768, 256), (300, 4096, 512)])
def test_boundary_in_several_rounds(rows, hidden, block):
    say(f"case: boundary over several rounds rows={rows} hidden={hidden} block={block}")
    d = synth.boundary_inputs(400 + rows, rows=rows, hidden=hidden, tp=2, mxfp8=True)
    h = handle_for(hidden, rows, tp=2, block=block)
    compare_boundary_outputs(gpu_boundary(h, d), oracle_boundary(d), f"rounds {rows}x{hidden}")
    assert h.errors() == 0


def test_no_handoff_errors_on_normal_calls():
    say("case: error word after config 1 and config 2 calls")
    h = handle_for(7168, 64, tp=8, top_k=8)
    gpu_boundary(h, synth.config(1))
    gpu_finalize(h, synth.config(2))
    _pre_call(h, synth.config(3))
    assert h.errors() == 0


def _bf16_nan(bits):
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0)


def test_many_handoffs_in_a_graph_all_complete():
    """Thousands of row handoffs back to back (a graph of 400 config-1 boundary calls and
    400 finalize calls over rotating buffers, replayed 5 times, with the handle's default
    handoff scope): no wait gives up, and every call's outputs equal the same call run
    eagerly, bit for bit."""
    say("case: 4000 boundary and finalize calls graph-replayed, default handoff scope")
    d1 = synth.config(1)
    d2 = synth.config(2)
    h = handle_for(7168, 64, tp=8, top_k=8)
    want_b = gpu_boundary(h, d1)
    want_f = gpu_finalize(h, d2)
    inb = {k: T(d1[k]) for k in ("x_partials", "residual", "post", "comb", "pre", "norm_weight")}
    inf = {k: T(d2[k]) for k in ("gemm2_permuted", "expert_weights",
                                 "expanded_idx_to_permuted_idx", "shared_output", "residual",
                                 "post", "comb", "pre", "norm_weight")}
    nb = 4
    outs_b = [{"so": torch.empty_like(inb["residual"]),
               "li": torch.empty((32, 7168), dtype=torch.bfloat16, device="cuda"),
               "md": torch.empty((32, 7168), dtype=torch.uint8, device="cuda"),
               "ms": torch.empty((32, 224), dtype=torch.uint8, device="cuda")} for _ in range(nb)]
    outs_f = [{"so": torch.empty_like(inf["residual"]),
               "li": torch.empty((64, 7168), dtype=torch.bfloat16, device="cuda"),
               "md": torch.empty((64, 7168), dtype=torch.uint8, device="cuda"),
               "ms": torch.empty((64, 224), dtype=torch.uint8, device="cuda")} for _ in range(nb)]

    def calls():
        for i in range(400):
            o = outs_b[i % nb]
            binding.boundary(h, inb["x_partials"], inb["residual"], inb["post"], inb["comb"],
                             inb["pre"], inb["norm_weight"], d1["eps"], mxfp8=True,
                             residual_out=o["so"], layer_input_out=o["li"],
                             mx_out=(o["md"], o["ms"]))
            o = outs_f[i % nb]
            binding.finalize(h, inf["gemm2_permuted"], inf["expert_weights"],
                             inf["expanded_idx_to_permuted_idx"], inf["shared_output"],
                             inf["residual"], inf["post"], inf["comb"], inf["pre"],
                             inf["norm_weight"], d2["eps"], mxfp8=True, residual_out=o["so"],
                             layer_input_out=o["li"], mx_out=(o["md"], o["ms"]))

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(5):
        g.replay()
        torch.cuda.synchronize()
        for o in outs_b:
            assert np.array_equal(N(o["so"]), want_b["residual"])
            assert np.array_equal(N(o["li"]), want_b["layer_input"])
            assert np.array_equal(N(o["md"]), want_b["mx_data"])
            assert np.array_equal(N(o["ms"]), want_b["mx_scale"])
        for o in outs_f:
            assert np.array_equal(N(o["li"]), want_f["layer_input"])
            assert np.array_equal(N(o["ms"]), want_f["mx_scale"])
    assert h.errors() == 0, "a handoff wait gave up"


def test_row_handoff_scopes_give_identical_outputs():
    """MHC_OPT_ROW_HANDOFF changes only how a row's workgroups exchange their partial sums:
    through the L2 of the row's XCD or at device scope, the boundary (config 1 with MXFP8,
    a ragged 5 x 1056 call in two rounds), the finalize (config 2), the first layer's entry
    and the head give the same bits, the first two also matching the oracle, and no wait
    gives up. A value outside the enum is rejected."""
    say("case: row handoff through the XCD's L2 against device scope")
    d1 = with_stated_comb(synth.config(1), 1001)
    d2 = with_stated_comb(synth.config(2), 1002)
    dr = synth.boundary_inputs(7, rows=5, hidden=1056, tp=3)
    h = handle_for(7168, 64, tp=8, top_k=8)
    hr = handle_for(1056, 5, tp=3)
    hr.set_option(binding.MHC_OPT_BOUNDARY_BLOCK, 128)
    rng = np.random.default_rng(5)
    x = codecs.f64_to_bf16_bits(rng.normal(0, 1, (32, 7168)))
    w = codecs.f64_to_bf16_bits(rng.normal(1, 0.1, 7168))
    outs = {}
    for mode in (binding.MHC_HANDOFF_DEVICE, binding.MHC_HANDOFF_XCD):
        try:
            h.set_option(binding.MHC_OPT_ROW_HANDOFF, mode)
            hr.set_option(binding.MHC_OPT_ROW_HANDOFF, mode)
        except binding.MhcError:
            assert mode == binding.MHC_HANDOFF_XCD
            pytest.skip("this device does not deal workgroup ids to its XCDs round-robin")
        o = {"b": gpu_boundary(h, d1), "f": gpu_finalize(h, d2), "r": gpu_boundary(hr, dr),
             "first": {k: N(v) for k, v in binding.first(h, T(x), T(w), 1e-6, mxfp8=True).items()},
             "head": {k: N(v) for k, v in binding.collapse_norm(
                 h, T(d1["residual"]), T(d1["pre"]), T(d1["norm_weight"]), 1e-6,
                 mxfp8=True).items()}}
        torch.cuda.synchronize()
        assert h.errors() == 0 and hr.errors() == 0, f"handoff {mode}: a wait gave up"
        outs[mode] = o
    a, b = outs[binding.MHC_HANDOFF_DEVICE], outs[binding.MHC_HANDOFF_XCD]
    for call in a:
        for k in a[call]:
            assert np.array_equal(a[call][k], b[call][k]), f"{call}.{k} differs between scopes"
    compare_boundary_outputs(b["b"], oracle_boundary(d1), "config 1, XCD handoff")
    compare_boundary_outputs(b["f"], oracle_finalize(d2), "config 2, XCD handoff")
    with pytest.raises(binding.MhcValueError):
        h.set_option(binding.MHC_OPT_ROW_HANDOFF, 2)


def test_zero_spin_limit_poisons_and_reset_recovers():
    """A spin limit of 0 polls once, so waits give up (counted; nothing hangs, every kernel
    exits). The data shows it: where a wait gave up the layer input is NaN, its E4M3 codes the
    NaN code and its E8M0 scale 0xFF; elsewhere it is right; the streams never depend on a
    wait and stay right. A row whose wait gave up is marked: every later call (plain or fused)
    skips that row's waits and poisons those outputs; clearing the count (a full reset of the
    handoff state) restores exact results."""
    say("case: spin limit 0 on config 1, poisoned outputs, then clear/reset")
    d = synth.config(1)
    o = oracle_boundary(d)
    h = handle_for(7168, 32, tp=8)
    h.set_option(binding.MHC_OPT_SPIN_LIMIT, 0)
    n, tries = 0, 0
    while n == 0 and tries < 8:  # the spin limit comes from the host: each call ends normally
        g = gpu_boundary(h, d)
        n = h.errors()
        tries += 1
    say(f"  waits that gave up with limit 0: {n} (after {tries} calls)")
    assert n > 0
    li = g["layer_input"]
    nan = _bf16_nan(li)
    say(f"  layer-input elements poisoned: {int(nan.sum())} of {nan.size}")
    assert nan.any()
    assert_bf16_close(g["residual"], o["residual"], "streams with waits given up")
    ok = ~nan
    gv, ov = codecs.bf16_bits_to_f64(li)[ok], codecs.bf16_bits_to_f64(o["layer_input"])[ok]
    assert np.all(np.abs(gv - ov) <= 2e-2 + 1e-2 * np.abs(ov)), "unpoisoned layer input"
    blk_nan = nan.reshape(32, -1, 32).any(axis=2)
    assert np.all(g["mx_scale"][blk_nan] == 0xFF), "poisoned blocks' scale byte"
    assert np.all((g["mx_data"][nan] & 0x7F) == 0x7F), "poisoned elements' E4M3 codes"
    codes, scales = codecs.mxfp8_quantize(np.where(nan, 0, li).astype(np.uint16))
    clean = ~np.repeat(blk_nan, 32, axis=1)  # elements of blocks without a poisoned element
    assert np.array_equal(g["mx_scale"][~blk_nan], scales[~blk_nan])
    assert np.array_equal(g["mx_data"][clean], codes[clean])
    # the marks stay: later calls, with the default limit, poison every wait-dependent output
    # of the marked rows (plain and fused), and the streams stay right
    h.set_option(binding.MHC_OPT_SPIN_LIMIT, 1 << 20)
    bad_rows = nan.any(axis=1)
    say(f"  rows marked: {int(bad_rows.sum())} of {len(bad_rows)}")
    g2 = gpu_boundary(h, d)
    assert _bf16_nan(g2["layer_input"][bad_rows]).all()
    assert np.all(g2["mx_scale"][bad_rows] == 0xFF)
    assert_bf16_close(g2["residual"], o["residual"], "streams of a poisoned handle")
    p3 = synth.pre_inputs(3, rows=1, hidden=7168)
    nxt = {"fn": T(p3["fn"]), "scale": T(p3["scale"]), "base": T(p3["base"]),
           "rms_eps": p3["rms_eps"], "pre_eps": p3["pre_eps"], "sinkhorn_eps": p3["sinkhorn_eps"],
           "post_alpha": p3["post_alpha"], "sinkhorn_iters": p3["sinkhorn_iters"]}
    f = binding.boundary_coeffs(h, T(d["x_partials"]), T(d["residual"]), T(d["post"]),
                                T(d["comb"]), T(d["pre"]), T(d["norm_weight"]), d["eps"], nxt,
                                mxfp8=True)
    torch.cuda.synchronize()
    assert _bf16_nan(N(f["layer_input"])[bad_rows]).all(), "fused call: marked rows' layer input"
    for t in f["next"]:
        assert np.isnan(N(t)[bad_rows]).all(), "fused call: marked rows' next coefficients"
    assert_bf16_close(N(f["residual"]), o["residual"], "fused streams of a poisoned handle")
    # clearing the count re-zeroes the handoff state: exact again
    h.errors(clear=True)
    assert h.errors() == 0
    compare_boundary_outputs(gpu_boundary(h, d), o, "after clearing the count")
    h.set_option(binding.MHC_OPT_SPIN_LIMIT, 0)
    gpu_boundary(h, d)
    h.set_option(binding.MHC_OPT_SPIN_LIMIT, 1 << 20)
    h.reset()
    compare_boundary_outputs(gpu_boundary(h, d), o, "after reset")
    assert h.errors() == 0
    with pytest.raises(binding.MhcValueError):
        h.set_option(binding.MHC_OPT_SPIN_LIMIT, -1)


def test_graph_replays_match_eager():
    """One graph with a boundary, a finalize and a coefficient call, replayed three times with
    eager work and synchronizations between the replays; every replay equals the eager run."""
    say("case: HIP graph replays of boundary + finalize + pre_coeffs")
    d1, d2, d3 = synth.config(1), synth.config(2), synth.config(3)
    h = handle_for(7168, 64, tp=8, top_k=8)
    a = {k: T(v) for k, v in d1.items() if isinstance(v, np.ndarray)}
    b = {k: T(v) for k, v in d2.items() if isinstance(v, np.ndarray)}
    c = {k: T(v) for k, v in d3.items() if isinstance(v, np.ndarray)}

    def step():
        o1 = binding.boundary(h, a["x_partials"], a["residual"], a["post"], a["comb"], a["pre"],
                              a["norm_weight"], d1["eps"], mxfp8=True)
        o2 = binding.finalize(h, b["gemm2_permuted"], b["expert_weights"],
                              b["expanded_idx_to_permuted_idx"], b["shared_output"], b["residual"],
                              b["post"], b["comb"], b["pre"], b["norm_weight"], d2["eps"], mxfp8=True)
        o3 = binding.pre_coeffs(h, c["residual"], c["fn"], c["scale"], c["base"], d3["rms_eps"],
                                d3["pre_eps"], d3["sinkhorn_eps"], d3["post_alpha"],
                                d3["sinkhorn_iters"])
        return [o1["residual"], o1["layer_input"], o1["mx_data"], o1["mx_scale"], o2["residual"],
                o2["layer_input"], o2["mx_data"], o2["mx_scale"], *o3]

    eager = [N(t) for t in step()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    for rep in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, eager)):
            assert np.array_equal(N(t), e), f"replay {rep}: output {i} differs from eager"
        step()  # eager work between replays
        torch.cuda.synchronize()
    assert h.errors() == 0


@pytest.mark.parametrize("block", [128, 256, 512])
def test_block_sizes_match_oracle(block):
    """Every layer-input block size: configs 1 and 2 and a ragged shape against the oracle."""
    say(f"case: block={block}: config 1, config 2, rows=5 hidden=1056 tp=3")
    for d, fin in ((synth.config(1), False), (synth.config(2), True),
                   (synth.boundary_inputs(77, rows=5, hidden=1056, tp=3, mxfp8=True), False)):
        rows, _, hidden = d["residual"].shape
        h = handle_for(hidden, rows, tp=8, top_k=8)
        h.set_option(binding.MHC_OPT_BOUNDARY_BLOCK, block)
        if fin:
            compare_boundary_outputs(gpu_finalize(h, d), oracle_finalize(d), "lane finalize")
        else:
            compare_boundary_outputs(gpu_boundary(h, d), oracle_boundary(d), "lane boundary")
        assert h.errors() == 0
