"""Pins of the oracle's boundary and coefficient path: closed forms, invariants, brute force.

CPU only. Each test is chosen so that a plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand, sum for mean, eps
outside the root, the wrong flatten order or scale group) fails at least one.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import codecs
from mhc_hyper_connection_02_amd import synth

bf = codecs.f64_to_bf16_bits
dec = codecs.bf16_bits_to_f64


def _tiny_boundary(seed=0, R=3, n=4, H=64, T=2):
    return synth.boundary_inputs(seed, rows=R, hidden=H, tp=T)


# ---------------------------------------------------------------------------
# a1 / a2: the sublayer output
# ---------------------------------------------------------------------------

def test_tp_reduce_order_invariant_and_single_slice_copy():
    d = _tiny_boundary(T=5)
    xp = d["x_partials"]
    a = oracle.tp_reduce(xp)
    b = oracle.tp_reduce(xp[::-1])
    assert np.array_equal(a, b)  # fp64 sums of 5 bf16 values are exact
    assert np.array_equal(oracle.tp_reduce(xp[:1]), dec(xp[0]))


def _golden_post_rounding(golden_dir):
    with open(os.path.join(golden_dir, "post_rounding_points.json")) as f:
        return json.load(f)


def _bits(hexes):
    return np.array([int(h, 16) for h in hexes], np.uint16)


def _flat_row(values, H=64):
    """bf16 bits of one row per value, every hidden element equal: [len(values), 1, H]."""
    return np.stack([np.full((1, H), int(bf(np.array(float(v)))), np.uint16) for v in values])


def test_tp_reduce_hand_derived_sums(golden_dir):
    """The slices are summed, not averaged (boundary page, module docstring): exact dyadic
    sums of two and three slices, hand-derived in the fixture."""
    g = _golden_post_rounding(golden_dir)
    for case in g["cases"]:
        parts = [eval(e, {}) for e in case["partials_expr"]]  # noqa: S307 (fixture literals)
        xp = _flat_row(parts)
        got = oracle.tp_reduce(xp)
        assert got.shape == (1, 64)
        assert np.all(got == eval(case["x_expr"], {})), case["name"]  # noqa: S307


def test_post_reads_the_bf16_rounded_sum_hand_derived(golden_dir):
    """D3: the new streams are bf16(post * bf16(x)) with x the exact sum of the slices, on
    inputs where skipping the rounding of x, or a mean instead of the sum, changes output
    bits (boundary page, Boundaries.post_only: the post kernel reads the reduced bf16
    tensor). Expected streams are the fixture's hand-derived bits."""
    g = _golden_post_rounding(golden_dir)
    n, H = 4, 64
    rng = np.random.default_rng(5)
    for case in g["cases"]:
        parts = [eval(e, {}) for e in case["partials_expr"]]  # noqa: S307
        xp = _flat_row(parts, H)
        res = bf(rng.normal(0, 1, (1, n, H)))
        post = np.array([case["post"]], np.float32)
        comb = np.zeros((1, n, n), np.float32)
        want = _bits(case["stream_bits"])
        for out in (oracle.residual_only(xp, res, post, comb),
                    oracle.boundary(xp, res, post, comb, np.full((1, n), 0.25, np.float32),
                                    bf(np.ones(H)), 1e-6)["residual"]):
            assert np.array_equal(out[0], np.repeat(want[:, None], H, axis=1)), case["name"]
        # the fixture's alternatives are real alternatives: each slip changes some stream
        assert not np.array_equal(_bits(case["if_mean_bits"]), want)
        if case["partials_expr"] != ["1.5", "2.25", "-0.75"]:
            assert not np.array_equal(_bits(case["if_unrounded_bits"]), want)
    for case in g["finalize_cases"]:
        sh = np.full((1, H), int(bf(np.array(eval(case["shared_expr"], {})))), np.uint16)  # noqa: S307
        gg = np.full((1, H), int(bf(np.array(eval(case["g_expr"], {})))), np.uint16)  # noqa: S307
        w = np.array([[case["w"]]], np.float32)
        idx = np.array([0], np.int32)
        res = bf(rng.normal(0, 1, (1, n, H)))
        post = np.array([case["post"]], np.float32)
        out = oracle.finalize(gg, w, idx, sh, res, post, np.zeros((1, n, n), np.float32), None,
                              None, 0.0)["residual"]
        want = _bits(case["stream_bits"])
        assert np.array_equal(out[0], np.repeat(want[:, None], H, axis=1)), case["name"]


def test_finalize_sum_brute_force():
    d = synth.finalize_inputs(1, rows=3, hidden=64, top_k=2)
    g, w, idx, sh = (d["gemm2_permuted"], d["expert_weights"],
                     d["expanded_idx_to_permuted_idx"], d["shared_output"])
    got = oracle.moe_finalize_sum(g, w, idx, sh)
    gv, shv = dec(g), dec(sh)
    for r in range(3):
        for h in range(64):
            acc = shv[r, h]
            for k in range(2):
                acc += float(w[r, k]) * gv[int(idx[r * 2 + k]), h]
            assert got[r, h] == pytest.approx(acc, rel=1e-15, abs=1e-300)


def test_finalize_one_hot_gather_is_bit_exact():
    """One-hot weights, zero shared output, comb = 0, post = 1: the streams are g[idx] exactly."""
    R, K, H, n = 4, 3, 96, 4
    d = synth.finalize_inputs(2, rows=R, hidden=H, top_k=K)
    rng = np.random.default_rng(0)
    pick = rng.integers(0, K, size=R)
    w = np.zeros((R, K), np.float32)
    w[np.arange(R), pick] = 1.0
    comb = np.zeros((R, n, n), np.float32)
    post = np.ones((R, n), np.float32)
    out = oracle.finalize(d["gemm2_permuted"], w, d["expanded_idx_to_permuted_idx"],
                          np.zeros((R, H), np.uint16), d["residual"], post, comb, None, None, 0.0)
    idx = d["expanded_idx_to_permuted_idx"]
    for r in range(R):
        want = d["gemm2_permuted"][idx[r * K + pick[r]]]
        for i in range(n):
            assert np.array_equal(out["residual"][r, i], want)


def test_finalize_out_of_range_index_contributes_nothing():
    d = synth.finalize_inputs(3, rows=2, hidden=32, top_k=2)
    idx = d["expanded_idx_to_permuted_idx"].copy()
    idx[1] = -1
    idx[2] = 10_000
    got = oracle.moe_finalize_sum(d["gemm2_permuted"], d["expert_weights"], idx, d["shared_output"])
    g, w, sh = dec(d["gemm2_permuted"]), d["expert_weights"].astype(np.float64), dec(d["shared_output"])
    want0 = sh[0] + w[0, 0] * g[idx[0]]
    want1 = sh[1] + w[1, 1] * g[idx[3]]
    assert np.allclose(got[0], want0, rtol=1e-15) and np.allclose(got[1], want1, rtol=1e-15)


# ---------------------------------------------------------------------------
# a3: the mHC post
# ---------------------------------------------------------------------------

def test_post_identity_comb_zero_post_is_identity():
    d = _tiny_boundary()
    R, n = d["post"].shape
    eye = np.broadcast_to(np.eye(n, dtype=np.float32), (R, n, n)).copy()
    out = oracle.boundary(d["x_partials"], d["residual"], np.zeros((R, n), np.float32), eye,
                          None, None, 0.0)
    assert np.array_equal(out["residual"], d["residual"])


def test_post_permutation_comb_moves_streams():
    """comb[r,i,j] = [j == pi(i)] sends input stream pi(i) to output stream i (bit-exact)."""
    d = _tiny_boundary()
    R, n = d["post"].shape
    pi = np.array([2, 0, 3, 1])  # not an involution: a transposed comb gives pi^-1 instead
    comb = np.zeros((R, n, n), np.float32)
    comb[:, np.arange(n), pi] = 1.0
    out = oracle.boundary(d["x_partials"], d["residual"], np.zeros((R, n), np.float32), comb,
                          None, None, 0.0)
    for i in range(n):
        assert np.array_equal(out["residual"][:, i], d["residual"][:, pi[i]])


def test_post_adds_post_times_rounded_x():
    d = _tiny_boundary()
    R, n = d["post"].shape
    post = np.tile(np.array([1.0, 2.0, -0.5, 0.25], np.float32), (R, 1))
    out = oracle.boundary(d["x_partials"], d["residual"], post, np.zeros((R, n, n), np.float32),
                          None, None, 0.0)
    x = dec(bf(oracle.tp_reduce(d["x_partials"])))  # x is rounded to bf16 first
    for i in range(n):
        assert np.array_equal(out["residual"][:, i], bf(post[0, i] * x))


def test_post_doubly_stochastic_conserves_stream_sum():
    d = _tiny_boundary(H=256)
    R, n = d["post"].shape
    out = oracle.boundary(d["x_partials"], d["residual"], np.zeros((R, n), np.float32), d["comb"],
                          None, None, 0.0)
    s_in = dec(d["residual"]).sum(axis=1)
    s_out = dec(out["residual"]).sum(axis=1)
    bound = n * 2.0 ** -8 * np.abs(dec(out["residual"])).max(axis=1) + 1e-6 * np.abs(s_in).max()
    assert np.all(np.abs(s_in - s_out) <= bound)


def test_post_uniform_comb_gives_stream_mean():
    d = _tiny_boundary()
    R, n = d["post"].shape
    comb = np.full((R, n, n), 1.0 / n, np.float32)  # 0.25 is exact
    out = oracle.boundary(d["x_partials"], d["residual"], np.zeros((R, n), np.float32), comb,
                          None, None, 0.0)
    m = oracle.collapse_mean(d["residual"])
    for i in range(n):
        assert np.array_equal(out["residual"][:, i], m)


# ---------------------------------------------------------------------------
# a4 / a5: collapse and RMSNorm
# ---------------------------------------------------------------------------

def test_collapse_unit_pre_selects_stream():
    d = _tiny_boundary()
    R, n = d["pre"].shape
    for k in range(n):
        pre = np.zeros((R, n), np.float32)
        pre[:, k] = 1.0
        assert np.array_equal(oracle.collapse(d["residual"], pre), dec(d["residual"][:, k]))


def test_rmsnorm_closed_forms():
    H = 64
    alt = np.where(np.arange(H) % 2 == 0, 1.0, -1.0)[None, :]
    one = bf(np.ones(H))
    # mean(y^2) = 1, eps = 3: out = +-1/sqrt(4) = +-0.5 (pins eps inside the root, mean not sum)
    assert np.array_equal(dec(oracle.rms_norm(alt, one, 3.0)), 0.5 * alt)
    # scale invariance without eps: c * alt -> +-1 for any c > 0
    assert np.array_equal(dec(oracle.rms_norm(37.5 * alt, one, 0.0)), alt)
    # the weight multiplies after normalizing
    two = bf(np.full(H, 2.0))
    assert np.array_equal(dec(oracle.rms_norm(alt, two, 0.0)), 2 * alt)
    # a constant row c with eps: c / sqrt(c^2 + eps)
    c, eps = 0.75, 0.4375  # c^2 + eps = 1
    got = dec(oracle.rms_norm(np.full((1, H), c), one, eps))
    assert np.array_equal(got, np.full((1, H), c))


def test_identity_premix_selects_stream_zero_rms_normed():
    """comb = I, post = 0, pre = e0: streams unchanged, layer input = RMSNorm(stream 0)."""
    R, n, H = 2, 4, 64
    rng = np.random.default_rng(11)
    res = bf(rng.normal(size=(R, n, H)))
    alt = np.where(np.arange(H) % 2 == 0, 1.0, -1.0)
    res[:, 0] = bf(np.stack([3.0 * alt, -0.5 * alt]))  # RMS 3 and 0.5: closed-form output +-1, -+1
    eye = np.broadcast_to(np.eye(n, dtype=np.float32), (R, n, n)).copy()
    pre = np.zeros((R, n), np.float32)
    pre[:, 0] = 1.0
    xp = bf(rng.normal(size=(1, R, H)))
    out = oracle.boundary(xp, res, np.zeros((R, n), np.float32), eye, pre, bf(np.ones(H)), 0.0)
    assert np.array_equal(out["residual"], res)
    assert np.array_equal(dec(out["layer_input"]), np.stack([alt, -alt]))


def test_layer_input_scale_invariance_of_premix():
    d = _tiny_boundary()
    a = oracle.boundary(d["x_partials"], d["residual"], d["post"], d["comb"], d["pre"],
                        d["norm_weight"], 0.0)
    b = oracle.boundary(d["x_partials"], d["residual"], d["post"], d["comb"], 4.0 * d["pre"],
                        d["norm_weight"], 0.0)
    assert np.array_equal(a["layer_input"], b["layer_input"])


# ---------------------------------------------------------------------------
# The first layer's entry and the head
# ---------------------------------------------------------------------------

def test_first_broadcasts_and_normalizes_the_embedding():
    """Streams: x in every stream, bit for bit. Layer input: closed forms of RMSNorm(x)
    (rows of +-c normalize to +-1 without eps, whatever c), equal to the boundary's layer
    input with comb = I, post = 0, pre = e0 on those streams, and MXFP8 of it."""
    R, H = 3, 64
    alt = np.where(np.arange(H) % 2 == 0, 1.0, -1.0)
    x = bf(np.stack([2.5 * alt, -0.125 * alt, 96.0 * alt]))
    w = bf(np.ones(H))
    out = oracle.first(x, w, 0.0, mxfp8=True)
    assert out["residual"].shape == (R, 4, H)
    for i in range(4):
        assert np.array_equal(out["residual"][:, i], x)
    assert np.array_equal(dec(out["layer_input"]), np.stack([alt, -alt, alt]))
    codes, scales = codecs.mxfp8_quantize(out["layer_input"])
    assert np.array_equal(out["mx_data"], codes) and np.array_equal(out["mx_scale"], scales)
    rng = np.random.default_rng(5)
    x = bf(rng.normal(0, 1, (R, H)))
    w = bf(rng.normal(1, 0.1, H))
    eye = np.broadcast_to(np.eye(4, dtype=np.float32), (R, 4, 4)).copy()
    pre = np.zeros((R, 4), np.float32)
    pre[:, 0] = 1.0
    b = oracle.boundary(bf(np.zeros((1, R, H))), np.repeat(x[:, None, :], 4, axis=1),
                        np.zeros((R, 4), np.float32), eye, pre, w, 1e-6)
    assert np.array_equal(oracle.first(x, w, 1e-6)["layer_input"], b["layer_input"])


def test_collapse_norm_closed_forms_and_invariances():
    """Constant streams c_j: y = sum_j pre_j c_j per row, normalized to sign(y) * w without
    eps; a power-of-two scale of every stream changes nothing (eps = 0); pre = e0 reduces
    the head to the first layer's normalization of stream 0."""
    R, H = 2, 32
    c = np.array([[1.0, -2.0, 0.5, 4.0], [-3.0, 1.0, 1.0, -1.0]])
    s = bf(np.repeat(c[:, :, None], H, axis=2))
    pre = np.array([[0.25, 0.5, 1.0, 0.125], [1.0, 0.5, 0.5, 2.0]], np.float32)
    w = bf(np.linspace(0.5, 1.5, H))
    y = (pre.astype(np.float64) * c).sum(axis=1)          # 0.25, -4.0
    got = dec(oracle.collapse_norm(s, pre, w, 0.0)["layer_input"])
    assert np.array_equal(got, np.sign(y)[:, None] * dec(w)[None, :])
    rng = np.random.default_rng(6)
    s = bf(rng.normal(0, 1, (3, 4, H)))
    pre = rng.uniform(0.1, 1.0, (3, 4)).astype(np.float32)
    a = oracle.collapse_norm(s, pre, w, 0.0, mxfp8=True)
    b = oracle.collapse_norm(bf(dec(s) * 2.0 ** -7), pre, w, 0.0, mxfp8=True)
    for k in a:
        assert np.array_equal(a[k], b[k])
    e0 = np.zeros((3, 4), np.float32)
    e0[:, 0] = 1.0
    assert np.array_equal(oracle.collapse_norm(s, e0, w, 1e-6)["layer_input"],
                          oracle.first(s[:, 0], w, 1e-6)["layer_input"])


def test_collapse_norm_rounds_the_collapse_once_before_the_norm():
    """y = [1.453125 + 2^-9, 0.90625] is not a bf16 number; the head normalizes its bf16
    rounding [1.453125, 0.90625] (ties to even), which decides the second output: 0.75,
    where normalizing the unrounded y would give 0.74609375 (worked out by hand: mean(y^2)
    = (1.453125^2 + 0.90625^2) / 2 = 1.4664306640625, and 0.90625 / sqrt of that
    = 0.74836..., which rounds to 0.75; with the unrounded y it is 0.74772... -> 0.74609375)."""
    s = bf(np.array([[[1.453125, 0.90625], [2.0 ** -9, 0.0], [0.0, 0.0], [0.0, 0.0]]]))
    pre = np.array([[1.0, 1.0, 0.0, 0.0]], np.float32)
    w = bf(np.ones(2))
    got = dec(oracle.collapse_norm(s, pre, w, 0.0)["layer_input"])
    assert np.array_equal(got, np.array([[1.203125, 0.75]]))


def test_residual_only_streams_equal_full_boundary_streams():
    d = _tiny_boundary()
    full = oracle.boundary(d["x_partials"], d["residual"], d["post"], d["comb"], d["pre"],
                           d["norm_weight"], d["eps"])
    ro = oracle.residual_only(d["x_partials"], d["residual"], d["post"], d["comb"])
    assert np.array_equal(full["residual"], ro)
    assert set(full) == {"residual", "layer_input"}


def test_mxfp8_output_is_quantized_layer_input():
    d = synth.boundary_inputs(4, rows=2, hidden=128, tp=3)
    out = oracle.boundary(d["x_partials"], d["residual"], d["post"], d["comb"], d["pre"],
                          d["norm_weight"], d["eps"], mxfp8=True)
    codes, scales = codecs.mxfp8_quantize(out["layer_input"])
    assert np.array_equal(out["mx_data"], codes) and np.array_equal(out["mx_scale"], scales)
    assert out["mx_scale"].shape == (2, 4)


def test_collapse_mean_of_identical_streams():
    rng = np.random.default_rng(2)
    s = bf(rng.normal(size=(3, 1, 40)))
    s4 = np.repeat(s, 4, axis=1)
    assert np.array_equal(oracle.collapse_mean(s4), s[:, 0])


# ---------------------------------------------------------------------------
# a9 - a12: the coefficient path
# ---------------------------------------------------------------------------

def _golden_sinkhorn(golden_dir):
    with open(os.path.join(golden_dir, "sinkhorn_2x2.json")) as f:
        return json.load(f)


def test_sinkhorn_one_iteration_golden(golden_dir):
    g = _golden_sinkhorn(golden_dir)
    logits = np.log(np.array(g["matrix"], np.float64))
    got = oracle.sinkhorn(logits, 1, 0.0)
    want = np.array([[eval(v) for v in row] for row in g["one_iteration"]])
    assert np.allclose(got, want, rtol=1e-14, atol=0)


def test_sinkhorn_converges_to_2x2_closed_form(golden_dir):
    g = _golden_sinkhorn(golden_dir)
    p = eval(g["converged_p_expr"], {"__builtins__": {}}, {})
    got = oracle.sinkhorn(np.log(np.array(g["matrix"], np.float64)), 200, 0.0)
    assert np.allclose(got, [[p, 1 - p], [1 - p, p]], rtol=0, atol=1e-13)


def test_sinkhorn_shift_invariance():
    """Row shifts of the logits scale rows of exp(logits): the first (row) step removes them at
    any iteration count. Column shifts are removed only in the limit (the unique scaling)."""
    rng = np.random.default_rng(3)
    z = rng.normal(size=(4, 4))
    rows = rng.normal(size=(4, 1))
    cols = rng.normal(size=(1, 4))
    assert np.allclose(oracle.sinkhorn(z, 7, 0.0), oracle.sinkhorn(z + rows, 7, 0.0),
                       rtol=1e-12, atol=1e-14)
    assert np.allclose(oracle.sinkhorn(z, 500, 0.0), oracle.sinkhorn(z + rows + cols, 500, 0.0),
                       rtol=1e-10, atol=1e-12)


def test_sinkhorn_columns_after_every_call_rows_only_at_convergence():
    rng = np.random.default_rng(4)
    eps = 1e-6
    for _ in range(20):
        z = rng.normal(0, 2, size=(4, 4))
        for iters in (1, 3, 20):
            # a column whose mass was S before its step sums to S / (S + eps) after it:
            # never above 1, and within 2 eps of 1 once S is near 1 (a few iterations in)
            A = oracle.sinkhorn(z, iters, eps)
            assert np.all(A.sum(axis=0) <= 1 + 1e-15)
            assert np.allclose(oracle.sinkhorn(z, iters, 0.0).sum(axis=0), 1, rtol=0, atol=1e-15)
        A = oracle.sinkhorn(z, 20, eps)
        assert np.all(np.abs(A.sum(axis=0) - 1) <= 2 * eps)
        A = oracle.sinkhorn(z, 1000, eps)
        assert np.all(np.abs(A.sum(axis=1) - 1) <= 1e-5)
        assert np.all(np.abs(A.sum(axis=0) - 1) <= 2 * eps)
    # the last half-step is the column one: after one iteration rows are generally off
    A = oracle.sinkhorn(np.array([[0.0, 3.0], [1.0, 0.0]]), 1, 0.0)
    assert np.allclose(A.sum(axis=0), 1, atol=1e-15) and not np.allclose(A.sum(axis=1), 1, atol=1e-3)


def test_sinkhorn_equal_logits_uniform():
    A = oracle.sinkhorn(np.full((4, 4), 0.7), 20, 1e-6)
    assert np.all(np.abs(A - 0.25) <= 1e-6)


def _pre_case(R=3, n=4, H=32, seed=0):
    return synth.pre_inputs(seed, rows=R, hidden=H, n=n)


def _call_pre(d, **kw):
    args = dict(d)
    args.update(kw)
    return oracle.pre_coeffs(args["residual"], args["fn"], args["scale"], args["base"],
                             args["rms_eps"], args["pre_eps"], args["sinkhorn_eps"],
                             args["post_alpha"], args["sinkhorn_iters"])


def test_pre_zero_fn_zero_base_closed_form():
    d = _pre_case()
    R, n = 3, 4
    fn0 = np.zeros_like(d["fn"])
    pre, post, comb = _call_pre(d, fn=fn0, base=np.zeros(24, np.float32))
    assert np.allclose(pre, 0.5 + d["pre_eps"], rtol=0, atol=1e-15)
    assert np.allclose(post, 1.0, rtol=0, atol=1e-15)  # alpha * sigmoid(0) = 2 * 0.5
    assert np.all(np.abs(comb - 0.25) <= 1e-6)


def test_pre_base_only_closed_form_and_group_order():
    """fn = 0 gives l' = base: pre = sigmoid(base[0:n]) + eps, post = alpha * sigmoid(base[n:2n])."""
    d = _pre_case()
    n = 4
    base = np.zeros(24, np.float32)
    base[:n] = [0.0, math.log(3.0), -math.log(3.0), 2.0]
    base[n:2 * n] = [math.log(3.0), 0.0, 0.0, -1.0]
    pre, post, comb = _call_pre(d, fn=np.zeros_like(d["fn"]), base=base)
    b = base.astype(np.float64)
    assert np.allclose(pre[0], [0.5 + 1e-6, 0.75 + 1e-6, 0.25 + 1e-6, 1 / (1 + math.exp(-b[3])) + 1e-6],
                       rtol=0, atol=1e-7)
    assert np.allclose(post[0], [1.5, 1.0, 1.0, 2 / (1 + math.e)], rtol=0, atol=1e-7)


def test_pre_one_hot_fn_pins_flatten_order_rms_and_scale_groups():
    """fn with one 1 per column picks v[k_c]: l_c = inv * v[k_c], k = i*H + h (stream-major)."""
    R, n, H = 2, 4, 32
    d = _pre_case(R=R, n=n, H=H, seed=9)
    nc = 2 * n + n * n
    ks = [(c * 5 + 3) % (n * H) for c in range(nc)]
    fn = np.zeros((n * H, nc))
    for c, k in enumerate(ks):
        fn[k, c] = 1.0
    scale = np.array([2.0, 0.5, 1.5], np.float32)
    base = np.linspace(-0.2, 0.3, nc).astype(np.float32)
    pre, post, comb = _call_pre(d, fn=bf(fn), scale=scale, base=base, sinkhorn_iters=0)
    s = dec(d["residual"])
    for r in range(R):
        v = [s[r, k // H, k % H] for k in range(n * H)]  # stream-major flatten by hand
        inv = 1.0 / math.sqrt(sum(x * x for x in v) / (n * H) + d["rms_eps"])
        lp = [inv * v[ks[c]] * float(scale[0 if c < n else 1 if c < 2 * n else 2]) + float(base[c])
              for c in range(nc)]
        for i in range(n):
            assert pre[r, i] == pytest.approx(1 / (1 + math.exp(-lp[i])) + d["pre_eps"], abs=1e-13)
            assert post[r, i] == pytest.approx(2 / (1 + math.exp(-lp[n + i])), abs=1e-13)
        # zero Sinkhorn iterations leave exp(l' - rowmax): row i, column j is column 2n + n*i + j
        for i in range(n):
            row = [lp[2 * n + n * i + j] for j in range(n)]
            m = max(row)
            for j in range(n):
                assert comb[r, i, j] == pytest.approx(math.exp(row[j] - m), abs=1e-13)


def test_pre_rms_scale_invariance():
    d = _pre_case(seed=5)
    a = _call_pre(d, rms_eps=0.0)
    b = _call_pre(d, residual=bf(4.0 * dec(d["residual"])), rms_eps=0.0)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=1e-13, atol=1e-15)


def test_pre_ranges():
    d = _pre_case(R=6, seed=6)
    pre, post, comb = _call_pre(d)
    assert np.all(pre > d["pre_eps"]) and np.all(pre < 1 + d["pre_eps"])
    assert np.all(post > 0) and np.all(post < d["post_alpha"])
    assert np.all(comb >= 0)
    assert np.all(np.abs(comb.sum(axis=1) - 1) <= 2 * d["sinkhorn_eps"])  # column sums


# ---------------------------------------------------------------------------
# The chained step's plumbing
# ---------------------------------------------------------------------------

def test_decode_chain_uses_the_delayed_pre():
    rows, hidden, n = 4, 64, 4
    emb = synth.chain_embedding(rows, hidden)
    subs = [synth.chain_sublayer(L, ffn, rows=rows, hidden=hidden, tp=2, top_k=2)
            for L in range(2) for ffn in (False, True)]
    p = synth.chain_params()
    rec = []
    streams, mean = oracle.decode_chain(emb, subs, p["rms_eps"], p["hc_eps"], p["post_alpha"],
                                        p["sinkhorn_iters"], p["norm_eps"], record=rec)
    assert len(rec) == 1 + len(subs)
    for b in range(1, len(subs)):
        prev, cur = rec[b - 1], rec[b]
        want = oracle.rms_norm(oracle.collapse(cur["residual"], prev["pre"].astype(np.float32)),
                               subs[b]["norm_w"], p["norm_eps"])
        assert np.array_equal(cur["layer_input"], want)
        assert ("mx_data" in cur) == subs[b]["mxfp8"]
    assert "layer_input" not in rec[-1]
    assert np.array_equal(mean, oracle.collapse_mean(streams))
