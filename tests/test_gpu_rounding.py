"""Bit-exact GPU checks of the kernels' narrowing conversions on inputs built to sit at
rounding ties and format edges (both sides round to nearest even; expected values come
from the oracle).

- fp32 -> bf16 of the reduced sublayer output: partial slices a + b whose exact sum is a
  bf16 tie, or one step either side of it, pass through the mix unchanged (post = 1,
  comb = 0), so the new streams are exactly the rounded sums.
- bf16 -> E4M3 / E8M0: with every stream equal to a power of two c, comb = I and
  pre = e0, eps = 0, the RMS of the collapse is |c| exactly and the layer input is the
  norm weight itself; the weight's 32-element blocks are built from E4M3 ties, the
  subnormal range, signed zeros, the 448 edge and the [fraction > 0.75] scale rule.
"""

import numpy as np
import pytest

import oracle
from oracle import codecs
from mhc_hyper_connection_02_amd import binding

from gpu_helpers import N, T, handle_for, say

pytestmark = pytest.mark.gpu


def bf16_bits(sign, exp2, frac7):
    """bf16 bit patterns of (-1)^sign * (1 + frac7/128) * 2^exp2 (normal numbers)."""
    sign = np.asarray(sign, np.uint32)
    e = np.asarray(exp2, np.int64) + 127
    assert (e >= 1).all() and (e <= 254).all()
    return ((sign << 15) | (e.astype(np.uint32) << 7) | np.asarray(frac7, np.uint32)).astype(np.uint16)


def tie_partials(rng, rows, hidden):
    """Two slices a, b: a = +-(1 + m/128) 2^j; b = +-(half a bf16 ulp of a) times one of
    1 (a tie), 1 - 2^-8 (just below) or 1 + 2^-7 (just above), same sign as a or opposite."""
    shape = (rows, hidden)
    s = rng.integers(0, 2, shape)
    j = rng.integers(-12, 13, shape)
    m = rng.integers(0, 128, shape)
    a = bf16_bits(s, j, m)
    kind = rng.integers(0, 3, shape)
    sb = np.where(rng.random(shape) < 0.75, s, 1 - s)
    # half ulp of a is 2^(j-8); the three b magnitudes as bf16: 2^(j-8), (2 - 2^-7) 2^(j-9),
    # (1 + 2^-7) 2^(j-8)
    b = np.where(kind == 0, bf16_bits(sb, j - 8, 0),
                 np.where(kind == 1, bf16_bits(sb, j - 9, 127), bf16_bits(sb, j - 8, 1)))
    return np.stack([a, b]).astype(np.uint16)


def unit_mixes(rows, n=4):
    post = np.ones((rows, n), np.float32)
    comb = np.zeros((rows, n, n), np.float32)
    pre = np.zeros((rows, n), np.float32)
    pre[:, 0] = 1.0
    return post, comb, pre


def test_bf16_rounding_of_the_reduced_output_is_bit_exact():
    rows, hidden = 8, 1024
    say(f"case: bf16 ties, boundary and residual-only, rows={rows} hidden={hidden} tp=2")
    rng = np.random.default_rng(11)
    xp = tie_partials(rng, rows, hidden)
    res = codecs.f64_to_bf16_bits(rng.normal(0, 1, (rows, 4, hidden)))
    post, comb, pre = unit_mixes(rows)
    w = codecs.f64_to_bf16_bits(np.ones(hidden))
    want = oracle.residual_only(xp, res, post, comb)
    # the rounded sums, repeated in every stream
    assert np.array_equal(want, np.repeat(codecs.f64_to_bf16_bits(
        codecs.bf16_bits_to_f64(xp[0]) + codecs.bf16_bits_to_f64(xp[1]))[:, None, :], 4, axis=1))
    h = handle_for(hidden, rows, tp=2)
    got = binding.boundary(h, T(xp), T(res), T(post), T(comb), T(pre), T(w), 1e-6)
    assert np.array_equal(N(got["residual"]), want), "boundary streams"
    got_ro = binding.residual_only(h, T(xp), T(res), T(post), T(comb))
    assert np.array_equal(N(got_ro), want), "residual-only streams"


def test_bf16_rounding_of_the_finalized_output_is_bit_exact():
    rows, hidden, top_k = 8, 1024, 2
    say(f"case: bf16 ties, finalize with and without pre, rows={rows} hidden={hidden}")
    rng = np.random.default_rng(12)
    ab = tie_partials(rng, rows, hidden)           # [2, rows, hidden]
    g = ab.transpose(1, 0, 2).reshape(rows * top_k, hidden).copy()
    perm = rng.permutation(rows * top_k).astype(np.int32)
    g_perm = np.empty_like(g)
    g_perm[perm] = g                               # slot e = r*K + k lands at perm[e]
    ew = np.ones((rows, top_k), np.float32)
    shared = np.zeros((rows, hidden), np.uint16)
    res = codecs.f64_to_bf16_bits(rng.normal(0, 1, (rows, 4, hidden)))
    post, comb, pre = unit_mixes(rows)
    w = codecs.f64_to_bf16_bits(np.ones(hidden))
    want = oracle.finalize(g_perm, ew, perm, shared, res, post, comb, None, None, 0.0)["residual"]
    h = handle_for(hidden, rows, tp=1, top_k=top_k)
    got = binding.finalize(h, T(g_perm), T(ew), T(perm), T(shared), T(res), T(post), T(comb),
                           T(pre), T(w), 1e-6)
    assert np.array_equal(N(got["residual"]), want), "finalize streams"
    got_ro = binding.finalize(h, T(g_perm), T(ew), T(perm), T(shared), T(res), T(post), T(comb))
    assert np.array_equal(N(got_ro["residual"]), want), "residual-only finalize streams"


def e4m3_edge_blocks(rng, nblocks):
    """Norm-weight blocks of 32 bf16 values, each block scaled by its own 2^eb."""
    out = np.zeros((nblocks, 32), np.float64)
    ties = [(1 + (2 * m + 1) / 16) * 2.0 ** j for j in range(-6, 8) for m in range(8)]
    ties += [(1 + (2 * m + 1) / 16) * 256.0 for m in range(6)]            # up to 432
    sub_ties = [(2 * k + 1) * 2.0 ** -10 for k in range(8)]                # incl. 15 * 2^-10
    exact = [(1 + m / 8) * 2.0 ** j for j in range(-6, 9) for m in range(8)
             if (1 + m / 8) * 2.0 ** j <= 448] + [k * 2.0 ** -9 for k in range(1, 8)]
    tiny = [2.0 ** -10, 2.0 ** -10 * (1 + 2 ** -7), 2.0 ** -11, 2.0 ** -12 * 3]
    pool = np.array(ties + sub_ties + exact + tiny)
    for b in range(nblocks):
        kind = b % 8
        eb = int(rng.integers(-30, 31))
        vals = rng.choice(pool, 32) * np.where(rng.random(32) < 0.5, -1.0, 1.0)
        if kind == 0:                      # amax exactly 448 * 2^eb
            vals[rng.integers(32)] = 448.0 * (1 if rng.random() < 0.5 else -1)
        elif kind == 1:                    # amax fraction just above 0.75: e = E - 7
            vals[rng.integers(32)] = (1 + 97 / 128) * 2.0 ** 8
            vals = np.clip(vals, -240, 240)
            vals[rng.integers(32)] = (1 + 97 / 128) * 2.0 ** 8
        elif kind == 2:                    # amax fraction exactly 0.75: e = E - 8
            vals = np.clip(vals, -224, 224)
            vals[rng.integers(32)] = -1.75 * 2.0 ** 7
        elif kind == 3:                    # signed zeros only: e = -127
            vals = np.where(rng.random(32) < 0.5, -0.0, 0.0)
        elif kind == 4:                    # zeros mixed in
            vals[rng.random(32) < 0.5] = -0.0
        elif kind == 5:                    # random bf16 magnitudes across 20 binades
            vals = codecs.bf16_bits_to_f64(codecs.f64_to_bf16_bits(
                rng.normal(0, 1, 32) * 2.0 ** rng.integers(-12, 8, 32)))
        elif kind == 6:                    # amax well below the E4M3 range: large 2^-e
            vals = vals * 2.0 ** -20
        out[b] = vals * 2.0 ** eb if kind != 3 else vals
    bits = codecs.f64_to_bf16_bits(out.reshape(-1))
    # every value is a bf16 number already (no rounding happened above), signs of zero kept
    assert np.array_equal(codecs.bf16_bits_to_f64(bits), out.reshape(-1))
    assert np.array_equal(np.signbit(codecs.bf16_bits_to_f64(bits)), np.signbit(out.reshape(-1)))
    return bits


def test_mxfp8_codes_and_scales_at_format_edges_are_bit_exact():
    rows, hidden = 3, 16384
    say(f"case: MXFP8 edge blocks, rows={rows} hidden={hidden}")
    rng = np.random.default_rng(13)
    w = e4m3_edge_blocks(rng, hidden // 32)
    c = codecs.f64_to_bf16_bits(np.array([1.0, -4.0, 2.0 ** -6])[:rows])
    res = np.repeat(np.repeat(c[:, None, None], 4, axis=1), hidden, axis=2).astype(np.uint16)
    xp = np.zeros((1, rows, hidden), np.uint16)
    post = np.zeros((rows, 4), np.float32)
    comb = np.tile(np.eye(4, dtype=np.float32), (rows, 1, 1))
    pre = np.zeros((rows, 4), np.float32)
    pre[:, 0] = 1.0
    want = oracle.boundary(xp, res, post, comb, pre, w, 0.0, mxfp8=True)
    # the layer input is sign(c) * w, so the quantizer sees the crafted blocks
    sign = np.signbit(codecs.bf16_bits_to_f64(c))
    assert np.array_equal(want["layer_input"], np.where(sign[:, None], w ^ np.uint16(0x8000), w))
    h = handle_for(hidden, rows, tp=1)
    got = binding.boundary(h, T(xp), T(res), T(post), T(comb), T(pre), T(w), 0.0, mxfp8=True)
    assert np.array_equal(N(got["layer_input"]), want["layer_input"]), "layer input"
    assert np.array_equal(N(got["mx_scale"]), want["mx_scale"]), "E8M0 scales"
    g, o = N(got["mx_data"]), want["mx_data"]
    bad = np.argwhere(g != o)
    assert bad.size == 0, (f"{len(bad)} E4M3 codes differ; first at {tuple(bad[0])}: gpu "
                           f"{g[tuple(bad[0])]:#04x} oracle {o[tuple(bad[0])]:#04x}")


def test_hand_derived_sum_and_rounding_of_x_bit_exact(golden_dir):
    """The hand-derived cases of tests/golden/post_rounding_points.json: the slices are
    summed (not averaged) and the sum is rounded to bf16 before post * x, so the new streams
    equal the fixture's bits exactly, through the boundary, residual-only and finalize."""
    import json
    import os
    with open(os.path.join(golden_dir, "post_rounding_points.json")) as f:
        g = json.load(f)
    n, H = 4, 1024
    rng = np.random.default_rng(17)
    for case in g["cases"]:
        parts = [eval(e, {}) for e in case["partials_expr"]]  # noqa: S307 (fixture literals)
        tp = len(parts)
        say(f"case: hand-derived post rounding '{case['name']}' tp={tp} hidden={H}")
        xp = np.stack([np.full((1, H), int(codecs.f64_to_bf16_bits(np.array(v))), np.uint16)
                       for v in parts])
        res = codecs.f64_to_bf16_bits(rng.normal(0, 1, (1, n, H)))
        post = np.array([case["post"]], np.float32)
        comb = np.zeros((1, n, n), np.float32)
        pre = np.full((1, n), 0.25, np.float32)
        w = codecs.f64_to_bf16_bits(np.ones(H))
        want = np.repeat(np.array([int(b, 16) for b in case["stream_bits"]], np.uint16)[:, None],
                         H, axis=1)
        h = handle_for(H, 1, tp=tp)
        full = binding.boundary(h, T(xp), T(res), T(post), T(comb), T(pre), T(w), 1e-6)
        ro = binding.residual_only(h, T(xp), T(res), T(post), T(comb))
        assert np.array_equal(N(full["residual"])[0], want), "boundary streams"
        assert np.array_equal(N(ro)[0], want), "residual-only streams"
    for case in g["finalize_cases"]:
        say(f"case: hand-derived finalize rounding '{case['name']}' hidden={H}")
        val = lambda e: int(codecs.f64_to_bf16_bits(np.array(eval(e, {}))))  # noqa: E731,S307
        sh = np.full((1, H), val(case["shared_expr"]), np.uint16)
        gg = np.full((1, H), val(case["g_expr"]), np.uint16)
        wt = np.array([[case["w"]]], np.float32)
        idx = np.array([0], np.int32)
        res = codecs.f64_to_bf16_bits(rng.normal(0, 1, (1, n, H)))
        post = np.array([case["post"]], np.float32)
        comb = np.zeros((1, n, n), np.float32)
        want = np.repeat(np.array([int(b, 16) for b in case["stream_bits"]], np.uint16)[:, None],
                         H, axis=1)
        h = handle_for(H, 1, tp=1, top_k=1)
        for pre in (None, np.full((1, n), 0.25, np.float32)):
            out = binding.finalize(h, T(gg), T(wt), T(idx), T(sh), T(res), T(post), T(comb),
                                   None if pre is None else T(pre),
                                   None if pre is None else T(codecs.f64_to_bf16_bits(np.ones(H))),
                                   1e-6)
            assert np.array_equal(N(out["residual"])[0], want), f"finalize streams pre={pre is not None}"
