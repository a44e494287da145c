"""Shared helpers of the GPU parity tests: run a case through the C ABI and compare it with
the oracle on the same seeded inputs."""

import sys

import numpy as np
import torch

import oracle
from oracle import codecs
from mhc_hyper_connection_02_amd import binding, synth

DEV = torch.device("cuda", 0)

# bf16 outputs: |gpu - oracle| <= 2e-2 + 1e-2 |oracle|; fp32 coefficients: 1e-5 + 1e-5 |oracle|
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL, F32_RTOL = 1e-5, 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def T(a):
    return synth.to_torch(a, DEV)


def N(t):
    return synth.to_numpy(t)


def assert_bf16_close(gpu_bits, ora_bits, what):
    g = codecs.bf16_bits_to_f64(gpu_bits)
    o = codecs.bf16_bits_to_f64(ora_bits)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    err = np.abs(g - o)
    bad = err > BF16_ATOL + BF16_RTOL * np.abs(o)
    if bad.any():
        i = np.unravel_index(np.argmax(err - BF16_RTOL * np.abs(o)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                             f"worst at {i}: gpu {g[i]} oracle {o[i]}")
    return float(np.mean(gpu_bits == ora_bits))  # fraction bit-identical


def assert_f32_close(gpu, ora, what):
    g = np.asarray(gpu, np.float64)
    o = np.asarray(ora, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    err = np.abs(g - o)
    bad = err > F32_ATOL + F32_RTOL * np.abs(o)
    if bad.any():
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; worst at "
                             f"{i}: gpu {g[i]} oracle {o[i]} (|d| = {err[i]:.3e})")
    return float(err.max())


def with_stated_comb(d, seed, iters=20, eps=1e-6):
    """The workload's comb as the configurations state it: per row, the Sinkhorn
    normalization (20 iterations, eps 1e-6) of exp(N(0,1) logits), computed by the oracle
    from logits drawn with their own seed (the seeded generator holds none of the method's
    arithmetic, so it draws a doubly-stochastic mixture instead). Returns a copy of d."""
    R = d["post"].shape[0]
    rng = np.random.default_rng(seed)
    logits = rng.normal(0.0, 1.0, size=(R, 4, 4))
    out = dict(d)
    out["comb"] = np.stack([oracle.sinkhorn(z, iters, eps) for z in logits]).astype(np.float32)
    return out


def handle_for(hidden, rows, tp=8, top_k=8, block=None):
    h = binding.Handle(hidden, 4, max_rows=max(rows, 1), max_tp=max(tp, 1), top_k=top_k)
    if block is not None:
        h.set_option(binding.MHC_OPT_BOUNDARY_BLOCK, block)
    return h


def gpu_boundary(h, d, mxfp8=None, residual_only=False):
    mx = d["mxfp8"] if mxfp8 is None else mxfp8
    if residual_only:
        out = binding.residual_only(h, T(d["x_partials"]), T(d["residual"]), T(d["post"]),
                                    T(d["comb"]))
        torch.cuda.synchronize()
        return {"residual": N(out)}
    out = binding.boundary(h, T(d["x_partials"]), T(d["residual"]), T(d["post"]), T(d["comb"]),
                           T(d["pre"]), T(d["norm_weight"]), d["eps"], mxfp8=mx)
    torch.cuda.synchronize()
    return {k: N(v) for k, v in out.items()}


def oracle_boundary(d, mxfp8=None, residual_only=False):
    mx = d["mxfp8"] if mxfp8 is None else mxfp8
    if residual_only:
        return {"residual": oracle.residual_only(d["x_partials"], d["residual"], d["post"], d["comb"])}
    return oracle.boundary(d["x_partials"], d["residual"], d["post"], d["comb"], d["pre"],
                           d["norm_weight"], d["eps"], mxfp8=mx)


def gpu_finalize(h, d, pre=True, mxfp8=None, num_permuted=None):
    mx = d["mxfp8"] if mxfp8 is None else mxfp8
    out = binding.finalize(h, T(d["gemm2_permuted"]), T(d["expert_weights"]),
                           T(d["expanded_idx_to_permuted_idx"]), T(d["shared_output"]),
                           T(d["residual"]), T(d["post"]), T(d["comb"]),
                           T(d["pre"]) if pre else None, T(d["norm_weight"]) if pre else None,
                           d["eps"], mxfp8=mx and pre)
    torch.cuda.synchronize()
    return {k: N(v) for k, v in out.items()}


def oracle_finalize(d, pre=True, mxfp8=None):
    mx = d["mxfp8"] if mxfp8 is None else mxfp8
    return oracle.finalize(d["gemm2_permuted"], d["expert_weights"],
                           d["expanded_idx_to_permuted_idx"], d["shared_output"], d["residual"],
                           d["post"], d["comb"], d["pre"] if pre else None,
                           d["norm_weight"] if pre else None, d["eps"], mxfp8=mx and pre)


def compare_boundary_outputs(g, o, what):
    """Streams and layer input within the bf16 tolerance; MXFP8 bit-exact against the oracle's
    quantizer applied to the GPU's own layer input, and the end-to-end mismatch count returned."""
    stats = {"residual_exact": assert_bf16_close(g["residual"], o["residual"], what + " streams")}
    if "layer_input" in o:
        stats["layer_exact"] = assert_bf16_close(g["layer_input"], o["layer_input"],
                                                 what + " layer input")
    if "mx_data" in o:
        codes, scales = codecs.mxfp8_quantize(g["layer_input"])
        assert np.array_equal(g["mx_scale"], scales), what + ": E8M0 scales differ from the quantizer"
        assert np.array_equal(g["mx_data"], codes), what + ": E4M3 codes differ from the quantizer"
        stats["scale_mismatch_vs_oracle"] = assert_scale_mismatches_at_the_edge(
            g["layer_input"], o["layer_input"], g["mx_scale"], o["mx_scale"], what)
        stats["code_mismatch_vs_oracle"] = int(np.sum(g["mx_data"] != o["mx_data"]))
        say(f"  {what}: E8M0 scales differing from the oracle's: "
            f"{stats['scale_mismatch_vs_oracle']} of {o['mx_scale'].size}")
    return stats


def assert_scale_mismatches_at_the_edge(g_li, o_li, g_scale, o_scale, what):
    """E8M0 scales against the oracle's own end-to-end scales (row-major [R, H/32]).

    The scale is the smallest e with amax <= 448 * 2^e, which is continuous in amax except
    at amax = 448 * 2^e (a mantissa of exactly 1.75). The GPU's layer input may differ from
    the oracle's by a bf16 ulp (fp32 against fp64 arithmetic), so a block's scale may differ
    only where the two layer inputs' block maxima lie on opposite sides of such an edge: the
    bytes then differ by one and the edge 448 * 2^e_lo sits in [min amax, max amax). Any
    other mismatch fails. Returns the number of mismatching blocks."""
    R, nb = o_scale.shape
    ga = np.abs(codecs.bf16_bits_to_f64(g_li)).reshape(R, nb, 32).max(axis=2)
    oa = np.abs(codecs.bf16_bits_to_f64(o_li)).reshape(R, nb, 32).max(axis=2)
    bad = np.argwhere(g_scale != o_scale)
    for r, b in bad:
        gs, os_ = int(g_scale[r, b]), int(o_scale[r, b])
        lo, hi = sorted((ga[r, b], oa[r, b]))
        edge = 448.0 * 2.0 ** (min(gs, os_) - 127)
        assert abs(gs - os_) == 1 and lo <= edge < hi, (
            f"{what}: E8M0 scale of row {r} block {b} is {gs} on the GPU and {os_} in the "
            f"oracle, with block maxima {ga[r, b]} and {oa[r, b]}: not a 1.75 * 2^E edge case")
    return int(len(bad))
