"""Seeded synthetic inputs for the boundary calls, shared by the tests and the benchmark.

This module only draws random numbers and rounds them to the dtypes the calls
take. It holds none of the boundary's arithmetic, so the oracle and the HIP
library can both be fed from it without sharing any of their computation.

Every tensor is drawn in fp64 from ``numpy.random.default_rng(seed)`` (PCG64)
in the order listed by each builder, then rounded to fp32 and, for bf16
tensors, to bfloat16 by torch's CPU conversion (round to nearest even).
Arrays are returned as numpy: bf16 as uint16 bit patterns, fp32 as float32,
indices as int32. ``N(mu, sigma)`` names a normal with standard deviation sigma.

Coefficient inputs of the boundary: ``post = 2 * logistic(N(0,1))`` and
``pre = logistic(N(0,1))`` (logit-normal draws via scipy's ``expit``), and
``comb`` a random doubly-stochastic matrix per row, built as a Dirichlet(1)
weighted mixture of n random permutation matrices (Birkhoff--von Neumann), so
that no normalization routine of the method is needed to produce it.
"""

import numpy as np
import torch
from scipy.special import expit

HC = 4


def to_bf16_bits(a):
    """fp64/fp32 array -> bfloat16 bit patterns (uint16), via fp32 and torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def normal_bf16(rng, shape, mu=0.0, sigma=1.0):
    return to_bf16_bits(rng.normal(mu, sigma, size=shape))


def doubly_stochastic(rng, rows, n=HC):
    """[rows, n, n] fp32: per row, sum_k w_k P_k with w ~ Dirichlet(1) and P_k random permutations."""
    out = np.zeros((rows, n, n), dtype=np.float64)
    for r in range(rows):
        w = rng.dirichlet(np.ones(n))
        for k in range(n):
            perm = rng.permutation(n)
            out[r, np.arange(n), perm] += w[k]
    return f32(out)


def coefficients(rng, rows, n=HC):
    """post [rows,n], pre [rows,n], comb [rows,n,n], all fp32, drawn in that order."""
    post = f32(2.0 * expit(rng.normal(0.0, 1.0, size=(rows, n))))
    pre = f32(expit(rng.normal(0.0, 1.0, size=(rows, n))))
    comb = doubly_stochastic(rng, rows, n)
    return post, pre, comb


def softmax_weights(rng, rows, top_k):
    z = rng.normal(0.0, 1.0, size=(rows, top_k))
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return f32(e / e.sum(axis=1, keepdims=True))


def boundary_inputs(seed, rows, hidden, tp, n=HC, x_sigma=1.0, eps=1e-6, mxfp8=False):
    """TP-partial boundary: x_partials [tp,rows,hidden], residual [rows,n,hidden],
    post, pre, comb, norm_weight [hidden] ~ N(1, 0.1), eps."""
    rng = np.random.default_rng(seed)
    d = {
        "x_partials": normal_bf16(rng, (tp, rows, hidden), 0.0, x_sigma),
        "residual": normal_bf16(rng, (rows, n, hidden)),
    }
    d["post"], d["pre"], d["comb"] = coefficients(rng, rows, n)
    d["norm_weight"] = normal_bf16(rng, (hidden,), 1.0, 0.1)
    d["eps"] = float(np.float32(eps))
    d["mxfp8"] = mxfp8
    return d


def finalize_inputs(seed, rows, hidden, top_k, n=HC, g_sigma=0.3, eps=1e-6, mxfp8=False,
                    num_permuted=None):
    """MoE-finalize boundary: gemm2_permuted [P,hidden], a random permutation of 0..P-1 as
    expanded_idx_to_permuted_idx [rows*top_k] (P = rows*top_k unless given, in which case a
    random choice without replacement), softmax expert_weights [rows,top_k], shared_output,
    residual, post/pre/comb, norm_weight."""
    rng = np.random.default_rng(seed)
    P = rows * top_k if num_permuted is None else num_permuted
    d = {"gemm2_permuted": normal_bf16(rng, (P, hidden), 0.0, g_sigma)}
    if num_permuted is None:
        d["expanded_idx_to_permuted_idx"] = rng.permutation(P).astype(np.int32)
    else:
        d["expanded_idx_to_permuted_idx"] = rng.choice(P, size=rows * top_k,
                                                       replace=False).astype(np.int32)
    d["expert_weights"] = softmax_weights(rng, rows, top_k)
    d["shared_output"] = normal_bf16(rng, (rows, hidden), 0.0, g_sigma)
    d["residual"] = normal_bf16(rng, (rows, n, hidden))
    d["post"], d["pre"], d["comb"] = coefficients(rng, rows, n)
    d["norm_weight"] = normal_bf16(rng, (hidden,), 1.0, 0.1)
    d["eps"] = float(np.float32(eps))
    d["mxfp8"] = mxfp8
    return d


def pre_inputs(seed, rows, hidden, n=HC, fn_sigma=0.02):
    """Coefficient path: residual [rows,n,hidden] ~ N(0,1), fn [n*hidden, 2n+n*n] ~ N(0,fn_sigma),
    scale [3] ~ U(0.5,1.5), base [2n+n*n] ~ N(0,0.1), and the scalar parameters."""
    rng = np.random.default_rng(seed)
    nc = 2 * n + n * n
    return {
        "residual": normal_bf16(rng, (rows, n, hidden)),
        "fn": normal_bf16(rng, (n * hidden, nc), 0.0, fn_sigma),
        "scale": f32(rng.uniform(0.5, 1.5, size=3)),
        "base": f32(rng.normal(0.0, 0.1, size=nc)),
        "rms_eps": float(np.float32(1e-6)),
        "pre_eps": float(np.float32(1e-6)),
        "sinkhorn_eps": float(np.float32(1e-6)),
        "post_alpha": 2.0,
        "sinkhorn_iters": 20,
    }


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def config(k):
    """Workload k (0..3) with seed k."""
    if k == 0:   # tiny boundary
        return boundary_inputs(0, rows=4, hidden=1024, tp=2, x_sigma=1.0, mxfp8=False)
    if k == 1:   # decode boundary, MXFP8 layer input
        return boundary_inputs(1, rows=32, hidden=7168, tp=8, x_sigma=0.5, mxfp8=True)
    if k == 2:   # MoE-finalize boundary, MXFP8 layer input
        return finalize_inputs(2, rows=64, hidden=7168, top_k=8, g_sigma=0.3, mxfp8=True)
    if k == 3:   # coefficient path
        return pre_inputs(3, rows=64, hidden=7168)
    raise ValueError("config 4 is built per sublayer: see chain_embedding / chain_sublayer")


CHAIN_LAYERS = 61
CHAIN_ROWS = 128
CHAIN_HIDDEN = 7168
CHAIN_TP = 8
CHAIN_TOP_K = 8


def chain_embedding(rows=CHAIN_ROWS, hidden=CHAIN_HIDDEN):
    rng = np.random.default_rng(np.random.SeedSequence([4]))
    return normal_bf16(rng, (rows, hidden))


def chain_sublayer(layer, ffn, rows=CHAIN_ROWS, hidden=CHAIN_HIDDEN, tp=CHAIN_TP,
                   top_k=CHAIN_TOP_K, n=HC):
    """Sublayer (layer, attn|ffn) of the chained decode step, seed SeedSequence([4, layer, ffn]).

    Draw order: fn, scale, base, norm weight, then the sublayer's output --
    attention: tp partials ~ N(0, 0.3); MoE: gemm2_permuted [rows*top_k, hidden] ~ N(0, 0.3),
    a permutation, softmax weights, shared ~ N(0, 0.3). Attention inputs are MXFP8 from
    layer 1 on; MoE inputs are bf16."""
    rng = np.random.default_rng(np.random.SeedSequence([4, layer, int(ffn)]))
    nc = 2 * n + n * n
    d = {
        "fn": normal_bf16(rng, (n * hidden, nc), 0.0, 0.02),
        "scale": f32(rng.uniform(0.5, 1.5, size=3)),
        "base": f32(rng.normal(0.0, 0.1, size=nc)),
        "norm_w": normal_bf16(rng, (hidden,), 1.0, 0.1),
        "mxfp8": (not ffn) and layer > 0,
    }
    if not ffn:
        d["output"] = {"partials": normal_bf16(rng, (tp, rows, hidden), 0.0, 0.3)}
    else:
        P = rows * top_k
        g = normal_bf16(rng, (P, hidden), 0.0, 0.3)
        idx = rng.permutation(P).astype(np.int32)
        w = softmax_weights(rng, rows, top_k)
        shared = normal_bf16(rng, (rows, hidden), 0.0, 0.3)
        d["output"] = {"finalize": (g, w, idx, shared)}
    return d


def chain_params():
    return {"rms_eps": float(np.float32(1e-6)), "hc_eps": float(np.float32(1e-6)),
            "post_alpha": 2.0, "sinkhorn_iters": 20, "norm_eps": float(np.float32(1e-6))}


# ---------------------------------------------------------------------------
# Moving the arrays into torch tensors (marshalling only)
# ---------------------------------------------------------------------------

def to_torch(a, device):
    """numpy -> torch on `device`: uint16 arrays become bfloat16 (same bits), float32 and
    int32 keep their dtype."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype in (np.float32, np.int32, np.uint8):
        return torch.from_numpy(a).to(device)
    raise TypeError(f"unsupported array dtype {a.dtype}")


def to_numpy(t):
    """torch -> numpy: bfloat16 comes back as uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
