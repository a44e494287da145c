"""The fused mHC boundary and the mhc_pre coefficient path, written out in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation: R rows (tokens), n = hc_mult residual streams, H hidden, T tensor-
parallel partial slices, K = top_k. bf16 tensors arrive as uint16 bit
patterns, fp32 ones as float32, indices as int32; everything is promoted to
fp64 exactly, and each bf16 output is rounded once, from fp64.

Rounding points (a reading: the pages print no arithmetic). A value is rounded
to bf16 exactly where the unfused composition on the boundary page materialises
a bf16 tensor: the reduced sublayer output x (the plain-tensor path of
``Boundaries.post_only`` all-reduces it before the separate post kernel), the
new residual streams (they are the tensor handed to the coefficient call in
``Boundaries.sublayer``), and the layer input. Everything between those points
stays in fp64.
"""

import numpy as np

from .codecs import bf16_bits_to_f64, f64_to_bf16_bits, mxfp8_quantize


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# The sublayer output x
# ----------------------------------------------------------------------------

def tp_reduce(x_partials_bits):
    """Sum of the tensor-parallel partial slices of a sublayer output, [T,R,H] -> [R,H] fp64.

    boundary page, module docstring: each sublayer leaves its output as partial slices
    over the tensor-parallel ranks, and the boundary after it adds them up. On one GPU
    the T slices are resident and the reduction is their plain sum.
    """
    xp = bf16_bits_to_f64(x_partials_bits)
    return xp.sum(axis=0)


def moe_finalize_sum(gemm2_permuted_bits, expert_weights, expanded_idx_to_permuted_idx,
                     shared_output_bits):
    """The finalized MoE output: shared + sum_k w[r,k] * g[idx[r*K+k]], [R,H] fp64.

    boundary page, ``Boundaries._reduce``: a MoE output left unfinalized is
    reduced by the kernel's ``finalize`` from ``gemm2_permuted``,
    ``expert_weights``, ``expanded_idx_to_permuted_idx`` and the shared
    expert's output (all_reduce page, ``BoundaryAllReduce.finalize``).
    Readings: the expanded index of (row r, slot k) is r*K + k, row-major over
    ``expert_weights[R, K]``; an index outside [0, num_permuted) contributes 0.
    """
    g = bf16_bits_to_f64(gemm2_permuted_bits)
    w = _f64(expert_weights)
    idx = np.asarray(expanded_idx_to_permuted_idx, dtype=np.int64)
    x = bf16_bits_to_f64(shared_output_bits).copy()
    R, K = w.shape
    P = g.shape[0]
    for r in range(R):
        for k in range(K):
            p = idx[r * K + k]
            if 0 <= p < P:
                x[r] += w[r, k] * g[p]
    return x


# ----------------------------------------------------------------------------
# mHC post, pre collapse, RMSNorm
# ----------------------------------------------------------------------------

def mhc_post(x_f64, residual_bits, post, comb):
    """New residual streams: s'[r,i] = bf16( sum_j comb[r,i,j] * s[r,j] + post[r,i] * x[r] ).

    boundary page, module docstring (the reduced output is mixed into the streams
    at the boundary) and ``BoundaryState`` (post and comb belong to the
    sublayer that produced the pending output). Reading: in comb[r,i,j], i is
    the output stream and j the input stream.
    x must already be bf16-valued (it is rounded after the reduction).
    """
    s = bf16_bits_to_f64(residual_bits)            # [R,n,H]
    c = _f64(comb)                                 # [R,n,n]
    p = _f64(post)                                 # [R,n]
    mixed = np.einsum("rij,rjh->rih", c, s) + p[:, :, None] * _f64(x_f64)[:, None, :]
    return f64_to_bf16_bits(mixed)


def collapse(streams_bits, pre):
    """Pre-mix collapse of the streams, y[r] = sum_j pre[r,j] * s[r,j], fp64 [R,H].

    boundary page, module docstring (the streams are collapsed to one hidden state,
    which becomes the following sublayer's input) and ``BoundaryState`` (pre is kept
    for the collapse at the following boundary).
    """
    s = bf16_bits_to_f64(streams_bits)
    return np.einsum("rj,rjh->rh", _f64(pre), s)


def rms_norm(y_f64, weight_bits, eps):
    """RMSNorm of each row: bf16( y * (mean_h y**2 + eps) ** -1/2 * w ).

    boundary page, ``Boundaries.sublayer``: the layer input is normalized with
    the sublayer's norm weight and ``variance_epsilon``. Reading: eps inside the
    square root, the weight applied after normalizing, one rounding at the end.
    """
    y = _f64(y_f64)
    w = bf16_bits_to_f64(weight_bits)
    ms = np.mean(y * y, axis=1, keepdims=True)
    return f64_to_bf16_bits(y / np.sqrt(ms + float(eps)) * w[None, :])


def _mhc_tail(x, residual_bits, post, comb, pre, norm_weight_bits, eps, mxfp8):
    x_bf16 = bf16_bits_to_f64(f64_to_bf16_bits(x))
    new_streams = mhc_post(x_bf16, residual_bits, post, comb)
    out = {"residual": new_streams}
    if pre is None:
        return out
    layer_input = rms_norm(collapse(new_streams, pre), norm_weight_bits, eps)
    out["layer_input"] = layer_input
    if mxfp8:
        out["mx_data"], out["mx_scale"] = mxfp8_quantize(layer_input)
    return out


def boundary(x_partials_bits, residual_bits, post, comb, pre, norm_weight_bits, eps,
             mxfp8=False):
    """The fused boundary on TP partials.

    boundary page, ``Boundaries._reduce`` / all_reduce page,
    ``BoundaryAllReduce.__call__``: reduce the partials, apply the mHC post,
    then (unless ``pre`` is None: residual-only) collapse with ``pre``,
    RMS-normalize, and optionally also emit the layer input as MXFP8.
    Returns a dict with "residual" and, with ``pre``, "layer_input" (and
    "mx_data", "mx_scale" with ``mxfp8``).
    """
    return _mhc_tail(tp_reduce(x_partials_bits), residual_bits, post, comb, pre,
                     norm_weight_bits, eps, mxfp8)


def finalize(gemm2_permuted_bits, expert_weights, expanded_idx_to_permuted_idx,
             shared_output_bits, residual_bits, post, comb, pre, norm_weight_bits, eps,
             mxfp8=False):
    """The fused boundary on an unfinalized MoE output.

    boundary page, ``Boundaries._reduce`` (MoE branch) / all_reduce page,
    ``BoundaryAllReduce.finalize``. Same outputs as :func:`boundary`.
    """
    x = moe_finalize_sum(gemm2_permuted_bits, expert_weights, expanded_idx_to_permuted_idx,
                         shared_output_bits)
    return _mhc_tail(x, residual_bits, post, comb, pre, norm_weight_bits, eps, mxfp8)


def residual_only(x_partials_bits, residual_bits, post, comb):
    """Reduce and mix only; the new streams are the one output.

    boundary page, ``Boundaries.post_only`` and ``Boundaries._reduce`` (no pre
    means residual-only): used before an Engram injection and for the final
    collapse.
    """
    return boundary(x_partials_bits, residual_bits, post, comb, None, None, 0.0)["residual"]


def collapse_mean(streams_bits):
    """Mean of the hc streams, bf16( (1/n) sum_i s[r,i] ), [R,H].

    boundary page, ``Boundaries.sublayer`` (the aux output is the streams' mean
    over the stream axis) and decode page, ``SpecializedDecode.run`` (the same
    mean after the final reduction).
    """
    s = bf16_bits_to_f64(streams_bits)
    return f64_to_bf16_bits(s.mean(axis=1))


def _with_mxfp8(out, mxfp8):
    if mxfp8:
        out["mx_data"], out["mx_scale"] = mxfp8_quantize(out["layer_input"])
    return out


def first(x_bits, norm_weight_bits, eps, hc_mult=4, mxfp8=False):
    """The first layer's entry: hc copies of the embedding as the streams, and the first
    sublayer's input.

    boundary page, ``Boundaries.first``: each of the hc streams starts as a copy of the
    embedding x, and the first pre-mix is the identity on stream 0, so the collapse is x itself
    and the layer input is x RMS-normalized with the sublayer's norm (``Boundaries._pre``
    receives x and the attention norm). Returns {"residual": [R,n,H] bf16 bits,
    "layer_input": [R,H] bf16 bits} (and "mx_data", "mx_scale" with ``mxfp8``).
    """
    x = np.asarray(x_bits, dtype=np.uint16)
    out = {"residual": np.repeat(x[:, None, :], hc_mult, axis=1),
           "layer_input": rms_norm(bf16_bits_to_f64(x), norm_weight_bits, eps)}
    return _with_mxfp8(out, mxfp8)


def collapse_norm(streams_bits, pre, norm_weight_bits, eps, mxfp8=False):
    """The head after the layers: the streams collapsed with the last pre-mix, then the
    final norm.

    decode page, ``_head`` (after ``Boundaries.post_only``): the hc streams are collapsed
    with ``state.pre`` into one hidden state, which the backbone's final norm normalizes.
    Reading: there the collapse is its own op and materializes a bf16 tensor, so y is
    rounded to bf16 once before the norm (inside the fused boundary, y goes straight into
    the norm). Returns {"layer_input": [R,H] bf16 bits} (and the MXFP8 pair with
    ``mxfp8``).
    """
    y = bf16_bits_to_f64(f64_to_bf16_bits(collapse(streams_bits, pre)))
    return _with_mxfp8({"layer_input": rms_norm(y, norm_weight_bits, eps)}, mxfp8)


# ----------------------------------------------------------------------------
# mhc_pre: the next coefficients
# ----------------------------------------------------------------------------

def sinkhorn(logits, iters, eps):
    """Sinkhorn normalization of exp(logits) for one [n,n] matrix, fp64.

    boundary page, ``Boundaries.sublayer``: the coefficient call takes
    ``hc_eps`` (a second time, after the pre eps) and ``hc_sinkhorn_iters``.
    Reading (the pages fix no convention): subtract each row's max before exp;
    then ``iters`` times divide every row by (its sum + eps), then every column
    by (its sum + eps). The last step normalizes columns.
    """
    z = _f64(logits)
    A = np.exp(z - z.max(axis=1, keepdims=True))
    for _ in range(int(iters)):
        A = A / (A.sum(axis=1, keepdims=True) + eps)
        A = A / (A.sum(axis=0, keepdims=True) + eps)
    return A


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def pre_coeffs(residual_bits, fn_bits, scale, base, rms_eps, pre_eps, sinkhorn_eps,
               post_alpha, sinkhorn_iters):
    """Coefficients (pre, post, comb) of the next sublayer from the streams, fp64.

    boundary page, ``Boundaries.sublayer`` and ``Boundaries._pre``: the call
    takes the streams, ``fn``, ``scale``, ``base``, ``rms_norm_eps``,
    ``hc_eps`` twice, ``hc_post_alpha`` and ``hc_sinkhorn_iters``. Steps:

    1. v = the row's streams flattened stream-major (k = i*H + h, the memory
       order of [R,n,H] and the row order of fn [n*H, 2n+n*n]);
    2. inv = (mean_k v**2 + rms_eps) ** -1/2 (no weight);
    3. l = inv * (v @ fn), 2n + n*n logits per row;
    4. l' = l * scale[g] + base, with g = 0 for the n pre columns, 1 for the n
       post columns and 2 for the n*n comb columns (comb row-major, column
       2n + n*i + j holds comb[i,j]);
    5. pre = sigmoid(l'_pre) + pre_eps; post = post_alpha * sigmoid(l'_post);
       comb = Sinkhorn(l'_comb) with ``sinkhorn_eps`` and ``sinkhorn_iters``.
    """
    s = bf16_bits_to_f64(residual_bits)             # [R,n,H]
    R, n, H = s.shape
    v = s.reshape(R, n * H)
    fn = bf16_bits_to_f64(fn_bits)                  # [n*H, 2n+n*n]
    if fn.shape != (n * H, 2 * n + n * n):
        raise ValueError("fn must be [n*H, 2n+n*n]")
    inv = 1.0 / np.sqrt(np.mean(v * v, axis=1) + float(rms_eps))
    logits = inv[:, None] * (v @ fn)
    sc = _f64(scale)
    group_scale = np.concatenate([np.full(n, sc[0]), np.full(n, sc[1]), np.full(n * n, sc[2])])
    lp = logits * group_scale[None, :] + _f64(base)[None, :]
    pre = _sigmoid(lp[:, :n]) + float(pre_eps)
    post = float(post_alpha) * _sigmoid(lp[:, n:2 * n])
    comb = np.stack([sinkhorn(lp[r, 2 * n:].reshape(n, n), sinkhorn_iters, float(sinkhorn_eps))
                     for r in range(R)])
    return pre, post, comb


# ----------------------------------------------------------------------------
# The chained decode step
# ----------------------------------------------------------------------------

def decode_chain(embedding_bits, sublayers, rms_eps, hc_eps, post_alpha, sinkhorn_iters,
                 norm_eps, hc_mult=4, record=None, progress=None, coeff_perturb=None):
    """One decode step's boundaries over all sublayers, fp64 per step.

    decode page, ``SpecializedDecode.run``: the first layer enters through
    ``Boundaries.first`` (every stream starts as a copy of the embedding); then every
    sublayer's output is reduced at the next boundary (``Boundaries.sublayer``),
    and after the last sublayer ``Boundaries.post_only`` reduces it
    residual-only, followed by the streams' mean.

    The pre-mix is delayed (boundary page, ``Boundaries.sublayer`` and
    ``BoundaryState``): a boundary collapses its new streams with the ``pre``
    the coefficient call returned at the previous boundary, and the call on the
    new streams returns the post/comb of the sublayer about to run plus the pre
    of the next collapse.

    ``sublayers`` is a sequence of dicts, one per sublayer in execution order,
    each with the coefficient weights "fn", "scale", "base", the norm weight
    "norm_w", a flag "mxfp8" for its layer input, and "output": the sublayer's
    output as {"partials": [T,R,H]} or {"finalize": (g, w, idx, shared)}.
    The first entry (:func:`first`) also yields the first sublayer's input, the
    normalized embedding. Coefficients pass between steps as fp32, as they do
    between the library's calls. Returns the final streams and their mean; with
    ``record`` (a list), appends the first entry's outputs with the first
    coefficients, and then each boundary's outputs. ``progress``, if given, is called
    with each sublayer's index after its boundary (reporting only). ``coeff_perturb``, if
    given, maps every (pre, post, comb) the coefficient calls return to the values passed
    on (for measuring how the chain responds to coefficient errors; None: unchanged).
    """
    emb = np.asarray(embedding_bits, dtype=np.uint16)
    head = sublayers[0]
    entry = first(emb, head["norm_w"], norm_eps, hc_mult, mxfp8=bool(head["mxfp8"]))
    streams = entry["residual"]
    pre, post, comb = pre_coeffs(streams, head["fn"], head["scale"], head["base"],
                                 rms_eps, hc_eps, hc_eps, post_alpha, sinkhorn_iters)
    if coeff_perturb is not None:
        pre, post, comb = coeff_perturb(pre, post, comb)
    if record is not None:
        entry.update({"pre": pre, "post": post, "comb": comb})
        record.append(entry)
    for idx in range(len(sublayers)):
        out = sublayers[idx]["output"]
        last = idx + 1 == len(sublayers)
        nxt = None if last else sublayers[idx + 1]
        p32 = pre.astype(np.float32)
        po32 = post.astype(np.float32)
        c32 = comb.astype(np.float32)
        if last:
            use_pre, w_bits, mx = None, None, False
        else:
            use_pre, w_bits, mx = p32, nxt["norm_w"], bool(nxt["mxfp8"])
        if "partials" in out:
            res = boundary(out["partials"], streams, po32, c32, use_pre, w_bits, norm_eps, mx)
        else:
            g, w, ix, sh = out["finalize"]
            res = finalize(g, w, ix, sh, streams, po32, c32, use_pre, w_bits, norm_eps, mx)
        streams = res["residual"]
        if not last:
            pre, post, comb = pre_coeffs(streams, nxt["fn"], nxt["scale"], nxt["base"],
                                         rms_eps, hc_eps, hc_eps, post_alpha, sinkhorn_iters)
            if coeff_perturb is not None:
                pre, post, comb = coeff_perturb(pre, post, comb)
            res.update({"pre": pre, "post": post, "comb": comb})
        if record is not None:
            record.append(res)
        if progress is not None:
            progress(idx)
    return streams, collapse_mean(streams)
