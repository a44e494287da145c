"""One decode step's boundaries over all layers, on the library's entry points.

decode page, ``SpecializedDecode.run``: the first layer enters through
``Boundaries.first`` (``mhc_first``: every one of the hc streams starts as a copy of the
embedding, and since the first pre-mix is the identity on stream 0 the first sublayer's
input is the embedding normalized; then the coefficient call runs on those copies); then
each sublayer's output is reduced at the
next boundary (``Boundaries.sublayer``: the fused kernel, then the coefficient
call on the new streams), and after the last sublayer ``Boundaries.post_only``
reduces it residual-only, followed by the streams' mean (the final collapse).

The pre-mix is delayed (boundary page, ``Boundaries.sublayer`` and
``BoundaryState``): a boundary collapses its new streams with the ``pre`` that
the coefficient call returned at the previous boundary; the call on the new
streams returns the post/comb of the sublayer about to run and the pre of the
next collapse. One coefficient buffer set therefore suffices: each boundary
reads it before the following coefficient call rewrites it, in stream order.

The streams are updated in place. Every buffer is allocated up front, so
``run`` allocates nothing and can be captured in a HIP graph. The sublayers'
outputs (attention partials, unfinalized MoE outputs) are inputs here: the
step covers the boundaries only.

Side stream (boundary page, ``Boundaries.sublayer`` and ``Boundaries.join``): the
coefficient call after a boundary may run on a second stream while the sublayer
computes on the layer input, joined before the next boundary. With
``standin=True`` each sublayer is stood in for by one bf16 GEMM of the layer input
([R, H] x [H, H], a projection's worth of work, outside the hot path and its
result unused), so that the overlap has something to hide under; ``standin_cols``
narrows it to [R, H] x [H, cols], a GEMM with few output tiles that leaves most CUs idle
(as a decode sublayer of few rows can).

Fused (``fused=True``): each boundary that is followed by a coefficient call runs as one
call with it (``mhc_boundary_coeffs`` / ``mhc_finalize_coeffs``), which reads the current
coefficients and writes the next ones in the same kernel, so the step alternates between
two coefficient buffer sets. With ``deferred=True`` as well, each fused call leaves the next
coefficients as partial sums, and the next fused call finishes them in its own kernel while
its loads are in flight (``mhc_coeff_args.deferred``).
"""

import torch

from . import binding, synth


class DecodeChain:
    def __init__(self, handle, embedding, sublayers, params, device, standin=False,
                 side_stream=False, deferred=False, fused=False, standin_cols=None):
        """embedding: [R,H] bf16 tensor; sublayers: list of dicts of device tensors as built by
        :meth:`from_synth`; params: rms_eps, hc_eps, post_alpha, sinkhorn_iters, norm_eps."""
        self.h = handle
        self.emb = embedding
        self.subs = sublayers
        self.p = params
        R, H = embedding.shape
        self.rows, self.hidden = R, H
        n = handle.hc_mult
        self.streams = torch.empty((R, n, H), dtype=torch.bfloat16, device=device)
        self.pre = torch.empty((R, n), dtype=torch.float32, device=device)
        self.post = torch.empty((R, n), dtype=torch.float32, device=device)
        self.comb = torch.empty((R, n, n), dtype=torch.float32, device=device)
        self.layer_input = torch.empty((R, H), dtype=torch.bfloat16, device=device)
        self.mx_data = torch.empty((R, H), dtype=torch.uint8, device=device)
        self.mx_scale = torch.empty((R, H // 32), dtype=torch.uint8, device=device)
        self.mean = torch.empty((R, H), dtype=torch.bfloat16, device=device)
        # deferred coefficient calls: each boundary finishes the coefficients it consumes
        self.deferred = deferred
        # fused: boundary and coefficient call in one kernel, two coefficient sets
        self.fused = fused
        self.sets = [(self.pre, self.post, self.comb)]
        if fused:
            if side_stream:
                raise ValueError("fused boundaries take no side-stream calls")
            self.sets.append((torch.empty_like(self.pre), torch.empty_like(self.post),
                              torch.empty_like(self.comb)))
        self.next_args = [None if i + 1 == len(sublayers) else {
            "fn": sublayers[i + 1]["fn"], "scale": sublayers[i + 1]["scale"],
            "base": sublayers[i + 1]["base"], "rms_eps": params["rms_eps"],
            "pre_eps": params["hc_eps"], "sinkhorn_eps": params["hc_eps"],
            "post_alpha": params["post_alpha"], "sinkhorn_iters": params["sinkhorn_iters"]}
            for i in range(len(sublayers))]
        self.side = torch.cuda.Stream(device=device) if side_stream else None
        self.standin_w = self.standin_out = None
        if standin:
            cols = H if standin_cols is None else standin_cols
            g = torch.Generator(device=device)
            g.manual_seed(1234)
            self.standin_w = (torch.randn((H, cols), generator=g, device=device) * H ** -0.5
                              ).to(torch.bfloat16)
            self.standin_out = torch.empty((R, cols), dtype=torch.bfloat16, device=device)
        # optional callback(index, stage, chain) around every boundary: stage "before", "after"
        # (the boundary's outputs), "coeffs" (the coefficient call that follows it); and once
        # with index -1, stage "first", after the first layer's entry
        self.record = None

    @classmethod
    def from_synth(cls, device, layers=synth.CHAIN_LAYERS, rows=synth.CHAIN_ROWS,
                   hidden=synth.CHAIN_HIDDEN, tp=synth.CHAIN_TP, top_k=synth.CHAIN_TOP_K,
                   handle=None, standin=False, side_stream=False, deferred=False, fused=False):
        """The chained step on the seeded synthetic inputs (see ``synth.chain_sublayer``)."""
        emb = synth.chain_embedding(rows, hidden)
        subs = (synth.chain_sublayer(layer, ffn, rows=rows, hidden=hidden, tp=tp, top_k=top_k)
                for layer in range(layers) for ffn in (False, True))
        return cls.from_arrays(device, emb, subs, tp=tp, top_k=top_k, handle=handle,
                               standin=standin, side_stream=side_stream, deferred=deferred,
                               fused=fused)

    @classmethod
    def from_arrays(cls, device, embedding, sublayers, tp=synth.CHAIN_TP, top_k=synth.CHAIN_TOP_K,
                    handle=None, **kw):
        """The chained step on host arrays: ``embedding`` [R,H] bf16 bits and ``sublayers``
        as ``synth.chain_sublayer`` returns them (uploaded here, one sublayer at a time)."""
        T = lambda a: synth.to_torch(a, device)  # noqa: E731
        rows, hidden = embedding.shape
        if handle is None:
            handle = binding.Handle(hidden, 4, max_rows=rows, max_tp=tp, top_k=top_k,
                                    device=device.index)
        subs = []
        for d in sublayers:
            t = {k: T(d[k]) for k in ("fn", "scale", "base", "norm_w")}
            t["mxfp8"] = d["mxfp8"]
            if "partials" in d["output"]:
                t["partials"] = T(d["output"]["partials"])
            else:
                g, w, idx, sh = d["output"]["finalize"]
                t["finalize"] = (T(g), T(w), T(idx), T(sh))
            subs.append(t)
        return cls(handle, T(embedding), subs, synth.chain_params(), device, **kw)

    def input_bytes(self):
        tot = self.emb.numel() * 2
        for s in self.subs:
            for k, v in s.items():
                if isinstance(v, torch.Tensor):
                    tot += v.numel() * v.element_size()
                elif isinstance(v, tuple):
                    tot += sum(x.numel() * x.element_size() for x in v)
        return tot

    def algorithmic_bytes(self):
        """Bytes the step must move: every boundary's and coefficient call's read-once inputs
        and written outputs, plus the broadcast (R*n*H written, R*H read) and the mean."""
        R, H, n = self.rows, self.hidden, self.h.hc_mult
        nc = 2 * n + n * n
        coef = R * (n + n + n * n) * 4
        tot = R * H * 2 + R * n * H * 2 + H * 2 + R * H * 2   # first: broadcast, layer input
        if self.subs[0]["mxfp8"]:
            tot += R * H + R * H // 32
        pre_call = R * n * H * 2 + n * H * nc * 2 + (3 + nc) * 4 + coef
        tot += pre_call                                       # first coefficients
        if self.fused:  # the coefficient calls take the streams from the boundary's registers
            pre_call -= R * n * H * 2
        for i, s in enumerate(self.subs):
            last = i + 1 == len(self.subs)
            nxt = None if last else self.subs[i + 1]
            b = 2 * R * n * H * 2 + coef                      # streams in/out + mixes
            if "partials" in s:
                b += s["partials"].numel() * 2
            else:
                g, w, idx, sh = s["finalize"]
                b += R * self.h.top_k * (H * 2 + 8) + R * H * 2
            if not last:
                b += H * 2 + R * H * 2                        # norm weight, layer input
                if nxt["mxfp8"]:
                    b += R * H + R * H // 32
                b += pre_call
            tot += b
        tot += R * n * H * 2 + R * H * 2                      # mean-collapse
        return tot

    def run(self):
        """One decode step: the first layer's entry, coefficients, 122 boundaries, final
        reduction, mean."""
        h, p = self.h, self.p
        first = self.subs[0]
        cur = 0
        self.pre, self.post, self.comb = self.sets[cur]
        binding.first(h, self.emb, first["norm_w"], p["norm_eps"], mxfp8=first["mxfp8"],
                      residual_out=self.streams, layer_input_out=self.layer_input,
                      mx_out=(self.mx_data, self.mx_scale) if first["mxfp8"] else None)
        if self.record is not None:
            self.record(-1, "first", self)
        binding.pre_coeffs(h, self.streams, first["fn"], first["scale"], first["base"],
                           p["rms_eps"], p["hc_eps"], p["hc_eps"], p["post_alpha"],
                           p["sinkhorn_iters"], out=(self.pre, self.post, self.comb),
                           deferred=self.deferred)
        for i, s in enumerate(self.subs):
            last = i + 1 == len(self.subs)
            nxt = None if last else self.subs[i + 1]
            kw = {}
            if not last:
                kw = dict(pre=self.pre, norm_weight=nxt["norm_w"], eps=p["norm_eps"],
                          mxfp8=nxt["mxfp8"], layer_input_out=self.layer_input,
                          mx_out=(self.mx_data, self.mx_scale) if nxt["mxfp8"] else None)
            if self.record is not None:
                self.record(i, "before", self)
            if self.fused and not last:
                kw.update(residual_out=self.streams, next_out=self.sets[1 - cur],
                          deferred=self.deferred)
                if "partials" in s:
                    binding.boundary_coeffs(h, s["partials"], self.streams, self.post, self.comb,
                                            nxt=self.next_args[i], **kw)
                else:
                    g, w, idx, sh = s["finalize"]
                    binding.finalize_coeffs(h, g, w, idx, sh, self.streams, self.post, self.comb,
                                            nxt=self.next_args[i], **kw)
                if self.record is not None:
                    self.record(i, "after", self)
                cur = 1 - cur
                self.pre, self.post, self.comb = self.sets[cur]
                if self.record is not None:
                    self.record(i, "coeffs", self)
                continue
            if "partials" in s:
                binding.boundary(h, s["partials"], self.streams, self.post, self.comb,
                                 residual_out=self.streams, **kw)
            else:
                g, w, idx, sh = s["finalize"]
                binding.finalize(h, g, w, idx, sh, self.streams, self.post, self.comb,
                                 residual_out=self.streams, **kw)
            if self.record is not None:
                self.record(i, "after", self)
            if not last:
                main = torch.cuda.current_stream()
                if self.side is not None:
                    # the coefficients of the next sublayer beside it, joined before the
                    # next boundary (which reads them)
                    self.side.wait_stream(main)
                    cs = self.side
                else:
                    cs = main
                binding.pre_coeffs(h, self.streams, nxt["fn"], nxt["scale"], nxt["base"],
                                   p["rms_eps"], p["hc_eps"], p["hc_eps"], p["post_alpha"],
                                   p["sinkhorn_iters"], out=(self.pre, self.post, self.comb),
                                   stream=cs, deferred=self.deferred)
                if self.standin_w is not None:
                    torch.matmul(self.layer_input, self.standin_w, out=self.standin_out)
                if self.side is not None:
                    main.wait_stream(self.side)
                if self.record is not None:
                    self.record(i, "coeffs", self)
        binding.collapse_mean(h, self.streams, out=self.mean)
        return self.mean
