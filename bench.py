#!/usr/bin/env python3
"""Benchmark of the fused mHC boundary on one MI355X.

Prints ONE JSON line. The headline is the decode boundary with the MXFP8 layer
input at rows=32, hidden=7168, hc_mult=4, tp=8: achieved HBM GB/s over the
algorithmic bytes of a call (read-once inputs plus written outputs), with the
inputs already resident in HBM. Every input and output rotates over enough
buffer sets (>= 512 MB) that no call finds its data in the 256 MB Infinity
Cache left there by an earlier call. The other calls of the path are timed the
same way and reported under "rows", as is the 61-layer chained decode step
(config 4: 122 boundaries plus their coefficient calls at rows=128).

Timing: W eager warm-up calls; then one HIP graph of EXACTLY K calls and one
of 2K calls (the caller's graph is how the path runs in a decode step), each
replayed five times, interleaved, between two events recorded on the launch
stream. The per-call time is the slope between the medians, (t(2K) - t(K)) / K:
the replay's fixed cost cancels, so it does not depend on K; t(K) / K, with
that cost, and the eager per-call time of K calls launched one by one are
reported beside it. Before each
timed region a spacer (the headline call over its own >= 512 MB of buffer
sets, twice the 256 MB Infinity Cache) evicts whatever the untimed work left
in the cache and keeps the GPU busy while the host enqueues the timed work.
Call i uses buffer set i mod B, B sets covering >= 512 MB, so no call finds
its data in the cache.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused mHC boundary µs/call + achieved HBM GB/s (rows=32, hidden=7168, hc=4)"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
COPY_CALIBRATION_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "boundary_decode_r32_h7168_traffic.json")
KSTATS_FILE = os.path.join(ROOT, "profiles", "boundary_decode_mxfp8_r32_h7168_kernel_stats.json")
KERNEL_SOURCES = ["boundary.hip", "device_common.h", "kernels.h"]
# the fused tile kernel's sources: the hash its counter summaries carry
TILE_SOURCES = ["boundary_tile.hip", "device_common.h", "kernels.h", "coeff_epilogue.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--block", type=int, default=None, help="boundary workgroup size (128/256/512)")
    ap.add_argument("--tile-placement", choices=("default", "per-xcd", "spread"),
                    default="default", help="MHC_OPT_TILE_PLACEMENT of the fused calls' kernel")
    ap.add_argument("--no-chain", action="store_true", help="skip the 61-layer chained step")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--no-rows", action="store_true", help="time only the headline call")
    ap.add_argument("--graph-only", action="store_true",
                    help="skip the eager timing loops (profiled runs: dispatches are then the "
                         "graph replays that the reported numbers time)")
    ap.add_argument("--chain-only", action="store_true",
                    help="run only the chained decode step and print its row")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 256 MiB, --steps times (to scale "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic bytes per call (read-once inputs + written outputs)
# ---------------------------------------------------------------------------

def bytes_boundary(rows, hidden, tp, n=4, pre=True, mxfp8=False):
    per_row = tp * hidden * 2 + 2 * n * hidden * 2 + (n + n * n) * 4
    if pre:
        per_row += n * 4 + hidden * 2
    if mxfp8:
        per_row += hidden + hidden // 32
    return rows * per_row + (hidden * 2 if pre else 0)


def bytes_finalize(rows, hidden, top_k, n=4, pre=True, mxfp8=False):
    # gathered expert rows + weights + indices + shared row replace the tp partials
    per_row = top_k * (hidden * 2 + 4 + 4) + hidden * 2 + 2 * n * hidden * 2 + (n + n * n) * 4
    if pre:
        per_row += n * 4 + hidden * 2
    if mxfp8:
        per_row += hidden + hidden // 32
    return rows * per_row + (hidden * 2 if pre else 0)


def bytes_floor(rows, hidden, tp, n=4):
    """What mhc_floor_boundary_traffic moves: the partials and streams read; the streams,
    a layer input, its E4M3 bytes and scale bytes written."""
    return rows * (tp * hidden * 2 + 2 * n * hidden * 2 + hidden * 2 + hidden + hidden // 32)


def bytes_pre(rows, hidden, n=4):
    nc = 2 * n + n * n
    return rows * n * hidden * 2 + n * hidden * nc * 2 + (3 + nc) * 4 + rows * nc * 4


def bytes_mean(rows, hidden, n=4):
    return rows * n * hidden * 2 + rows * hidden * 2


def bytes_first(rows, hidden, n=4, mxfp8=False):
    """Embedding read, norm weight, n streams and the layer input written (+ MXFP8)."""
    b = rows * hidden * 2 + hidden * 2 + rows * n * hidden * 2 + rows * hidden * 2
    return b + (rows * hidden + rows * hidden // 32 if mxfp8 else 0)


def bytes_collapse_norm(rows, hidden, n=4):
    """Streams and pre read, norm weight, the normalized collapse written."""
    return rows * n * hidden * 2 + rows * n * 4 + hidden * 2 + rows * hidden * 2


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

GRAPH_ONLY = False
_SPACER = []
REPEATS = 5  # replays of each graph; the medians give the slope


def set_spacer(torch, calls):
    """The cache flush of every timed region: one graph of `calls`, headline boundary calls
    on a pool of buffer sets (>= 512 MB) that no timed call uses."""
    for c in calls:
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    # the graph holds raw addresses: keep the launchers, and with them the buffers they
    # hold, alive as long as the graph (freed buffers would be handed out again while the
    # spacer still writes them)
    _SPACER[:] = [g, list(calls)]


def flush(torch):
    """Enqueue the spacer: it evicts the timed buffers from the 256 MB Infinity Cache with
    the same kind of work as the timed calls, and occupies the GPU while the host enqueues
    what follows. (A foreign 1 GiB read or copy in its place was measured to slow the
    boundary calls after it by ~0.45 us each, for milliseconds, even calls whose data sits
    in the cache; a spin kernel that touches no memory left them unchanged.)"""
    _SPACER[0].replay()


def _timed(torch, fn):
    """Milliseconds between two events on the current stream around fn(), behind a flush."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush(torch)
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def time_calls(torch, calls, steps, warmup):
    """calls: zero-argument launchers, one per buffer set; call i uses set i % len(calls).

    Returns (eager, graph, graph_single) microseconds per call. graph: the slope between one
    HIP graph of exactly `steps` calls and one of 2 * `steps` (the second continuing over the
    buffer sets), each replayed REPEATS times, interleaved, each replay behind a cache flush,
    from the median times: the replay's fixed cost cancels, so the figure does not depend on
    `steps`. graph_single: the `steps`-call graph's median time per call, that fixed cost
    included. eager: `steps` calls launched one by one (None under --graph-only)."""
    nset = len(calls)
    for i in range(warmup):
        calls[i % nset]()
    torch.cuda.synchronize()
    eager_ms = None
    if not GRAPH_ONLY:
        eager_ms = _timed(torch, lambda: [calls[i % nset]() for i in range(steps)])

    graphs = []
    for n in (steps, 2 * steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                calls[i % nset]()
        g.replay()  # untimed: the first replay uploads the graph
        graphs.append(g)
    torch.cuda.synchronize()
    t1, t2 = [], []
    for _ in range(REPEATS):  # interleaved, each behind its own spacer
        t1.append(_timed(torch, graphs[0].replay))
        t2.append(_timed(torch, graphs[1].replay))
    del graphs
    m1, m2 = sorted(t1)[REPEATS // 2], sorted(t2)[REPEATS // 2]
    eager_us = None if eager_ms is None else eager_ms / steps * 1e3
    return eager_us, (m2 - m1) / steps * 1e3, m1 / steps * 1e3


def n_sets(bytes_per_set):
    return max(2, int((2 * MALL_BYTES + bytes_per_set - 1) // bytes_per_set))


def row_entry(name, nbytes, t, sets):
    """t: time_calls' (eager, graph slope, single graph) microseconds per call."""
    us_eager, us, us_single = t
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us_per_call": round(us, 3), "us_per_call_single_graph": round(us_single, 3),
            "us_per_call_eager": None if us_eager is None else round(us_eager, 3),
            "algorithmic_bytes": int(nbytes), "gb_per_s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "buffer_sets": sets}


def time_entry(t, note):
    """A row without bytes: time_calls' microseconds per call."""
    us_eager, us, us_single = t
    return {"us_per_call": round(us, 3), "us_per_call_single_graph": round(us_single, 3),
            "us_per_call_eager": None if us_eager is None else round(us_eager, 3),
            "note": note}


def source_hash(files=None):
    """Short hash of the headline kernel's sources (or of `files`, names under csrc/), which
    a profile summary carries so that a stale one is recognised."""
    h = hashlib.sha256()
    for f in files or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mhc_hyper_connection_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_stats():
    """The headline kernel's rocprofv3 per-dispatch durations from the committed summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(KSTATS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    return t


def measured_traffic(block):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on
    the current kernel source at this block size; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash() or t.get("block") != block:
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# the benchmark
# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path has no "
              "collectives: each GPU would run this kernel on its own tensor-parallel share after "
              "an exchange of the partial slices.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from mhc_hyper_connection_02_amd import binding, synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    T = lambda a: synth.to_torch(a, dev)  # noqa: E731

    if args.copy_calibration:
        n = COPY_CALIBRATION_BYTES
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": args.steps}), flush=True)
        return

    global GRAPH_ONLY
    GRAPH_ONLY = args.graph_only

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    def chain_rows():
        """The chained step, then the same step with a stand-in sublayer (one bf16 GEMM of the
        layer input per sublayer), coefficient calls inline and on a side stream."""
        from mhc_hyper_connection_02_amd import chain as chain_mod
        log("chain: generating 122 sublayers of synthetic inputs")
        t0 = time.time()
        step = chain_mod.DecodeChain.from_synth(dev)
        if placement is not None:
            step.h.set_option(binding.MHC_OPT_TILE_PLACEMENT, placement)
        log(f"  inputs ready in {time.time() - t0:.1f} s ({step.input_bytes() / 1e9:.2f} GB)")
        k = max(3, args.steps // 40)
        out = {}
        s5 = chain_mod.DecodeChain(step.h, step.emb, step.subs, step.p, dev, fused=True,
                                   deferred=True)
        e5, g5, _ = time_calls(torch, [s5.run], k, 2)
        out["chain_decode_step"] = {
            "us_per_step": round(g5, 1), "us_per_step_eager": None if e5 is None else round(e5, 1),
            "algorithmic_bytes": int(s5.algorithmic_bytes()),
            "gb_per_s": round(s5.algorithmic_bytes() / g5 / 1e3, 1),
            "note": "each boundary and the coefficient call after it in one kernel, which "
                    "leaves the coefficients as partial sums for the next one to finish "
                    "(mhc_boundary_coeffs / mhc_finalize_coeffs, deferred)"}
        log(f"  chain (fused, deferred) {out['chain_decode_step']}")
        del s5
        s4 = chain_mod.DecodeChain(step.h, step.emb, step.subs, step.p, dev, fused=True)
        e4, g4, _ = time_calls(torch, [s4.run], k, 2)
        out["chain_decode_step_fused"] = {
            "us_per_step": round(g4, 1), "us_per_step_eager": None if e4 is None else round(e4, 1),
            "gb_per_s": round(s4.algorithmic_bytes() / g4 / 1e3, 1),
            "note": "fused calls that finish the next coefficients themselves"}
        log(f"  chain (fused) {out['chain_decode_step_fused']}")
        del s4
        us_e, us_g, _ = time_calls(torch, [step.run], k, 2)
        out["chain_decode_step_unfused"] = {
            "us_per_step": round(us_g, 1),
            "us_per_step_eager": None if us_e is None else round(us_e, 1),
            "algorithmic_bytes": int(step.algorithmic_bytes()),
            "gb_per_s": round(step.algorithmic_bytes() / us_g / 1e3, 1),
            "note": "boundary calls, each followed by a separate mhc_pre_coeffs call"}
        log(f"  chain (unfused) {out['chain_decode_step_unfused']}")
        s3 = chain_mod.DecodeChain(step.h, step.emb, step.subs, step.p, dev, deferred=True)
        e3, g3, _ = time_calls(torch, [s3.run], k, 2)
        out["chain_decode_step_deferred"] = {
            "us_per_step": round(g3, 1), "us_per_step_eager": None if e3 is None else round(e3, 1),
            "gb_per_s": round(step.algorithmic_bytes() / g3 / 1e3, 1),
            "note": "coefficient calls deferred: each boundary finishes the coefficients it "
                    "consumes (no epilogue launch)"}
        log(f"  chain deferred {out['chain_decode_step_deferred']}")
        del s3

        for cols, tag in ((None, ""), (1024, "_narrow")):
            for side in (False, True):
                s2 = chain_mod.DecodeChain(step.h, step.emb, step.subs, step.p, dev, standin=True,
                                           side_stream=side, standin_cols=cols)
                e2, g2, _ = time_calls(torch, [s2.run], k, 2)
                name = f"chain_standin{tag}_" + ("side_stream" if side else "inline")
                shape = "[R,H]x[H,H]" if cols is None else f"[R,H]x[H,{cols}]"
                out[name] = {"us_per_step": round(g2, 1),
                             "us_per_step_eager": None if e2 is None else round(e2, 1),
                             "note": f"boundaries + one {shape} bf16 GEMM per sublayer as a "
                                     "stand-in; coefficient calls " + (
                                         "on a side stream, joined before the next boundary"
                                         if side else "inline")}
                log(f"  {name} {out[name]}")
                del s2
        del step
        return out

    def fused_rows(h):
        Rc, nc = 128, 24
        cq = synth.pre_inputs(12, rows=1, hidden=H)
        nxt = {"fn": T(cq["fn"]), "scale": T(cq["scale"]), "base": T(cq["base"]),
               "rms_eps": cq["rms_eps"], "pre_eps": cq["pre_eps"],
               "sinkhorn_eps": cq["sinkhorn_eps"], "post_alpha": cq["post_alpha"],
               "sinkhorn_iters": cq["sinkhorn_iters"]}
        extra = 4 * H * nc * 2 + (3 + nc) * 4 + Rc * nc * 4  # fn, scale/base, coefficients
        out = {}
        for kind in ("boundary", "finalize"):
            mx = kind == "finalize"
            if kind == "boundary":
                d = synth.boundary_inputs(11, rows=Rc, hidden=H, tp=TP, x_sigma=0.5)
                nb = bytes_boundary(Rc, H, TP, mxfp8=mx)
            else:
                d = synth.finalize_inputs(13, rows=Rc, hidden=H, top_k=8)
                nb = bytes_finalize(Rc, H, 8, mxfp8=mx)
            ns = n_sets(nb)
            co = {k: T(d[k]) for k in ("post", "comb", "pre", "norm_weight")}
            src = {k: T(d[k]) for k in ("x_partials", "gemm2_permuted", "shared_output")
                   if k in d}
            small = {k: T(d[k]) for k in ("expert_weights", "expanded_idx_to_permuted_idx")
                     if k in d}
            res = T(d["residual"])
            bufs = []
            for _ in range(ns):
                b = {k: v.clone() for k, v in src.items()}
                b["s"] = res.clone()
                b["li"] = torch.empty((Rc, H), dtype=torch.bfloat16, device=dev)
                b["mx"] = ((torch.empty((Rc, H), dtype=torch.uint8, device=dev),
                            torch.empty((Rc, H // 32), dtype=torch.uint8, device=dev))
                           if mx else None)
                b["nx"] = (torch.empty((Rc, 4), device=dev), torch.empty((Rc, 4), device=dev),
                           torch.empty((Rc, 4, 4), device=dev))
                bufs.append(b)

            def fused(b):
                kw = dict(mxfp8=mx, residual_out=b["s"], layer_input_out=b["li"],
                          mx_out=b["mx"], next_out=b["nx"])
                if kind == "boundary":
                    return binding.boundary_coeffs(h, b["x_partials"], b["s"], co["post"],
                                                   co["comb"], co["pre"], co["norm_weight"],
                                                   d["eps"], nxt, **kw)
                return binding.finalize_coeffs(h, b["gemm2_permuted"], small["expert_weights"],
                                               small["expanded_idx_to_permuted_idx"],
                                               b["shared_output"], b["s"], co["post"],
                                               co["comb"], co["pre"], co["norm_weight"],
                                               d["eps"], nxt, **kw)

            def two(b):
                kw = dict(mxfp8=mx, residual_out=b["s"], layer_input_out=b["li"], mx_out=b["mx"])
                if kind == "boundary":
                    binding.boundary(h, b["x_partials"], b["s"], co["post"], co["comb"],
                                     co["pre"], co["norm_weight"], d["eps"], **kw)
                else:
                    binding.finalize(h, b["gemm2_permuted"], small["expert_weights"],
                                     small["expanded_idx_to_permuted_idx"], b["shared_output"],
                                     b["s"], co["post"], co["comb"], co["pre"],
                                     co["norm_weight"], d["eps"], **kw)
                binding.pre_coeffs(h, b["s"], nxt["fn"], nxt["scale"], nxt["base"],
                                   nxt["rms_eps"], nxt["pre_eps"], nxt["sinkhorn_eps"],
                                   nxt["post_alpha"], nxt["sinkhorn_iters"], out=b["nx"])

            t = time_calls(torch, [(lambda b=b: fused(b)) for b in bufs], args.steps,
                              args.warmup)
            name = f"{kind}_coeffs_r128" + ("_mxfp8" if mx else "")
            out[name] = row_entry(name, nb + extra, t, ns)
            out[name]["note"] = ("boundary + the next coefficient call in one kernel "
                                 "(no second read of the streams)")
            log(f"  {name} {out[name]}")
            t = time_calls(torch, [(lambda b=b: two(b)) for b in bufs], args.steps,
                              args.warmup)
            name2 = f"{kind}_then_coeffs_r128" + ("_mxfp8" if mx else "")
            out[name2] = row_entry(name2, nb + extra + Rc * 4 * H * 2, t, ns)
            out[name2]["note"] = "the same work as two calls (boundary, then mhc_pre_coeffs)"
            log(f"  {name2} {out[name2]}")

            # deferred and chained: call i takes call i-1's coefficients (finishing them in
            # its kernel) and leaves its own as partial sums
            for b in bufs:
                for t, src_t in zip(b["nx"], (co["pre"], co["post"], co["comb"])):
                    t.copy_(src_t)

            def chained(i):
                b, (pp, qq, cc) = bufs[i], bufs[i - 1]["nx"]
                kw = dict(mxfp8=mx, residual_out=b["s"], layer_input_out=b["li"],
                          mx_out=b["mx"], next_out=b["nx"], deferred=True)
                if kind == "boundary":
                    return binding.boundary_coeffs(h, b["x_partials"], b["s"], qq, cc, pp,
                                                   co["norm_weight"], d["eps"], nxt, **kw)
                return binding.finalize_coeffs(h, b["gemm2_permuted"], small["expert_weights"],
                                               small["expanded_idx_to_permuted_idx"],
                                               b["shared_output"], b["s"], qq, cc, pp,
                                               co["norm_weight"], d["eps"], nxt, **kw)

            t = time_calls(torch, [(lambda i=i: chained(i)) for i in range(ns)],
                              args.steps, args.warmup)
            binding.pre_coeffs_flush(h)  # the last call's coefficients, before the buffers go
            torch.cuda.synchronize()
            name3 = f"{kind}_coeffs_deferred_r128" + ("_mxfp8" if mx else "")
            out[name3] = row_entry(name3, nb + extra, t, ns)
            out[name3]["note"] = ("as " + name + ", chained: each call finishes the previous "
                                  "call's coefficients in its kernel and leaves its own as "
                                  "partial sums (mhc_coeff_args.deferred)")
            log(f"  {name3} {out[name3]}")
            del bufs
        return out

    # --- headline: config 1, decode boundary + MXFP8 --------------------------------
    R, H, TP = 32, 7168, 8
    d1 = synth.config(1)
    h = binding.Handle(H, 4, max_rows=128, max_tp=8, top_k=8)
    if args.block:
        h.set_option(binding.MHC_OPT_BOUNDARY_BLOCK, args.block)
    placement = {"per-xcd": binding.MHC_TILE_PER_XCD, "spread": binding.MHC_TILE_SPREAD}.get(
        args.tile_placement)
    if placement is not None:
        h.set_option(binding.MHC_OPT_TILE_PLACEMENT, placement)
    # the handle's choice for 32 rows: 512 threads at two elements per lane (the same seven
    # workgroups per row as 128 threads at eight); a fixed block size runs eight per lane
    block = args.block or 512
    lane_elems = 8 if args.block else 2
    nb = bytes_boundary(R, H, TP, pre=True, mxfp8=True)
    sets = n_sets(nb)
    base = {k: T(d1[k]) for k in ("x_partials", "residual", "post", "comb", "pre", "norm_weight")}

    def buffer_sets(n):
        return [{"x": base["x_partials"].clone(), "s": base["residual"].clone(),
                 "so": torch.empty_like(base["residual"]),
                 "li": torch.empty((R, H), dtype=torch.bfloat16, device=dev),
                 "md": torch.empty((R, H), dtype=torch.uint8, device=dev),
                 "ms": torch.empty((R, H // 32), dtype=torch.uint8, device=dev)}
                for _ in range(n)]

    def mk(b):
        return lambda: binding.boundary(h, b["x"], b["s"], base["post"], base["comb"], base["pre"],
                                        base["norm_weight"], d1["eps"], mxfp8=True,
                                        residual_out=b["so"], layer_input_out=b["li"],
                                        mx_out=(b["md"], b["ms"]))

    # the flush before every timed region: the headline call on its own pool of buffer sets
    set_spacer(torch, [mk(b) for b in buffer_sets(sets)])
    if args.chain_only:
        print(json.dumps({"rows": chain_rows()}), flush=True)
        return
    bufs = buffer_sets(sets)
    log(f"headline: boundary rows={R} hidden={H} tp={TP} mxfp8, {sets} buffer sets, block {block}")

    t = time_calls(torch, [mk(b) for b in bufs], args.steps, args.warmup)
    rows = {"boundary_decode_mxfp8": row_entry("boundary", nb, t, sets)}
    log(f"  {rows['boundary_decode_mxfp8']}")
    if not args.no_rows:
        # the same call on one buffer set: its 8 MB stay in the 256 MB Infinity Cache between
        # calls (the case of a producer that has just written the partials); context only,
        # the headline is the cold figure above
        t = time_calls(torch, [mk(bufs[0])], args.steps, args.warmup)
        rows["boundary_decode_mxfp8_warm"] = row_entry("boundary_warm", nb, t, 1)
        rows["boundary_decode_mxfp8_warm"]["note"] = (
            "one buffer set reused every call (inputs resident in the Infinity Cache); "
            "context, not the headline")
        log(f"  warm {rows['boundary_decode_mxfp8_warm']}")
        # floors on the same box, timed the same way: a device copy moving the headline's
        # bytes (half read, half written) over rotating cold buffers, and a one-element fill
        # (the cost of a launch in a graph)
        half = (nb // 2 + 15) // 16 * 16
        cs = n_sets(2 * half)
        cbufs = [(torch.empty(half, dtype=torch.uint8, device=dev),
                  torch.empty(half, dtype=torch.uint8, device=dev)) for _ in range(cs)]
        calls = [(lambda a=a, b=b: b.copy_(a)) for a, b in cbufs]
        t = time_calls(torch, calls, args.steps, args.warmup)
        rows["copy_floor_8mb"] = row_entry("copy", 2 * half, t, cs)
        rows["copy_floor_8mb"]["note"] = ("device copy of the headline's bytes (read + written), "
                                          "cold buffers: the floor of an 8 MB pass")
        log(f"  copy floor {rows['copy_floor_8mb']}")
        del cbufs, calls
        one = torch.empty(1, dtype=torch.float32, device=dev)
        t = time_calls(torch, [one.zero_], args.steps, args.warmup)
        rows["launch_floor"] = time_entry(t, "a one-element fill kernel: the cost of one launch")
        log(f"  launch floor {rows['launch_floor']}")
    # the in-house floors of the headline's launch geometry (include/mhc_floor.h), on the
    # headline's own buffer sets: its bytes moved with its grid and access kind but without
    # its arithmetic or row handoff, and the same grid doing nothing
    nfl = bytes_floor(R, H, TP)
    t = time_calls(torch, [(lambda b=b: binding.floor_boundary_traffic(
        b["x"], b["s"], b["so"], b["li"], b["md"], b["ms"])) for b in bufs], args.steps,
        args.warmup)
    rows["floor_boundary_traffic"] = row_entry("floor_traffic", nfl, t, sets)
    rows["floor_boundary_traffic"]["note"] = (
        "mhc_floor_boundary_traffic: the headline's bytes with its grid (224 x 512 threads), "
        "non-temporal 4-byte loads and stores, no arithmetic, no row handoff")
    log(f"  floor (traffic) {rows['floor_boundary_traffic']}")
    t = time_calls(torch, [lambda: binding.floor_empty(R, H)], args.steps, args.warmup)
    rows["floor_empty_grid"] = time_entry(t, "mhc_floor_empty: the headline's grid, doing nothing")
    log(f"  floor (empty grid) {rows['floor_empty_grid']}")
    del bufs

    if not args.no_rows:
        # the same boundary without the MXFP8 form of the layer input
        nb16 = bytes_boundary(R, H, TP, pre=True, mxfp8=False)
        s1 = n_sets(nb16)
        bufs = [{"x": base["x_partials"].clone(), "s": base["residual"].clone(),
                 "so": torch.empty_like(base["residual"]),
                 "li": torch.empty((R, H), dtype=torch.bfloat16, device=dev)} for _ in range(s1)]
        calls = [(lambda b=b: binding.boundary(h, b["x"], b["s"], base["post"], base["comb"],
                                               base["pre"], base["norm_weight"], d1["eps"],
                                               residual_out=b["so"], layer_input_out=b["li"]))
                 for b in bufs]
        t = time_calls(torch, calls, args.steps, args.warmup)
        rows["boundary_decode_bf16"] = row_entry("boundary_bf16", nb16, t, s1)
        log(f"  bf16-only {rows['boundary_decode_bf16']}")
        del bufs, calls

        # residual-only at config 1
        nro = bytes_boundary(R, H, TP, pre=False)
        s2 = n_sets(nro)
        bufs = [{"x": base["x_partials"].clone(), "s": base["residual"].clone(),
                 "so": torch.empty_like(base["residual"])} for _ in range(s2)]
        calls = [(lambda b=b: binding.residual_only(h, b["x"], b["s"], base["post"], base["comb"],
                                                    residual_out=b["so"])) for b in bufs]
        t = time_calls(torch, calls, args.steps, args.warmup)
        rows["residual_only_decode"] = row_entry("residual_only", nro, t, s2)
        log(f"  residual-only {rows['residual_only_decode']}")
        del bufs, calls

        # the headline's call at 512 rows (context: the per-launch costs spread over 16x the
        # bytes)
        R5 = 512
        d5 = synth.boundary_inputs(11, rows=R5, hidden=H, tp=TP, x_sigma=0.5, mxfp8=True)
        h5 = binding.Handle(H, 4, max_rows=R5, max_tp=TP, top_k=8)
        b5 = {k: T(d5[k]) for k in ("post", "comb", "pre", "norm_weight")}
        n5 = bytes_boundary(R5, H, TP, pre=True, mxfp8=True)
        s5b = n_sets(n5)
        bufs = [{"x": T(d5["x_partials"]), "s": T(d5["residual"]),
                 "so": torch.empty((R5, 4, H), dtype=torch.bfloat16, device=dev),
                 "li": torch.empty((R5, H), dtype=torch.bfloat16, device=dev),
                 "md": torch.empty((R5, H), dtype=torch.uint8, device=dev),
                 "ms": torch.empty((R5, H // 32), dtype=torch.uint8, device=dev)}
                for _ in range(s5b)]
        del d5
        calls = [(lambda b=b: binding.boundary(h5, b["x"], b["s"], b5["post"], b5["comb"],
                                               b5["pre"], b5["norm_weight"], 1e-6, mxfp8=True,
                                               residual_out=b["so"], layer_input_out=b["li"],
                                               mx_out=(b["md"], b["ms"])))
                 for b in bufs]
        t = time_calls(torch, calls, args.steps, args.warmup)
        rows["boundary_mxfp8_r512"] = row_entry("boundary_r512", n5, t, s5b)
        rows["boundary_mxfp8_r512"]["note"] = ("the headline's call at 512 rows (seed 11): "
                                               "context, where one launch carries 16x the bytes")
        log(f"  boundary r512 {rows['boundary_mxfp8_r512']}")
        del bufs, calls, h5

        # finalize at config 2
        d2 = synth.config(2)
        R2, K2 = 64, 8
        nf = bytes_finalize(R2, H, K2, pre=True, mxfp8=True)
        s3 = n_sets(nf)
        c2 = {k: T(d2[k]) for k in ("expert_weights", "expanded_idx_to_permuted_idx", "post",
                                     "comb", "pre", "norm_weight")}
        g0, sh0, r0 = T(d2["gemm2_permuted"]), T(d2["shared_output"]), T(d2["residual"])
        bufs = [{"g": g0.clone(), "sh": sh0.clone(), "s": r0.clone(), "so": torch.empty_like(r0),
                 "li": torch.empty((R2, H), dtype=torch.bfloat16, device=dev),
                 "md": torch.empty((R2, H), dtype=torch.uint8, device=dev),
                 "ms": torch.empty((R2, H // 32), dtype=torch.uint8, device=dev)}
                for _ in range(s3)]
        calls = [(lambda b=b: binding.finalize(
            h, b["g"], c2["expert_weights"], c2["expanded_idx_to_permuted_idx"], b["sh"], b["s"],
            c2["post"], c2["comb"], c2["pre"], c2["norm_weight"], d2["eps"], mxfp8=True,
            residual_out=b["so"], layer_input_out=b["li"], mx_out=(b["md"], b["ms"])))
            for b in bufs]
        t = time_calls(torch, calls, args.steps, args.warmup)
        rows["finalize_moe_mxfp8"] = row_entry("finalize", nf, t, s3)
        log(f"  finalize {rows['finalize_moe_mxfp8']}")
        del bufs, calls

        # coefficient path at config 3
        d3 = synth.config(3)
        npb = bytes_pre(64, H)
        s4 = n_sets(npb)
        sc, bs = T(d3["scale"]), T(d3["base"])
        r3, fn3 = T(d3["residual"]), T(d3["fn"])
        bufs = [{"s": r3.clone(), "fn": fn3.clone(),
                 "o": (torch.empty((64, 4), device=dev), torch.empty((64, 4), device=dev),
                       torch.empty((64, 4, 4), device=dev))} for _ in range(s4)]
        calls = [(lambda b=b: binding.pre_coeffs(h, b["s"], b["fn"], sc, bs, d3["rms_eps"],
                                                 d3["pre_eps"], d3["sinkhorn_eps"],
                                                 d3["post_alpha"], d3["sinkhorn_iters"],
                                                 out=b["o"])) for b in bufs]
        t = time_calls(torch, calls, args.steps, args.warmup)
        rows["pre_coeffs"] = row_entry("pre_coeffs", npb, t, s4)
        log(f"  pre_coeffs {rows['pre_coeffs']}")
        del bufs, calls

        # the first layer's entry at the decode boundary's 32 rows, with MXFP8
        nfi = bytes_first(R, H, mxfp8=True)
        s6 = n_sets(nfi)
        emb = T(synth.chain_embedding(R, H))
        bufs = [{"x": emb.clone(), "so": torch.empty((R, 4, H), dtype=torch.bfloat16, device=dev),
                 "li": torch.empty((R, H), dtype=torch.bfloat16, device=dev),
                 "md": torch.empty((R, H), dtype=torch.uint8, device=dev),
                 "ms": torch.empty((R, H // 32), dtype=torch.uint8, device=dev)}
                for _ in range(s6)]
        calls = [(lambda b=b: binding.first(h, b["x"], base["norm_weight"], d1["eps"], mxfp8=True,
                                            residual_out=b["so"], layer_input_out=b["li"],
                                            mx_out=(b["md"], b["ms"]))) for b in bufs]
        t = time_calls(torch, calls, args.steps, args.warmup)
        rows["first_decode_mxfp8"] = row_entry("first", nfi, t, s6)
        log(f"  first {rows['first_decode_mxfp8']}")
        del bufs, calls

        # the head (collapse with the last pre-mix + final norm) at the chained step's 128 rows
        nhd = bytes_collapse_norm(128, H)
        s7 = n_sets(nhd)
        dh = synth.boundary_inputs(7, rows=128, hidden=H, tp=1)
        sh, ph, wh = T(dh["residual"]), T(dh["pre"]), T(dh["norm_weight"])
        bufs = [{"s": sh.clone(), "o": torch.empty((128, H), dtype=torch.bfloat16, device=dev)}
                for _ in range(s7)]
        calls = [(lambda b=b: binding.collapse_norm(h, b["s"], ph, wh, dh["eps"], out=b["o"]))
                 for b in bufs]
        t = time_calls(torch, calls, args.steps, args.warmup)
        rows["collapse_norm_r128"] = row_entry("collapse_norm", nhd, t, s7)
        log(f"  collapse_norm {rows['collapse_norm_r128']}")
        del bufs, calls

        # mean-collapse at the chained step's 128 rows
        nm = bytes_mean(128, H)
        s5 = n_sets(nm)
        sm = T(synth.boundary_inputs(5, rows=128, hidden=H, tp=1)["residual"])
        bufs = [{"s": sm.clone(), "o": torch.empty((128, H), dtype=torch.bfloat16, device=dev)}
                for _ in range(s5)]
        calls = [(lambda b=b: binding.collapse_mean(h, b["s"], out=b["o"])) for b in bufs]
        t = time_calls(torch, calls, args.steps, args.warmup)
        rows["collapse_mean_r128"] = row_entry("collapse_mean", nm, t, s5)
        log(f"  collapse_mean {rows['collapse_mean_r128']}")
        del bufs, calls

        # the boundary fused with the next coefficient call, against the two calls, at the
        # chained step's 128 rows: the attention boundary (TP partials, bf16 layer input) and
        # the MoE boundary (finalize, MXFP8 layer input)
        rows.update(fused_rows(h))

    if not args.no_chain and not args.no_rows:
        rows.update(chain_rows())

    head = rows["boundary_decode_mxfp8"]
    us = head["us_per_call"]
    achieved = head["gb_per_s"]
    traffic = measured_traffic(block)
    ks = kernel_stats()
    rocprof = None
    if ks is not None:
        rocprof = {"kernel": ks["kernel"], "dispatches": ks["dispatches"],
                   "avg_us": ks["avg_us"], "median_us": ks["median_us"],
                   "frac_avg": round(nb / (ks["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "frac_median": round(nb / (ks["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "source": os.path.relpath(KSTATS_FILE, ROOT)}
    out = {
        "metric": METRIC,
        "value": achieved,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "us_per_call": us,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode boundary + MXFP8 layer input: rows=32 hidden=7168 "
                               "hc_mult=4 tp=8 (bf16 in/out, fp32 arithmetic)",
                   "rows": R, "hidden": H, "hc_mult": 4, "tp": TP, "mxfp8": True,
                   "block": block, "lane_elems": lane_elems, "buffer_sets": head["buffer_sets"],
                   "timing": "slope between the median times of one HIP graph of exactly K "
                             "calls and one of 2K, each replayed 5 times between two events "
                             "on the launch stream behind a cache-evicting spacer (the same "
                             "call on >= 512 MB of other buffers); call i on buffer set i mod "
                             "buffer_sets (>= 512 MB)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": nb,
                     "kernel_time_rocprof": rocprof},
        "rows": rows,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(d1, nb, args.cpu_seconds, log)
    print(json.dumps(out), flush=True)
    h.close()


def cpu_baseline(d, nbytes, seconds, log):
    """The oracle as it stands (numpy fp64) on the same config-1 inputs, repeated for about
    `seconds` of host time. Its boundary is numpy element-wise and einsum loops, which run on
    one thread whatever cores and BLAS threads the host offers (both reported)."""
    import oracle
    host_cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = sum(i.get("num_threads", 0) for i in threadpool_info()
                   if i.get("user_api") == "blas")
    except Exception:  # noqa: BLE001 (threadpoolctl missing or failing: report unknown)
        blas = None
    log(f"cpu baseline: oracle boundary on config 1, ~{seconds:.0f} s")
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.boundary(d["x_partials"], d["residual"], d["post"], d["comb"], d["pre"],
                        d["norm_weight"], d["eps"], mxfp8=True)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    return {"value": round(nbytes / per / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "ms_per_call": round(per * 1e3, 2), "host_cores_available": host_cores,
            "blas_threads": blas,
            "sample": f"{n} full calls of the config-1 boundary (32 rows, MXFP8) in {el:.1f} s; "
                      "numpy fp64 element-wise and einsum loops, which use one thread "
                      f"({host_cores} host cores available, BLAS threads {blas}, unused here)"}


if __name__ == "__main__":
    main()
