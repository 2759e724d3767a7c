#!/usr/bin/env python3
"""MoE-layer tokens/s on one MI355X: single-token decode and 512-token
prefill of one routed-expert layer at real shape (hidden 2048, 512 experts,
top-10, width 512, 2-bit block weights), with the roofline fraction of each
path's dominant kernel and the CPU oracle timed beside it.

A step is 256 independent single-token decode calls (router, top-k, lookup,
gate/up, down, ordered sum for each token) on seeded synthetic inputs already
resident in HBM; the 256 calls of a step are captured once as a HIP graph and
replayed.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published
METRIC = "MoE-layer tokens/sec (decode, prefill@512) + % HBM roofline"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=256, help="decode calls per step")
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=100,
                    help="untimed back-to-back chunks before the prefill timings (about 25 ms: "
                         "the chunk time settles only after some tens of milliseconds of load)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cache-flushed timings and the HBM read ceiling")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--eager", action="store_true", help="no HIP graph for the decode step")
    ap.add_argument("--no-stacks", action="store_true",
                    help="skip the 48-layer stacks of the default line (decode_48l, prefill_48l 2-bit, "
                         "the bounded-pool decode by the native driver with and without prefetch)")
    ap.add_argument("--stacks", action="store_true",
                    help="also time prefill_48l with 3-bit weights and the other bounded-pool decode "
                         "variants (Python loop, early-out path, sticky flag)")
    ap.add_argument("--slope", action="store_true",
                    help="only the decode expert stages against top_k = 1..k (warm and cache-flushed) "
                         "with a line fitted per stage, as one JSON line; nothing else runs")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB three times (the known-size "
                         "kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def stored_traffic(tag):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from
    profiles/traffic_<tag>.md, or None when the file is missing or the
    kernel's sources no longer hash to the value the counters were taken at."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        k, sep, v = line.strip().partition(": ")
        if sep and k in ("sources", "source_sha256", "fetch_bytes", "write_bytes"):
            kv[k] = v.strip()
    if len(kv) < 4:
        return None
    h = hashlib.sha256()
    for src in kv["sources"].split(","):
        f = os.path.join(ROOT, src)
        if not os.path.exists(f):
            return None
        h.update(open(f, "rb").read())
    if h.hexdigest() != kv["source_sha256"]:
        return None
    return int(kv["fetch_bytes"]) + int(kv["write_bytes"])


def event_ms(fn, stream, reps):
    """Average milliseconds of fn() over reps calls bracketed by HIP events
    recorded on the stream the kernels run on."""
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        fn()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) / reps


def cold_ms(items, flush, stream, reps=5):
    """Milliseconds per item with the Infinity Cache flushed before each: a
    graph of (flush, item) pairs and a graph of the flushes alone, replayed
    reps times each; the difference of their medians over the item count."""
    import torch

    def cap(with_items):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for it in items:
                flush.add_(1.0)
                if with_items:
                    it()
        g.replay()
        return g
    gp, gf = cap(True), cap(False)
    tp, tf = [], []
    for _ in range(reps):
        with torch.cuda.stream(stream):
            tp.append(event_ms(gp.replay, stream, 1))
            tf.append(event_ms(gf.replay, stream, 1))
    del gp, gf
    return (sorted(tp)[reps // 2] - sorted(tf)[reps // 2]) / len(items)


def slope(args, model, X, stream):
    """Decode expert stages against top_k = 1 .. k of the same layer (same
    router, pool and tokens; only the descriptor's top_k changes): warm time
    per launch over a graph of T launches, cold time by cold_ms over 32, and a
    least-squares line t = a + b*k per stage, so the per-expert streaming
    cost b separates from the fixed latency a."""
    import ctypes as C

    import numpy as np
    import torch

    from quantized_routed_expert_rl_amd import binding as B
    from quantized_routed_expert_rl_amd.device import RouteBuffers

    w, lib = model.w, B.lib
    T = min(args.tokens, 128)
    flush = torch.zeros(512 << 18, device="cuda")
    W0, res, pool = model.router[0].data_ptr(), model.residency.data_ptr(), model.pool.data_ptr()
    tb = B.rl_tensor_bytes(model.desc)
    rows = []
    for k in range(1, w.top_k + 1):
        dk = B.desc(w.hidden, w.n_experts, k, w.width, 1, w.qbits, model.desc.n_slots)
        sbk = B.rl_decode_scratch_bytes(dk)
        scr = torch.zeros(T, sbk, dtype=torch.uint8, device="cuda")
        rb = RouteBuffers.alloc(T, k, w.n_experts, with_logits=False)
        mc = torch.zeros(T, dtype=torch.int32, device="cuda")     # per token: calls stay independent
        eo = torch.zeros(T, dtype=torch.int32, device="cuda")
        outs = [B.route_out(rb.ids[t], rb.weights[t], rb.slots[t], mc[t:t + 1], eo[t:t + 1])
                for t in range(T)]
        Y = torch.empty(T, w.hidden, device="cuda")

        def stage(sg, t, dk=dk, scr=scr, outs=outs, Y=Y, sbk=sbk):
            return lambda: lib.rl_decode_stage(C.byref(dk), sg, 0, X[t].data_ptr(), W0, None, res,
                                               pool, C.byref(outs[t]), scr[t].data_ptr(), sbk,
                                               Y[t].data_ptr(),
                                               torch.cuda.current_stream().cuda_stream)
        with torch.cuda.stream(stream):
            for t in range(T):
                for sg in (0, 1, 2):
                    assert stage(sg, t)() == 0
        stream.synchronize()
        row = {"k": k}
        for sg, name in ((1, "gateup"), (2, "down")):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for t in range(T):
                    stage(sg, t)()
            g.replay()
            with torch.cuda.stream(stream):
                row[name + "_us"] = round(event_ms(g.replay, stream, 5) * 1e3 / T, 3)
                row[name + "_cold_us"] = round(
                    cold_ms([stage(sg, t) for t in range(32)], flush, stream) * 1e3, 3)
            del g
        assert int(mc.sum().cpu()) == 0 and int(eo.sum().cpu()) == 0
        rows.append(row)
        del scr, rb, mc, eo, outs, Y
    ks = np.array([r["k"] for r in rows], float)
    fits = {}
    for name, per_expert in (("gateup", 2 * tb), ("down", tb)):
        for kind in ("", "_cold"):
            b, a = np.polyfit(ks, [r[name + kind + "_us"] for r in rows], 1)
            fits[name + kind] = {"intercept_us": round(float(a), 3),
                                 "us_per_expert": round(float(b), 4),
                                 "expert_bytes": int(per_expert),
                                 "gbs_per_expert_slope": round(per_expert / (b * 1e-6) / 1e9, 1)}
    print(json.dumps({"mode": "slope", "workload": f"decode_1l, top_k 1..{w.top_k}, {T} tokens",
                      "rows": rows, "fits": fits}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import ctypes as C

    import numpy as np
    import torch

    from quantized_routed_expert_rl_amd import binding as B
    from quantized_routed_expert_rl_amd import synth, workloads
    from quantized_routed_expert_rl_amd.device import DeviceModel, RouteBuffers, to_dev

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    lib = B.lib
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ------------------------------------------------------------ decode
    w = workloads.get("decode_1l")
    model = DeviceModel(w)
    T = args.tokens
    X = to_dev(synth.activations(w, T, stream=1))
    if args.slope:
        slope(args, model, X, stream)
        return
    Y = torch.empty(T, w.hidden, device="cuda")
    rb = RouteBuffers.alloc(T, w.top_k, w.n_experts, with_logits=False)
    outs = [B.route_out(rb.ids[t], rb.weights[t], rb.slots[t], rb.miss_count, rb.early_out)
            for t in range(T)]
    scratch = model.decode_scratch()
    d = model.desc
    xp = [X[t].data_ptr() for t in range(T)]
    yp = [Y[t].data_ptr() for t in range(T)]
    W0, res, pool = model.router[0].data_ptr(), model.residency.data_ptr(), model.pool.data_ptr()
    sp, sb = scratch.data_ptr(), scratch.numel()

    def decode_step():
        st = torch.cuda.current_stream().cuda_stream
        for t in range(T):
            rc = lib.moe_decode_layer(C.byref(d), 0, xp[t], W0, None, res, pool,
                                      C.byref(outs[t]), sp, sb, yp[t], st)
            if rc:
                raise B.RlError(f"moe_decode_layer {rc}")

    with torch.cuda.stream(stream):
        for _ in range(max(args.warmup, 1)):
            decode_step()
    stream.synchronize()
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            decode_step()
        for _ in range(args.warmup):
            graph.replay()
    torch.cuda.synchronize()
    run = graph.replay if graph is not None else decode_step
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            run()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / args.steps
    decode_tps = T * args.steps / dt
    assert int(rb.early_out.cpu()[0]) == 0 and torch.isfinite(Y).all()

    # eager timing of the same step (host launch overhead included)
    with torch.cuda.stream(stream):
        eager_ms = event_ms(decode_step, stream, 3)

    # dominant kernel: top-k + gate/up GEMVs + SwiGLU of the 10 selected
    # experts, one launch per token; each token has its own scratch holding
    # its own router logits, so every launch streams that token's experts
    sb_tok = scratch.numel()
    scr = torch.zeros(T, sb_tok, dtype=torch.uint8, device="cuda")
    rb2 = RouteBuffers.alloc(T, w.top_k, w.n_experts, with_logits=False)
    outs2 = [B.route_out(rb2.ids[t], rb2.weights[t], rb2.slots[t], rb2.miss_count[0:1],
                         rb2.early_out[0:1]) for t in range(T)]
    with torch.cuda.stream(stream):
        st = stream.cuda_stream
        for t in range(T):
            B.rl_decode_stage(d, 0, 0, X[t], model.router[0], None, model.residency, model.pool,
                              outs2[t], scr[t], sb_tok, Y[t], st)

    def gateup_all():
        st = torch.cuda.current_stream().cuda_stream
        for t in range(T):
            lib.rl_decode_stage(C.byref(d), 1, 0, xp[t], W0, None, res, pool, C.byref(outs2[t]),
                                scr[t].data_ptr(), sb_tok, None, st)

    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        gateup_all()
    with torch.cuda.graph(g2, stream=stream):
        gateup_all()
    g2.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        gu_ms = event_ms(g2.replay, stream, 5) / T
    tb = B.rl_tensor_bytes(d)
    # codes of the 10 experts' gate and up tensors, x, logits, residency row, h
    gu_bytes = (w.top_k * 2 * tb + w.hidden * 4 + w.n_experts * 4 * 2
                + w.top_k * w.width * 4)
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
    layer_bytes = w.top_k * 3 * tb + w.n_experts * w.hidden * 4 + 2 * w.hidden * 4
    expert_gu_bytes = w.top_k * 2 * tb               # the ten experts' gate and up codes alone

    # The same launches with the 256 MB Infinity Cache flushed before each one
    # (a 512 MiB read-modify-write of another buffer).  One graph holds M pairs
    # (flush, launch i) and another the M flushes alone; the difference of
    # their replay times over M is the cold time per launch, with the same
    # back-to-back launch structure as the warm figure (a graph of a single
    # launch would mostly time the graph's own launch).
    flush = None if args.no_cold else torch.zeros(512 << 18, device="cuda")

    def cold_per_item_ms(items, reps=5):
        return cold_ms(items, flush, stream, reps)

    gu_cold_ms = None
    if flush is not None:
        def gu_launch(t):
            return lambda: lib.rl_decode_stage(C.byref(d), 1, 0, xp[t], W0, None, res, pool,
                                               C.byref(outs2[t]), scr[t].data_ptr(), sb_tok, None,
                                               torch.cuda.current_stream().cuda_stream)
        gu_cold_ms = cold_per_item_ms([gu_launch(t) for t in range(32)])

    line = {
        "metric": METRIC,
        "value": round(decode_tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode_1l: single-token decode of one MoE layer, hidden 2048, "
                        "512 experts all resident, top-10, width 512, 2-bit block weights; "
                        f"{T} independent tokens per step, HIP-graph replay"
                        + (" (eager)" if graph is None else ""),
            "tokens_per_step": T,
            "layer_bytes_per_token": layer_bytes,
            "us_per_token": round(ms_per_step * 1e3 / T, 3),
            "eager_us_per_token": round(eager_ms * 1e3 / T, 3),
        },
        "roofline": {
            "kernel": ("decode_topk_gateup_mfma_kernel<8, 8, 2, 4>" if w.width % 256 == 0
                       else "decode_topk_gateup_kernel<8, 2, 64>"),
            "bound": "hbm",
            "achieved": round(gu_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gu_gbs / PEAK_HBM_GBS, 4),
            "traffic": stored_traffic("decode_topk_gateup"),
            "bytes_per_launch": gu_bytes,
            "us_per_launch": round(gu_ms * 1e3, 3),
            "expert_bytes_per_launch": expert_gu_bytes,
            "frac_expert_bytes": round(expert_gu_bytes / (gu_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "cold": None if gu_cold_ms is None else {
                "us_per_launch": round(gu_cold_ms * 1e3, 3),
                "achieved": round(gu_bytes / (gu_cold_ms * 1e-3) / 1e9, 1),
                "frac": round(gu_bytes / (gu_cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "how": "Infinity Cache flushed (512 MiB read-modify-write) before each of 32 "
                       "launches: graph of (flush, launch) pairs minus a graph of the flushes alone, "
                       "HIP events, median of 5"},
        },
    }

    def graph_of(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        g.replay()
        return g

    # ------------------------------------------- decode, 3-bit block weights
    # the same single-token decode with the heavier 3-bit format (eight code
    # levels): 1.45x the expert bytes per token
    del g2, scr, outs2, rb2
    w3b = workloads.get("decode_1l", 3)
    m3b = DeviceModel(w3b)
    T3b = min(T, 128)
    X3b = to_dev(synth.activations(w3b, T3b, stream=1))
    Y3b = torch.empty(T3b, w3b.hidden, device="cuda")
    rb3 = RouteBuffers.alloc(T3b, w3b.top_k, w3b.n_experts, with_logits=False)
    outs3 = [B.route_out(rb3.ids[t], rb3.weights[t], rb3.slots[t], rb3.miss_count, rb3.early_out)
             for t in range(T3b)]
    sc3 = m3b.decode_scratch()
    d3b = m3b.desc

    def decode3():
        st = torch.cuda.current_stream().cuda_stream
        for t in range(T3b):
            rc = lib.moe_decode_layer(C.byref(d3b), 0, X3b[t].data_ptr(), m3b.router[0].data_ptr(),
                                      None, m3b.residency.data_ptr(), m3b.pool.data_ptr(),
                                      C.byref(outs3[t]), sc3.data_ptr(), sc3.numel(),
                                      Y3b[t].data_ptr(), st)
            if rc:
                raise B.RlError(f"moe_decode_layer {rc}")

    with torch.cuda.stream(stream):
        decode3()
        stream.synchronize()
        g3 = graph_of(decode3)
        ms3 = event_ms(g3.replay, stream, 5)
    assert int(rb3.early_out.cpu()[0]) == 0 and torch.isfinite(Y3b).all()
    line["decode_3bit"] = {
        "tokens_per_s": round(T3b / (ms3 * 1e-3), 1), "us_per_token": round(ms3 * 1e3 / T3b, 3),
        "layer_bytes_per_token": w3b.top_k * 3 * B.rl_tensor_bytes(d3b) + w3b.n_experts * w3b.hidden * 4
                                 + 2 * w3b.hidden * 4,
        "workload": f"decode_1l with 3-bit block weights: {T3b} independent tokens per graph replay"}
    del g3, m3b, X3b, Y3b, rb3, outs3, sc3
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ prefill
    if not args.no_prefill:
        w3 = workloads.get("prefill_1l")
        m3 = DeviceModel(w3)
        T3 = 512
        X3 = to_dev(synth.activations(w3, T3))
        Y3 = torch.empty(T3, w3.hidden, device="cuda")
        r3 = RouteBuffers.alloc(T3, w3.top_k, w3.n_experts, with_logits=False)
        s3 = m3.prefill_scratch(T3)
        def chunk():
            m3.prefill(0, X3, w3.plan_cap, r3, s3, Y3)

        with torch.cuda.stream(stream):
            for _ in range(max(2, args.prefill_warmup)):
                chunk()
            stream.synchronize()
            p_eager_ms = event_ms(chunk, stream, args.prefill_reps)
            # the chunk's launches captured once and replayed, as for decode
            p_ms = event_ms(graph_of(chunk).replay, stream, args.prefill_reps)
            stage_ms = {}
            for stg, name in [(1, "gateup"), (2, "down")]:
                gs = graph_of(lambda: B.rl_prefill_stage(m3.desc, stg, 0, T3, w3.plan_cap, X3,
                                                         m3.residency, m3.pool, r3.c(), s3,
                                                         s3.numel(), Y3))
                stage_ms[name] = event_ms(gs.replay, stream, args.prefill_reps)
        plan = m3.read_plan(s3, T3)
        U = plan["n_buckets"]
        tb3 = B.rl_tensor_bytes(m3.desc)
        P = T3 * w3.top_k
        gb = {"gateup": U * 2 * tb3 + T3 * w3.hidden * 4 + P * w3.width * 4,
              "down": U * tb3 + P * w3.width * 4 + P * w3.hidden * 4}
        dom = max(stage_ms, key=stage_ms.get)
        ach = gb[dom] / (stage_ms[dom] * 1e-3) / 1e9
        stage_cold_ms = None
        if flush is not None:
            stage = 1 if dom == "gateup" else 2
            stage_cold_ms = cold_per_item_ms(
                [lambda: B.rl_prefill_stage(m3.desc, stage, 0, T3, w3.plan_cap, X3, m3.residency,
                                            m3.pool, r3.c(), s3, s3.numel(), Y3)] * 8)
        chunk_bytes = U * 3 * tb3 + w3.n_experts * w3.hidden * 4 + 2 * T3 * w3.hidden * 4
        line["prefill"] = {
            "value": round(T3 / (p_ms * 1e-3), 1),
            "unit": "tokens/s",
            "ms_per_chunk": round(p_ms, 4),
            "eager_ms_per_chunk": round(p_eager_ms, 4),
            "config": {"workload": "prefill_1l: one 512-token chunk, 5120 pairs, plan cap 512, "
                                   "same layer shape", "distinct_experts": U,
                       "chunk_bytes": chunk_bytes,
                       "chunk_frac_of_hbm": round(chunk_bytes / (p_ms * 1e-3) / 1e9
                                                  / PEAK_HBM_GBS, 4)},
            "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
            "roofline": {"kernel": {"gateup": "quantize_rows_kernel<true> + prefill_expert_kernel<true, 2>",
                                    "down": "quantize_rows_kernel<true> + prefill_expert_kernel<false, 2>"
                                    }[dom] if w3.qbits == 2 and w3.width % 256 == 0 else f"prefill {dom} stage",
                         "bound": "hbm",
                         "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_GBS, 4),
                         "traffic": stored_traffic("prefill_" + dom),
                         "bytes_per_launch": gb[dom],
                         "us_per_launch": round(stage_ms[dom] * 1e3, 2),
                         "cold": None if stage_cold_ms is None else {
                             "us_per_launch": round(stage_cold_ms * 1e3, 2),
                             "achieved": round(gb[dom] / (stage_cold_ms * 1e-3) / 1e9, 1),
                             "frac": round(gb[dom] / (stage_cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "how": "Infinity Cache flushed before each of 8 stage launches (graph "
                                    "of flush + stage pairs minus the flushes alone)"}},
        }

    # ------------------------------------- cold caches and the HBM read ceiling
    # The figures above are warm: the experts a launch streams may still sit in
    # the 256 MB Infinity Cache from an earlier replay.  Here each timed run
    # follows a 512 MiB read-modify-write of another buffer, which evicts them,
    # and a plain streaming read of 1 GiB gives the ceiling HBM reaches on
    # this box.
    if not args.no_cold:
        def token(t):
            return lambda: lib.moe_decode_layer(C.byref(d), 0, xp[t], W0, None, res, pool,
                                                C.byref(outs[t]), sp, sb, yp[t],
                                                torch.cuda.current_stream().cuda_stream)
        cold_tok_ms = cold_per_item_ms([token(t) for t in range(32)])
        big = torch.ones(1 << 28, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        with torch.cuda.stream(stream):
            read = lambda: B.rl_stream_read(big, big.numel() * 4, sink, stream.cuda_stream)
            read()
            read_ms = event_ms(read, stream, 5)
        cold = {"decode_us_per_token": round(cold_tok_ms * 1e3, 3),
                "decode_tokens_per_s": round(1e3 / cold_tok_ms, 1),
                "how": "Infinity Cache flushed before each of 32 tokens (graph of flush + token "
                       "pairs minus the flushes alone)",
                "hbm_read_ceiling_gbs": round(big.numel() * 4 / (read_ms * 1e-3) / 1e9, 1),
                "read_ceiling_kernel": "rl_stream_read over 1 GiB"}
        if not args.no_prefill:
            cold_chunk_ms = cold_per_item_ms([chunk] * 8)
            cold["prefill_ms_per_chunk"] = round(cold_chunk_ms, 4)
            cold["prefill_tokens_per_s"] = round(T3 / (cold_chunk_ms * 1e-3), 1)
        line["cold"] = cold
        del flush, big
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ stacks
    # decode_48l and prefill_48l (2-bit) by default; 3-bit prefill and the
    # bounded-pool decode stacks with --stacks
    if args.stacks or not args.no_stacks:
        from quantized_routed_expert_rl_amd.stack import DecodeStack, PrefillStack
        stacks = {}
        wd = workloads.get("decode_48l")
        md = DeviceModel(wd)
        ds = DecodeStack(md)
        Xd = to_dev(synth.activations(wd, wd.tokens))
        xin = torch.empty(wd.hidden, device="cuda")
        with torch.cuda.stream(stream):
            xin.copy_(Xd[0])
            ds.token(xin)
            gd = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gd, stream=stream):
                ds.token(xin)
            stream.synchronize()
            t0 = time.perf_counter()
            for t in range(wd.tokens):
                xin.copy_(Xd[t])
                gd.replay()
            stream.synchronize()
            dt = time.perf_counter() - t0
        flags = torch.stack([r.early_out for r in ds.routes]).cpu().numpy().ravel()
        stacks["decode_48l"] = {
            "tokens_per_s": round(wd.tokens / dt, 1), "us_per_token": round(dt * 1e6 / wd.tokens, 2),
            "layers": wd.n_layers, "flagged_layers_last_token": int(flags.sum()),
            "workload": "256 sequential tokens through 48 decode layers, Zipf-biased routing, "
                        "4608 of 24576 experts resident; one HIP graph per token"}
        del gd, md, ds
        torch.cuda.empty_cache()
        for qb in ((2, 3) if args.stacks else (2,)):
            wp = workloads.get("prefill_48l", qb)
            mp_ = DeviceModel(wp)
            ps = PrefillStack(mp_, wp.chunks, wp.plan_cap)
            Xp = to_dev(synth.activations(wp, wp.tokens))
            with torch.cuda.stream(stream):
                ps.prompt(Xp)
                stream.synchronize()
                reps = 3
                t0 = time.perf_counter()
                for _ in range(reps):
                    ps.prompt(Xp)
                stream.synchronize()
                dt = (time.perf_counter() - t0) / reps
            stacks[f"prefill_48l_{qb}bit"] = {
                "prompt_tokens_per_s": round(wp.tokens / dt, 1), "ms_per_prompt": round(dt * 1e3, 3),
                "token_layers_per_s": round(wp.tokens * wp.n_layers / dt, 1),
                "workload": f"1100-token prompt in chunks 512/512/76 through 48 prefill layers, "
                            f"Zipf-biased routing, all experts resident, {qb}-bit block weights"}
            del mp_, ps
            torch.cuda.empty_cache()
    if args.stacks or not args.no_stacks:
        # decode with a bounded pool (each layer's 224 most popular experts
        # resident) and miss service, without and with the pre-gated prefetch:
        # the native driver on the default line, the Python loop and the
        # early-out-path variants with --stacks
        from quantized_routed_expert_rl_amd.stack import (HostExpertStore, NativeServicedDecode,
                                                          ServicedDecodeStack)
        wh = workloads.get("decode_48l_hot")
        store = HostExpertStore(wh)
        Xh = to_dev(synth.activations(wh, wh.tokens))
        runs = [("_native", dict(native=True)), ("_native_prefetch", dict(native=True, prefetch=True))]
        if args.stacks:
            runs += [("", dict()), ("_prefetch", dict(prefetch=True)),
                     ("_early_out_path", dict(early_out_limit=1 << 30)),
                     ("_early_out_path_sticky", dict(early_out_limit=1 << 30, sticky=True)),
                     ("_native_early_out_path_sticky",
                      dict(native=True, early_out_limit=1 << 30, sticky=True))]
        for tag, kw in runs:
            mh = DeviceModel(wh, pool=store.device_pool(synth.residency(wh)))
            kw = dict(kw)
            native = kw.pop("native", False)
            sv = (NativeServicedDecode if native else ServicedDecodeStack)(mh, store, **kw)
            pf = kw.get("prefetch", False)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for t in range(wh.tokens):
                sv.token(Xh[t])
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            st = sv.stats
            n = st["tokens"]
            stacks["decode_48l_hot" + tag] = {
                "tokens_per_s": round(n / dt, 1), "ms_per_token": round(dt * 1e3 / n, 3),
                "early_outs_per_token": round(st["early_outs"] / n, 2),
                "critical_loads_per_token": round(st["loads"] / n, 2),
                "prefetch_loads_per_token": round(st["prefetch_loads"] / n, 2),
                "run_time_hit_rate": round(1 - st["loads"] / (n * wh.n_layers * wh.top_k), 4),
                "prediction_precision": (round(st["predicted_selected"]
                                               / (st["predictions"] * wh.top_k), 4)
                                         if st["predictions"] else None),
                "synchronous_tokens": st["sync_tokens"],
                "workload": f"{wh.tokens} sequential tokens through 48 decode layers, Zipf-biased "
                            "routing, 10752 slots seeded with each layer's 224 most popular experts, "
                            "misses loaded from host memory into least recently used slots"
                            + ("; next layer's experts predicted and prefetched" if pf else "")
                            + ("; early-out path on every token" if "early_out_limit" in kw else "")
                            + ("; one shared sticky flag" if kw.get("sticky") else "")
                            + ("; token loop in the library's native driver" if native
                               else "; token loop in Python")}
            del sv, mh
            torch.cuda.empty_cache()
        del store
    if args.stacks or not args.no_stacks:
        line["stacks"] = stacks

    # -------------------------------------------------------- cpu oracle
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import moe_oracle as O
        host_pool = synth.build_pool(w, model.table)
        Wr = synth.router_weights(w, 0)
        xs = synth.activations(w, T, stream=1)
        shape = O.LayerShape(w.hidden, w.n_experts, w.top_k, w.width, w.qbits)
        n = 0
        t0 = time.perf_counter()
        while n < T and (time.perf_counter() - t0 < args.cpu_seconds or n == 0):
            O.decode_layer(shape, xs[n], Wr, None, model.table[0], lambda s: host_pool[s])
            n += 1
        cdt = time.perf_counter() - t0
        blas = [i.get("num_threads", 1) for i in threadpool_info()]
        from threadpoolctl import threadpool_limits
        n1 = 0
        with threadpool_limits(1):
            t1 = time.perf_counter()
            while n1 < T and (time.perf_counter() - t1 < args.cpu_seconds / 3 or n1 == 0):
                O.decode_layer(shape, xs[n1], Wr, None, model.table[0], lambda s: host_pool[s])
                n1 += 1
            cdt1 = time.perf_counter() - t1
        cpu_model = next((l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                          if l.startswith("model name")), "unknown")
        line["cpu_baseline"] = {
            "value": round(n / cdt, 3), "unit": "tokens/s", "cores": max(blas + [1]),
            "kind": "oracle", "cpu_model": cpu_model, "logical_cpus": os.cpu_count(),
            "sample": f"first {n} of the {T} decode_1l tokens through oracle.decode_layer "
                      f"({cdt:.1f} s); float64 NumPy, BLAS threads {max(blas + [1])}, "
                      f"host has {os.cpu_count()} logical CPUs",
            "value_1_thread": round(n1 / cdt1, 3),
            "sample_1_thread": f"first {n1} tokens with BLAS limited to one thread ({cdt1:.1f} s)"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
