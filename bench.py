#!/usr/bin/env python3
"""Throughput of the 1.58-bit linear layer on one MI355X.

One step is one pass of the whole path over one layer's synthetic inputs,
already resident in HBM: tern_quantize_pack (fp32 weights -> codes, scales
and packed bytes in one pass), tern_unpack, and tern_gemm (bf16 X times the
packed ternary weights, fused scale epilogue); --separate-quantize runs
tern_quantize and tern_pack as two calls instead.  The reported value is whole-step throughput
in effective TFLOP/s, 2*M*N*K per step; the roofline object describes the
dominant kernel (tern_gemm) measured with HIP events on the stream it is
launched on; the CPU baseline is the oracle timed on this host on a bounded
sample of the same step.

After the timed steps, every layer shape of the five workloads is timed on its
own ("rows"): tern_gemm per launch, and tern_gemm_ex with the bias and GELU
of the layers that have them, as effective TFLOP/s, GB/s and the fraction of
the bound that applies (MFMA or HBM); "dx_rows" time the input gradient
(tern_gemm_dx, tern_pack_transposed) on the backward shapes; "a8_rows" time
the 8-bit-activation layer (tern_quantize_act, tern_gemm_a8) on the forward
shapes against the int8 matrix peak.  The two few-token layers
cycle through a pool of distinct packed weights larger than every cache, so
that each launch streams its weights from HBM.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload flux_qkv]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tern_gemm effective TFLOP/s + % of MFMA/HBM roofline, FLUX linears M=4608"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
PEAK_I8_TOPS = 5000.0       # MI355X dense int8 matrix peak
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
CSRC = os.path.join(ROOT, "ternary_weight_quantized_tern_amd", "csrc")
GEMM_SRCS = [os.path.join(CSRC, f) for f in ("gemm.hip", "gemm_small.hip", "gemm_common.h")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="flux_qkv")
    ap.add_argument("--layers", type=int, default=0,
                    help="use only the first L layers of a multi-layer workload (0 = all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle's layer-output sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a device copy of this size (for counter calibration)")
    ap.add_argument("--gemm-only-reps", type=int, default=0,
                    help="after the steps, launch tern_gemm alone this many times (profiling)")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-layer-shape tables")
    ap.add_argument("--rows", choices=("all", "fwd", "dx", "a8"), default="all",
                    help="which per-layer-shape tables to time: the forward layer, the input "
                         "gradient, the 8-bit-activation layer, or all")
    ap.add_argument("--separate-quantize", action="store_true",
                    help="run quantize and pack as two calls in the step instead of the fused pass")
    ap.add_argument("--row-reps", type=int, default=30, help="timed launches per row")
    ap.add_argument("--pool-mib", type=int, default=1024,
                    help="packed-weight pool cycled by the few-token rows")
    return ap.parse_args()


def gemm_alg_bytes(m, k, n):
    return 2 * m * k + n * k // 4 + 4 * n + 2 * m * n


def source_digest(paths=GEMM_SRCS):
    """sha256 over the GEMM kernel sources, in a fixed order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload):
    """HBM bytes per tern_gemm launch from committed counter summaries, if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"tern_gemm_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("gemm_source_sha256") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(layers, inputs, target_s):
    """The oracle, as it stands, on this host: all weights of every layer go
    through quantize, pack and unpack; the layer output is computed for a
    leading sample of X rows and scaled to all M rows."""
    import oracle
    import tern_inputs
    cores = min(len(os.sched_getaffinity(0)), 16)
    t_weights = 0.0
    t_gemm = 0.0
    rows_used = []
    flops = 0
    for layer, (x, w) in zip(layers, inputs):
        t0 = time.perf_counter()
        t_ref, s_ref = oracle.oracle_quantize(w.numpy())
        p_ref = oracle.oracle_pack(t_ref)
        oracle.oracle_unpack(p_ref, layer.k)
        t_weights += time.perf_counter() - t0
        xb = tern_inputs.bf16_bits(x)
        pilot = min(8, layer.m)
        t0 = time.perf_counter()
        oracle.oracle_gemm(xb[:pilot], p_ref, s_ref, nthreads=cores)
        dt = time.perf_counter() - t0
        per_row = dt / pilot
        rows = int(max(pilot, min(layer.m, (target_s / len(layers)) / max(per_row, 1e-9))))
        if rows > pilot:
            t0 = time.perf_counter()
            oracle.oracle_gemm(xb[:rows], p_ref, s_ref, nthreads=cores)
            dt = time.perf_counter() - t0
        t_gemm += dt * layer.m / rows
        rows_used.append(rows)
        flops += 2 * layer.m * layer.n * layer.k
    t_step = t_weights + t_gemm
    return {
        "value": flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "seconds_per_step_extrapolated": t_step,
        "sample": (f"oracle quantize+pack+unpack on all weights ({t_weights:.2f} s), oracle layer "
                   f"output on the first {rows_used} X rows of M={[l.m for l in layers]} "
                   f"scaled to all rows; {cores} threads"),
    }


def roofline_of(flops, byts, seconds):
    """Effective rates and the fraction of the bound that applies."""
    tf = flops / seconds / 1e12
    gbs = byts / seconds / 1e9
    bound = "mfma" if flops / byts >= RIDGE else "hbm"
    t_ideal = max(flops / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9))
    return {"tflops": tf, "gbs": gbs, "pct_mfma": 100 * tf / PEAK_BF16_TFLOPS,
            "pct_hbm": 100 * gbs / PEAK_HBM_GBS, "bound": bound,
            "pct_roofline": 100 * t_ideal / seconds}


def time_rows(tern, tern_inputs, torch, dev, reps, pool_mib):
    """The layer on every layer shape of the workloads (layer 0 inputs of each
    shape): tern_gemm, and tern_gemm_ex where the layer's consumer applies a
    bias and the tanh-form GELU (the MLP up-projections; the single-stream
    in-projection, whose GELU covers only its MLP columns from 9216 on).
    Few-token shapes cycle through a pool of distinct packed weights of at
    least pool_mib MiB (seeded normal weights quantized on the GPU), one
    launch per pool entry."""
    import statistics
    W = tern_inputs.WORKLOADS
    shapes = [("single", W["single"][0], None),
              ("flux_qkv", W["flux_qkv"][0], None),
              ("flux_mlp.up", W["flux_mlp"][0], None),
              ("flux_mlp.up+gelu", W["flux_mlp"][0], (False, 0)),
              ("flux_mlp.down", W["flux_mlp"][1], None),
              ("flux_single_stream.in_proj", W["flux_single_stream"][0], None),
              ("flux_single_stream.in_proj+bias+gelu[9216:]", W["flux_single_stream"][0],
               (True, 9216)),
              ("flux_single_stream.out_proj", W["flux_single_stream"][1], None)]
    for l in W["dit"]:
        shapes.append((l.name, l, None))
        if ".up." in l.name:
            shapes.append((l.name + "+bias+gelu", l, (True, 0)))
    rows = []
    for name, layer, epi in shapes:
        x, w = tern_inputs.draw_layer(layer)
        xd = x.to(dev)
        ldp = tern.packed_row_bytes(layer.k)
        y = torch.empty((layer.m, layer.n), dtype=torch.bfloat16, device=dev)
        if epi is None:
            def launch(p_i, s_i, xd=xd, y=y, k=layer.k):
                tern.tern_gemm(xd, p_i, s_i, y, k)
        else:
            bias = None
            if epi[0]:
                gb = torch.Generator().manual_seed(layer.seed + 7)
                bias = (torch.randn(layer.n, generator=gb) * 0.02).to(dev)

            def launch(p_i, s_i, xd=xd, y=y, k=layer.k, bias=bias, act_from=epi[1]):
                tern.tern_gemm_ex(xd, p_i, s_i, y, bias, tern.TERN_ACT_GELU_TANH, act_from, k)
        pool = layer.m <= 64 and layer.n * layer.k >= (1 << 20)
        if pool:
            per = layer.n * ldp + 4 * layer.n
            count = max(1, -(-(pool_mib << 20) // per))
            gen = torch.Generator(device=dev).manual_seed(layer.seed)
            ps = torch.empty((count, layer.n, ldp), dtype=torch.uint8, device=dev)
            ss = torch.empty((count, layer.n), dtype=torch.float32, device=dev)
            t = torch.empty((layer.n, layer.k), dtype=torch.int8, device=dev)
            for i in range(count):
                wi = torch.randn((layer.n, layer.k), generator=gen, device=dev) * tern_inputs.W_STD
                tern.tern_quantize(wi, t, ss[i])
                tern.tern_pack(t, ps[i], layer.k)
            operands = [(ps[i], ss[i]) for i in range(count)]
            launches = count
        else:
            t, s = tern.quantize(w.to(dev))
            operands = [(tern.pack(t), s)]
            launches = reps
        for i in range(min(5, launches)):
            p_i, s_i = operands[i % len(operands)]
            launch(p_i, s_i)
        torch.cuda.synchronize()
        # Per-launch durations with events around each launch (they include
        # the host's submission gaps), and the same launches captured in a
        # HIP graph and replayed back to back (no host in the loop).
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(launches)]
        for i in range(launches):
            p_i, s_i = operands[i % len(operands)]
            ev[i][0].record()
            launch(p_i, s_i)
            ev[i][1].record()
        torch.cuda.synchronize()
        d = [a.elapsed_time(b) * 1e-3 for a, b in ev]
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            launch(*operands[0])
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            for i in range(launches):
                p_i, s_i = operands[i % len(operands)]
                launch(p_i, s_i)
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        graph.replay()
        g1.record()
        torch.cuda.synchronize()
        per_launch = g0.elapsed_time(g1) * 1e-3 / launches
        del graph
        med = statistics.median(d)
        flops = 2 * layer.m * layer.n * layer.k
        byts = gemm_alg_bytes(layer.m, layer.k, layer.n)
        if epi is not None and epi[0]:
            byts += 4 * layer.n  # the fp32 bias
        # The table's rate is the back-to-back (graph) time per launch unless
        # the event-bracketed median is lower.
        t = min(per_launch, med)
        row = {"layer": name, "m": layer.m, "k": layer.k, "n": layer.n,
               "launches": launches, "us_per_launch": t * 1e6,
               "graph_us_per_launch": per_launch * 1e6, "event_median_us": med * 1e6,
               "event_min_us": min(d) * 1e6, "alg_flops": flops, "alg_bytes": byts,
               "entry": "tern_gemm" if epi is None else "tern_gemm_ex"}
        if epi is not None:
            row["epilogue"] = {"bias": bool(epi[0]), "act": "gelu_tanh", "act_from": epi[1]}
        row.update(roofline_of(flops, byts, t))
        if pool:
            row["weight_pool_mib"] = round(launches * per / 2**20, 1)
        rows.append(row)
        print(f"# row {name}: {t * 1e6:.1f} us per launch, {row['tflops']:.0f} TFLOP/s, "
              f"{row['gbs']:.0f} GB/s, {row['pct_roofline']:.1f}% of roofline",
              file=sys.stderr, flush=True)
        del operands
        torch.cuda.empty_cache()
    return rows


def time_graph(torch, fn, launches):
    """Seconds per call of fn() with `launches` calls captured in one HIP graph
    and replayed back to back (after one eager warm-up call on a side stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(launches):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    del graph
    return g0.elapsed_time(g1) * 1e-3 / launches


def time_dx_rows(tern, tern_inputs, torch, dev, reps):
    """The input gradient of the layer, dX = bf16((dY * s) . T), on the backward
    shapes of the DiT and FLUX layers (dY [m, n] of the forward's output, dX
    [m, k]): tern_gemm_dx (the scaling pass and the ternary GEMM over n), and
    tern_pack_transposed of the layer's codes.  Seeded normal weights quantized
    on the GPU, dY ~ N(0, 1) in bf16; graph-replayed launches."""
    names = ["dit.up.m2048", "dit.down.m2048", "flux_qkv", "flux_mlp.up", "flux_mlp.down"]
    layers = {l.name: l for wl in tern_inputs.WORKLOADS.values() for l in wl}
    rows = []
    for name in names:
        layer = layers[name]
        m, k, n = layer.m, layer.k, layer.n
        _, w = tern_inputs.draw_layer(layer)
        p, s = tern.quantize_pack(w.to(dev))
        pt = torch.zeros((k, tern.packed_row_bytes(n)), dtype=torch.uint8, device=dev)
        g = torch.Generator(device=dev).manual_seed(layer.seed + 500)
        dy = torch.randn((m, n), generator=g, device=dev).to(torch.bfloat16)
        u = torch.empty_like(dy)
        dx = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
        tern.tern_pack_transposed(p, pt, n, k)
        t_pt = time_graph(torch, lambda: tern.tern_pack_transposed(p, pt, n, k), reps)
        t_dx = time_graph(torch, lambda: tern.tern_gemm_dx(dy, pt, s, u, dx, k), reps)
        flops = 2 * m * n * k
        # algorithmic bytes: dY, the codes, the scales and dX (the bf16 workspace
        # u, written once and read once, is the implementation's own traffic)
        byts = 2 * m * n + n * k // 4 + 4 * n + 2 * m * k
        row = {"layer": name + ".dx", "m": m, "n": n, "k": k, "us_per_launch": t_dx * 1e6,
               "alg_flops": flops, "alg_bytes": byts, "workspace_bytes": 4 * m * n,
               "entry": "tern_gemm_dx",
               "pack_transposed_us": t_pt * 1e6,
               "pack_transposed_gbs": 2 * (n * k // 4) / t_pt / 1e9}
        row.update(roofline_of(flops, byts, t_dx))
        rows.append(row)
        print(f"# dx row {name}: {t_dx * 1e6:.1f} us per launch, {row['tflops']:.0f} TFLOP/s, "
              f"{row['pct_roofline']:.1f}% of roofline; pack_transposed {t_pt * 1e6:.1f} us",
              file=sys.stderr, flush=True)
        del p, s, pt, dy, u, dx
        torch.cuda.empty_cache()
    return rows


def time_a8_rows(tern, tern_inputs, torch, dev, reps, pool_mib):
    """The 8-bit-activation layer on the forward shapes: tern_quantize_act
    (bf16 X -> int8 codes and per-token scales) and tern_gemm_a8, each
    graph-replayed, and the two together as the layer.  Rates against the
    int8 peak (5.0 POP/s) and the bf16 peak (the unquantized layer's bound).
    The few-token shapes cycle through at least pool_mib MiB of copies of the
    arranged weights, one launch per copy, so that every launch streams its
    weights from HBM; their rate is also given in GB/s."""
    W = tern_inputs.WORKLOADS
    shapes = [("flux_qkv", W["flux_qkv"][0], None),
              ("flux_mlp.up", W["flux_mlp"][0], None),
              ("flux_mlp.up+gelu", W["flux_mlp"][0], (False, 0)),
              ("flux_mlp.down", W["flux_mlp"][1], None),
              ("flux_single_stream.in_proj", W["flux_single_stream"][0], None),
              ("flux_single_stream.out_proj", W["flux_single_stream"][1], None),
              ("dit.up.m2048", W["dit"][0], None), ("dit.down.m2048", W["dit"][1], None),
              ("dit.up.m8", W["dit"][2], None), ("dit.down.m8", W["dit"][3], None)]
    rows = []
    for name, layer, epi in shapes:
        m, k, n = layer.m, layer.k, layer.n
        x, w = tern_inputs.draw_layer(layer)
        xd = x.to(dev)
        p, s = tern.quantize_pack(w.to(dev))
        p8 = tern.pack_a8(p, k)
        q, xs = tern.quantize_act(xd)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        act = tern.TERN_ACT_NONE if epi is None else tern.TERN_ACT_GELU_TANH
        af = 0 if epi is None else epi[1]

        pool = m <= 64
        p8s = [p8]
        if pool:
            count = max(1, -(-(pool_mib << 20) // (p8.numel() + 4 * n)))
            p8s = [p8.clone() for _ in range(count)]
        it = [0]

        def gemm():
            tern.tern_gemm_a8(q, xs, p8s[it[0] % len(p8s)], s, y, None, act, af, k)
            it[0] += 1

        def quant():
            tern.tern_quantize_act(xd, q, xs)

        def layer_fn():
            quant()
            gemm()

        launches = len(p8s) if pool else reps
        t_g = time_graph(torch, gemm, launches)
        t_q = time_graph(torch, quant, reps)
        t_l = time_graph(torch, layer_fn, launches)
        flops = 2 * m * n * k
        byts = m * k + n * k // 4 + 4 * n + 4 * m + 2 * m * n
        q_bytes = 2 * m * k + m * k + 4 * m
        row = {"layer": name, "m": m, "k": k, "n": n, "entry": "tern_gemm_a8",
               "us_per_launch": t_g * 1e6, "tops": flops / t_g / 1e12,
               "pct_i8_peak": 100 * flops / t_g / 1e12 / PEAK_I8_TOPS,
               "pct_bf16_peak": 100 * flops / t_g / 1e12 / PEAK_BF16_TFLOPS,
               "gbs": byts / t_g / 1e9, "alg_flops": flops, "alg_bytes": byts,
               "quantize_act_us": t_q * 1e6, "quantize_act_gbs": q_bytes / t_q / 1e9,
               "layer_us": t_l * 1e6, "layer_tops": flops / t_l / 1e12}
        if epi is not None:
            row["epilogue"] = {"bias": False, "act": "gelu_tanh", "act_from": af}
        if pool:
            row["weight_pool_mib"] = round(len(p8s) * (p8.numel() + 4 * n) / 2**20, 1)
        rows.append(row)
        print(f"# a8 row {name}: gemm {t_g * 1e6:.1f} us {row['tops']:.0f} TOP/s "
              f"({row['pct_i8_peak']:.1f}% of int8 peak); quantize_act {t_q * 1e6:.1f} us "
              f"{row['quantize_act_gbs']:.0f} GB/s; layer {t_l * 1e6:.1f} us",
              file=sys.stderr, flush=True)
        del p, p8, p8s, q, xs, y, xd
        torch.cuda.empty_cache()
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the ternary linear layer is measured on one MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch
    import tern_inputs
    import ternary_weight_quantized_tern_amd as tern

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    layers = list(tern_inputs.iter_layers(args.workload))
    if args.layers:
        layers = layers[: args.layers]
    print(f"# workload {args.workload}: {len(layers)} layer(s), drawing inputs", file=sys.stderr,
          flush=True)
    host_inputs = [tern_inputs.draw_layer(layer) for layer in layers]

    bufs = []
    for layer, (x, w) in zip(layers, host_inputs):
        ldp = tern.packed_row_bytes(layer.k)
        bufs.append(dict(
            x=x.to(dev), w=w.to(dev),
            t=torch.empty((layer.n, layer.k), dtype=torch.int8, device=dev),
            s=torch.empty((layer.n,), dtype=torch.float32, device=dev),
            p=torch.zeros((layer.n, ldp), dtype=torch.uint8, device=dev),
            tu=torch.empty((layer.n, layer.k), dtype=torch.int8, device=dev),
            y=torch.empty((layer.m, layer.n), dtype=torch.bfloat16, device=dev),
        ))
    torch.cuda.synchronize()

    # A step runs every row of the path on every layer: quantize and pack
    # (one fused pass, writing the codes, the scales and the packed bytes),
    # unpack, and the layer.  --separate-quantize runs quantize and pack as two
    # calls instead.
    if args.separate_quantize:
        names = ("tern_quantize", "tern_pack", "tern_unpack", "tern_gemm")
    else:
        names = ("tern_quantize_pack", "tern_unpack", "tern_gemm")

    def step(events=None):
        for li, (layer, b) in enumerate(zip(layers, bufs)):
            ev = events[li] if events is not None else None
            if ev:
                ev[0].record()
            j = 1
            if args.separate_quantize:
                tern.tern_quantize(b["w"], b["t"], b["s"])
                if ev:
                    ev[j].record()
                j += 1
                tern.tern_pack(b["t"], b["p"], layer.k)
            else:
                tern.tern_quantize_pack(b["w"], b["t"], b["p"], b["s"])
            if ev:
                ev[j].record()
            j += 1
            tern.tern_unpack(b["p"], b["tu"], layer.k)
            if ev:
                ev[j].record()
            j += 1
            tern.tern_gemm(b["x"], b["p"], b["s"], b["y"], layer.k)
            if ev:
                ev[j].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    per_step_events = [[[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
                        for _ in layers] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(per_step_events[i])
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps

    kern_ms = {nm: 0.0 for nm in names}
    gemm_launch_ms = []
    for i in range(args.steps):
        for li in range(len(layers)):
            ev = per_step_events[i][li]
            for j, nm in enumerate(names):
                d = ev[j].elapsed_time(ev[j + 1])
                kern_ms[nm] += d
                if nm == "tern_gemm":
                    gemm_launch_ms.append(d)
    launches = args.steps * len(layers)
    for nm in names:
        kern_ms[nm] /= launches

    flops_step = sum(2 * l.m * l.n * l.k for l in layers)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # Dominant kernel: tern_gemm.  Algorithmic work per launch, averaged over layers.
    gemm_flops = flops_step / len(layers)
    gemm_bytes = sum(gemm_alg_bytes(l.m, l.k, l.n) for l in layers) / len(layers)
    gemm_ms = kern_ms["tern_gemm"]
    ai = gemm_flops / gemm_bytes
    if ai >= RIDGE:
        achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS}
    else:
        achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
    roof["traffic"] = load_traffic(args.workload)
    roof["kernel"] = "tern_gemm"
    roof["avg_launch_ms"] = gemm_ms
    roof["alg_flops_per_launch"] = gemm_flops
    roof["alg_bytes_per_launch"] = gemm_bytes
    roof["gbs"] = gemm_bytes / (gemm_ms * 1e-3) / 1e9

    # The separate quantize and pack entry points, timed after the step loop
    # on the same buffers (not part of the step when the fused pass is used):
    # ten back-to-back launches of each between two events, queued behind one
    # layer so that the host's launch latency stays off the GPU's clock.
    if not args.separate_quantize:
        reps = 10
        b0, l0 = bufs[0], layers[0]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        tern.tern_gemm(b0["x"], b0["p"], b0["s"], b0["y"], l0.k)
        e[0].record()
        for _ in range(reps):
            tern.tern_quantize(b0["w"], b0["t"], b0["s"])
        e[1].record()
        for _ in range(reps):
            tern.tern_pack(b0["t"], b0["p"], l0.k)
        e[2].record()
        torch.cuda.synchronize()
        kern_ms["tern_quantize"] = e[0].elapsed_time(e[1]) / reps
        kern_ms["tern_pack"] = e[1].elapsed_time(e[2]) / reps
    # The fused conversion from bf16 weights (the 16-bit checkpoints the pages
    # start from), on the first layer's weights rounded to bf16, same timing.
    reps = 10
    b0, l0 = bufs[0], layers[0]
    w16 = b0["w"].to(torch.bfloat16)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    tern.tern_gemm(b0["x"], b0["p"], b0["s"], b0["y"], l0.k)
    e[0].record()
    for _ in range(reps):
        tern.tern_quantize_pack(w16, b0["t"], b0["p"], b0["s"])
    e[1].record()
    torch.cuda.synchronize()
    kern_ms["tern_quantize_pack.bf16_w"] = e[0].elapsed_time(e[1]) / reps
    del w16

    kernels = {}
    for nm in kern_ms:
        d = {"avg_ms": kern_ms[nm]}
        if nm in ("tern_quantize", "tern_pack"):
            d["in_step"] = bool(args.separate_quantize)
        if nm == "tern_quantize_pack.bf16_w":
            d["in_step"] = False
            byts = l0.n * l0.k * 2 + l0.n * l0.k + l0.n * ((l0.k + 3) // 4) + 4 * l0.n
        elif nm == "tern_quantize_pack":
            byts = sum(l.n * l.k * 4 + l.n * l.k + l.n * ((l.k + 3) // 4) + 4 * l.n
                       for l in layers) / len(layers)
        elif nm == "tern_quantize":
            ls = layers if args.separate_quantize else layers[:1]
            byts = sum(l.n * l.k * 4 + l.n * l.k + 4 * l.n for l in ls) / len(ls)
        elif nm == "tern_pack":
            ls = layers if args.separate_quantize else layers[:1]
            byts = sum(l.n * l.k + l.n * ((l.k + 3) // 4) for l in ls) / len(ls)
        elif nm == "tern_unpack":
            byts = sum(l.n * ((l.k + 3) // 4) + l.n * l.k for l in layers) / len(layers)
        else:
            byts = gemm_bytes
            d["tflops"] = gemm_flops / (kern_ms[nm] * 1e-3) / 1e12
        d["alg_bytes"] = byts
        d["gbs"] = byts / (kern_ms[nm] * 1e-3) / 1e9
        kernels[nm] = d

    if args.gemm_only_reps:
        b, layer = bufs[0], layers[0]
        for _ in range(args.gemm_only_reps):
            tern.tern_gemm(b["x"], b["p"], b["s"], b["y"], layer.k)
        torch.cuda.synchronize()
    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy calibration: {nbytes} bytes read and written", file=sys.stderr)

    rows = dx_rows = a8_rows = None
    if not args.no_rows and args.rows in ("all", "fwd"):
        print("# timing tern_gemm on every layer shape", file=sys.stderr, flush=True)
        rows = time_rows(tern, tern_inputs, torch, dev, args.row_reps, args.pool_mib)
    if not args.no_rows and args.rows in ("all", "dx"):
        print("# timing the input gradient on the backward shapes", file=sys.stderr, flush=True)
        dx_rows = time_dx_rows(tern, tern_inputs, torch, dev, args.row_reps)
    if not args.no_rows and args.rows in ("all", "a8"):
        print("# timing the 8-bit-activation layer on the forward shapes", file=sys.stderr,
              flush=True)
        a8_rows = time_a8_rows(tern, tern_inputs, torch, dev, args.row_reps, args.pool_mib)

    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(layers, host_inputs, args.cpu_seconds)

    shape = layers[0]
    config = {"workload": args.workload, "layers": len(layers), "m": shape.m, "k": shape.k,
              "n": shape.n, "step": "+".join(names),
              "x": f"bf16 {shape.x_dist}", "w": "fp32 N(0, 0.02^2)", "seed": shape.seed}
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "rows": rows,
        "dx_rows": dx_rows,
        "a8_rows": a8_rows,
        "peaks": {"bf16_mfma_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS,
                  "i8_mfma_tops": PEAK_I8_TOPS},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
