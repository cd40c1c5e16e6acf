"""Benchmark of the block-FP8 MoE layer on one MI355X.

A step is one pass of the whole layer (router, activation quantisation,
routed FP8 experts, SwiGLU, shared expert, gate, combine) on one bf16 row of
the decode layer (H 2048, 256 experts top-8, I = Is = 512). Steps rotate over
40 independently generated layers and rows (32.5 GB of weights), so the
256 MB Infinity Cache cannot hold the working set (one layer touches 32.5 MB). The K timed steps
are captured once in a HIP graph (the way a frame step runs) and replayed.

The JSON line's `value` is the decode layer's algorithmic HBM bytes per step
divided by the time per step, in TB/s; `us_per_layer` is that time. The
decode layer is one kernel launch; its own duration is also timed live with
HIP events around eager launches on the stream it runs on, which gives the
roofline's `achieved`. `traffic` comes from the committed rocprofv3 counter
summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size)
when the kernel sources still hash to the value recorded with it, else null.
The same run also times 1024-row chunks (uniform, skewed and all-on-16-experts
routing) and reports FP8 TFLOP/s; times the per-frame stack (the 40 layers
chained on one row with an RMS renormalisation between layers); and times
the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import statistics
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import block_fp8_mixture_router_amd as moe  # noqa: E402
from block_fp8_mixture_router_amd import inputs  # noqa: E402

METRIC = "decode µs/layer + HBM TB/s; 1024-row chunk FP8 TFLOP/s (% of peak)"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0  # dense MFMA, no sparsity


def decode_bytes(shape, rows=1, experts_touched=None, shared_fp8=False) -> int:
    """Algorithmic HBM bytes of one layer pass: every touched expert's codes
    and scales once, shared expert (bf16, or block-FP8 codes and scales),
    router, gate vector, x and y."""
    k = shape.top_k * rows if experts_touched is None else experts_touched
    routed = k * shape.expert_bytes()
    h, i_s = shape.hidden, shape.shared_inter
    shared = (3 * h * i_s + 3 * (h // 128) * (i_s // 128) * 4) if shared_fp8 else 3 * h * i_s * 2
    router = shape.n_experts * shape.hidden * 2
    return routed + shared + router + shape.hidden * 2 + rows * shape.hidden * 2 * 2


def fp8_flops(shape, rows) -> int:
    return 2 * rows * shape.top_k * 3 * shape.hidden * shape.inter


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "block_fp8_mixture_router_amd", "csrc")


DECODE_SOURCES = ("decode.hip", "topk.h", "common.h", "kernels.h")


def source_hash(files=DECODE_SOURCES) -> str:
    """Hash of the HIP sources a kernel is built from (its counters are void
    once these change)."""
    h = hashlib.sha256()
    for name in sorted(files):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str, src_hash: str):
    """HBM bytes per launch from a committed counter summary, if still valid."""
    path = os.path.join(PROFILES, name)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def kernel_time_live(step_fn, n, stream, batches=5):
    """Average duration of one launch, from HIP events on the stream the
    kernel runs on, each pair bracketing n back-to-back eager launches (a
    spin kernel keeps the GPU busy while the host enqueues, so no host gap
    lands inside a bracket). Returns (mean, min) over the batches."""
    per = []
    for b in range(batches):
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(50e6))
            a_ev.record(stream)
            for i in range(n):
                step_fn(b * n + i)
            b_ev.record(stream)
        torch.cuda.synchronize()
        per.append(a_ev.elapsed_time(b_ev) / 1e3 / n)
    return sum(per) / len(per), min(per)


def copy_calibration(nbytes=256 << 20, reps=10):
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters (run this under rocprofv3 --pmc)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def graph_time(step_fn, n_steps, warmup, stream, replays=5):
    """Capture n_steps calls in one graph, replay it `replays` times (each
    replay timed by HIP events on the stream); returns (median seconds per
    replay, the graph, every replay's seconds)."""
    torch.cuda.synchronize()  # inputs were prepared on the default stream
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step_fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n_steps):
            step_fn(i)
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            start.record(stream)
            g.replay()
            end.record(stream)
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) / 1e3)
    return statistics.median(times), g, times


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, host_layers, reps=5):
    """The oracle, as it stands, timed on the host cores: the decode row
    (config 1, also the 40-layer stack's per-layer step), and rows of the
    uniform and skewed 1024-row chunks (configs 2 and 3), at every thread
    the oracle gets by default and at one thread. Each figure is the median
    of `reps` timed calls on a bounded sample of rows (the oracle's time is
    linear in rows: every (row, slot) pair and every row is computed on its
    own), scaled to the config's unit."""
    import oracle
    nproc = oracle.num_threads()
    layer = host_layers[0]
    x_dec = inputs.make_x(shape, 256, seed=99)
    x_chunk = inputs.make_x(shape, 1024, seed=1)
    import dataclasses
    skewed = dataclasses.replace(layer, router_bias=inputs.skew_bias(shape.n_experts))
    oracle.forward(shape, layer, x_dec[:1])  # warm

    def med_per_row(lw, x, rows):
        per = []
        for r in range(reps):
            xs = x[(r * rows) % x.shape[0]:][:rows]
            t0 = time.perf_counter()
            oracle.forward(shape, lw, xs)
            per.append((time.perf_counter() - t0) / xs.shape[0])
        return statistics.median(per)

    figures = {}
    for threads in (nproc, 1):
        oracle.set_num_threads(threads)
        rows = 256 if threads > 1 else 8
        dec = med_per_row(layer, x_dec, rows)
        uni = med_per_row(layer, x_chunk, rows)
        skw = med_per_row(skewed, x_chunk, rows)
        # one row per call, layer after layer: the stack's per-layer step
        # (the renormalisation between layers costs microseconds)
        per = []
        for r in range(reps):
            t0 = time.perf_counter()
            oracle.forward(shape, host_layers[r % len(host_layers)], x_dec[r:r + 1])
            per.append(time.perf_counter() - t0)
        one = statistics.median(per)
        figures[f"threads{threads}"] = {
            "decode_1row_us_per_row_batched": round(dec * 1e6, 1),
            "decode_1row_tbs_batched": round(decode_bytes(shape) / dec / 1e12, 6),
            "stack40_decode_us_per_layer": round(one * 1e6, 1),
            "chunk1024_uniform_ms_per_chunk": round(uni * 1024 * 1e3, 1),
            "chunk1024_skewed_ms_per_chunk": round(skw * 1024 * 1e3, 1),
            "chunk1024_uniform_fp8_tflops": round(fp8_flops(shape, 1024) / (uni * 1024) / 1e12,
                                                  6),
            "rows_per_sample": rows,
        }
    oracle.set_num_threads(nproc)
    head = figures[f"threads{nproc}"]
    return {
        "value": head["decode_1row_tbs_batched"],
        "unit": "TB/s",
        "us_per_layer": head["decode_1row_us_per_row_batched"],
        "cores": nproc,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"median of {reps} oracle calls per figure: {figures[f'threads{nproc}']['rows_per_sample']}"
                  f" rows per call at {nproc} threads, 8 at 1 thread (decode rows; rows of "
                  "the uniform and skewed 1024-row chunks, scaled to 1024 rows); the stack "
                  "figure is one-row calls on successive layers; value = the decode layer's "
                  "bytes over the per-row time of batched decode rows",
        "figures": figures,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1600)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--stack-passes", type=int, default=25)
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--chunk-steps", type=int, default=16)
    ap.add_argument("--no-chunk", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-addnorm", action="store_true")
    ap.add_argument("--no-gemv", action="store_true",
                    help="skip the one-row bf16 projections")
    ap.add_argument("--no-control", action="store_true",
                    help="skip the chunks of the two variants (no activation quantisation, "
                    "block-FP8 shared expert)")
    ap.add_argument("--live-launches", type=int, default=200)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        torch.cuda.set_device(0)
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is benchmarked at its single-GPU shape)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if not moe.supported(0):
        raise SystemExit("cuda:0 is not a gfx950 GPU")
    shape = inputs.DECODE
    L = args.layers
    print(f"[bench] generating {L} decode layers", file=sys.stderr, flush=True)
    layers = [inputs.make_layer(shape, seed=0, layer=l, device="cuda") for l in range(L)]
    wstructs = [moe.weights_struct(lw) for lw in layers]
    xs = inputs.make_x(shape, L, seed=0, device="cuda")
    ys = torch.empty_like(xs)
    cfg = moe.config(shape)
    ws = moe.alloc_workspace(cfg, 1024)
    stream = torch.cuda.Stream()

    def step(i):
        j = i % L
        moe.forward(cfg, layers[j], xs[j:j + 1], y=ys[j:j + 1], workspace=ws,
                    wstruct=wstructs[j], stream=stream)

    nbytes = decode_bytes(shape)
    rec = {
        "metric": METRIC, "value": None, "unit": "TB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": "decode_1row", "hidden": shape.hidden,
                   "experts": shape.n_experts, "top_k": shape.top_k, "inter": shape.inter,
                   "shared_inter": shape.shared_inter, "rows": 1, "layers_rotated": L},
    }
    if not args.no_decode:
        print(f"[bench] decode: {args.steps} steps", file=sys.stderr, flush=True)
        secs, _, reps = graph_time(step, args.steps, args.warmup, stream)
        us = secs / args.steps * 1e6
        gbs = nbytes / (us * 1e-6) / 1e9
        rec["value"] = round(gbs / 1e3, 4)
        rec["ms_per_step"] = secs / args.steps * 1e3
        rec["us_per_layer"] = round(us, 3)
        rec["decode_replays_us_per_layer"] = [round(t / args.steps * 1e6, 3) for t in reps]
        rec["decode_timing"] = (f"median of {len(reps)} replays of one graph of {args.steps} "
                                "layer calls on 40 rotated layers")
        # the decode layer is one kernel launch: time those launches live
        k_avg, k_min = kernel_time_live(step, args.live_launches, stream)
        kgbs = nbytes / k_avg / 1e9
        traffic = measured_traffic("decode_fused_kernel.decode_1row.pmc.json", source_hash())
        rec["roofline"] = {"bound": "hbm", "achieved": round(kgbs, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                           "traffic": traffic,
                           "kernel": "moe::decode_fused_kernel (the whole layer, one launch)",
                           "bytes_per_launch": nbytes,
                           "kernel_us_avg": round(k_avg * 1e6, 3),
                           "kernel_us_min_batch": round(k_min * 1e6, 3),
                           "launches_timed": 5 * args.live_launches}
    if not args.no_decode and not args.no_control:
        # one row through the expert-grouped kernels (MOE_FORCE_GROUPED): the
        # chunk-invariant way to run a row, its bytes equal to that row's
        # inside any chunk; same 40 rotated layers as the decode line
        cfg_g = moe.config(shape, moe.FORCE_GROUPED)

        def gstep1(i):
            j = i % L
            moe.forward(cfg_g, layers[j], xs[j:j + 1], y=ys[j:j + 1], workspace=ws,
                        wstruct=wstructs[j], stream=stream)

        n1 = max(L, args.steps // 8)
        print(f"[bench] one row, grouped kernels: {n1} steps", file=sys.stderr, flush=True)
        g1secs, _, _ = graph_time(gstep1, n1, L, stream)
        rec["row1_grouped_invariant"] = {"us_per_layer": round(g1secs / n1 * 1e6, 3),
                                         "note": "one row on the grouped kernels "
                                                 "(chunk-invariant bytes)"}
        # the two switches on the one-row kernel: the block-FP8 shared expert
        # (on as many rotated layers, its shared matrices block-FP8) and the
        # no-activation-quantisation control
        cfg_sf = moe.config(shape, moe.SHARED_FP8)
        ws_sf = moe.alloc_workspace(cfg_sf, 1)
        lsf = [inputs.make_layer(shape, seed=0, layer=l, device="cuda", shared_fp8=True)
               for l in range(L)]
        wsf = [moe.weights_struct(lw) for lw in lsf]
        cfg_nq = moe.config(shape, moe.NO_ACT_QUANT)
        ws_nq = moe.alloc_workspace(cfg_nq, 1)

        def sfstep(i):
            j = i % L
            moe.forward(cfg_sf, lsf[j], xs[j:j + 1], y=ys[j:j + 1], workspace=ws_sf,
                        wstruct=wsf[j], stream=stream)

        def nqstep(i):
            j = i % L
            moe.forward(cfg_nq, layers[j], xs[j:j + 1], y=ys[j:j + 1], workspace=ws_nq,
                        wstruct=wstructs[j], stream=stream)

        n2 = max(L, args.steps // 4)
        print(f"[bench] one row, switches: {n2} steps each", file=sys.stderr, flush=True)
        sfsecs, _, _ = graph_time(sfstep, n2, L, stream)
        sf_us = sfsecs / n2 * 1e6
        sf_bytes = decode_bytes(shape, shared_fp8=True)
        rec["decode_1row_shared_fp8"] = {
            "us_per_layer": round(sf_us, 3), "bytes_per_layer": sf_bytes,
            "tbs_algorithmic": round(sf_bytes / (sf_us * 1e-6) / 1e12, 4),
            "note": "block-FP8 shared expert as slot K of the one-row kernel"}
        nqsecs, _, _ = graph_time(nqstep, n2, L, stream)
        rec["decode_1row_no_act_quant"] = {
            "us_per_layer": round(nqsecs / n2 * 1e6, 3),
            "note": "fidelity control on the one-row kernel (bf16 x and h, decoded e4m3 weights)"}
        del lsf, wsf, ws_sf, ws_nq
    if not args.no_chunk:
        chunk = {}
        xc = inputs.make_x(shape, 1024, seed=1, device="cuda")
        yc = torch.empty_like(xc)
        nrot = min(4, L)
        # the uniform and skewed chunks are HBM-bound; the concentrated one (all
        # rows on 16 experts, ~512 rows each) is bound by the FP8 matrix cores
        for name, bias_fn in (("chunk1024_uniform", None),
                              ("chunk1024_skewed", inputs.skew_bias),
                              ("chunk1024_16experts", inputs.concentrated_bias)):
            bias = bias_fn(shape.n_experts).cuda() if bias_fn else None
            skew = bias is not None
            ls = []
            for l in range(nrot):
                lw = layers[l]
                if skew:
                    import dataclasses
                    lw = dataclasses.replace(lw, router_bias=bias)
                ls.append((lw, moe.weights_struct(lw)))
            ids, _, _ = moe.route(cfg, xc, ls[0][0].router_w, bias,
                                  logits=torch.empty(1024, shape.n_experts, device="cuda"))
            touched = int(torch.unique(ids).numel())

            def cstep(i, ls=ls):
                lw, wsr = ls[i % nrot]
                moe.forward(cfg, lw, xc, y=yc, workspace=ws, wstruct=wsr, stream=stream)

            print(f"[bench] {name}: {args.chunk_steps} steps", file=sys.stderr, flush=True)
            csecs, _, _ = graph_time(cstep, args.chunk_steps, 2, stream)
            cus = csecs / args.chunk_steps * 1e6
            fl = fp8_flops(shape, 1024)
            cb = decode_bytes(shape, rows=1024, experts_touched=touched)
            tflops = fl / (cus * 1e-6) / 1e12
            attain = min(FP8_PEAK_TFLOPS, fl / cb * HBM_PEAK_GBS / 1e3)
            chunk[name] = {"us_per_chunk": round(cus, 2), "fp8_tflops": round(tflops, 1),
                           "pct_fp8_peak": round(100 * tflops / FP8_PEAK_TFLOPS, 2),
                           "roofline_attainable_tflops": round(attain, 1),
                           "pct_of_attainable": round(100 * tflops / attain, 1),
                           "hbm_tbs_algorithmic": round(cb / (cus * 1e-6) / 1e12, 3),
                           "experts_touched": touched, "algorithmic_bytes": cb}
        if not args.no_control:
            # the no-activation-quantisation control on the uniform chunk
            # (bf16 x and h times decoded e4m3 weights; untuned kernels)
            cfg_nq = moe.config(shape, moe.NO_ACT_QUANT)
            ws_nq = moe.alloc_workspace(cfg_nq, 1024)
            lsu = [(layers[l], moe.weights_struct(layers[l])) for l in range(nrot)]

            def nstep(i):
                lw, wsr = lsu[i % nrot]
                moe.forward(cfg_nq, lw, xc, y=yc, workspace=ws_nq, wstruct=wsr, stream=stream)

            print(f"[bench] control: {args.chunk_steps} steps", file=sys.stderr, flush=True)
            nsecs, _, _ = graph_time(nstep, args.chunk_steps, 2, stream)
            chunk["chunk1024_uniform_no_act_quant"] = {
                "us_per_chunk": round(nsecs / args.chunk_steps * 1e6, 2),
                "note": "fidelity control: bf16 activations, decoded e4m3 weights"}
            del ws_nq
            # the block-FP8 shared-expert variant on the uniform chunk (the
            # shared matrices as one more grouped FP8 expert over every row)
            cfg_sf = moe.config(shape, moe.SHARED_FP8)
            ws_sf = moe.alloc_workspace(cfg_sf, 1024)
            lsf = []
            for l in range(nrot):
                lw = inputs.make_layer(shape, seed=0, layer=l, device="cuda", shared_fp8=True)
                lsf.append((lw, moe.weights_struct(lw)))

            def fstep(i):
                lw, wsr = lsf[i % nrot]
                moe.forward(cfg_sf, lw, xc, y=yc, workspace=ws_sf, wstruct=wsr, stream=stream)

            print(f"[bench] shared fp8: {args.chunk_steps} steps", file=sys.stderr, flush=True)
            fsecs, _, _ = graph_time(fstep, args.chunk_steps, 2, stream)
            chunk["chunk1024_uniform_shared_fp8"] = {
                "us_per_chunk": round(fsecs / args.chunk_steps * 1e6, 2),
                "note": "variant: block-FP8 shared expert run as a grouped expert"}
            del ws_sf, lsf
        rec["chunk"] = chunk
    if not args.no_stack and L >= 2:
        # the per-frame stack: L independent decode layers chained on one row,
        # RMS-renormalised between layers; moe_forward_stack launches one
        # kernel per layer, each later layer renormalising its predecessor's
        # output in its prologue (L launches per pass)
        arr = moe.weights_array(wstructs)
        x0 = inputs.make_x(shape, 1, seed=7, device="cuda")
        y_st = torch.empty_like(x0)

        def spass(i):
            moe.forward_stack(cfg, arr, x0, y=y_st, eps=1e-6, workspace=ws, stream=stream)

        print(f"[bench] stack of {L} layers: {args.stack_passes} passes", file=sys.stderr,
              flush=True)
        ssecs, _, _ = graph_time(spass, args.stack_passes, 2, stream)
        sus = ssecs / args.stack_passes * 1e6
        rec["stack"] = {"workload": f"stack{L}_decode", "layers": L,
                        "us_per_pass": round(sus, 2), "us_per_layer": round(sus / L, 3),
                        "hbm_tbs_algorithmic": round(L * nbytes / (sus * 1e-6) / 1e12, 4),
                        "launches_per_pass": L,
                        "passes_timed": args.stack_passes}
    if not args.no_addnorm:
        # the step in front of the layer: residual add + RMS norm + 1x128 FP8
        # groups of the normed rows, one row and a 1024-row chunk, 8 rotated
        # buffer sets (HBM-bound: bytes per launch below)
        an = {}
        H = shape.hidden
        for rows in (1, 1024):
            sets = []
            for k in range(8):
                g = torch.Generator(device="cuda").manual_seed(500 + k)
                hs = torch.randn(rows, H, device="cuda", generator=g).to(torch.bfloat16)
                rs = torch.randn(rows, H, device="cuda", generator=g).to(torch.bfloat16)
                outs = (torch.empty_like(rs), torch.empty_like(hs),
                        torch.empty(rows, H, dtype=torch.uint8, device="cuda"),
                        torch.empty(rows, H // 128, dtype=torch.float32, device="cuda"))
                sets.append((hs, rs, outs))
            nw = torch.ones(H, dtype=torch.bfloat16, device="cuda")

            def astep(i, sets=sets, nw=nw):
                hs, rs, (ro, xo, qo, so) = sets[i % len(sets)]
                moe.add_rmsnorm_quant(hs, rs, nw, eps=1e-6, residual_out=ro, x=xo, q=qo,
                                      scales=so, stream=stream)

            n = 800 if rows == 1 else 200
            asecs, _, _ = graph_time(astep, n, 8, stream)
            aus = asecs / n * 1e6
            abytes = rows * (4 * H + 4 * H + H + (H // 128) * 4) + 2 * H
            an[f"rows{rows}"] = {"us": round(aus, 3), "bytes": abytes,
                                 "hbm_tbs": round(abytes / (aus * 1e-6) / 1e12, 3)}
        rec["add_rmsnorm_quant"] = an
    if not args.no_gemv:
        # one-row bf16 projections of the rest of the backbone row (sizes
        # around hidden 2048), each over enough rotated weight copies (more
        # than 256 MiB) that no cache holds them between launches
        gv = {}
        K0 = shape.hidden
        for (N, K) in ((4096, K0), (K0, 2 * K0), (8 * K0, K0)):
            ncopy = max(4, -(-(384 << 20) // (N * K * 2)))
            g = torch.Generator(device="cuda").manual_seed(N + K)
            Ws = [(torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
                  for _ in range(ncopy)]
            xg = torch.randn(1, K, device="cuda", generator=g).to(torch.bfloat16)
            yg = torch.empty(1, N, dtype=torch.bfloat16, device="cuda")

            def gstep(i, Ws=Ws, xg=xg, yg=yg):
                moe.bf16_gemv(Ws[i % len(Ws)], xg, y=yg, stream=stream)

            n = 4 * ncopy
            gsecs, _, _ = graph_time(gstep, n, ncopy, stream)
            gus = gsecs / n * 1e6
            gbytes = N * K * 2 + K * 2 + N * 2
            tbs = gbytes / (gus * 1e-6) / 1e12
            gv[f"N{N}_K{K}_rows1"] = {"us": round(gus, 3), "bytes": gbytes,
                                      "hbm_tbs": round(tbs, 3),
                                      "frac_hbm_peak": round(tbs * 1e3 / HBM_PEAK_GBS, 3)}
            del Ws
        rec["bf16_gemv"] = gv
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(shape, [layers[l].to("cpu") for l in range(min(5, L))])
    rec["source_hash"] = source_hash()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
