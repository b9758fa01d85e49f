#!/usr/bin/env python3
"""Benchmark: ternary FFN weight-stream throughput on one MI355X.

Workload: a 64-layer FFN weight stream with the 27B model's FFN shapes
(hidden 5120, intermediate 17408). The layers are independently seeded
synthetic ternary blocks: 2-bit codes with one fp16 scale per 128 weights,
4,545,576,960 bytes in all, about 17x the 256 MiB last-level cache. A step is
one pass over the 64 layers, in order, on one stream. Each layer runs
tb_rotate_quant_i8(x), tb_ffn_gateup_silu and tb_ffn_down. The layers are
not overlapped and no work is hoisted out of a step.

Printed (stdout, one JSON line): weight GB/s at M=1 (the value), us/layer,
% of the 8 TB/s HBM peak; the same at M=8; the 1-bit sign stream; the
roofline of the dominant kernel (gate/up GEMV), timed with HIP events on
its own stream; and the scalar CPU oracle timed on a bounded sample on
this host.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ternary FFN GEMV weight GB/s (% HBM peak) + µs/layer at M=1 and M=8"
HBM_PEAK_GBS = 8000.0
LAYERS = 64
SEED = 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=LAYERS)
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    p.add_argument("--skip-sign", action="store_true")
    p.add_argument("--skip-m8", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--profile-only", action="store_true",
                   help="one eager M=1 pass and exit (for rocprofv3 counter runs)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="only run a device copy of this many MiB (counter calibration)")
    return p.parse_args()


class Stream64:
    """Device weights and buffers of the layer stream at m rows."""

    def __init__(self, tb, layers_dev, xs, m, torch):
        self.tb, self.layers, self.m = tb, layers_dev, m
        dev = "cuda"
        k = layers_dev[0][0].k
        n = layers_dev[0][0].n
        self.x = [torch.from_numpy(x[:m].copy()).to(dev) for x in xs]
        self.q = torch.empty(m, k, dtype=torch.int8, device=dev)
        self.dq = torch.empty(m, k // 128, dtype=torch.float32, device=dev)
        self.h = torch.empty(m, n, dtype=torch.float32, device=dev)
        self.qh = torch.empty(m, n, dtype=torch.int8, device=dev)
        self.dqh = torch.empty(m, n // 128, dtype=torch.float32, device=dev)
        self.y = torch.empty(len(layers_dev), m, k, dtype=torch.float32, device=dev)

    def step(self):
        tb = self.tb
        for l, (wg, wu, wd) in enumerate(self.layers):
            tb.tb_rotate_quant_i8(self.x[l], self.q, self.dq)
            tb.tb_ffn_gateup_silu(wg, wu, self.q, self.dq, self.h)
            tb.tb_ffn_down(wd, self.h, self.qh, self.dqh, self.y[l])


def time_stream(torch, s: Stream64, steps: int, warmup: int, use_graph: bool):
    graph = None
    if use_graph:
        s.step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            s.step()
        torch.cuda.synchronize()
    run = graph.replay if graph else s.step
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps, graph


def gateup_event_timing(torch, s: Stream64, reps: int):
    """Mean gate/up kernel duration (s): HIP events around back-to-back gate/up launches.

    One pass launches tb_ffn_gateup_silu once per layer, over every layer's weights
    in turn (so each launch streams its 47 MB from HBM), on the current stream, with
    one event before and one after the whole pass. Kernels on one stream run back to
    back, so the mean is the kernel's own duration, comparable with the per-dispatch
    durations of a kernel trace.
    """
    tb = s.tb
    tb.tb_rotate_quant_i8(s.x[0], s.q, s.dq)
    torch.cuda.synchronize()
    n = len(s.layers)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total = 0.0
    for _ in range(reps):
        e0.record()
        for wg, wu, _wd in s.layers:
            tb.tb_ffn_gateup_silu(wg, wu, s.q, s.dq, s.h)
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1) * 1e-3
    return total / (reps * n)


def cpu_baseline(layers_host, xs, seconds: float):
    """The scalar oracle, single-threaded, on the first layers of the same stream."""
    import oracle
    o = oracle.default()
    t0 = time.perf_counter()
    done, nbytes = 0, 0
    while True:
        l = done % len(layers_host)
        o.ffn(layers_host[l], xs[l][:1])
        done += 1
        nbytes += layers_host[l].nbytes
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} FFN layers of the same 64-layer stream at M=1 "
                      f"({nbytes} weight bytes, {dt:.1f} s, 1 thread)"}


def copy_probe(torch, mib: int):
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy probe: {mib} MiB read + {mib} MiB written per copy, 3 copies")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("bench.py: only --gpus 1 is supported (the path is single-GPU; see the design notes)")
        sys.exit(2)

    import numpy as np
    import torch

    import ternary_weight_int8_tb_amd as tb
    from ternary_weight_int8_tb_amd import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib)
        return

    t0 = time.perf_counter()
    layers = synth.ffn_stream(SEED, args.layers, synth.FMT_TERNARY2, threads=16)
    xs = [synth.normal_rows(8, synth.HIDDEN, SEED, l) for l in range(args.layers)]
    layer_bytes = layers[0].nbytes
    step_bytes = layer_bytes * args.layers
    log(f"generated {args.layers} layers ({step_bytes} B) in {time.perf_counter() - t0:.1f} s")

    def upload(ls):
        return [tuple(tb.Matrix.upload(w) for w in (L.gate, L.up, L.down)) for L in ls]

    dev_layers = upload(layers)
    torch.cuda.synchronize()

    s1 = Stream64(tb, dev_layers, xs, 1, torch)
    if args.profile_only:
        s1.step()
        torch.cuda.synchronize()
        log("profile pass done")
        return

    use_graph = not args.no_graph
    t1, _ = time_stream(torch, s1, args.steps, args.warmup, use_graph)
    gb1 = step_bytes / t1 / 1e9
    log(f"M=1: {t1 * 1e3:.3f} ms/step, {t1 / args.layers * 1e6:.2f} us/layer, {gb1:.1f} GB/s")

    t_eager1, _ = time_stream(torch, s1, max(3, args.steps // 4), 1, False)
    gu_s = gateup_event_timing(torch, s1, max(2, args.steps // 4))
    gu_bytes = layers[0].gate.nbytes + layers[0].up.nbytes
    gu_gbs = gu_bytes / gu_s / 1e9
    log(f"gate/up kernel: {gu_s * 1e6:.2f} us/launch, {gu_gbs:.1f} GB/s (events, back to back)")

    res_m8 = None
    if not args.skip_m8:
        s8 = Stream64(tb, dev_layers, xs, 8, torch)
        t8, _ = time_stream(torch, s8, args.steps, args.warmup, use_graph)
        gb8 = step_bytes / t8 / 1e9
        gu8 = gateup_event_timing(torch, s8, max(2, args.steps // 4))
        res_m8 = {"value": round(gb8, 2), "unit": "GB/s", "ms_per_step": round(t8 * 1e3, 4),
                  "us_per_layer": round(t8 / args.layers * 1e6, 3),
                  "pct_hbm_peak": round(100 * gb8 / HBM_PEAK_GBS, 2),
                  "gateup_us": round(gu8 * 1e6, 3)}
        log(f"M=8: {t8 * 1e3:.3f} ms/step, {t8 / args.layers * 1e6:.2f} us/layer, {gb8:.1f} GB/s")
        del s8

    res_sign = None
    if not args.skip_sign:
        del dev_layers, s1
        torch.cuda.empty_cache()
        sl = synth.ffn_stream(SEED + 100, args.layers, synth.FMT_SIGN1, threads=16)
        sbytes = sl[0].nbytes * args.layers
        sdev = upload(sl)
        res_sign = {"bytes_per_step": sbytes}
        for m in (1, 8):
            ss = Stream64(tb, sdev, xs, m, torch)
            ts, _ = time_stream(torch, ss, args.steps, args.warmup, use_graph)
            res_sign[f"m{m}"] = {"value": round(sbytes / ts / 1e9, 2), "unit": "GB/s",
                                 "us_per_layer": round(ts / args.layers * 1e6, 3),
                                 "pct_hbm_peak": round(100 * sbytes / ts / 1e9 / HBM_PEAK_GBS, 2)}
            log(f"sign M={m}: {ts / args.layers * 1e6:.2f} us/layer, {sbytes / ts / 1e9:.1f} GB/s")
            del ss
        del sdev, sl

    cpu = cpu_baseline(layers[:4], xs, args.cpu_seconds)
    log(f"cpu oracle: {cpu['value']} GB/s ({cpu['sample']})")

    out = {
        "metric": METRIC,
        "value": round(gb1, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t1 * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"ffn_weight_stream_{args.layers}_layers_m1",
                   "layers": args.layers, "hidden": synth.HIDDEN, "intermediate": synth.INTER,
                   "rows": 1, "format": "ternary 2-bit, 128-weight blocks, fp16 scales",
                   "bytes_per_step": step_bytes,
                   "launch": "hip graph replay" if use_graph else "eager"},
        "us_per_layer": round(t1 / args.layers * 1e6, 3),
        "pct_hbm_peak": round(100 * gb1 / HBM_PEAK_GBS, 2),
        "eager_us_per_layer": round(t_eager1 / args.layers * 1e6, 3),
        "m8": res_m8,
        "sign1_stream": res_sign,
        "roofline": {"bound": "hbm", "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gemv_ring_kernel<1,TERNARY2,GATEUP> (tb_ffn_gateup_silu)",
                     "bytes_per_launch": gu_bytes, "us_per_launch": round(gu_s * 1e6, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
