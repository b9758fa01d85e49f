#!/usr/bin/env python3
"""Benchmark: ternary FFN weight-stream throughput on one MI355X.

Workload: a 64-layer FFN weight stream with the 27B model's FFN shapes
(hidden 5120, intermediate 17408). The layers are independently seeded
synthetic ternary blocks: 2-bit codes with one fp16 scale per 128 weights,
4,545,576,960 bytes in all, about 17x the 256 MiB last-level cache. Each layer
takes its own N(0,1) activation rows. A step is one pass over the 64 layers,
in order: per layer rotate + quantise x, gate/up + SiLU gate, rotate +
quantise h, down. Nothing is hoisted out of a step.

Two complete paths are timed at M=1, both with strict layer order (layer l+1
starts after every output of layer l is written; no layer is overlapped with
another and no work is hoisted out of a step): the fused entry point
tb_ffn_layers (one persistent launch per 32 layers), and the three separate
calls per layer (tb_rotate_quant_i8, tb_ffn_gateup_silu, tb_ffn_down) replayed
from a HIP graph (and eagerly). The value is the faster of the two; the JSON
names it. Also printed: the same at M=8; the 1-bit sign stream; the roofline
of the headline path's dominant kernel, timed with HIP events on the stream it
runs on; a 4 GiB streaming-read probe; and the scalar CPU oracle timed on a
bounded sample on this host.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

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


class Fused64:
    """The same stream through tb_ffn_layers: one call per step (one launch per 32 layers)."""

    def __init__(self, tb, layers_dev, xs, m, torch):
        self.tb, self.m = tb, m
        dev = "cuda"
        k = layers_dev[0][0].k
        n = layers_dev[0][0].n
        self.arr = tb.FfnLayers(layers_dev)
        self.x = torch.from_numpy(np.stack([x[:m] for x in xs])).to(dev)
        self.y = torch.empty(len(layers_dev), m, k, dtype=torch.float32, device=dev)
        self.ws = torch.empty(tb.tb_ffn_workspace_bytes(m, k, n), dtype=torch.uint8, device=dev)
        tb.tb_ffn_workspace_init(self.ws)

    def step(self):
        self.tb.tb_ffn_layers(self.arr, self.x, self.ws, self.y)

    def check(self):
        err = self.tb.tb_ffn_workspace_error(self.ws)
        if err:
            raise RuntimeError(f"tb_ffn_layers reported error {err}: not all workgroups resident")


def time_stream(torch, s, steps: int, warmup: int, use_graph: bool):
    """Time `steps` passes after `warmup` untimed ones.

    Returns (mean seconds per step over the whole timed region, bracketed by device
    synchronisation; per-step seconds from HIP events recorded between the steps)."""
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
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        run()
        ev[i + 1].record()
    torch.cuda.synchronize()
    total = (time.perf_counter() - t0) / steps
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(steps)]
    return total, per


def read_probe(torch, nbytes: int, reps: int = 5):
    """Achievable HBM read bandwidth: a 16-byte non-temporal streaming read of nbytes."""
    import ctypes
    from ternary_weight_int8_tb_amd import build as tb_build
    path = os.path.join(ROOT, "ternary_weight_int8_tb_amd", "libtb_probe.so")
    if not os.path.exists(path):
        tb_build.build()
    P = ctypes.CDLL(path)
    P.tbp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    best = 0.0
    for grid in (256, 512, 1024):
        P.tbp_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, st)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            P.tbp_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, st)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best


def gateup_event_timing(torch, s: Stream64, reps: int):
    """Mean gate/up kernel duration (s): HIP events around back-to-back gate/up launches
    over every layer's weights (each launch streams its 47 MB from HBM), on the current
    stream, which is the stream the library launches on."""
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


def call_breakdown(torch, s: Stream64, layer_s: float, reps: int):
    """Per-call device time of the separate-call stream, without a tracer.

    Each call type is captured 64 times back to back (one per layer's weights) in a HIP
    graph and timed with HIP events around `reps` replays, so a figure is the kernel's
    duration plus the dependency between two launches on one stream. The stream's layer
    time minus the sum of its three calls is what changes when the calls alternate
    (caches, launch shapes). Returns microseconds per call and kernel-only GB/s."""
    tb, n = s.tb, len(s.layers)
    tb.tb_rotate_quant_i8(s.x[0], s.q, s.dq)
    tb.tb_ffn_gateup_silu(*s.layers[0][:2], s.q, s.dq, s.h)
    tb.tb_rotate_quant_i8(s.h, s.qh, s.dqh)
    torch.cuda.synchronize()
    calls = {
        "rotate_quant_x": lambda l, w: tb.tb_rotate_quant_i8(s.x[l], s.q, s.dq),
        "gateup_silu": lambda l, w: tb.tb_ffn_gateup_silu(w[0], w[1], s.q, s.dq, s.h),
        "rotate_quant_h": lambda l, w: tb.tb_rotate_quant_i8(s.h, s.qh, s.dqh),
        "down_gemv": lambda l, w: tb.tb_gemv_ternary(w[2], s.qh, s.dqh, s.y[l]),
        "ffn_down": lambda l, w: tb.tb_ffn_down(w[2], s.h, s.qh, s.dqh, s.y[l]),
    }
    out = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, call in calls.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l, w in enumerate(s.layers):
                call(l, w)
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1e-3 / (reps * n)
        del g
    w = s.layers[0]
    gu_bytes = w[0].nbytes + w[1].nbytes
    res = {k + "_us": round(v * 1e6, 3) for k, v in out.items()}
    summed = out["rotate_quant_x"] + out["gateup_silu"] + out["ffn_down"]
    res.update({
        "layer_us": round(layer_s * 1e6, 3),
        "sum_of_calls_us": round(summed * 1e6, 3),
        "layer_minus_sum_us": round((layer_s - summed) * 1e6, 3),
        "gateup_kernel_only_gbs": round(gu_bytes / out["gateup_silu"] / 1e9, 1),
        "down_gemv_kernel_only_gbs": round(w[2].nbytes / out["down_gemv"] / 1e9, 1),
        "note": "HIP events around graph replays of 64 back-to-back calls of one kind; "
                "kernel-only GB/s counts weight bytes"})
    return res


def fused_event_timing(torch, f: Fused64, reps: int):
    """Mean duration (s) of one fused launch (32 layers), from HIP events on its stream.

    tb_ffn_layers launches on the current stream (the default argument), which is the
    stream torch.cuda.Event records on. Each repetition is one step (two back-to-back
    launches of 32 layers) between two events; kernels on one stream run back to
    back, so the mean per launch compares with the per-dispatch durations of a kernel
    trace.
    """
    f.step()
    torch.cuda.synchronize()
    launches = (len(f.arr) + 31) // 32
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total = 0.0
    for _ in range(reps):
        e0.record()
        f.step()
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1) * 1e-3
    return total / (reps * launches)


def measured_traffic(kernel_key: str):
    """HBM bytes per launch of `kernel_key` from the committed counter summary, or None.

    profiles/ffn64_stream_traffic.json holds calibrated FETCH_SIZE + WRITE_SIZE bytes per
    launch with a sha256 of the kernel sources they were taken on; once the sources
    change, the figure no longer describes the kernel and None is returned."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "ffn64_stream_traffic.json")
    if not os.path.exists(path):
        return None
    doc = json.load(open(path))
    h = hashlib.sha256()
    for f in doc["source_files"]:
        path_f = os.path.join(ROOT, f)
        if not os.path.exists(path_f):
            return None
        with open(path_f, "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != doc["source_sha256"] or kernel_key not in doc["kernels"]:
        return None
    return int(doc["kernels"][kernel_key]["traffic_bytes_per_launch"])


def cpu_baseline(layers_host, xs, seconds: float, m: int = 1):
    """The scalar oracle, single-threaded, on the first layers of the same stream at m rows."""
    import oracle
    o = oracle.default()
    t0 = time.perf_counter()
    done, nbytes = 0, 0
    while True:
        l = done % len(layers_host)
        o.ffn(layers_host[l], xs[l][:m])
        done += 1
        nbytes += layers_host[l].nbytes
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} FFN layers of the same 64-layer stream at M={m} "
                      f"({nbytes} weight bytes, {dt:.1f} s, 1 thread)"}


def gpu_clocks(torch, work=None):
    """The GPU's clock lines from `amd-smi metric --clock`, run as a child process after the
    timed region; while it runs, `work` (the M=1 stream step) is replayed so the reading is
    taken under load. None when the tool is missing or refuses."""
    import re
    import subprocess
    try:
        proc = subprocess.Popen(["amd-smi", "metric", "--clock"], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.perf_counter()
    while proc.poll() is None and time.perf_counter() - t0 < 30:
        if work is not None:
            for _ in range(4):
                work()
            torch.cuda.synchronize()
        else:
            time.sleep(0.05)
    try:
        out, _ = proc.communicate(timeout=5)
    except subprocess.SubprocessError:
        proc.kill()
        return None
    if proc.returncode != 0:
        return None
    lines = [" ".join(x.split()) for x in out.splitlines() if re.search(r"GFX_\d|CLK:|MEM", x)]
    return lines[:16] or None


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

    f1 = Fused64(tb, dev_layers, xs, 1, torch)
    s1 = Stream64(tb, dev_layers, xs, 1, torch)
    if args.profile_only:
        f1.step()
        s1.step()
        torch.cuda.synchronize()
        f1.check()
        log("profile pass done (one fused step, one pass of separate calls)")
        return

    def summary(total, per):
        per = sorted(per)
        return {"value": round(step_bytes / total / 1e9, 2), "unit": "GB/s",
                "ms_per_step": round(total * 1e3, 4),
                "us_per_layer": round(total / args.layers * 1e6, 3),
                "pct_hbm_peak": round(100 * step_bytes / total / 1e9 / HBM_PEAK_GBS, 2),
                "event_median_ms": round(per[len(per) // 2] * 1e3, 4),
                "event_min_ms": round(per[0] * 1e3, 4)}

    use_graph = not args.no_graph
    paths = {}
    tf, pf = time_stream(torch, f1, args.steps, args.warmup, False)
    f1.check()
    paths["fused"] = summary(tf, pf)
    log(f"fused M=1: {tf / args.layers * 1e6:.2f} us/layer, {step_bytes / tf / 1e9:.1f} GB/s")
    ts, ps = time_stream(torch, s1, args.steps, args.warmup, use_graph)
    paths["separate"] = summary(ts, ps)
    log(f"separate calls M=1 ({'graph' if use_graph else 'eager'}): {ts / args.layers * 1e6:.2f} "
        f"us/layer, {step_bytes / ts / 1e9:.1f} GB/s")
    te, pe = time_stream(torch, s1, max(3, args.steps // 4), 1, False)
    paths["separate_eager"] = summary(te, pe)
    log(f"separate calls M=1 (eager): {te / args.layers * 1e6:.2f} us/layer")
    head = "fused" if tf <= ts else "separate"
    t1 = tf if head == "fused" else ts

    # roofline of the dominant kernel of the headline path, timed with HIP events on the
    # stream it is launched on (the current stream)
    if head == "fused":
        launch_layers = min(32, args.layers)
        k_s = fused_event_timing(torch, f1, max(3, args.steps // 4))
        k_bytes = launch_layers * (layer_bytes + 2 * synth.HIDDEN * 4)
        k_name = "ffn_layers_kernel<1,TERNARY2> (tb_ffn_layers, 32 layers per launch)"
        k_key = "ffn_layers_kernel<1, 0>"
    else:
        k_s = gateup_event_timing(torch, s1, max(2, args.steps // 4))
        k_bytes = layers[0].gate.nbytes + layers[0].up.nbytes + synth.HIDDEN + 40 * 4 + synth.INTER * 4
        k_name = "gemv_ring_kernel<1,TERNARY2,GATEUP> (tb_ffn_gateup_silu)"
        k_key = "gemv_ring_kernel<1, 0, 1>"
    k_gbs = k_bytes / k_s / 1e9
    log(f"dominant kernel {k_name}: {k_s * 1e6:.2f} us/launch, {k_gbs:.1f} GB/s")
    breakdown = call_breakdown(torch, s1, ts / args.layers, max(3, args.steps // 4))
    log("M=1 calls (graph, us): " + ", ".join(f"{k[:-3]} {v}" for k, v in breakdown.items()
                                               if k.endswith("_us")))
    clocks = gpu_clocks(torch, s1.step)
    log("clocks (under the M=1 stream): " + (" | ".join(clocks) if clocks else "amd-smi unavailable"))
    del f1, s1

    res_m8 = None
    if not args.skip_m8:
        m8 = {}
        f8 = Fused64(tb, dev_layers, xs, 8, torch)
        t8, p8 = time_stream(torch, f8, args.steps, args.warmup, False)
        f8.check()
        m8["fused"] = summary(t8, p8)
        del f8
        s8 = Stream64(tb, dev_layers, xs, 8, torch)
        t8s, p8s = time_stream(torch, s8, args.steps, args.warmup, use_graph)
        m8["separate"] = summary(t8s, p8s)
        del s8
        best = "fused" if t8 <= t8s else "separate"
        res_m8 = dict(m8[best], entry_point=best, paths=m8)
        log(f"M=8: fused {t8 / args.layers * 1e6:.2f} us/layer, separate "
            f"{t8s / args.layers * 1e6:.2f} us/layer")

    res_sign = None
    if not args.skip_sign:
        del dev_layers
        torch.cuda.empty_cache()
        sl = synth.ffn_stream(SEED + 100, args.layers, synth.FMT_SIGN1, threads=16)
        sbytes = sl[0].nbytes * args.layers
        sdev = upload(sl)
        res_sign = {"bytes_per_step": sbytes}
        for m in (1, 8):
            row = {}
            fs = Fused64(tb, sdev, xs, m, torch)
            tfs, _ = time_stream(torch, fs, args.steps, args.warmup, False)
            fs.check()
            row["fused_us_per_layer"] = round(tfs / args.layers * 1e6, 3)
            del fs
            ss = Stream64(tb, sdev, xs, m, torch)
            tss, _ = time_stream(torch, ss, args.steps, args.warmup, use_graph)
            row["separate_us_per_layer"] = round(tss / args.layers * 1e6, 3)
            del ss
            tb_ = min(tfs, tss)
            row.update({"value": round(sbytes / tb_ / 1e9, 2), "unit": "GB/s",
                        "us_per_layer": round(tb_ / args.layers * 1e6, 3),
                        "pct_hbm_peak": round(100 * sbytes / tb_ / 1e9 / HBM_PEAK_GBS, 2),
                        "entry_point": "fused" if tfs <= tss else "separate"})
            res_sign[f"m{m}"] = row
            log(f"sign M={m}: fused {tfs / args.layers * 1e6:.2f}, separate "
                f"{tss / args.layers * 1e6:.2f} us/layer")
        del sdev, sl
        torch.cuda.empty_cache()

    probe = read_probe(torch, 4 << 30)
    log(f"read probe (4 GiB): {probe:.1f} GB/s")
    gb1 = step_bytes / t1 / 1e9

    cpu = cpu_baseline(layers[:4], xs, args.cpu_seconds)
    cpu8 = cpu_baseline(layers[:4], xs, args.cpu_seconds / 2, m=8)
    cpu["m8"] = {"value": cpu8["value"], "unit": cpu8["unit"], "sample": cpu8["sample"]}
    log(f"cpu oracle: {cpu['value']} GB/s ({cpu['sample']}); M=8 {cpu8['value']} GB/s "
        f"({cpu8['sample']})")

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
                   "entry_point": {"fused": "tb_ffn_layers (one persistent launch per 32 layers)",
                                   "separate": "tb_rotate_quant_i8 + tb_ffn_gateup_silu + "
                                               "tb_ffn_down per layer, "
                                               + ("hip graph replay" if use_graph else "eager")}[head],
                   "layer_order": "strict: layer l+1 starts after layer l's outputs are written"},
        "us_per_layer": round(t1 / args.layers * 1e6, 3),
        "pct_hbm_peak": round(100 * gb1 / HBM_PEAK_GBS, 2),
        "read_probe_gbs": round(probe, 1),
        "pct_of_read_probe": round(100 * gb1 / probe, 2),
        "paths_m1": paths,
        "m8": res_m8,
        "sign1_stream": res_sign,
        "roofline": {"bound": "hbm", "achieved": round(k_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(k_key),
                     "kernel": k_name, "bytes_per_launch": k_bytes,
                     "us_per_launch": round(k_s * 1e6, 3)},
        "cpu_baseline": cpu,
        "m1_call_breakdown": breakdown,
        "gpu_clocks_amd_smi": clocks,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
