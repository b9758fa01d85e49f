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
tb_ffn_layers (one persistent launch per 32 layers), and the separate calls per
layer (tb_ffn_gateup_silu_x, which rotates x inside its launch where that
applies, and tb_ffn_down_split, which at M=1 runs tb_ffn_down's kernels and
from 4 rows splits the down stage over k) replayed from a HIP graph (and
eagerly). The value is the faster of the two; the JSON names it. Also printed: the same at M=8; the 1-bit sign stream; the roofline
of the headline path's dominant kernel, timed with HIP events on the stream it
runs on; a 4 GiB streaming-read probe; and the scalar CPU oracle timed on this
host's cores.

The timed outputs are checked: after timing, the y of every layer from the
timed graph replay must equal, byte for byte, that of the same calls run
eagerly and that of the fused launch; and the CPU-baseline leg (the oracle run
over all 64 layers on every host core) checks every layer's y against the
oracle within the chained-layer bound. Any mismatch prints the JSON line with
parity_checked false and exits with status 3.
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
    p.add_argument("--skip-batch", action="store_true", help="no M=16 / M=32 stream")
    p.add_argument("--skip-attn", action="store_true", help="no attention-projection stream")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="target CPU time of the single-thread oracle sample")
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="host threads of the all-cores oracle pass (0: the usable cores, "
                        "at most 16)")
    p.add_argument("--skip-oracle-m8", action="store_true",
                   help="no all-cores oracle pass (and oracle parity check) at M=8")
    p.add_argument("--profile-only", action="store_true",
                   help="one eager pass of each path and exit (for rocprofv3 counter runs)")
    p.add_argument("--profile-m", default="1,8,32",
                   help="rows of the --profile-only passes, comma-separated (1..8: the fused "
                        "and the separate paths; 9..32: the *_batch calls)")
    p.add_argument("--profile-fmt", choices=("ternary", "sign"), default="ternary",
                   help="weight format of the --profile-only passes")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="only run a device copy of this many MiB (counter calibration)")
    return p.parse_args()


class Stream64:
    """Device weights and buffers of the layer stream at m rows.

    Every layer writes its own q, dq, h, rotquant(h) and y (the same kernels and bytes as
    with shared buffers), so all of a timed step's intermediates can be checked after it."""

    def __init__(self, tb, layers_dev, xs, m, torch, batch=False):
        self.tb, self.layers, self.m, self.batch = tb, layers_dev, m, batch
        dev = "cuda"
        k = layers_dev[0][0].k
        n = layers_dev[0][0].n
        L = len(layers_dev)
        self.x = [torch.from_numpy(x[:m].copy()).to(dev) for x in xs]
        self.q = torch.empty(L, m, k, dtype=torch.int8, device=dev)
        self.dq = torch.empty(L, m, k // 128, dtype=torch.float32, device=dev)
        self.h = torch.empty(L, m, n, dtype=torch.float32, device=dev)
        self.qh = torch.empty(L, m, n, dtype=torch.int8, device=dev)
        self.dqh = torch.empty(L, m, n // 128, dtype=torch.float32, device=dev)
        self.y = torch.empty(L, m, k, dtype=torch.float32, device=dev)
        # the step partials of tb_ffn_down_split(_batch) (one workspace: the calls are in order)
        self.ws = tb.tb_ffn_down_split_workspace(layers_dev[0][2], m, batch=batch)

    def step(self):
        tb = self.tb
        if self.batch:   # the *_batch calls (up to 32 rows)
            for l, (wg, wu, wd) in enumerate(self.layers):
                tb.tb_rotate_quant_i8_batch(self.x[l], self.q[l], self.dq[l])
                tb.tb_ffn_gateup_silu_batch(wg, wu, self.q[l], self.dq[l], self.h[l])
                tb.tb_ffn_down_split_batch(wd, self.h[l], self.qh[l], self.dqh[l], self.y[l], self.ws)
            return
        for l, (wg, wu, wd) in enumerate(self.layers):
            tb.tb_ffn_gateup_silu_x(wg, wu, self.x[l], self.q[l], self.dq[l], self.h[l])
            tb.tb_ffn_down_split(wd, self.h[l], self.qh[l], self.dqh[l], self.y[l], self.ws)

    def outputs(self):
        """Every intermediate and output of the last step, on the host."""
        return {name: getattr(self, name).cpu().numpy().copy()
                for name in ("q", "dq", "h", "qh", "dqh", "y")}


class AttnStream:
    """Second workload: the full-attention projections of the model's 16 full-attention
    layers at m rows. Per layer: the fused query/gate/key/value GEMV (9216 x 5120) of the
    rotated, quantised x, and the output GEMV (5120 x 4096) of the rotated, quantised
    attention output (stand-in rows), each one tb_gemv_ternary_x call. Every layer writes
    its own outputs."""

    def __init__(self, tb, mats_dev, xs, os_, m, torch):
        self.tb, self.mats, self.m = tb, mats_dev, m
        dev = "cuda"
        L = len(mats_dev)
        H, Q, G = mats_dev[0][0].k, mats_dev[0][1].k, mats_dev[0][0].n
        self.x = [torch.from_numpy(v[:m].copy()).to(dev) for v in xs]
        self.oin = [torch.from_numpy(v[:m].copy()).to(dev) for v in os_]
        self.q = torch.empty(L, m, H, dtype=torch.int8, device=dev)
        self.dq = torch.empty(L, m, H // 128, dtype=torch.float32, device=dev)
        self.qo = torch.empty(L, m, Q, dtype=torch.int8, device=dev)
        self.dqo = torch.empty(L, m, Q // 128, dtype=torch.float32, device=dev)
        self.yg = torch.empty(L, m, G, dtype=torch.float32, device=dev)
        self.y = torch.empty(L, m, H, dtype=torch.float32, device=dev)

    def step(self):
        tb = self.tb
        for l, (wg, wo) in enumerate(self.mats):
            tb.tb_gemv_ternary_x(wg, self.x[l], self.q[l], self.dq[l], self.yg[l])
            tb.tb_gemv_ternary_x(wo, self.oin[l], self.qo[l], self.dqo[l], self.y[l])

    def outputs(self):
        return {name: getattr(self, name).cpu().numpy().copy()
                for name in ("q", "dq", "yg", "qo", "dqo", "y")}


def attn_oracle_parity(mats_host, xs, os_, got, m, which):
    """Layers `which` of the attention stream against the oracle: rotquant of both inputs
    bit-exact, both GEMVs within 1e-4 * sum|terms|. Returns (ok, worst y over its bound)."""
    import oracle
    from tests import bounds
    o = oracle.default()
    ok, worst = True, 0.0
    for l in which:
        q, dq = o.rotate_quant(xs[l][:m])
        qo, dqo = o.rotate_quant(os_[l][:m])
        ok &= np.array_equal(got["q"][l], q) and np.array_equal(got["dq"][l], dq)
        ok &= np.array_equal(got["qo"][l], qo) and np.array_equal(got["dqo"][l], dqo)
        for key, w, qq, dd in (("yg", mats_host[l].qkvg, q, dq), ("y", mats_host[l].o, qo, dqo)):
            yo, sabs = o.gemv(w, qq, dd)
            g_ok, g_w = bounds.gemv_ok(got[key][l], yo, sabs)
            ok &= g_ok
            worst = max(worst, g_w)
    return bool(ok), worst


class Fused64:
    """The same stream through tb_ffn_layers: one call per step (one launch per 32 layers).

    chain=True runs the layers chained (layer l+1 takes layer l's y), the real decode
    dependency; chain=False gives every layer its own input, like Stream64."""

    def __init__(self, tb, layers_dev, xs, m, torch, chain=False):
        self.tb, self.m, self.chain = tb, m, chain
        dev = "cuda"
        k = layers_dev[0][0].k
        n = layers_dev[0][0].n
        self.arr = tb.FfnLayers(layers_dev)
        x = xs[0][:m] if chain else np.stack([x[:m] for x in xs])
        self.x = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        self.y = torch.empty(len(layers_dev), m, k, dtype=torch.float32, device=dev)
        self.ws = torch.empty(tb.tb_ffn_workspace_bytes(m, k, n), dtype=torch.uint8, device=dev)
        tb.tb_ffn_workspace_init(self.ws)

    def step(self):
        self.tb.tb_ffn_layers(self.arr, self.x, self.ws, self.y, chain=self.chain)

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
    s.graph = graph   # kept for replays after the timed region (clock reading)
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


def shader_clock(torch, replay, rounds: int = 4):
    """The shader clock while the M=1 stream runs, measured on the GPU: the clock probe (one
    wave per CU, 50 us of real time) is launched on a second stream, at the default priority,
    while about 20 graph replays are queued on the current one, so its waves share the CUs
    with the stream's kernels; per workgroup, shader-clock ticks over 100 MHz real-time
    ticks. The same probe on the idle GPU is reported beside it. MHz: median, min, max."""
    import ctypes
    from ternary_weight_int8_tb_amd import build as tb_build
    path = os.path.join(ROOT, "ternary_weight_int8_tb_amd", "libtb_probe.so")
    if not os.path.exists(path):
        tb_build.build()
    P = ctypes.CDLL(path)
    P.tbp_clock.argtypes = [ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    grid = 256
    out = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()

    def run(busy: bool):
        mhz = []
        for _ in range(rounds):
            torch.cuda.synchronize()
            if busy:
                for _ in range(20):
                    replay()
            rc = P.tbp_clock(5000, out.data_ptr(), grid, side.cuda_stream)
            torch.cuda.synchronize()
            if rc != 0:
                return None
            o = out.view(grid, 2).cpu().numpy().astype(np.float64)
            mhz += list(o[:, 0] / np.maximum(o[:, 1], 1.0) * 100.0)
        mhz = np.sort(np.array(mhz))
        return {"median": round(float(np.median(mhz)), 1), "min": round(float(mhz[0]), 1),
                "max": round(float(mhz[-1]), 1), "samples": int(mhz.size)}
    return {"while_m1_stream_runs": run(True), "idle": run(False),
            "method": "s_memtime ticks over s_memrealtime (100 MHz) ticks in a 50 us probe "
                      "wave per CU, launched beside the replayed M=1 graph"}


def gateup_event_timing(torch, s: Stream64, reps: int):
    """Mean duration (s) of the gate/up launch of the separate-call path at M=1 (the
    rotation of x inside it): back-to-back launches over every layer's weights (each
    launch streams its 47 MB from HBM) captured in a HIP graph, and HIP events around
    `reps` replays on the current stream, which the replay runs on. The graph keeps the
    host's launch rate out of the figure (eager launches through the binding can trail
    the GPU on a slow host)."""
    tb = s.tb
    torch.cuda.synchronize()
    n = len(s.layers)

    def launches():
        for wg, wu, _wd in s.layers:
            tb.tb_ffn_gateup_silu_x(wg, wu, s.x[0], s.q[0], s.dq[0], s.h[0])

    launches()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launches()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total = 0.0
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1) * 1e-3
    del g
    return total / (reps * n)


def call_breakdown(torch, s: Stream64, layer_s: float, reps: int):
    """Per-call device time of the separate-call stream, without a tracer.

    Each call type is captured 64 times back to back (one per layer's weights) in a HIP
    graph and timed with HIP events around `reps` replays, so a figure is the kernel's
    duration plus the dependency between two launches on one stream. The stream's layer
    time minus the sum of its two calls (gate/up from x, down) is what changes when the
    calls alternate (caches, launch shapes). The int8-input calls and the separate
    rotations are timed beside them. Returns microseconds per call and kernel-only GB/s."""
    tb, n = s.tb, len(s.layers)
    tb.tb_rotate_quant_i8(s.x[0], s.q[0], s.dq[0])
    tb.tb_ffn_gateup_silu(*s.layers[0][:2], s.q[0], s.dq[0], s.h[0])
    tb.tb_rotate_quant_i8(s.h[0], s.qh[0], s.dqh[0])
    torch.cuda.synchronize()
    calls = {
        "rotate_quant_x": lambda l, w: tb.tb_rotate_quant_i8(s.x[l], s.q[l], s.dq[l]),
        "gateup_silu": lambda l, w: tb.tb_ffn_gateup_silu(w[0], w[1], s.q[0], s.dq[0], s.h[l]),
        "gateup_silu_x": lambda l, w: tb.tb_ffn_gateup_silu_x(w[0], w[1], s.x[0], s.q[l], s.dq[l],
                                                              s.h[l]),
        "rotate_quant_h": lambda l, w: tb.tb_rotate_quant_i8(s.h[0], s.qh[l], s.dqh[l]),
        "down_gemv": lambda l, w: tb.tb_gemv_ternary(w[2], s.qh[0], s.dqh[0], s.y[l]),
        "ffn_down": lambda l, w: tb.tb_ffn_down(w[2], s.h[0], s.qh[l], s.dqh[l], s.y[l]),
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
    summed = out["gateup_silu_x"] + out["ffn_down"]
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads(requested: int) -> int:
    if requested > 0:
        return requested
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_single_thread(layers_host, xs, seconds: float, m: int = 1):
    """The scalar oracle, one thread, on the first layers of the same stream at m rows."""
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
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "sample": f"{done} FFN layers of the 64-layer stream at M={m} "
                      f"({nbytes} weight bytes, {dt:.1f} s, 1 thread)"}


def cpu_all_cores(layers_host, xs, m: int, threads: int, which=None):
    """The oracle over every layer of the stream (or the layers in `which`) at m rows, one
    layer per task on `threads` host threads (its C calls release the GIL). Returns
    (results per layer, or None for layers not run; seconds)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    o = oracle.default()
    which = list(range(len(layers_host))) if which is None else list(which)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        part = list(ex.map(lambda l: o.ffn(layers_host[l], xs[l][:m]), which))
    res = [None] * len(layers_host)
    for l, r in zip(which, part):
        res[l] = r
    return res, time.perf_counter() - t0


def lut_comparison(torch, tb, synth, sdev, layers: int):
    """The lookup-table GEMV (row-interleaved sign weights) against the bit-mask kernel on
    the same matrices: the gate and down projections of the first `layers` sign layers,
    each call kind captured back to back in a graph and timed with events, at one and
    two rows. Checks that both produce the same y bytes. Returns the report dict."""
    out = {"layers": layers, "note": "graph replay of back-to-back calls, us per call; "
           "tb_gemv_ternary on TB_FMT_SIGN1 (bit-mask decode) and on TB_FMT_SIGN1_RI4 "
           "(lookup tables through v_perm_b32)"}
    same = True
    for label, pick in (("gate_17408x5120", 0), ("down_5120x17408", 2)):
        ws = [sdev[l][pick] for l in range(layers)]
        ri = [tb.tb_sign_interleave(w) for w in ws]
        k, n = ws[0].k, ws[0].n
        for m in (1, 2):
            x = torch.from_numpy(synth.student_t_rows(m, k, SEED + 300, pick)).cuda()
            q = torch.empty(m, k, dtype=torch.int8, device="cuda")
            dq = torch.empty(m, k // 128, dtype=torch.float32, device="cuda")
            tb.tb_rotate_quant_i8(x, q, dq)
            row = {}
            ys = {}
            for name, mats in (("bitmask", ws), ("lut", ri)):
                y = torch.empty(layers, m, n, device="cuda")
                for l, w in enumerate(mats):
                    tb.tb_gemv_ternary(w, q, dq, y[l])
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for l, w in enumerate(mats):
                        tb.tb_gemv_ternary(w, q, dq, y[l])
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / 10 / layers * 1e3
                row[name + "_us"] = round(us, 3)
                row[name + "_gbs"] = round(ws[0].nbytes / us / 1e3, 1)
                ys[name] = y.cpu().numpy().tobytes()
                del g
            same = same and ys["bitmask"] == ys["lut"]
            out[f"{label}_m{m}"] = row
        del ri
    return out, same


def oracle_parity(layers_host, res, got, threads: int):
    """Every layer of a timed step against the oracle, stagewise (the bars of the tests):
      q, dq                  bit-exact against the oracle's rotquant(x);
      h                      within the h bound propagated from the 1e-4 fold bar;
      rotquant(h), its dq    bit-exact against the oracle's rotquant of the GPU's own h;
      y                      within 1e-4 * sum|terms| of the oracle's down GEMV on that q_h.
    res: the oracle's ffn() of every layer (from the timed all-cores pass); got: the timed
    step's outputs [L][m][...] (Stream64.outputs()). Returns (all pass, worst h error over
    its bound, worst y error over its bound, failures as text)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from tests import bounds
    o = oracle.default()

    def one(l):
        r, bad = res[l], []
        if not np.array_equal(got["q"][l], r["q"]):
            bad.append("q")
        if got["dq"][l].view(np.uint32).tobytes() != r["dq"].view(np.uint32).tobytes():
            bad.append("dq")
        tol_h = bounds.h_tolerance(r["g"], r["u"], r["sg"], r["su"])
        wh = float(np.max(np.abs(got["h"][l].astype(np.float64) - r["h"]) / tol_h))
        if not wh <= 1.0:
            bad.append("h")
        d = o.ffn_down(layers_host[l].down, got["h"][l])
        if not np.array_equal(got["qh"][l], d["qh"]):
            bad.append("qh")
        if got["dqh"][l].view(np.uint32).tobytes() != d["dqh"].view(np.uint32).tobytes():
            bad.append("dqh")
        ok_y, wy = bounds.gemv_ok(got["y"][l], d["y"], d["sabs"])
        if not ok_y:
            bad.append("y")
        return bad, wh, wy

    which = [l for l in range(len(res)) if res[l] is not None]
    with ThreadPoolExecutor(threads) as ex:
        out = list(ex.map(one, which))
    fails = [f"layer {l}: {','.join(b)}" for l, (b, _, _) in zip(which, out) if b]
    return (not fails, max(w for _, w, _ in out), max(w for _, _, w in out), fails[:8])


def gpu_clocks(torch, replay):
    """The GPU's clock lines from `amd-smi metric --clock`, read while `replay` (one graph
    replay of the M=1 stream, about 1.5 ms) is queued back to back, 200 at a time, so
    the GPU is busy the whole time the tool runs. None when the tool is missing."""
    import re
    import subprocess
    try:
        proc = subprocess.Popen(["amd-smi", "metric", "--clock"], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.perf_counter()
    bursts = 0
    while proc.poll() is None and time.perf_counter() - t0 < 30:
        for _ in range(200):
            replay()
        torch.cuda.synchronize()
        bursts += 1
    try:
        out, _ = proc.communicate(timeout=5)
    except subprocess.SubprocessError:
        proc.kill()
        return None
    if proc.returncode != 0:
        return None
    lines = [" ".join(x.split()) for x in out.splitlines() if re.search(r"GFX_\d|CLK:|MEM", x)]
    return {"lines": lines[:16], "replays_while_reading": bursts * 200,
            "seconds": round(time.perf_counter() - t0, 2)}


def copy_probe(torch, mib: int):
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy probe: {mib} MiB read + {mib} MiB written per copy, 3 copies")


def timed_outputs(torch, s):
    """The y of every layer as left by the last timed step, on the host."""
    torch.cuda.synchronize()
    return s.y.cpu().numpy().copy()


def eager_reference(torch, s):
    """The same calls run once more eagerly (no graph) into poisoned outputs."""
    s.y.fill_(float("nan"))
    s.step()
    torch.cuda.synchronize()
    return s.y.cpu().numpy().copy()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU only; --gpus must be 1",
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
    fmt = synth.FMT_SIGN1 if args.profile_only and args.profile_fmt == "sign" else synth.FMT_TERNARY2
    layers = synth.ffn_stream(SEED, args.layers, fmt, threads=16)
    xs = [synth.normal_rows(32, synth.HIDDEN, SEED, l) for l in range(args.layers)]
    layer_bytes = layers[0].nbytes
    step_bytes = layer_bytes * args.layers
    log(f"generated {args.layers} layers ({step_bytes} B) in {time.perf_counter() - t0:.1f} s")

    def upload(ls):
        return [tuple(tb.Matrix.upload(w) for w in (L.gate, L.up, L.down)) for L in ls]

    dev_layers = upload(layers)
    torch.cuda.synchronize()

    if args.profile_only:
        for pm in (int(v) for v in args.profile_m.split(",")):
            if pm > 8:
                sp = Stream64(tb, dev_layers, xs, pm, torch, batch=True)
                sp.step()
                torch.cuda.synchronize()
                del sp
                log(f"profile pass done at M={pm} (one pass of the *_batch calls)")
                continue
            fp = Fused64(tb, dev_layers, xs, pm, torch)
            sp = Stream64(tb, dev_layers, xs, pm, torch)
            fp.step()
            sp.step()
            torch.cuda.synchronize()
            fp.check()
            del fp, sp
            log(f"profile pass done at M={pm} (one fused step, one pass of separate calls)")
        return
    f1 = Fused64(tb, dev_layers, xs, 1, torch)
    s1 = Stream64(tb, dev_layers, xs, 1, torch)

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
    parity = {}
    tf, pf = time_stream(torch, f1, args.steps, args.warmup, False)
    f1.check()
    y_fused1 = timed_outputs(torch, f1)
    paths["fused"] = summary(tf, pf)
    log(f"fused M=1: {tf / args.layers * 1e6:.2f} us/layer, {step_bytes / tf / 1e9:.1f} GB/s")
    fc = Fused64(tb, dev_layers, xs, 1, torch, chain=True)
    tfc, pfc = time_stream(torch, fc, args.steps, args.warmup, False)
    fc.check()
    paths["fused_chained"] = summary(tfc, pfc)
    log(f"fused M=1 chained (layer l+1 takes layer l's y): {tfc / args.layers * 1e6:.2f} us/layer")
    del fc
    ts, ps = time_stream(torch, s1, args.steps, args.warmup, use_graph)
    torch.cuda.synchronize()
    got1 = s1.outputs()
    y_sep1 = got1["y"]
    paths["separate"] = summary(ts, ps)
    log(f"separate calls M=1 ({'graph' if use_graph else 'eager'}): {ts / args.layers * 1e6:.2f} "
        f"us/layer, {step_bytes / ts / 1e9:.1f} GB/s")
    graph1 = s1.graph
    te, pe = time_stream(torch, s1, max(3, args.steps // 4), 1, False)
    paths["separate_eager"] = summary(te, pe)
    log(f"separate calls M=1 (eager): {te / args.layers * 1e6:.2f} us/layer")
    y_eager1 = eager_reference(torch, s1)
    parity["m1_timed_graph_equals_eager"] = bool(y_sep1.tobytes() == y_eager1.tobytes())
    parity["m1_fused_equals_separate"] = bool(y_fused1.tobytes() == y_eager1.tobytes())
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
        # weights, x read, its int8 copy and block scales written, h written
        k_bytes = (layers[0].gate.nbytes + layers[0].up.nbytes + synth.HIDDEN * 4 + synth.HIDDEN
                   + (synth.HIDDEN // 128) * 4 + synth.INTER * 4)
        k_name = "gemv_ring_kernel<1,TERNARY2,GATEUP,ROTX> (tb_ffn_gateup_silu_x)"
        k_key = "gemv_ring_kernel<1, 0, 1, true>"
    k_gbs = k_bytes / k_s / 1e9
    log(f"dominant kernel {k_name}: {k_s * 1e6:.2f} us/launch, {k_gbs:.1f} GB/s")
    breakdown = call_breakdown(torch, s1, ts / args.layers, max(3, args.steps // 4))
    log("M=1 calls (graph, us): " + ", ".join(f"{k[:-3]} {v}" for k, v in breakdown.items()
                                               if k.endswith("_us")))
    clocks = gpu_clocks(torch, graph1.replay) if graph1 is not None else None
    sclk = shader_clock(torch, graph1.replay) if graph1 is not None else None
    if sclk:
        log(f"shader clock (probe beside the M=1 stream): {sclk['while_m1_stream_runs']} MHz; "
            f"idle: {sclk['idle']} MHz")
    log("clocks (while the M=1 graph replays): "
        + (" | ".join(clocks["lines"]) if clocks else "amd-smi unavailable"))
    del f1, s1, graph1

    res_m8 = None
    y_sep8 = None
    if not args.skip_m8:
        m8 = {}
        f8 = Fused64(tb, dev_layers, xs, 8, torch)
        t8, p8 = time_stream(torch, f8, args.steps, args.warmup, False)
        f8.check()
        y_fused8 = timed_outputs(torch, f8)
        m8["fused"] = summary(t8, p8)
        del f8
        s8 = Stream64(tb, dev_layers, xs, 8, torch)
        t8s, p8s = time_stream(torch, s8, args.steps, args.warmup, use_graph)
        torch.cuda.synchronize()
        got8 = s8.outputs()
        y_sep8 = got8["y"]
        m8["separate"] = summary(t8s, p8s)
        y_eager8 = eager_reference(torch, s8)
        parity["m8_timed_graph_equals_eager"] = bool(y_sep8.tobytes() == y_eager8.tobytes())
        parity["m8_fused_equals_separate"] = bool(y_fused8.tobytes() == y_eager8.tobytes())
        del s8
        best = "fused" if t8 <= t8s else "separate"
        res_m8 = dict(m8[best], entry_point=best, paths=m8)
        log(f"M=8: fused {t8 / args.layers * 1e6:.2f} us/layer, separate "
            f"{t8s / args.layers * 1e6:.2f} us/layer")

    res_big = None
    got_big = {}   # m -> the timed stream's outputs, checked against the oracle below
    if not args.skip_batch:
        res_big = {}
        for m in (16, 32):
            sb = Stream64(tb, dev_layers, xs, m, torch, batch=True)
            tb_s, pb = time_stream(torch, sb, args.steps, args.warmup, use_graph)
            torch.cuda.synchronize()
            gotb = sb.outputs()
            ye = eager_reference(torch, sb)
            parity[f"m{m}_timed_graph_equals_eager"] = bool(gotb["y"].tobytes() == ye.tobytes())
            got_big[m] = gotb
            del sb, gotb
            res_big[f"m{m}"] = dict(summary(tb_s, pb), entry_point="tb_rotate_quant_i8_batch + tb_ffn_gateup_silu_batch + "
                                "tb_ffn_down_split_batch per layer, hip graph replay")
            log(f"M={m} (batch calls): {tb_s / args.layers * 1e6:.2f} us/layer, "
                f"{step_bytes / tb_s / 1e9:.1f} GB/s")

    # ---- second workload: the full-attention projections (16 layers)
    res_attn = None
    attn_got = {}
    if not args.skip_attn:
        al = synth.attn_stream(SEED + 200, synth.ATTN_LAYERS, synth.FMT_TERNARY2, threads=16)
        axs = [synth.normal_rows(8, synth.HIDDEN, SEED + 200, l) for l in range(len(al))]
        aos = [synth.normal_rows(8, synth.ATTN_Q, SEED + 200, l, synth.T_ATTN_OUT) for l in range(len(al))]
        adev = [(tb.Matrix.upload(a.qkvg), tb.Matrix.upload(a.o)) for a in al]
        abytes = al[0].nbytes * len(al)
        res_attn = {"layers": len(al), "bytes_per_step": abytes,
                    "shapes": {"qkvg": [synth.ATTN_QKVG, synth.HIDDEN], "o": [synth.HIDDEN, synth.ATTN_Q]}}
        for m in (1, 8):
            st = AttnStream(tb, adev, axs, aos, m, torch)
            ta, pa = time_stream(torch, st, args.steps, args.warmup, use_graph)
            torch.cuda.synchronize()
            attn_got[m] = st.outputs()
            st.y.fill_(float("nan"))
            st.step()
            torch.cuda.synchronize()
            parity[f"attn_m{m}_timed_graph_equals_eager"] = bool(
                attn_got[m]["y"].tobytes() == st.y.cpu().numpy().tobytes())
            del st
            res_attn[f"m{m}"] = {"value": round(abytes / ta / 1e9, 2), "unit": "GB/s",
                                 "us_per_layer": round(ta / len(al) * 1e6, 3),
                                 "pct_hbm_peak": round(100 * abytes / ta / 1e9 / HBM_PEAK_GBS, 2)}
            log(f"attention projections M={m}: {ta / len(al) * 1e6:.2f} us/layer, "
                f"{abytes / ta / 1e9:.1f} GB/s")
        del adev
        torch.cuda.empty_cache()

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
            yf = timed_outputs(torch, fs)
            row["fused_us_per_layer"] = round(tfs / args.layers * 1e6, 3)
            del fs
            ss = Stream64(tb, sdev, xs, m, torch)
            tss, _ = time_stream(torch, ss, args.steps, args.warmup, use_graph)
            ys = timed_outputs(torch, ss)
            ye = eager_reference(torch, ss)
            parity[f"sign_m{m}_timed_graph_equals_eager"] = bool(ys.tobytes() == ye.tobytes())
            parity[f"sign_m{m}_fused_equals_separate"] = bool(yf.tobytes() == ye.tobytes())
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
        res_sign["lookup_table_gemv"], lut_same = lut_comparison(torch, tb, synth, sdev, 16)
        parity["sign_lut_equals_bitmask"] = bool(lut_same)
        log("sign GEMV, bit-mask vs lookup table (us/call): " + ", ".join(
            f"{k} {v['bitmask_us']}/{v['lut_us']}" for k, v in res_sign["lookup_table_gemv"].items()
            if isinstance(v, dict)) + f"; same bytes: {lut_same}")
        del sdev, sl
        torch.cuda.empty_cache()

    probe = read_probe(torch, 4 << 30)
    log(f"read probe (4 GiB): {probe:.1f} GB/s")
    gb1 = step_bytes / t1 / 1e9

    # ---- CPU baseline leg: the oracle on this host, which also checks the timed outputs
    threads = host_threads(args.cpu_threads)
    single = cpu_single_thread(layers[:4], xs, args.cpu_seconds)
    res1, dt1 = cpu_all_cores(layers, xs, 1, threads)
    ok1, wh1, wy1, f1s = oracle_parity(layers, res1, got1, threads)
    parity["m1_oracle_all_layers"] = ok1
    parity["m1_oracle_worst_h_over_bound"] = round(wh1, 4)
    parity["m1_oracle_worst_y_over_bound"] = round(wy1, 4)
    if f1s:
        parity["m1_oracle_failures"] = f1s
    del res1, got1
    cpu = {"value": round(step_bytes / dt1 / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle",
           "sample": f"all {args.layers} layers of the stream at M=1, one layer per task on "
                     f"{threads} threads ({dt1:.1f} s; CPU: {cpu_model()}, "
                     f"{os.cpu_count()} logical CPUs)",
           "single_thread": single}
    log(f"cpu oracle: {cpu['value']} GB/s on {threads} threads ({dt1:.1f} s); single thread "
        f"{single['value']} GB/s; M=1 parity vs oracle: {ok1} (worst h {wh1:.3g}, "
        f"y {wy1:.3g} of bound)")
    if y_sep8 is not None and not args.skip_oracle_m8:
        res8, dt8 = cpu_all_cores(layers, xs, 8, threads)
        ok8, wh8, wy8, f8s = oracle_parity(layers, res8, got8, threads)
        parity["m8_oracle_all_layers"] = ok8
        parity["m8_oracle_worst_h_over_bound"] = round(wh8, 4)
        parity["m8_oracle_worst_y_over_bound"] = round(wy8, 4)
        if f8s:
            parity["m8_oracle_failures"] = f8s
        del res8, got8
        cpu["m8"] = {"value": round(step_bytes / dt8 / 1e9, 4), "unit": "GB/s",
                     "cores": threads,
                     "sample": f"all {args.layers} layers at M=8 on {threads} threads ({dt8:.1f} s)"}
        log(f"cpu oracle M=8: {cpu['m8']['value']} GB/s; M=8 parity vs oracle: {ok8} "
            f"(worst h {wh8:.3g}, y {wy8:.3g} of bound)")
    for m, gotb in sorted(got_big.items()):
        # sampled layers (8 at M=16, 4 at M=32), so the oracle's share of the run stays small
        sample = list(range(0, args.layers, max(1, args.layers // (128 // m))))
        resb, _ = cpu_all_cores(layers, xs, m, threads, which=sample)
        okb, whb, wyb, fbs = oracle_parity(layers, resb, gotb, threads)
        parity[f"m{m}_oracle_layers"] = sample
        parity[f"m{m}_oracle_ok"] = okb
        parity[f"m{m}_oracle_worst_y_over_bound"] = round(wyb, 4)
        if fbs:
            parity[f"m{m}_oracle_failures"] = fbs
        log(f"M={m} parity vs oracle on layers {sample}: {okb} (worst y {wyb:.3g} of bound)")
        del resb
    got_big.clear()
    for m, got in attn_got.items():
        a_ok, a_w = attn_oracle_parity(al, axs, aos, got, m, (0, len(al) - 1))
        parity[f"attn_m{m}_oracle_layers_0_15"] = a_ok
        parity[f"attn_m{m}_oracle_worst_y_over_bound"] = round(a_w, 4)
        log(f"attention M={m} parity vs oracle (layers 0, {len(al) - 1}): {a_ok} (worst {a_w:.3g})")
    parity_ok = all(v for k, v in parity.items() if isinstance(v, bool))
    parity["all_ok"] = parity_ok

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
                                   "separate": "tb_ffn_gateup_silu_x + tb_ffn_down_split per layer, "
                                               + ("hip graph replay" if use_graph else "eager")}[head],
                   "layer_order": "strict: layer l+1 starts after layer l's outputs are written"},
        "us_per_layer": round(t1 / args.layers * 1e6, 3),
        "pct_hbm_peak": round(100 * gb1 / HBM_PEAK_GBS, 2),
        "read_probe_gbs": round(probe, 1),
        "pct_of_read_probe": round(100 * gb1 / probe, 2),
        "paths_m1": paths,
        "m8": res_m8,
        "sign1_stream": res_sign,
        "batch_m16_m32": res_big,
        "attention_projections": res_attn,
        "roofline": {"bound": "hbm", "achieved": round(k_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(k_key),
                     "kernel": k_name, "bytes_per_launch": k_bytes,
                     "us_per_launch": round(k_s * 1e6, 3)},
        "cpu_baseline": cpu,
        "parity_checked": parity,
        "m1_call_breakdown": breakdown,
        "gpu_clocks_amd_smi": clocks,
        "gpu_shader_clock_mhz": sclk,
    }
    print(json.dumps(out), flush=True)
    if not parity_ok:
        log("bench.py: a timed output failed its check: " + json.dumps(parity))
        sys.exit(3)


if __name__ == "__main__":
    main()
