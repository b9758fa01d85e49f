"""Summaries of rocprofv3 output for profiles/: kernel statistics and calibrated HBM traffic.

    python -m ternary_weight_int8_tb_amd.profsum --stats DIR --pmc DIR --bench FILE --out profiles
    python -m ternary_weight_int8_tb_amd.profsum --sq DIR --out profiles

--stats: the directory of a `rocprofv3 --kernel-trace --stats --output-format csv -o bench`
run of bench.py; --pmc: the parent directory of the four counter runs pmc_FETCH_SIZE,
pmc_WRITE_SIZE (bench.py --profile-only: one pass of each path at M=1 and at M=8, and of the
batch calls at M=32) and pmc_copy_FETCH_SIZE, pmc_copy_WRITE_SIZE
(bench.py --copy-probe-mib 1024); --bench: the JSON line of an untraced bench.py run of
the same code. Writes ffn64_stream_kernel_stats.md, ffn64_stream_traffic.md and
ffn64_stream_traffic.json. --sq: the parent directory of two SQ counter runs (pmc_sq_a,
pmc_sq_b; the counter sets are in SQ_SETS) over the same profile pass; writes
ffn64_stream_sq_counters.md. The traffic file carries a sha256 of the kernel sources, and
bench.py reports the traffic figure only while the sources still hash to it.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ["ternary_weight_int8_tb_amd/csrc/tb.hip", "ternary_weight_int8_tb_amd/csrc/tb_device.h",
           "ternary_weight_int8_tb_amd/csrc/tb_layers.h", "ternary_weight_int8_tb_amd/csrc/tb_lut.h"]
COPY_BYTES = 1 << 30

HIDDEN, INTER, LAYERS = 5120, 17408, 64
NB_H, NB_N = HIDDEN // 128, INTER // 128
MATRIX_BYTES = INTER * HIDDEN // 4 + INTER * NB_H * 2   # codes + fp16 scales, ternary


def source_sha256() -> str:
    h = hashlib.sha256()
    for f in SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    """'void (anonymous namespace)::gemv_ring_kernel<1, 0, 1>(GemvArgs)' -> 'gemv_ring_kernel<1, 0, 1>'."""
    m = re.search(r"(\w+_kernel)(<[^>]*>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else name


# Algorithmic bytes per launch at M=1 (weights + activations read + outputs written).
ALGORITHMIC = {
    # gate/up with the rotation of x inside: x read, its int8 copy and scales written
    "gemv_ring_kernel<1, 0, 1, true>": 2 * MATRIX_BYTES + HIDDEN * 4 + HIDDEN + NB_H * 4 + INTER * 4,
    "gemv_ring_kernel<1, 0, 1, false>": 2 * MATRIX_BYTES + HIDDEN + NB_H * 4 + INTER * 4,
    "gemv_ring_kernel<1, 0, 0, false>": MATRIX_BYTES + INTER + NB_N * 4 + HIDDEN * 4,
    "ffn_layers_kernel<1, 0>": 32 * (3 * MATRIX_BYTES + 2 * HIDDEN * 4),
    # M=8: matrix-core kernels with two blocks per MFMA; the down stage split over k reads
    # h, writes rotquant(h) and its step partials (17 steps), which the fold reads
    "gemv_mfma_pack_kernel<8, 0, 1, false>": 2 * MATRIX_BYTES + 8 * (HIDDEN + NB_H * 4 + INTER * 4),
    "gemv_mfma_pack_kernel<8, 0, 0, true>": MATRIX_BYTES + 8 * (INTER * 4 + INTER + NB_N * 4)
    + 17 * 8 * HIDDEN * 4,
    "ffn_layers_kernel<8, 0>": 32 * (3 * MATRIX_BYTES + 8 * 2 * HIDDEN * 4),
    # M=32 (batch calls): gate/up in one launch (k staged in two phases) and the down stage
    # split over k in one launch, both with two 16-column groups
    "gemv_mfma_kernel<32, 0, 1, false, true>": 2 * MATRIX_BYTES + 32 * (HIDDEN + NB_H * 4 + INTER * 4),
    "gemv_mfma_kernel<32, 0, 0, true, false>": MATRIX_BYTES + 32 * (INTER * 4 + INTER + NB_N * 4)
    + 17 * 32 * HIDDEN * 4,
}
WHAT = {
    "gemv_ring_kernel<1, 0, 1, true>": "tb_ffn_gateup_silu_x at M=1 (gate and up, 47,349,760 weight "
                                       "bytes, the rotation of x inside)",
    "gemv_ring_kernel<1, 0, 1, false>": "tb_ffn_gateup_silu at M=1 (gate and up, 47,349,760 weight bytes)",
    "gemv_ring_kernel<1, 0, 0, false>": "the GEMV of tb_ffn_down at M=1 (23,674,880 weight bytes)",
    "ffn_layers_kernel<1, 0>": "one tb_ffn_layers launch of 32 layers at M=1",
    "gemv_mfma_pack_kernel<8, 0, 1, false>": "tb_ffn_gateup_silu at M=8 (matrix cores)",
    "gemv_mfma_pack_kernel<8, 0, 0, true>": "the down GEMV of tb_ffn_down_split at M=8 (split over k, "
                                            "rotation of h inside; matrix cores)",
    "ffn_layers_kernel<8, 0>": "one tb_ffn_layers launch of 32 layers at M=8",
    "gemv_mfma_kernel<32, 0, 1, false, true>": "tb_ffn_gateup_silu_batch at M=32 (matrix cores, two 16-column "
                                               "groups, k staged in two phases)",
    "gemv_mfma_kernel<32, 0, 0, true, false>": "the down GEMV of tb_ffn_down_split_batch at M=32 (split over k, "
                                        "rotation of h inside, two 16-column groups; matrix cores)",
}


def read_stats(d: str):
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = []
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            rows.append({"name": r["Name"], "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    rows.sort(key=lambda r: -r["pct"])
    return rows


SIGN_MATRIX_BYTES = INTER * HIDDEN // 8 + INTER * NB_H * 2
# the kernels of one layer of the separate-call stream (tb_ffn_gateup_silu_x,
# tb_ffn_down_split), each with the weight bytes it streams: at M=1 the gate/up launch
# rotates x itself and the down call is rotquant(h) + GEMV; at M=8 gate/up is rotquant +
# GEMV and the down call the split GEMV (rotation of h inside) + the fold
STREAMS = {
    "ternary M=1": [("gemv_ring_kernel<1, 0, 1, true>", 2 * MATRIX_BYTES), ("rotquant_kernel", 0),
                    ("gemv_ring_kernel<1, 0, 0, false>", MATRIX_BYTES)],
    "ternary M=8": [("rotquant_kernel", 0), ("gemv_mfma_pack_kernel<8, 0, 1, false>", 2 * MATRIX_BYTES),
                    ("gemv_mfma_pack_kernel<8, 0, 0, true>", MATRIX_BYTES), ("split_fold_kernel", 0)],
    "sign M=1": [("gemv_ring_kernel<1, 1, 1, true>", 2 * SIGN_MATRIX_BYTES), ("rotquant_kernel", 0),
                 ("gemv_ring_kernel<1, 1, 0, false>", SIGN_MATRIX_BYTES)],
    "sign M=8": [("rotquant_kernel", 0), ("gemv_mfma_pack_kernel<8, 1, 1, false>", 2 * SIGN_MATRIX_BYTES),
                 ("gemv_mfma_pack_kernel<8, 1, 0, true>", SIGN_MATRIX_BYTES), ("split_fold_kernel", 0)],
    # batch calls: rotquant, gate/up (one or two 16-row passes), the down split, the fold
    "ternary M=16": [("rotquant_kernel", 0), ("gemv_mfma_kernel<16, 0, 1, false, false>", 2 * MATRIX_BYTES),
                     ("gemv_mfma_kernel<16, 0, 0, true, false>", MATRIX_BYTES), ("split_fold_kernel", 0)],
    "ternary M=32": [("rotquant_kernel", 0), ("gemv_mfma_kernel<32, 0, 1, false, true>", 2 * MATRIX_BYTES),
                     ("gemv_mfma_kernel<32, 0, 0, true, false>", MATRIX_BYTES), ("split_fold_kernel", 0)],
}


def median(v):
    v = sorted(v)
    return v[len(v) // 2] if v else float("nan")


def stream_passes(d: str):
    """Graph passes of each 64-layer stream in a kernel trace.

    A pass is 64 layers of consecutive dispatches in the layer order above. Eager passes (host
    launch gaps between kernels) are dropped: a graph pass is one whose median gap between
    consecutive dispatches is at most zero. Returns, per stream, the number of passes
    and per position the median duration and the median gap to the next dispatch (us),
    plus the median pass span and busy time per layer."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        return {}
    with open(files[0]) as fh:
        seq = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short_name(r["Kernel_Name"]))
                      for r in csv.DictReader(fh)))
    names = [n for _, _, n in seq]
    out = {}
    for label, layer in STREAMS.items():
        per = len(layer)
        pat = [name for name, _ in layer] * LAYERS
        passes, i = [], 0
        while i + len(pat) <= len(seq):
            if names[i:i + len(pat)] == pat:
                p = seq[i:i + len(pat)]
                if median([p[j + 1][0] - p[j][1] for j in range(len(p) - 1)]) <= 0:
                    passes.append(p)
                i += len(pat)
            else:
                i += 1
        if not passes:
            continue
        pos = []
        for k in range(per):
            dur = [(p[j][1] - p[j][0]) / 1e3 for p in passes for j in range(k, len(pat), per)]
            gap = [(p[j + 1][0] - p[j][1]) / 1e3 for p in passes for j in range(k, len(pat) - 1, per)]
            pos.append((pat[k], median(dur), median(gap), sum(gap) / len(gap), layer[k][1]))
        span = median([(p[-1][1] - p[0][0]) / 1e3 / LAYERS for p in passes])
        busy = median([sum(e - b for b, e, _ in p) / 1e3 / LAYERS for p in passes])
        out[label] = {"passes": len(passes), "positions": pos, "span_us": span, "busy_us": busy}
    return out


def read_counter(d: str, counter: str):
    """Per kernel (short name): list of the counter's value per dispatch (KiB)."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            per.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def copy_factor(d: str, counter: str, true_bytes: int) -> float:
    """Counter bytes over true bytes for the largest dispatches of the copy probe."""
    per = read_counter(d, counter)
    best = max(((sum(v) / len(v), k) for k, v in per.items()), key=lambda t: t[0])
    return best[0] * 1024 / true_bytes


SQ_SETS = {
    "a": "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_VMEM_RD SQ_INSTS_SALU "
         "SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "b": "SQ_WAVE_CYCLES SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT "
         "SQ_ACTIVE_INST_LDS SQ_WAIT_INST_ANY SQ_WAIT_ANY GRBM_GUI_ACTIVE",
}
CUS = 256


def read_all_counters(d: str):
    """Per kernel (short name): {counter: mean over dispatches}, and the dispatch count."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            key = (short_name(r["Kernel_Name"]), r["Dispatch_Id"])
            d_ = per.setdefault(key, {})
            d_[r["Counter_Name"]] = d_.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    agg = {}
    for (k, _), cs in per.items():
        e = agg.setdefault(k, {"n": 0, "sum": {}})
        e["n"] += 1
        for c, v in cs.items():
            e["sum"][c] = e["sum"].get(c, 0.0) + v
    return {k: ({c: v / e["n"] for c, v in e["sum"].items()}, e["n"]) for k, e in agg.items()}


def write_sq(sq_dir: str, out: str, sign: bool = False):
    """SQ counters of the M=1, M=8 and M=32 kernels (sign weights: M=1 and M=8):
    instruction mix per wave and where wave time goes (waiting on memory counters, waiting
    to issue, issuing VALU)."""
    a = read_all_counters(os.path.join(sq_dir, "pmc_sq_a"))
    b = read_all_counters(os.path.join(sq_dir, "pmc_sq_b"))
    keep = [k for k in a if k in b and ("gemv" in k or "ffn_layers" in k)]
    what = "Sign-weight" if sign else "FFN"
    ms = "M=1 and M=8" if sign else "M=1, M=8 and M=32"
    extra = " --profile-fmt sign --profile-m 1,8" if sign else ""
    lines = [f"# {what} 64-layer stream: SQ counters of the {ms} kernels", "",
             "Commands (on the MI355X host, from /tmp with TMPDIR=/tmp; one counter set per run):", "", "```"]
    for name, cs in SQ_SETS.items():
        lines.append(f"rocprofv3 --pmc {cs} --output-format csv -d <out>/pmc_sq_{name} -o run -- "
                     f"python3 /root/repo/bench.py --profile-only{extra}")
    lines += ["```", "",
              "Means per dispatch over every dispatch of the kernel in one pass of each path at M=1 "
              + ("and M=8 (bench.py --profile-only --profile-fmt sign). " if sign else
                 "and M=8, and of the batch calls at M=32 (bench.py --profile-only). ") +
              "Instruction counts are wave instructions per wave. "
              "SQ_WAVE_CYCLES, SQ_WAIT_ANY (waiting on s_waitcnt: memory and LDS counters), "
              "SQ_WAIT_INST_ANY (waiting to issue the next instruction) and SQ_ACTIVE_INST_VALU "
              "share one unit (quad-cycles), so their ratios are fractions of resident wave time. "
              f"Bank conflicts and MFMA busy cycles are per CU ({CUS} CUs). Wave time is "
              "SQ_WAVE_CYCLES x 4 / waves, in shader cycles (about 2.1 GHz under load; counter "
              "runs serialise dispatches, so these kernels run a little slower than in the "
              "stream).", "",
              "| kernel | dispatches | waves | VALU / wave | MFMA / wave | LDS / wave | VMEM loads / wave "
              "| wave time (kcycles) | waiting on memory % | waiting to issue % | VALU active % "
              "| LDS bank-conflict cycles / CU | MFMA busy cycles / CU |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(keep, key=lambda k: (("<8" in k), k)):
        ca, n = a[k]
        cb, _ = b[k]
        w = ca["SQ_WAVES"]
        wc = cb["SQ_WAVE_CYCLES"]
        lines.append(
            f"| `{k}` | {n} | {w:.0f} | {ca['SQ_INSTS_VALU'] / w:.0f} | {ca['SQ_INSTS_MFMA'] / w:.0f} | "
            f"{ca['SQ_INSTS_LDS'] / w:.0f} | {ca['SQ_INSTS_VMEM_RD'] / w:.0f} | {wc * 4 / w / 1e3:.1f} | "
            f"{100 * cb['SQ_WAIT_ANY'] / wc:.0f} | {100 * cb['SQ_WAIT_INST_ANY'] / wc:.0f} | "
            f"{100 * cb['SQ_ACTIVE_INST_VALU'] / wc:.0f} | {cb['SQ_LDS_BANK_CONFLICT'] / CUS:.0f} | "
            f"{cb['SQ_VALU_MFMA_BUSY_CYCLES'] / CUS:.0f} |")
    lines += ["", "Kernel names as in the kernel statistics: gemv_ring_kernel<M, FMT, MODE, ROTX> "
              "(dot products), gemv_mfma_pack_kernel<M, FMT, MODE, KS> and gemv_mfma_kernel<M, FMT, "
              "MODE, KS, KP> (matrix cores; KS true = the down stage split over k, KP true = k "
              "staged in two phases), "
              "ffn_layers_kernel<M, FMT> (32 layers per launch)."]
    name = "sign1_stream_sq_counters.md" if sign else "ffn64_stream_sq_counters.md"
    with open(os.path.join(out, name), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out}/{name}")


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--stats")
    p.add_argument("--pmc")
    p.add_argument("--bench")
    p.add_argument("--sq", help="parent directory of the SQ counter runs pmc_sq_a and pmc_sq_b")
    p.add_argument("--sq-sign", help="the same for the sign-weight runs (--profile-fmt sign)")
    p.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = p.parse_args()
    if a.sq:
        write_sq(a.sq, a.out)
    if a.sq_sign:
        write_sq(a.sq_sign, a.out, sign=True)
    if not a.stats:
        return

    bench = None
    with open(a.bench) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("{"):
                bench = json.loads(line)
    stats = read_stats(a.stats)

    cmd_stats = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
                 "-d <out>/prof -o bench -- python3 /root/repo/bench.py --steps 5 --warmup 2")
    lines = ["# FFN 64-layer weight stream (hidden 5120, intermediate 17408): kernel statistics",
             "", "Command (on the MI355X host; /root/repo is the repository):", "", "```", cmd_stats, "```",
             "", "Kernel statistics (all dispatches of the run: both paths, M=1 and M=8, ternary and sign):",
             "", "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in stats[:16]:
        lines.append(f"| `{r['name']}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} | {r['pct']:.1f} |")
    lines += ["", "Template arguments: gemv_ring_kernel<M, FMT, MODE[, ROTX]>, FMT 0 = ternary, 1 = sign; "
              "MODE 0 = single GEMV (down), 1 = gate/up + SiLU, 2 = block-sum export; ROTX true = "
              "the fp32 input rotated and quantised inside the launch. "
              "gemv_mfma_pack_kernel<M, FMT, MODE, KS> (two blocks per MFMA, M <= 8; KS true = the "
              "down stage split over k, each workgroup one step of one row group, rotating its "
              "blocks of h itself; split_fold_kernel adds its step partials) and "
              "gemv_mfma_kernel<M, FMT, MODE, KS, KP> (one block per MFMA, batches above 8 rows; KS "
              "true = the batch's down stage split over k, KP true = gate/up with k staged in two "
              "phases; 32 rows in two 16-column groups) run on the "
              "matrix cores (ternary: gate/up for M >= 5, a single GEMV for M >= 6; sign: gate/up "
              "for M >= 5, a single GEMV for M >= 7). "
              "ffn_layers_kernel<M, FMT> is one tb_ffn_layers launch of up to 32 whole layers. "
              "stream_read_kernel is the 4 GiB read probe."]
    if bench:
        keep = {k: bench.get(k) for k in ("value", "unit", "ms_per_step", "us_per_layer", "pct_hbm_peak",
                                           "read_probe_gbs")}
        keep["entry_point"] = bench.get("config", {}).get("entry_point")
        lines += ["", "Bench line of an untraced run of the same code (bench.py without the profiler; "
                  "headline fields and roofline):", "", "```",
                  json.dumps(keep), json.dumps(bench.get("roofline")), "```"]
    passes = stream_passes(a.stats)
    if passes:
        lines += ["", "Graph passes of the 64-layer separate-call stream in the same trace (per layer: "
                  "tb_ffn_gateup_silu_x, then tb_ffn_down_split; at M=1 the gate/up launch rotates x "
                  "itself and the down call is rotquant + GEMV, at M=8 gate/up is rotquant + GEMV and "
                  "the down call the split GEMV + fold). Durations and gaps are medians over "
                  "every layer of every graph pass; a negative gap means the tracer stamped the next "
                  "start before the previous end. Kernel-only GB/s counts weight bytes over the "
                  "traced duration. The tracer's completion signal per dispatch lengthens passes, "
                  "at M=1 most of all, so span per layer here exceeds the untraced figure below.",
                  "", "| stream | passes | kernel | median us | kernel-only GB/s | median gap after us "
                  "| mean gap after us |", "|---|---|---|---|---|---|---|"]
        for label, r in passes.items():
            for name, dur, gap, mgap, wb in r["positions"]:
                gbs = f"{wb / dur / 1e3:.0f}" if wb else "-"
                lines.append(f"| {label} | {r['passes']} | `{name}` | {dur:.2f} | {gbs} | {gap:.2f} | "
                             f"{mgap:.2f} |")
        lines += ["", "| stream | traced span per layer us | traced kernel busy per layer us |",
                  "|---|---|---|"]
        for label, r in passes.items():
            lines.append(f"| {label} | {r['span_us']:.2f} | {r['busy_us']:.2f} |")
    if bench and bench.get("m1_call_breakdown"):
        lines += ["", "Untraced per-call device time at M=1 from that bench run (HIP events around "
                  "graph replays of 64 back-to-back calls of one kind):", "", "```",
                  json.dumps(bench["m1_call_breakdown"]), "```"]
    os.makedirs(a.out, exist_ok=True)
    with open(os.path.join(a.out, "ffn64_stream_kernel_stats.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    ff = copy_factor(os.path.join(a.pmc, "pmc_copy_FETCH_SIZE"), "FETCH_SIZE", COPY_BYTES)
    wf = copy_factor(os.path.join(a.pmc, "pmc_copy_WRITE_SIZE"), "WRITE_SIZE", COPY_BYTES)
    fetch = read_counter(os.path.join(a.pmc, "pmc_FETCH_SIZE"), "FETCH_SIZE")
    write = read_counter(os.path.join(a.pmc, "pmc_WRITE_SIZE"), "WRITE_SIZE")
    doc = {"source_sha256": source_sha256(), "source_files": SOURCES,
           "calibration": {"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "kernels": {}}
    rows = []
    for key, alg in ALGORITHMIC.items():
        if key not in fetch or key not in write:
            continue
        fk = sum(fetch[key]) / len(fetch[key])
        wk = sum(write[key]) / len(write[key])
        fb = int(fk * 1024 / ff)
        wb = int(wk * 1024 / wf)
        doc["kernels"][key] = {"fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                               "traffic_bytes_per_launch": fb + wb, "algorithmic_bytes_per_launch": alg,
                               "traffic_over_algorithmic": round((fb + wb) / alg, 4),
                               "fetch_raw_kib": round(fk, 1), "write_raw_kib": round(wk, 1),
                               "dispatches": len(fetch[key])}
        rows.append(f"| `{key}` | {fk:.1f} | {wk:.1f} | {fb} | {wb} | {alg} | {(fb + wb) / alg:.4f} |")
    with open(os.path.join(a.out, "ffn64_stream_traffic.json"), "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    cmds = []
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cmds.append(f"rocprofv3 --pmc {c} --output-format csv -d <out>/pmc_{c} -o run -- "
                    "python3 /root/repo/bench.py --profile-only")
        cmds.append(f"rocprofv3 --pmc {c} --output-format csv -d <out>/pmc_copy_{c} -o run -- "
                    "python3 /root/repo/bench.py --copy-probe-mib 1024")
    md = ["# HBM traffic per launch: 64-layer FFN stream at M=1 and M=8 (hidden 5120, intermediate 17408)", "",
          "Commands (on the MI355X host, from /tmp with TMPDIR=/tmp; one counter per run; the copy runs "
          "calibrate the counters):", "", "```", *cmds, "```", "",
          f"Calibration: a device copy of 1 GiB (reads 1 GiB, writes 1 GiB) reads FETCH_SIZE x{ff:.4f} "
          f"and WRITE_SIZE x{wf:.4f} of its true bytes; the factors below scale the counters.", "",
          "| kernel | FETCH raw KiB | WRITE raw KiB | fetched B (scaled) | written B | algorithmic B | "
          "traffic / algorithmic |", "|---|---|---|---|---|---|---|", *rows, ""]
    for key in doc["kernels"]:
        md.append(f"- `{key}`: {WHAT[key]}.")
    md += ["", "Algorithmic bytes: weights + activations read + outputs written. Per-dispatch averages "
           "over every dispatch of the kernel in the run.", "",
           f"Kernel sources hashed (sha256 over {', '.join(SOURCES)}): `{doc['source_sha256']}`. "
           "bench.py reports these bytes as `roofline.traffic` only while the sources hash to this value."]
    with open(os.path.join(a.out, "ffn64_stream_traffic.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(f"wrote {a.out}/ffn64_stream_kernel_stats.md, ffn64_stream_traffic.md/.json")


if __name__ == "__main__":
    main()
