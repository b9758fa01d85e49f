"""The fused multi-layer entry point tb_ffn_layers against the separate calls and the oracle.

tb_ffn_layers runs, per layer, the same device code as tb_rotate_quant_i8 ->
tb_ffn_gateup_silu -> tb_ffn_down, so its y must be bit-identical to those three
calls (which test_gpu_parity.py holds to the oracle); the first layer of each case is
also checked against the oracle here. Shapes span ragged last steps (hidden 640 and
inter 2176 are not multiples of the 16-chunk step), waves with no down rows, the full
5120 x 17408 layer, more than 32 layers (two launches), chaining, graph replay and
the bounded-wait error path (forced from the host with a tiny spin limit).
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import ternary_weight_int8_tb_amd as tb
from tests import bounds
from tests import gpu_util as gu
from ternary_weight_int8_tb_amd import synth

pytestmark = pytest.mark.gpu

TERN, SIGN = synth.FMT_TERNARY2, synth.FMT_SIGN1


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


def make_layers(seed, count, hidden, inter, fmt):
    host_layers, dev_layers = [], []
    for l in range(count):
        lay = synth.ffn_layer(seed, l, fmt, hidden=hidden, inter=inter)
        host_layers.append(lay)
        dev_layers.append(gu.GpuLayer(lay))
    return host_layers, dev_layers


def workspace(m, hidden, inter, spin_ticks=0):
    nb = tb.tb_ffn_workspace_bytes(m, hidden, inter)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=gu.DEV)
    tb.tb_ffn_workspace_init(ws, spin_ticks)
    return ws


def fused(dev_layers, x: np.ndarray, m, ws, chain=False, stream=None):
    """x: [L][m][H] or [m][H] (chain). Returns y [L][m][H] as numpy."""
    arr = tb.FfnLayers([(g.gate, g.up, g.down) for g in dev_layers])
    H = dev_layers[0].hidden
    y = gu.f32_out(len(dev_layers), m, H)
    tb.tb_ffn_layers(arr, gu.dev(x), ws, y, chain=chain, stream=stream)
    return gu.host(y)


def separate(dev_layers, xs, m, chain=False):
    """The three separate calls per layer. xs: [L][m][H] or [m][H] (chain)."""
    ys = []
    prev = None
    for l, g in enumerate(dev_layers):
        x = (xs if l == 0 else prev) if chain else xs[l]
        got = gu.LayerRun(g, m).run(x)
        ys.append(got["y"])
        prev = got["y"]
    return np.stack(ys)


def check_first_layer_vs_oracle(o, layer, x, y):
    r = o.ffn(layer, x)
    # y of the fused call equals the separate calls bit for bit; its distance to the
    # oracle is bounded like a chained layer (rotquant(h) may flip codes near ties)
    tol_h = bounds.h_tolerance(r["g"], r["u"], r["sg"], r["su"])
    wd = layer.down
    isum_or = o.block_sums(wd, r["qh"])
    *_, extra = bounds.chain_bounds(r["h"], tol_h, r["qh"], r["dqh"], isum_or,
                                    bounds.nonzero_weights(wd),
                                    wd.scales_f32().astype(np.float64), float(o.dq_unit()))
    err = np.abs(y.astype(np.float64) - r["y"])
    tol = bounds.GEMV_REL * (r["sabs"] + extra) + extra
    assert np.all(err <= tol), f"y worst {np.max(err / tol):.3g}"


CASES = [
    # (hidden, inter, layers, fmt, m)
    (256, 384, 3, TERN, 1),
    (256, 384, 3, SIGN, 2),
    (640, 2176, 3, TERN, 3),
    (640, 2176, 3, SIGN, 8),
    (1152, 640, 2, TERN, 8),
    (1152, 640, 2, SIGN, 5),
    (1152, 640, 2, SIGN, 6),   # sign on 8 waves from 6 rows (12 for 2 to 5, 16 for 1)
]


@pytest.mark.parametrize("hidden,inter,count,fmt,m", CASES)
def test_fused_matches_separate_calls(o, hidden, inter, count, fmt, m):
    say(f"fused: H={hidden} N={inter} L={count} fmt={fmt} M={m}")
    hl, dl = make_layers(20 + fmt, count, hidden, inter, fmt)
    xs = np.stack([synth.normal_rows(m, hidden, 20 + fmt, l) for l in range(count)])
    ws = workspace(m, hidden, inter)
    y = fused(dl, xs, m, ws)
    ref = separate(dl, xs, m)
    assert y.tobytes() == ref.tobytes()
    assert tb.tb_ffn_workspace_error(ws) == 0
    check_first_layer_vs_oracle(o, hl[0], xs[0], y[0])
    # the workspace is ready for the next call: run again and get the same bytes
    y2 = fused(dl, xs, m, ws)
    assert y2.tobytes() == y.tobytes()


@pytest.mark.parametrize("fmt,m", [(TERN, 1), (TERN, 8), (SIGN, 1), (SIGN, 8)])
def test_fused_full_size_layers(o, fmt, m):
    say(f"fused: 5120 x 17408, 2 layers, fmt={fmt} M={m}")
    hl, dl = make_layers(30 + fmt, 2, synth.HIDDEN, synth.INTER, fmt)
    xs = np.stack([synth.student_t_rows(m, synth.HIDDEN, 30 + fmt, l) for l in range(2)])
    ws = workspace(m, synth.HIDDEN, synth.INTER)
    y = fused(dl, xs, m, ws)
    ref = separate(dl, xs, m)
    assert y.tobytes() == ref.tobytes()
    check_first_layer_vs_oracle(o, hl[0], xs[0], y[0])


# Shapes whose steps are whole (hidden and intermediate multiples of 1024 for ternary, 2048
# for sign), with shares of 1 to 8 row tiles per CU, at one and two rows.
WHOLE_STEP_CASES = [
    # (hidden, inter, layers, fmt, m)
    (1024, 2048, 3, TERN, 1),
    (2048, 8192, 3, TERN, 2),
    (1024, 3072, 4, TERN, 2),
    (2048, 4096, 3, SIGN, 1),
    (2048, 4096, 3, SIGN, 2),
]


@pytest.mark.parametrize("hidden,inter,count,fmt,m", WHOLE_STEP_CASES)
@pytest.mark.parametrize("chain", [False, True])
def test_fused_whole_step_shapes(o, hidden, inter, count, fmt, m, chain):
    say(f"fused {hidden}x{inter} layers={count} fmt={fmt} m={m} chain={chain}")
    hl, dl = make_layers(90 + fmt, count, hidden, inter, fmt)
    if chain:
        x = synth.normal_rows(m, hidden, 90 + fmt, 0)
    else:
        x = np.stack([synth.normal_rows(m, hidden, 90 + fmt, l) for l in range(count)])
    y = fused(dl, x, m, workspace(m, hidden, inter), chain=chain)
    ref = separate(dl, x, m, chain=chain)
    assert y.tobytes() == ref.tobytes()
    check_first_layer_vs_oracle(o, hl[0], x if chain else x[0], y[0])


def test_fused_one_row_more_than_32_layers_and_replay():
    say("fused: one row, 34 layers (two launches), then graph replays")
    _, dl = make_layers(95, 34, 1024, 2048, TERN)
    xs = np.stack([synth.normal_rows(1, 1024, 95, l) for l in range(34)])
    ws = workspace(1, 1024, 2048)
    ref = separate(dl, xs, 1)
    assert fused(dl, xs, 1, ws).tobytes() == ref.tobytes()
    arr = tb.FfnLayers([(g.gate, g.up, g.down) for g in dl])
    xd = gu.dev(xs)
    y = gu.f32_out(34, 1, 1024)
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            tb.tb_ffn_layers(arr, xd, ws, y, stream=cs)
    torch.cuda.current_stream().wait_stream(cs)
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        assert gu.host(y).tobytes() == ref.tobytes(), rep


def test_fused_rows_bit_identical_to_row_alone():
    say("fused: M=8 rows vs each row alone")
    _, dl = make_layers(40, 2, 640, 2176, TERN)
    xs = np.stack([synth.normal_rows(8, 640, 40, l) for l in range(2)])
    y8 = fused(dl, xs, 8, workspace(8, 640, 2176))
    ws1 = workspace(1, 640, 2176)
    for r in range(8):
        y1 = fused(dl, np.ascontiguousarray(xs[:, r:r + 1]), 1, ws1)
        assert y1[:, 0].tobytes() == y8[:, r].tobytes(), r


@pytest.mark.parametrize("fmt", [TERN, SIGN])
def test_fused_chain(fmt):
    say(f"fused chain: 5 layers, fmt={fmt}")
    _, dl = make_layers(50 + fmt, 5, 640, 2176, fmt)
    x = synth.normal_rows(3, 640, 50 + fmt, 0)
    y = fused(dl, x, 3, workspace(3, 640, 2176), chain=True)
    ref = separate(dl, x, 3, chain=True)
    assert y.tobytes() == ref.tobytes()


@pytest.mark.parametrize("chain", [False, True])
def test_fused_more_than_32_layers(chain):
    say(f"fused: 35 layers (two launches), chain={chain}")
    _, dl = make_layers(60, 35, 256, 384, TERN)
    if chain:
        x = synth.normal_rows(2, 256, 60, 0)
    else:
        x = np.stack([synth.normal_rows(2, 256, 60, l) for l in range(35)])
    y = fused(dl, x, 2, workspace(2, 256, 384), chain=chain)
    ref = separate(dl, x, 2, chain=chain)
    assert y.tobytes() == ref.tobytes()


def test_fused_graph_replay():
    say("fused: graph replay x3 with eager work between")
    _, dl = make_layers(70, 3, 640, 2176, TERN)
    m = 4
    xs = np.stack([synth.normal_rows(m, 640, 70, l) for l in range(3)])
    ws = workspace(m, 640, 2176)
    ref = fused(dl, xs, m, ws)
    arr = tb.FfnLayers([(g.gate, g.up, g.down) for g in dl])
    xd = gu.dev(xs)
    y = gu.f32_out(3, m, 640)
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            tb.tb_ffn_layers(arr, xd, ws, y, stream=cs)
    torch.cuda.current_stream().wait_stream(cs)
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        got = gu.host(y)
        assert got.tobytes() == ref.tobytes(), rep
        # eager work on the same workspace between replays
        again = fused(dl, xs, m, ws)
        assert again.tobytes() == ref.tobytes(), rep


def test_fused_wait_limit_sets_sticky_error():
    say("fused: a 1-tick spin limit runs out; the error is sticky until re-init")
    _, dl = make_layers(80, 2, synth.HIDDEN, synth.INTER, TERN)
    m = 1
    xs = np.stack([synth.normal_rows(m, synth.HIDDEN, 80, l) for l in range(2)])
    ws = workspace(m, synth.HIDDEN, synth.INTER, spin_ticks=1)
    fused(dl, xs, m, ws)                       # outputs undefined; must finish
    assert tb.tb_ffn_workspace_error(ws) == 1
    y = fused(dl, xs, m, ws)                   # does nothing while the error is set
    assert np.isnan(y).all()
    assert tb.tb_ffn_workspace_error(ws) == 1
    tb.tb_ffn_workspace_init(ws, 0)
    y = fused(dl, xs, m, ws)
    assert tb.tb_ffn_workspace_error(ws) == 0
    assert y.tobytes() == separate(dl, xs, m).tobytes()
