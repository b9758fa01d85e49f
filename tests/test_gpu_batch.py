"""Batches above 8 rows (the *_batch calls, 1..32 rows) against the oracle, on MI355X.

Bars, as for the 1..8-row calls: block sums bit-exact; y within 1e-4 * sum|terms|;
h within the propagated bound; rotquant codes and scales bit-exact; and every row
of a batch bit-identical to the same row run alone through the 1..8-row calls.
The shapes are the FFN's (gate/up 17408 x 5120, down 5120 x 17408), where gate/up
runs 16 rows per matrix-core launch (ternary from 17 rows: one launch, k staged in two
phases) and the down GEMV chunks of 8, plus ragged shapes whose block count takes the
chunks-of-8 route.
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
FFN_SHAPES = [(synth.INTER, synth.HIDDEN), (synth.HIDDEN, synth.INTER)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert tb.tb_abi_version() == tb.ABI_VERSION
    yield


@pytest.fixture(scope="module")
def mats():
    return {(fmt, n, k): synth.matrix(fmt, n, k, 31, 0, synth.T_GATE)
            for fmt in (TERN, SIGN) for (n, k) in FFN_SHAPES}


def _rows(fmt, m, k, seed):
    return (synth.student_t_rows if fmt == SIGN else synth.normal_rows)(m, k, seed, 0)


def gemv_batch(w, q, dq):
    y = gu.f32_out(q.shape[0], w.n)
    tb.tb_gemv_ternary_batch(w, gu.dev(q), gu.dev(dq), y)
    return gu.host(y)


def block_sums_batch(w, q):
    out = gu.i32_out(q.shape[0], w.n, w.k // 128)
    tb.tb_gemv_block_sums_batch(w, gu.dev(q), out)
    return gu.host(out)


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("n,k", FFN_SHAPES)
@pytest.mark.parametrize("m", [9, 16, 17, 32])
def test_batch_gemv_full_shape(o, mats, fmt, n, k, m):
    say(f"batch gemv fmt={fmt} n={n} k={k} m={m}")
    w = mats[(fmt, n, k)]
    wd = tb.Matrix.upload(w)
    q, dq = o.rotate_quant(_rows(fmt, m, k, 40 + m))
    y = gemv_batch(wd, q, dq)
    yo, sabs = o.gemv(w, q, dq)
    ok, worst = bounds.gemv_ok(y, yo, sabs)
    say(f"  worst err / (1e-4 sum|tau|) = {worst:.3g}")
    assert ok
    for r in range(m):
        assert gu.gemv(wd, q[r:r + 1], dq[r:r + 1])[0].tobytes() == y[r].tobytes(), f"row {r}"
    if m <= 17:
        got = block_sums_batch(wd, q)
        want = o.block_sums(w, q)
        assert np.array_equal(got, want), f"block sums differ at {np.argwhere(got != want)[:5]}"


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("m", [16, 32])
def test_batch_gateup_and_down_full_shape(o, fmt, m):
    say(f"batch gate/up + down fmt={fmt} m={m}")
    layer = synth.ffn_layer(32, 0, fmt)
    g = gu.GpuLayer(layer)
    x = _rows(fmt, m, synth.HIDDEN, 50 + m)
    q = gu.i8_out(m, synth.HIDDEN)
    dq = gu.f32_out(m, synth.HIDDEN // 128)
    tb.tb_rotate_quant_i8_batch(gu.dev(x), q, dq)
    qn, dqn = gu.host(q), gu.host(dq)
    qo, dqo = o.rotate_quant(x)
    assert np.array_equal(qn, qo) and np.array_equal(dqn.view(np.uint32), dqo.view(np.uint32))
    h = gu.f32_out(m, synth.INTER)
    tb.tb_ffn_gateup_silu_batch(g.gate, g.up, q, dq, h)
    hn = gu.host(h)
    r = o.gateup_silu(layer.gate, layer.up, qo, dqo)
    tol = bounds.h_tolerance(r["g"], r["u"], r["sg"], r["su"])
    assert np.all(np.abs(hn.astype(np.float64) - r["h"]) <= tol)
    # down on the GPU's own h: rotquant(h) bit-exact, y within the fold bar
    qh, dqh, y = gu.i8_out(m, synth.INTER), gu.f32_out(m, synth.INTER // 128), gu.f32_out(m, synth.HIDDEN)
    tb.tb_ffn_down_batch(g.down, h, qh, dqh, y)
    d = o.ffn_down(layer.down, hn)
    assert np.array_equal(gu.host(qh), d["qh"])
    assert np.array_equal(gu.host(dqh).view(np.uint32), d["dqh"].view(np.uint32))
    yn = gu.host(y)
    assert bounds.gemv_ok(yn, d["y"], d["sabs"])[0]
    # each row alone through the 1..8-row calls
    for row in (0, 7, 8, m - 1):
        one = gu.LayerRun(g, 1).run(x[row:row + 1])
        assert one["h"][0].tobytes() == hn[row].tobytes(), f"h row {row}"
        assert one["y"][0].tobytes() == yn[row].tobytes(), f"y row {row}"


@pytest.mark.parametrize("fmt,n,k", [(TERN, 65, 640), (SIGN, 96, 1280), (TERN, 2176, 640),
                                     (SIGN, 1152, 5120), (TERN, 100, 1280)])
@pytest.mark.parametrize("m", [9, 24, 32])
def test_batch_ragged_shapes(o, fmt, n, k, m):
    # k/128 = 5 or 10 (sign): the matrix-core kernel cannot take these, so chunks of <= 8 run
    say(f"batch ragged fmt={fmt} n={n} k={k} m={m}")
    w = synth.matrix(fmt, n, k, 33, 0, synth.T_GATE)
    wd = tb.Matrix.upload(w)
    q, dq = o.rotate_quant(_rows(fmt, m, k, 60 + m))
    y = gemv_batch(wd, q, dq)
    yo, sabs = o.gemv(w, q, dq)
    assert bounds.gemv_ok(y, yo, sabs)[0]
    assert np.array_equal(block_sums_batch(wd, q), o.block_sums(w, q))
    for r in range(m):
        assert gu.gemv(wd, q[r:r + 1], dq[r:r + 1])[0].tobytes() == y[r].tobytes(), f"row {r}"


def test_batch_small_m_equals_the_1_to_8_calls(o):
    # up to 8 rows the batch calls run the same kernels as the calls without the suffix
    w = synth.matrix(TERN, 2176, 5120, 34, 0, synth.T_GATE)
    wd = tb.Matrix.upload(w)
    q, dq = o.rotate_quant(synth.normal_rows(8, 5120, 34, 0))
    for m in (1, 5, 8):
        assert gemv_batch(wd, q[:m], dq[:m]).tobytes() == gu.gemv(wd, q[:m], dq[:m]).tobytes()


def gateup_batch(wg, wu, q, dq):
    h = gu.f32_out(q.shape[0], wg.n)
    tb.tb_ffn_gateup_silu_batch(wg, wu, gu.dev(q), gu.dev(dq), h)
    return gu.host(h)


# k = 5120, 4096, 2304, 1280, 1024: 5, 4, 3, 2, 1 steps (the phases split them 3 + 2,
# 2 + 2, 2 + 1, 1 + 1 and 1 + 0); n with a partial 16-row tile in a workgroup
@pytest.mark.parametrize("n,k", [(synth.INTER, synth.HIDDEN), (1030, 4096), (100, 2304), (1030, 1280),
                                 (260, 1024)])
@pytest.mark.parametrize("m", [17, 24, 32])
def test_batch_gateup_one_launch_equals_chunks(o, n, k, m):
    # ternary gate/up of 17..32 rows runs as one launch with k staged in two phases; every
    # row must equal the same row through calls of at most 16 rows (and the oracle's bound)
    say(f"batch gate/up one launch n={n} k={k} m={m}")
    wg = synth.matrix(TERN, n, k, 35, 0, synth.T_GATE)
    wu = synth.matrix(TERN, n, k, 35, 0, synth.T_UP)
    g, u = tb.Matrix.upload(wg), tb.Matrix.upload(wu)
    q, dq = o.rotate_quant(synth.normal_rows(m, k, 36 + m, 0))
    h = gateup_batch(g, u, q, dq)
    for a in range(0, m, 16):
        b = min(a + 16, m)
        part = gateup_batch(g, u, q[a:b], dq[a:b])
        bad = np.argwhere(part.view(np.uint32) != h[a:b].view(np.uint32))
        assert bad.size == 0, f"rows {a}..{b - 1} differ from the one-launch batch at {bad[:5]}"
    r = o.gateup_silu(wg, wu, q, dq)
    tol = bounds.h_tolerance(r["g"], r["u"], r["sg"], r["su"])
    assert np.all(np.abs(h.astype(np.float64) - r["h"]) <= tol)
