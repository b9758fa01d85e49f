"""The rotation inside the GEMV launch (tb_ffn_gateup_silu_x, and tb_ffn_down up to 4 rows).

For up to 4 rows on the dot-product core, every workgroup rotates and quantises the
fp32 input itself and workgroup 0 writes the int8 copy out. Bars: that copy (codes and
block scales) bit-exact against the oracle; h and y bit-identical to the separate
launches (tb_rotate_quant_i8, then tb_ffn_gateup_silu or tb_gemv_ternary), which the
other GPU tests hold to the oracle; and h within the propagated bound of the oracle's.
Rows 5..8 and shapes past the ring kernel take the two launches inside the call, and
are checked the same way.
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
    assert tb.tb_abi_version() == tb.ABI_VERSION
    yield


def _rows(fmt, m, k, seed):
    return (synth.student_t_rows if fmt == SIGN else synth.normal_rows)(m, k, seed, 0)


def gateup_x(wg, wu, x):
    m, k = x.shape
    qx, dqx, h = gu.i8_out(m, k), gu.f32_out(m, k // 128), gu.f32_out(m, wg.n)
    tb.tb_ffn_gateup_silu_x(wg, wu, gu.dev(x), qx, dqx, h)
    return gu.host(qx), gu.host(dqx), gu.host(h)


def gateup_two(wg, wu, x):
    q, dq = gu.rotquant(x)
    h = gu.f32_out(x.shape[0], wg.n)
    tb.tb_ffn_gateup_silu(wg, wu, gu.dev(q), gu.dev(dq), h)
    return gu.host(h)


def check_copy(o, x, q, dq):
    qo, dqo = o.rotate_quant(x)
    assert np.array_equal(q, qo), f"codes differ at {np.argwhere(q != qo)[:5]}"
    assert np.array_equal(dq.view(np.uint32), dqo.view(np.uint32)), "block scales differ"


@pytest.fixture(scope="module")
def ffn():
    return {fmt: synth.ffn_layer(90, 0, fmt) for fmt in (TERN, SIGN)}


@pytest.fixture(scope="module")
def ffn_dev(ffn):
    return {fmt: gu.GpuLayer(layer) for fmt, layer in ffn.items()}


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
def test_gateup_x_full_shape(o, ffn, ffn_dev, fmt, m):
    say(f"gate/up from x fmt={fmt} m={m}")
    g, layer = ffn_dev[fmt], ffn[fmt]
    x = _rows(fmt, m, synth.HIDDEN, 91 + m)
    q, dq, h = gateup_x(g.gate, g.up, x)
    check_copy(o, x, q, dq)
    assert h.tobytes() == gateup_two(g.gate, g.up, x).tobytes()
    r = o.gateup_silu(layer.gate, layer.up, q, dq)
    tol = bounds.h_tolerance(r["g"], r["u"], r["sg"], r["su"])
    assert np.all(np.abs(h.astype(np.float64) - r["h"]) <= tol)


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("m", [1, 2, 4, 6, 8])
def test_down_full_shape_equals_two_launches(o, ffn, ffn_dev, fmt, m):
    say(f"down (rotation inside) fmt={fmt} m={m}")
    g, layer = ffn_dev[fmt], ffn[fmt]
    h = _rows(fmt, m, synth.INTER, 95 + m).astype(np.float32)
    qh, dqh, y = gu.down(g.down, h)
    check_copy(o, h, qh, dqh)
    assert y.tobytes() == gu.gemv(g.down, qh, dqh).tobytes()
    d = o.ffn_down(layer.down, h)
    assert bounds.gemv_ok(y, d["y"], d["sabs"])[0]


# n not a multiple of the 4-row tile, k/128 odd (5) or not a multiple of 4 (10, sign),
# one 128-block (k = 128), fewer row tiles than CUs
RAGGED = [(TERN, 65, 640), (SIGN, 96, 1280), (TERN, 2176, 640), (SIGN, 1153, 5120),
          (TERN, 100, 128), (SIGN, 7, 384)]


@pytest.mark.parametrize("fmt,n,k", RAGGED)
@pytest.mark.parametrize("m", [1, 3, 4, 7])
def test_ragged_shapes(o, fmt, n, k, m):
    say(f"rotation inside, ragged fmt={fmt} n={n} k={k} m={m}")
    wg = synth.matrix(fmt, n, k, 96, 0, synth.T_GATE)
    wu = synth.matrix(fmt, n, k, 96, 0, synth.T_UP)
    gd, ud = tb.Matrix.upload(wg), tb.Matrix.upload(wu)
    x = _rows(fmt, m, k, 97 + m)
    q, dq, h = gateup_x(gd, ud, x)
    check_copy(o, x, q, dq)
    assert h.tobytes() == gateup_two(gd, ud, x).tobytes()
    # the same matrix as a down projection (k inputs, n outputs)
    qh, dqh, y = gu.down(gd, x)
    check_copy(o, x, qh, dqh)
    assert y.tobytes() == gu.gemv(gd, qh, dqh).tobytes()
    yo, sabs = o.gemv(wg, qh, dqh)
    assert bounds.gemv_ok(y, yo, sabs)[0]


def test_zero_and_constant_rows(o, ffn_dev):
    # an all-zero row quantises to codes 0 and scale 0; a constant row rotates to one
    # nonzero coefficient per block
    g = ffn_dev[TERN]
    x = np.zeros((3, synth.HIDDEN), np.float32)
    x[1] = 0.75
    x[2, ::2] = -1.5
    q, dq, h = gateup_x(g.gate, g.up, x)
    check_copy(o, x, q, dq)
    assert not q[0].any() and not dq[0].any()
    assert h.tobytes() == gateup_two(g.gate, g.up, x).tobytes()


def test_stream_of_calls_matches_separate_launches(o, ffn_dev):
    # one stream of x-calls and down calls, back to back, against the separate launches
    g = ffn_dev[TERN]
    xs = [synth.normal_rows(1, synth.HIDDEN, 98, i) for i in range(4)]
    run = gu.LayerRun(g, 1)
    for x in xs:
        want = run.run(x)
        q, dq, h = gateup_x(g.gate, g.up, x)
        assert h.tobytes() == want["h"].tobytes()
        qh, dqh, y = gu.down(g.down, h)
        assert y.tobytes() == want["y"].tobytes()
        assert qh.tobytes() == want["qh"].tobytes()
