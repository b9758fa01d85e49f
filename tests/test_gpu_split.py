"""tb_ffn_down_split on MI355X: the down stage split over k (matrix cores: a GEMV launch
whose workgroups rotate their own step of h, then a fold launch). It is taken from 4 rows
while the unsplit GEMV would use the dot-product kernel, and on the matrix cores for
k >= 8192; elsewhere the call runs tb_ffn_down.

qh and dqh must be bit-identical to the oracle's rotate-quantise of h. y must be
bit-identical to tb_ffn_down on the same h: the rotation arithmetic, each row's step
partial and the step-order fold are the same. y must also lie within 1e-4 * sum|terms|
of the oracle's down GEMV.

Cases:
  * shapes: the FFN down shape (5120 x 17408); k >= 8192 with a partial 16-row tile
    (n = 1030, 100); k below 8192 (taken up to 5 rows: n = 1030, k = 1024; one step,
    k = 512); twice the FFN k (34 steps of 7 row groups); odd block counts (k = 2176,
    640, 128), which the split does not take;
  * both formats, 1..8 rows, zero and constant rows of h;
  * two calls in a row on one workspace;
  * a captured graph replayed three times, with eager work between the replays, every
    replay checked.

tb_ffn_down_split_batch (1 ... 32 rows): from 9 rows and k >= 8192 the batch runs on the
matrix-core kernel split over k (ternary: one launch, 16 or 32 B columns; sign: chunks of
up to 16 rows), with one fold launch. Every row's y, qh and dqh must be bit-identical to tb_ffn_down_batch (whose rows
are bit-identical to each row run alone, tests/test_gpu_batch.py) and, for sampled rows,
to tb_ffn_down on the row alone; y within the oracle's bound at the FFN shape for 16
and 32 rows. Shapes below k = 8192 and odd block counts take tb_ffn_down_batch.
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
SHAPES = [(synth.HIDDEN, synth.INTER), (1028, 2176), (1030, 640), (1030, 1024), (96, 1280),
          (64, 128), (256, 512), (260, 4096), (1030, 10240), (100, 8192)]


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


def hidden_rows(m, k, seed):
    h = synth.normal_rows(m, k, seed, 0, synth.T_HIDDEN)
    if m >= 3:
        h[1] = 0.0       # dq = 0 blocks
        h[2] = 0.75      # a constant row: one nonzero rotated element per block
    if m >= 8:
        h[7, :256] = 0.0  # zero blocks inside a row
    return h


def down_ref(wd, h):
    m, k = h.shape
    qh, dqh, y = gu.i8_out(m, k), gu.f32_out(m, k // 128), gu.f32_out(m, wd.n)
    tb.tb_ffn_down(wd, h, qh, dqh, y)
    return gu.host(qh).copy(), gu.host(dqh).copy(), gu.host(y).copy()


def down_split(wd, h, ws):
    m, k = h.shape
    qh, dqh, y = gu.i8_out(m, k), gu.f32_out(m, k // 128), gu.f32_out(m, wd.n)
    tb.tb_ffn_down_split(wd, h, qh, dqh, y, ws)
    return gu.host(qh).copy(), gu.host(dqh).copy(), gu.host(y).copy()


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8])
def test_down_split_equals_down(fmt, n, k, m):
    say(f"down split fmt={fmt} n={n} k={k} m={m}")
    wd = tb.Matrix.upload(synth.matrix(fmt, n, k, 31, 0, synth.T_DOWN))
    h = gu.dev(hidden_rows(m, k, 32 + m))
    want = down_ref(wd, h)
    ws = tb.tb_ffn_down_split_workspace(wd, m)
    for rep in range(2):   # the second call reuses the workspace the first one wrote
        got = down_split(wd, h, ws)
        assert np.array_equal(got[0], want[0]), f"qh differs (call {rep})"
        assert got[1].tobytes() == want[1].tobytes(), f"dqh differs (call {rep})"
        bad = np.argwhere(got[2].view(np.uint32) != want[2].view(np.uint32))
        assert bad.size == 0, f"y differs from tb_ffn_down at {bad[:5]} (call {rep})"


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("n,k,m", [(synth.HIDDEN, synth.INTER, 8), (synth.HIDDEN, synth.INTER, 5),
                                   (1030, 10240, 6), (1030, 1024, 4)])
def test_down_split_against_oracle(o, fmt, n, k, m):
    say(f"down split vs oracle fmt={fmt} n={n} k={k} m={m}")
    w = synth.matrix(fmt, n, k, 33, 0, synth.T_DOWN)
    wd = tb.Matrix.upload(w)
    h = hidden_rows(m, k, 34)
    qh, dqh, y = down_split(wd, gu.dev(h), tb.tb_ffn_down_split_workspace(wd, m))
    r = o.ffn_down(w, h)
    assert np.array_equal(qh, r["qh"])
    assert np.array_equal(dqh.view(np.uint32), r["dqh"].view(np.uint32))
    ok, worst = bounds.gemv_ok(y, r["y"], r["sabs"])
    say(f"  worst err / (1e-4 sum|tau|) = {worst:.3g}")
    assert ok


def test_down_split_many_steps():
    # 34 steps: 7 row groups of 183 tiles (the largest group LDS plan), 238 workgroups
    n, k = synth.HIDDEN, 2 * synth.INTER
    wd = tb.Matrix.upload(synth.matrix(TERN, n, k, 35, 0, synth.T_DOWN))
    h = gu.dev(hidden_rows(8, k, 36))
    want = down_ref(wd, h)
    got = down_split(wd, h, tb.tb_ffn_down_split_workspace(wd, 8))
    assert np.array_equal(got[0], want[0])
    assert got[2].tobytes() == want[2].tobytes()


def test_down_split_graph_replays():
    n, k, m = synth.HIDDEN, synth.INTER, 8
    wd = tb.Matrix.upload(synth.matrix(TERN, n, k, 37, 0, synth.T_DOWN))
    ws = tb.tb_ffn_down_split_workspace(wd, m)
    h = gu.dev(hidden_rows(m, k, 38))
    qh, dqh, y = gu.i8_out(m, k), gu.f32_out(m, k // 128), gu.f32_out(m, n)
    tb.tb_ffn_down_split(wd, h, qh, dqh, y, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tb.tb_ffn_down_split(wd, h, qh, dqh, y, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        h.copy_(gu.dev(hidden_rows(m, k, 100 + rep)))   # eager work between the replays
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = down_ref(wd, h)
        assert np.array_equal(gu.host(qh), want[0]), rep
        assert gu.host(y).tobytes() == want[2].tobytes(), rep


def down_batch_ref(wd, h):
    m, k = h.shape
    qh, dqh, y = gu.i8_out(m, k), gu.f32_out(m, k // 128), gu.f32_out(m, wd.n)
    tb.tb_ffn_down_batch(wd, h, qh, dqh, y)
    return gu.host(qh).copy(), gu.host(dqh).copy(), gu.host(y).copy()


def down_split_batch(wd, h, ws):
    m, k = h.shape
    qh, dqh, y = gu.i8_out(m, k), gu.f32_out(m, k // 128), gu.f32_out(m, wd.n)
    tb.tb_ffn_down_split_batch(wd, h, qh, dqh, y, ws)
    return gu.host(qh).copy(), gu.host(dqh).copy(), gu.host(y).copy()


BATCH_SHAPES = [(synth.HIDDEN, synth.INTER), (1030, 10240), (100, 8192), (1030, 1024),
                (260, 4096), (1028, 2176)]


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("n,k", BATCH_SHAPES)
@pytest.mark.parametrize("m", [1, 8, 9, 12, 16, 17, 24, 32])
def test_down_split_batch_equals_batch(fmt, n, k, m):
    say(f"down split batch fmt={fmt} n={n} k={k} m={m}")
    wd = tb.Matrix.upload(synth.matrix(fmt, n, k, 41, 0, synth.T_DOWN))
    hh = hidden_rows(m, k, 42 + m)
    h = gu.dev(hh)
    want = down_batch_ref(wd, h)
    ws = tb.tb_ffn_down_split_workspace(wd, m, batch=True)
    assert ws.numel() == tb.tb_ffn_down_split_batch_workspace_bytes(wd, m)
    for rep in range(2):   # the second call reuses the workspace the first one wrote
        got = down_split_batch(wd, h, ws)
        assert np.array_equal(got[0], want[0]), f"qh differs (call {rep})"
        assert got[1].tobytes() == want[1].tobytes(), f"dqh differs (call {rep})"
        bad = np.argwhere(got[2].view(np.uint32) != want[2].view(np.uint32))
        assert bad.size == 0, f"y differs from tb_ffn_down_batch at {bad[:5]} (call {rep})"
    for r in sorted({0, m // 2, m - 1}):   # rows alone through the 1 ... 8-row call
        alone = down_ref(wd, gu.dev(hh[r:r + 1]))
        assert np.array_equal(got[0][r], alone[0][0]), f"qh row {r} differs from the row alone"
        assert got[2][r].tobytes() == alone[2][0].tobytes(), f"y row {r} differs from the row alone"


@pytest.mark.parametrize("fmt,m", [(TERN, 16), (TERN, 32), (SIGN, 16), (SIGN, 32)])
def test_down_split_batch_against_oracle(o, fmt, m):
    n, k = synth.HIDDEN, synth.INTER
    say(f"down split batch vs oracle fmt={fmt} m={m}")
    w = synth.matrix(fmt, n, k, 43, 0, synth.T_DOWN)
    wd = tb.Matrix.upload(w)
    h = hidden_rows(m, k, 44)
    qh, dqh, y = down_split_batch(wd, gu.dev(h), tb.tb_ffn_down_split_workspace(wd, m, batch=True))
    r = o.ffn_down(w, h)
    assert np.array_equal(qh, r["qh"])
    assert np.array_equal(dqh.view(np.uint32), r["dqh"].view(np.uint32))
    ok, worst = bounds.gemv_ok(y, r["y"], r["sabs"])
    say(f"  worst err / (1e-4 sum|tau|) = {worst:.3g}")
    assert ok


def test_down_split_batch_many_steps():
    # 34 steps: 7 row groups, 238 workgroups per chunk, two chunks of 10 rows
    n, k, m = synth.HIDDEN, 2 * synth.INTER, 20
    wd = tb.Matrix.upload(synth.matrix(TERN, n, k, 45, 0, synth.T_DOWN))
    h = gu.dev(hidden_rows(m, k, 46))
    want = down_batch_ref(wd, h)
    got = down_split_batch(wd, h, tb.tb_ffn_down_split_workspace(wd, m, batch=True))
    assert np.array_equal(got[0], want[0])
    assert got[2].tobytes() == want[2].tobytes()


def test_down_split_batch_graph_replays():
    n, k, m = synth.HIDDEN, synth.INTER, 32
    wd = tb.Matrix.upload(synth.matrix(TERN, n, k, 47, 0, synth.T_DOWN))
    ws = tb.tb_ffn_down_split_workspace(wd, m, batch=True)
    h = gu.dev(hidden_rows(m, k, 48))
    qh, dqh, y = gu.i8_out(m, k), gu.f32_out(m, k // 128), gu.f32_out(m, n)
    tb.tb_ffn_down_split_batch(wd, h, qh, dqh, y, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tb.tb_ffn_down_split_batch(wd, h, qh, dqh, y, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        h.copy_(gu.dev(hidden_rows(m, k, 200 + rep)))   # eager work between the replays
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = down_batch_ref(wd, h)
        assert np.array_equal(gu.host(qh), want[0]), rep
        assert gu.host(y).tobytes() == want[2].tobytes(), rep
