"""The lookup-table GEMV over row-interleaved sign weights (TB_FMT_SIGN1_RI4), on MI355X.

tb_sign_interleave must produce exactly the byte permutation the layout defines (checked
against numpy). Through the interleaved matrix, tb_gemv_ternary runs the lookup-table
kernel: its y must be bit-identical to the bit-mask kernel on the original matrix (same
integer sums, same fold), within 1e-4 * sum|terms| of the oracle, and its block sums
(tb_gemv_block_sums) bit-exact against the oracle, also for int8 inputs over the full
range -128..127. Shapes: the FFN's, and ragged block counts (a partial last step of 16
blocks), one block, and fewer 4-row groups than CUs. One and two rows.
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

SIGN = synth.FMT_SIGN1
SHAPES = [(synth.INTER, synth.HIDDEN), (synth.HIDDEN, synth.INTER), (96, 1280), (1152, 640),
          (64, 128), (1028, 2176)]


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


def interleave_host(w: synth.PackedMatrix):
    """The layout's definition: byte r of word j of (quad, block) = byte j of row 4 quad + r."""
    nb = w.k // 128
    c = w.codes.reshape(w.n // 4, 4, nb, 16)              # [quad][r][b][j]
    codes = np.ascontiguousarray(c.transpose(0, 2, 3, 1))  # [quad][b][j][r]
    s = w.scales.reshape(w.n // 4, 4, nb)
    scales = np.ascontiguousarray(s.transpose(0, 2, 1))    # [quad][b][r]
    return codes.reshape(-1), scales.reshape(-1)


@pytest.mark.parametrize("n,k", [(64, 384), (1028, 2176)])
def test_interleave_layout(n, k):
    w = synth.matrix(SIGN, n, k, 120, 0, synth.T_GATE)
    wd = tb.Matrix.upload(w)
    ri = tb.tb_sign_interleave(wd)
    codes, scales = interleave_host(w)
    assert np.array_equal(gu.host(ri.codes).reshape(-1), codes)
    assert np.array_equal(gu.host(ri.scales).view(np.uint16).reshape(-1), scales)
    assert ri.fmt == tb.TB_FMT_SIGN1_RI4


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2])
def test_lut_gemv(o, n, k, m):
    say(f"lookup-table GEMV n={n} k={k} m={m}")
    w = synth.matrix(SIGN, n, k, 121, 0, synth.T_GATE)
    wd = tb.Matrix.upload(w)
    ri = tb.tb_sign_interleave(wd)
    q, dq = o.rotate_quant(synth.student_t_rows(m, k, 122, 0))
    y = gu.gemv(ri, q, dq)
    assert y.tobytes() == gu.gemv(wd, q, dq).tobytes(), "differs from the bit-mask kernel"
    yo, sabs = o.gemv(w, q, dq)
    ok, worst = bounds.gemv_ok(y, yo, sabs)
    say(f"  worst err / (1e-4 sum|tau|) = {worst:.3g}")
    assert ok
    got = gu.block_sums(ri, q)
    want = o.block_sums(w, q)
    assert np.array_equal(got, want), f"block sums differ at {np.argwhere(got != want)[:5]}"
    if m == 2:
        for r in range(2):
            assert gu.gemv(ri, q[r:r + 1], dq[r:r + 1])[0].tobytes() == y[r].tobytes(), r


@pytest.mark.parametrize("n,k", [(1152, 640), (synth.HIDDEN, synth.INTER)])
def test_lut_block_sums_full_int8_range(o, n, k):
    # every nibble split: -128 .. 127, the extremes in whole blocks
    w = synth.matrix(SIGN, n, k, 123, 0, synth.T_GATE)
    ri = tb.tb_sign_interleave(tb.Matrix.upload(w))
    rng = np.random.default_rng(124)
    q = rng.integers(-128, 128, size=(2, k), dtype=np.int64).astype(np.int8)
    q[0, :128] = -128
    q[1, 128:256] = 127
    got = gu.block_sums(ri, q)
    assert np.array_equal(got, o.block_sums(w, q))


def test_lut_limits():
    w = synth.matrix(SIGN, 64, 256, 125, 0, synth.T_GATE)
    wd = tb.Matrix.upload(w)
    ri = tb.tb_sign_interleave(wd)
    q = gu.dev(np.zeros((3, 256), np.int8))
    dq = gu.dev(np.zeros((3, 2), np.float32))
    y = gu.f32_out(3, 64)
    with pytest.raises(tb.TbError) as e:
        tb.tb_gemv_ternary(ri, q, dq, y)
    assert e.value.status == tb.TB_EUNSUPPORTED
    h = gu.f32_out(1, 64)
    with pytest.raises(tb.TbError) as e:
        tb.tb_ffn_gateup_silu(ri, ri, q[:1], dq[:1], h)
    assert e.value.status == tb.TB_EUNSUPPORTED
