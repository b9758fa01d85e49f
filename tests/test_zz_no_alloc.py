"""tb_ffn_down_noalloc (static scratch, no allocation) against tb_ffn_down, on MI355X.

Two calls in a row through the C ABI, the second with a smaller input: y must equal
tb_ffn_down's y byte for byte (same kernels and fold), and rotquant(h) from
tb_ffn_down's workspace must match the oracle. An input beyond the scratch limit is
rejected with TB_ESCRATCH and launches nothing. Runs alone in a fresh process and
after the other tests (the scratch keeps the previous call's contents, which no
call reads).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import ternary_weight_int8_tb_amd as tb
from tests import bounds
from tests import gpu_util as gu
from ternary_weight_int8_tb_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert tb.tb_abi_version() == tb.ABI_VERSION
    yield


@pytest.mark.parametrize("fmt", [synth.FMT_TERNARY2, synth.FMT_SIGN1])
def test_noalloc_down_matches_workspace_down(fmt):
    o = oracle.default()
    # first call: the full down shape at 8 rows; second: a smaller matrix and 3 rows
    for (n, k, m, seed) in ((synth.HIDDEN, synth.INTER, 8, 70), (640, 2176, 3, 71)):
        print(f"noalloc down fmt={fmt} n={n} k={k} m={m}", flush=True)
        w = synth.matrix(fmt, n, k, seed, 0, synth.T_DOWN)
        wd = tb.Matrix.upload(w)
        h = synth.normal_rows(m, k, seed, 0, synth.T_HIDDEN)
        hd = gu.dev(h)
        y_na = gu.f32_out(m, n)
        tb.tb_ffn_down_noalloc(wd, hd, y_na)
        qh, dqh, y_ws = gu.i8_out(m, k), gu.f32_out(m, k // 128), gu.f32_out(m, n)
        tb.tb_ffn_down(wd, hd, qh, dqh, y_ws)
        a, b = gu.host(y_na), gu.host(y_ws)
        assert a.tobytes() == b.tobytes(), "tb_ffn_down_noalloc differs from tb_ffn_down"
        d = o.ffn_down(w, h)
        assert np.array_equal(gu.host(qh), d["qh"])
        assert bounds.gemv_ok(a, d["y"], d["sabs"])[0]


def test_noalloc_rejects_inputs_beyond_the_scratch():
    # 8 rows of k = 127104 need 1,048,608 bytes of scratch, 32 more than it has
    n, k, m = 64, 127104, 8
    w = synth.matrix(synth.FMT_TERNARY2, n, k, 72, 0, synth.T_DOWN)
    wd = tb.Matrix.upload(w)
    h = torch.zeros(m, k, dtype=torch.float32, device="cuda")
    y = gu.f32_out(m, n)
    with pytest.raises(tb.TbError) as e:
        tb.tb_ffn_down_noalloc(wd, h, y)
    assert e.value.status == tb.TB_ESCRATCH
    assert torch.isnan(y).all()
