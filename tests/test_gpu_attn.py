"""Second workload: the full-attention projections of the same model, on MI355X.

The fused query/gate/key/value projection (9216 x 5120) and the output
projection (5120 x 4096) through the same C ABI: rotate-quantise the input,
then the GEMV. Bars as for the FFN: rotquant and block sums bit-exact, y within
1e-4 * sum|terms|, batched rows bit-identical to rows alone. The attention
itself is not part of this path; the output projection takes stand-in rows.
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


@pytest.fixture(scope="module")
def layers():
    return {fmt: synth.attn_layer(80, 0, fmt) for fmt in (TERN, SIGN)}


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("which", ["qkvg", "o"])
@pytest.mark.parametrize("m", [1, 8])
def test_attention_projection(o, layers, fmt, which, m):
    w = getattr(layers[fmt], which)
    say(f"attention {which} fmt={fmt} n={w.n} k={w.k} m={m}")
    tensor = synth.T_ACT if which == "qkvg" else synth.T_ATTN_OUT
    x = synth.normal_rows(8, w.k, 81, 0, tensor)[:m]
    q, dq = gu.rotquant(x)
    qo, dqo = o.rotate_quant(x)
    assert np.array_equal(q, qo) and np.array_equal(dq.view(np.uint32), dqo.view(np.uint32))
    wd = tb.Matrix.upload(w)
    assert np.array_equal(gu.block_sums(wd, q), o.block_sums(w, q))
    y = gu.gemv(wd, q, dq)
    yo, sabs = o.gemv(w, q, dq)
    ok, worst = bounds.gemv_ok(y, yo, sabs)
    say(f"  worst err / (1e-4 sum|tau|) = {worst:.3g}")
    assert ok
    if m > 1:
        for r in range(m):
            assert gu.gemv(wd, q[r:r + 1], dq[r:r + 1])[0].tobytes() == y[r].tobytes(), r


@pytest.mark.parametrize("fmt", [TERN, SIGN])
def test_attention_projection_batch16(o, layers, fmt):
    w = layers[fmt].qkvg
    x = synth.normal_rows(16, w.k, 82, 0)
    q, dq = o.rotate_quant(x)
    wd = tb.Matrix.upload(w)
    y = gu.f32_out(16, w.n)
    tb.tb_gemv_ternary_batch(wd, gu.dev(q), gu.dev(dq), y)
    yn = gu.host(y)
    yo, sabs = o.gemv(w, q, dq)
    assert bounds.gemv_ok(yn, yo, sabs)[0]
    for r in (0, 9, 15):
        assert gu.gemv(wd, q[r:r + 1], dq[r:r + 1])[0].tobytes() == yn[r].tobytes(), r


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("which", ["qkvg", "o"])
@pytest.mark.parametrize("m", [1, 4, 8])
def test_attention_projection_from_fp32(o, layers, fmt, which, m):
    # tb_gemv_ternary_x (the rotation inside the GEMV's launch up to 4 rows) against the
    # oracle's rotquant and the two separate calls
    w = getattr(layers[fmt], which)
    say(f"attention {which} from fp32 fmt={fmt} m={m}")
    tensor = synth.T_ACT if which == "qkvg" else synth.T_ATTN_OUT
    x = synth.normal_rows(8, w.k, 83, 0, tensor)[:m]
    wd = tb.Matrix.upload(w)
    qx, dqx, y = gu.i8_out(m, w.k), gu.f32_out(m, w.k // 128), gu.f32_out(m, w.n)
    tb.tb_gemv_ternary_x(wd, gu.dev(x), qx, dqx, y)
    qn, dqn, yn = gu.host(qx), gu.host(dqx), gu.host(y)
    qo, dqo = o.rotate_quant(x)
    assert np.array_equal(qn, qo) and np.array_equal(dqn.view(np.uint32), dqo.view(np.uint32))
    assert yn.tobytes() == gu.gemv(wd, qo, dqo).tobytes()
    yo, sabs = o.gemv(w, qo, dqo)
    assert bounds.gemv_ok(yn, yo, sabs)[0]
