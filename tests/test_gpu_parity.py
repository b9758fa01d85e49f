"""Parity of the HIP path (through the C ABI) with the CPU oracle, on MI355X.

Bars:
  * q, dq (rotate-quantise), isum (block sums), qh, dqh: bit-exact;
  * y: |err| <= 1e-4 * sum|terms| per output;
  * h: the propagated bound of tests/bounds.py;
  * a batched row is bit-identical to the same row run alone, for every output;
  * rotquant(h) of a chained layer: every code within the interval an h within tolerance
    can produce, and y within the matching bound.
Inputs are seeded synthetic data from ternary_weight_int8_tb_amd.synth.
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


def _x(kind: str, m: int, k: int, seed: int) -> np.ndarray:
    if kind == "normal":
        return synth.normal_rows(m, k, seed, 0)
    if kind == "student":
        return synth.student_t_rows(m, k, seed, 0)
    x = synth.normal_rows(m, k, seed, 0)
    if kind == "special":
        x[0] = 0.0                                    # all-zero row: q = 0, dq = 0
        if m > 1:
            x[1] = 0.0
            x[1, 7] = -3.25                          # spike: |u| equal everywhere
        if m > 2:
            x[2] *= np.float32(2.0 ** -100)          # tiny magnitudes
    return x


# ----------------------------------------------------------------- a1, a2: rotate + quantise
@pytest.mark.parametrize("k", [128, 256, 640, 2176, 5120, 17408])
@pytest.mark.parametrize("m", [1, 3, 8])
@pytest.mark.parametrize("kind", ["normal", "student", "special"])
def test_rotquant_bitexact(o, k, m, kind):
    say(f"rotquant k={k} m={m} kind={kind}")
    x = _x(kind, m, k, 100 + k + m)
    q, dq = gu.rotquant(x)
    qo, dqo = o.rotate_quant(x)
    assert np.array_equal(q, qo), f"q mismatch at {np.argwhere(q != qo)[:5]}"
    assert np.array_equal(dq.view(np.uint32), dqo.view(np.uint32))


def test_rotquant_ties(o):
    # a block whose rotation is exactly 127, 2.5, 3.5, ... (see the oracle pins)
    u_t = np.zeros(128)
    u_t[:9] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -3.5, 126.5]
    x = (bounds.H @ u_t / 128).astype(np.float32)[None, :]
    q, dq = gu.rotquant(x)
    qo, dqo = o.rotate_quant(x)
    assert np.array_equal(q, qo) and np.array_equal(dq, dqo)
    assert list(q[0, :9]) == [127, 2, 4, -2, 0, 2, 0, -4, 126]


# ----------------------------------------------------------------- a3, a4, a7, a9: GEMV
SHAPES = [(256, 512), (1, 128), (63, 256), (65, 640), (257, 2176), (2176, 640), (96, 17408)]


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", range(1, 9))   # the dot-product and matrix-core routes
def test_block_sums_and_gemv(o, fmt, n, k, m):
    say(f"gemv fmt={fmt} n={n} k={k} m={m}")
    w = synth.matrix(fmt, n, k, 7 + n + k, 0, synth.T_GATE)
    x = synth.normal_rows(m, k, 7 + n + k, 0)
    q, dq = o.rotate_quant(x)
    wd = tb.Matrix.upload(w)
    isum = gu.block_sums(wd, q)
    assert np.array_equal(isum, o.block_sums(w, q)), "block sums differ"
    y = gu.gemv(wd, q, dq)
    yo, sabs = o.gemv(w, q, dq)
    ok, worst = bounds.gemv_ok(y, yo, sabs)
    say(f"  worst err / (1e-4 sum|tau|) = {worst:.3g}")
    assert ok


@pytest.fixture(scope="module")
def full_mats():
    """The two FFN matrix shapes (gate/up 17408x5120, down 5120x17408) in both formats."""
    return {(fmt, n, k): synth.matrix(fmt, n, k, 21, 0, synth.T_GATE)
            for fmt in (TERN, SIGN) for (n, k) in ((synth.INTER, synth.HIDDEN),
                                                   (synth.HIDDEN, synth.INTER))}


@pytest.mark.parametrize("fmt", [TERN, SIGN])
@pytest.mark.parametrize("n,k", [(synth.INTER, synth.HIDDEN), (synth.HIDDEN, synth.INTER)])
@pytest.mark.parametrize("m", [5, 6, 7, 8])
def test_block_sums_matrix_core_full_shape(o, full_mats, fmt, n, k, m):
    # From M = 5 on the export runs the matrix-core integer core (v_mfma_i32_16x16x64_i8,
    # lane swaps, the D layout) that gate/up and the down GEMV run in production; its sums
    # must equal the oracle's bit for bit at the FFN shapes.
    say(f"block sums (matrix cores) fmt={fmt} n={n} k={k} m={m}")
    w = full_mats[(fmt, n, k)]
    x = (synth.student_t_rows if fmt == SIGN else synth.normal_rows)(m, k, 22 + m, 0)
    q, _ = o.rotate_quant(x)
    got = gu.block_sums(tb.Matrix.upload(w), q)
    want = o.block_sums(w, q)
    assert np.array_equal(got, want), f"block sums differ at {np.argwhere(got != want)[:5]}"


@pytest.mark.parametrize("fmt", [TERN, SIGN])
def test_sliced_and_streaming_kernels_fold_alike(o, fmt):
    # k = 24576: at M=8 the activation does not fit in LDS, so the sliced kernel runs; the
    # row alone (M=1) runs on the streaming kernel. Both fold every row in the same order,
    # so the batched rows must equal the rows alone bit for bit.
    n, k = 96, 24576
    say(f"sliced vs streaming fmt={fmt} n={n} k={k}")
    w = synth.matrix(fmt, n, k, 11, 0, synth.T_GATE)
    x = synth.normal_rows(8, k, 11, 0)
    q, dq = o.rotate_quant(x)
    wd = tb.Matrix.upload(w)
    y8 = gu.gemv(wd, q, dq)
    yo, sabs = o.gemv(w, q, dq)
    assert bounds.gemv_ok(y8, yo, sabs)[0]
    for r in range(8):
        y1 = gu.gemv(wd, q[r:r + 1], dq[r:r + 1])
        assert y1[0].tobytes() == y8[r].tobytes(), r


@pytest.mark.parametrize("fmt,n,k", [(TERN, 1, 256), (TERN, 100, 1280), (TERN, 2180, 1280),
                                     (TERN, 1152, 5120), (SIGN, 3, 512), (SIGN, 100, 1536),
                                     (SIGN, 2180, 1536), (SIGN, 1152, 5120)])
def test_matrix_core_and_dot_kernels_fold_alike(o, fmt, n, k):
    # Gate/up from M = 5 on, and a single GEMV from M = 6 (ternary)
    # or 7 (sign) on, run on the matrix cores (16-row tiles, rows past a CU's range masked;
    # the k = 1280 ternary and k = 1536 sign rows end in a ragged step); a row alone runs on
    # the dot-product kernel. Both fold every row in the same order, so the batched rows
    # must equal the rows alone bit for bit.
    say(f"matrix-core vs dot-product fmt={fmt} n={n} k={k}")
    wg = synth.matrix(fmt, n, k, 13, 0, synth.T_GATE)
    wu = synth.matrix(fmt, n, k, 13, 0, synth.T_UP)
    dg, du = tb.Matrix.upload(wg), tb.Matrix.upload(wu)

    def gateup(qm, dqm):
        h = gu.f32_out(qm.shape[0], n)
        tb.tb_ffn_gateup_silu(dg, du, gu.dev(qm), gu.dev(dqm), h)
        return gu.host(h)

    x = synth.normal_rows(8, k, 13, 0)
    q, dq = o.rotate_quant(x)
    alone = [gateup(q[r:r + 1], dq[r:r + 1])[0].tobytes() for r in range(8)]
    for m in (4, 5, 6, 7, 8):
        h = gateup(q[:m], dq[:m])
        for r in range(m):
            assert h[r].tobytes() == alone[r], f"M={m} row {r}"
    r = o.gateup_silu(wg, wu, q, dq)
    tol = bounds.h_tolerance(r["g"], r["u"], r["sg"], r["su"])
    assert np.all(np.abs(h.astype(np.float64) - r["h"]) <= tol)
    # one matrix (tb_gemv_ternary, the down GEMV's kernel)
    y_alone = [gu.gemv(dg, q[row:row + 1], dq[row:row + 1])[0].tobytes() for row in range(8)]
    for m in (6, 7, 8):
        y = gu.gemv(dg, q[:m], dq[:m])
        for row in range(m):
            assert y[row].tobytes() == y_alone[row], f"M={m} row {row}"
    yo, sabs = o.gemv(wg, q, dq)
    assert bounds.gemv_ok(y, yo, sabs)[0]


def test_code3_and_zero_cases(o):
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 4, (130, 384)).astype(np.uint8)     # includes the unused code 3
    w = synth.pack_ternary(codes, rng.lognormal(-4, 0.5, (130, 3)))
    x = synth.normal_rows(3, 384, 5, 0)
    q, dq = o.rotate_quant(x)
    wd = tb.Matrix.upload(w)
    assert np.array_equal(gu.block_sums(wd, q), o.block_sums(w, q))
    # x = 0 gives y = 0 exactly; all-zero codes give y = 0 exactly
    qz, dqz = o.rotate_quant(np.zeros((2, 384), np.float32))
    assert not gu.gemv(wd, qz, dqz).any()
    z = tb.Matrix.upload(synth.pack_ternary(np.zeros((33, 384), np.uint8), np.ones((33, 3))))
    assert not gu.gemv(z, q, dq).any()


# ----------------------------------------------------------------- a5: gate/up + SiLU
@pytest.mark.parametrize("fmt", [TERN, SIGN])
# the full gate/up shape at M = 5, where gate/up moves to the matrix cores
@pytest.mark.parametrize("n,k,m", [(384, 256, 1), (2176, 640, 3), (1152, 5120, 8),
                                   (17408, 5120, 5)])
def test_gateup_silu(o, fmt, n, k, m):
    say(f"gateup fmt={fmt} n={n} k={k} m={m}")
    layer = synth.ffn_layer(11, 0, fmt, hidden=k, inter=n)
    g = gu.GpuLayer(layer)
    x = synth.normal_rows(m, k, 11, 0)
    q, dq = o.rotate_quant(x)
    h = gu.gateup(g, q, dq)
    r = o.gateup_silu(layer.gate, layer.up, q, dq)
    tol = bounds.h_tolerance(r["g"], r["u"], r["sg"], r["su"])
    err = np.abs(h.astype(np.float64) - r["h"])
    say(f"  worst h err / tol = {np.max(err / tol):.3g}")
    assert np.all(err <= tol)


# ----------------------------------------------------------------- a6, a7: down stage
@pytest.mark.parametrize("fmt", [TERN, SIGN])
# full down shape at M = 6 and 7: where the down GEMV moves to the matrix cores
@pytest.mark.parametrize("n,k,m", [(65, 2176, 2), (5120, 17408, 1), (5120, 17408, 6),
                                   (5120, 17408, 7), (5120, 17408, 8)])
def test_down_stage(o, fmt, n, k, m):
    say(f"down fmt={fmt} n={n} k={k} m={m}")
    wd = synth.matrix(fmt, n, k, 12, 0, synth.T_DOWN)
    h = synth.normal_rows(m, k, 12, 0, synth.T_HIDDEN)
    qh, dqh, y = gu.down(tb.Matrix.upload(wd), h)
    r = o.ffn_down(wd, h)
    assert np.array_equal(qh, r["qh"])
    assert np.array_equal(dqh.view(np.uint32), r["dqh"].view(np.uint32))
    ok, worst = bounds.gemv_ok(y, r["y"], r["sabs"])
    say(f"  worst err / (1e-4 sum|tau|) = {worst:.3g}")
    assert ok


# ----------------------------------------------------------------- whole layers
def check_chain(o, layer, x, got, label):
    """Stagewise parity of one chained layer run (got: dict from LayerRun.run)."""
    r = o.ffn(layer, x)
    assert np.array_equal(got["q"], r["q"]), label
    assert np.array_equal(got["dq"].view(np.uint32), r["dq"].view(np.uint32)), label
    tol_h = bounds.h_tolerance(r["g"], r["u"], r["sg"], r["su"])
    err_h = np.abs(got["h"].astype(np.float64) - r["h"])
    assert np.all(err_h <= tol_h), f"{label}: h worst {np.max(err_h / tol_h):.3g}"
    wd = layer.down
    t_abs = bounds.nonzero_weights(wd)
    isum_or = o.block_sums(wd, r["qh"])
    q_lo, q_hi, dq_lo, dq_hi, extra = bounds.chain_bounds(
        r["h"], tol_h, r["qh"], r["dqh"], isum_or, t_abs,
        wd.scales_f32().astype(np.float64), float(o.dq_unit()))
    qg = got["qh"].astype(np.float64)
    assert np.all((q_lo <= qg) & (qg <= q_hi)), f"{label}: qh code outside its interval"
    dqg = got["dqh"].astype(np.float64)
    assert np.all((dq_lo <= dqg) & (dqg <= dq_hi)), f"{label}: dqh outside its interval"
    flips = int(np.count_nonzero(got["qh"] != r["qh"]))
    err_y = np.abs(got["y"].astype(np.float64) - r["y"])
    tol_y = bounds.GEMV_REL * (r["sabs"] + extra) + extra
    say(f"  {label}: qh flips {flips}/{qg.size}, worst h {np.max(err_h / tol_h):.3g}, "
        f"worst y {np.max(err_y / tol_y):.3g}")
    assert np.all(err_y <= tol_y), f"{label}: y worst {np.max(err_y / tol_y):.3g}"
    return r


@pytest.fixture(scope="module")
def layer1():
    return synth.ffn_layer(0, 0, TERN, keep_draw=False)


@pytest.fixture(scope="module")
def layer1_gpu(layer1):
    return gu.GpuLayer(layer1)


def test_config0_tiny_gemv(o):
    say("config 0: W 256x512, seed 0")
    w = synth.ternary_matrix(256, 512, 0, 0, synth.T_GATE)
    x = synth.normal_rows(1, 512, 0, 0)
    q, dq = gu.rotquant(x)
    qo, dqo = o.rotate_quant(x)
    assert np.array_equal(q, qo) and np.array_equal(dq, dqo)
    wd = tb.Matrix.upload(w)
    assert np.array_equal(gu.block_sums(wd, q), o.block_sums(w, q))
    y = gu.gemv(wd, q, dq)
    yo, sabs = o.gemv(w, q, dq)
    assert bounds.gemv_ok(y, yo, sabs)[0]


def test_config1_layer_m1(o, layer1, layer1_gpu):
    say("config 1: one FFN layer, M=1, seed 0")
    x = synth.normal_rows(1, synth.HIDDEN, 0, 0)
    got = gu.LayerRun(layer1_gpu, 1).run(x)
    check_chain(o, layer1, x, got, "config1 M=1")


def test_config1_stagewise_down(o, layer1, layer1_gpu):
    say("config 1: down stage from generated h")
    h = synth.normal_rows(1, synth.INTER, 0, 0, synth.T_HIDDEN)
    qh, dqh, y = gu.down(layer1_gpu.down, h)
    r = o.ffn_down(layer1.down, h)
    assert np.array_equal(qh, r["qh"]) and np.array_equal(dqh, r["dqh"])
    assert bounds.gemv_ok(y, r["y"], r["sabs"])[0]


@pytest.fixture(scope="module")
def layer2():
    return synth.ffn_layer(1, 0, TERN)


@pytest.fixture(scope="module")
def layer2_gpu(layer2):
    return gu.GpuLayer(layer2)


def test_config2_batched_bit_identical(o, layer2, layer2_gpu):
    say("config 2: M in {2,4,8} vs each row alone, seed 1")
    x8 = synth.normal_rows(8, synth.HIDDEN, 1, 0)
    alone = [gu.LayerRun(layer2_gpu, 1).run(x8[r:r + 1]) for r in range(8)]
    for m in (2, 4, 8):
        got = gu.LayerRun(layer2_gpu, m).run(x8[:m])
        for name in ("q", "dq", "h", "qh", "dqh", "y"):
            for r in range(m):
                a = got[name][r].tobytes()
                b = alone[r][name][0].tobytes()
                assert a == b, f"M={m} row {r}: {name} differs from the row alone"
    check_chain(o, layer2, x8, got, "config2 M=8")


@pytest.mark.parametrize("m", [1, 8])
def test_config4_sign_outliers(o, m):
    say(f"config 4: sign weights, Student-t + outliers, M={m}")
    layer = synth.ffn_layer(4, 0, SIGN)
    g = gu.GpuLayer(layer)
    x = synth.student_t_rows(8, synth.HIDDEN, 4, 0)[:m]
    got = gu.LayerRun(g, m).run(x)
    r = check_chain(o, layer, x, got, f"config4 M={m}")
    if m == 8:
        for row in range(8):
            one = gu.LayerRun(g, 1).run(x[row:row + 1])
            for name in ("q", "dq", "h", "qh", "dqh", "y"):
                assert got[name][row].tobytes() == one[name][0].tobytes(), (row, name)
    # reported, not gated: rotated vs unrotated int8 error on the outlier inputs
    xb = x.reshape(m, -1, 128).astype(np.float64)
    rot = np.einsum("ij,rbj->rbi", bounds.H, xb) / np.sqrt(128)
    deq = r["q"].reshape(xb.shape) * r["dq"][:, :, None]
    err_rot = np.linalg.norm(deq - rot) / np.linalg.norm(rot)
    amax = np.abs(xb).max(axis=2, keepdims=True)
    plain = np.rint(xb / amax * 127) * amax / 127
    err_plain = np.linalg.norm(plain - xb) / np.linalg.norm(xb)
    say(f"  relative int8 error: rotated {err_rot:.4f} vs unrotated {err_plain:.4f}")


@pytest.mark.parametrize("m", [1, 8])
def test_config3_sampled_layers(o, m):
    say(f"config 3: 64-layer stream, sampled layers, M={m}")
    for l in (0, 37, 63):
        layer = synth.ffn_layer(3, l, TERN)
        g = gu.GpuLayer(layer)
        x = synth.normal_rows(m, synth.HIDDEN, 3, l)
        got = gu.LayerRun(g, m).run(x)
        check_chain(o, layer, x, got, f"config3 layer {l} M={m}")
        del g


# ----------------------------------------------------------------- determinism
def test_determinism_streams_and_graph(layer2_gpu):
    say("determinism: reruns, another stream, graph replay A -> zero -> A")
    x = synth.normal_rows(4, synth.HIDDEN, 9, 0)
    run = gu.LayerRun(layer2_gpu, 4)
    ref = run.run(x)
    for _ in range(4):
        again = run.run(x)
        for name in ref:
            assert ref[name].tobytes() == again[name].tobytes(), name
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        other = run.run(x, stream=s)
    for name in ref:
        assert ref[name].tobytes() == other[name].tobytes(), name
    # graph capture of the three calls; outputs are zeroed by eager kernels between replays
    run.x.copy_(torch.from_numpy(x))
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            run.launch(stream=cs)
    torch.cuda.current_stream().wait_stream(cs)
    for rep in range(3):
        for t in (run.q, run.dq, run.h, run.qh, run.dqh, run.y):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        got = run.fetch()
        for name in ref:
            assert ref[name].tobytes() == got[name].tobytes(), (rep, name)


def test_invalid_arguments_launch_nothing():
    y = gu.f32_out(1, 64)
    w = tb.Matrix.upload(synth.ternary_matrix(64, 256, 1, 0, 0))
    q = gu.dev(np.zeros((9, 256), np.int8))
    dq = gu.dev(np.zeros((9, 2), np.float32))
    with pytest.raises(tb.TbError) as e:
        tb.tb_gemv_ternary(w, q, dq, y)               # 9 rows
    assert e.value.status == tb.TB_EINVAL
    assert torch.isnan(y).all()
