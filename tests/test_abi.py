"""The C ABI without a GPU: the library loads, exports every declared symbol, and rejects
bad arguments before touching HIP. No call here reaches a kernel launch."""

import ctypes
import os
import re

import pytest

import ternary_weight_int8_tb_amd as tb
from ternary_weight_int8_tb_amd import build as tb_build

HEADER = os.path.join(os.path.dirname(tb.PKG), "include", "tb.h")
ALIGNED = 0x10000          # fake, 16-byte aligned addresses: never dereferenced
ALIGNED2 = 0x4000000
ALIGNED3 = 0x8000000
ALIGNED4 = 0xC000000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tb.LIB_PATH):
        tb_build.build()
    return tb.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tb_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(tb.ABI_SYMBOLS)


def test_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.tb_abi_version() == tb.ABI_VERSION


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, 12345):
        assert isinstance(tb.tb_status_str(code), str) and tb.tb_status_str(code)


def mat(codes=ALIGNED, scales=ALIGNED2, n=256, k=512, fmt=0):
    return tb.CMatrix(codes, scales, n, k, fmt)


def rq(L, x=ALIGNED, m=1, k=512, q=ALIGNED2, dq=ALIGNED3):
    return L.tb_rotate_quant_i8(x, m, k, q, dq, None)


def test_rotate_quant_validation(L):
    assert rq(L, m=0) == tb.TB_EINVAL
    assert rq(L, m=9) == tb.TB_EINVAL
    assert rq(L, k=100) == tb.TB_EINVAL
    assert rq(L, k=0) == tb.TB_EINVAL
    assert rq(L, x=0) == tb.TB_EINVAL
    assert rq(L, q=0) == tb.TB_EINVAL
    assert rq(L, x=ALIGNED + 4) == tb.TB_EALIGN
    assert rq(L, dq=ALIGNED3 + 8) == tb.TB_EALIGN
    assert rq(L, q=ALIGNED + 512) == tb.TB_EINVAL            # q overlaps x


def test_gemv_validation(L):
    def g(w, q=ALIGNED3, dq=ALIGNED4, m=1, y=ALIGNED4 + 0x100000):
        return L.tb_gemv_ternary(ctypes.byref(w), q, dq, m, y, None)
    assert L.tb_gemv_ternary(None, ALIGNED3, ALIGNED4, 1, ALIGNED4 + 0x100000, None) == tb.TB_EINVAL
    assert g(mat(), m=0) == tb.TB_EINVAL
    assert g(mat(), m=9) == tb.TB_EINVAL
    assert g(mat(k=500)) == tb.TB_EINVAL
    assert g(mat(k=0)) == tb.TB_EINVAL
    assert g(mat(n=0)) == tb.TB_EINVAL
    assert g(mat(fmt=3)) == tb.TB_EINVAL
    assert g(mat(codes=0)) == tb.TB_EINVAL
    assert g(mat(codes=ALIGNED + 2)) == tb.TB_EALIGN
    assert g(mat(), q=0) == tb.TB_EINVAL
    assert g(mat(), q=ALIGNED3 + 1) == tb.TB_EALIGN
    assert g(mat(), y=ALIGNED + 64) == tb.TB_EINVAL          # y overlaps the codes
    assert g(mat(), y=ALIGNED4) == tb.TB_EINVAL               # y overlaps dq


def test_gateup_validation(L):
    def gu(wg, wu, m=1, h=0x20000000):
        return L.tb_ffn_gateup_silu(ctypes.byref(wg), ctypes.byref(wu), ALIGNED3, ALIGNED4, m, h,
                                    None)
    up = mat(codes=0x10000000, scales=0x14000000)
    assert gu(mat(), mat(codes=0x10000000, scales=0x14000000, n=128)) == tb.TB_EINVAL
    assert gu(mat(), mat(codes=0x10000000, scales=0x14000000, fmt=1)) == tb.TB_EINVAL
    assert gu(mat(), up, m=0) == tb.TB_EINVAL
    assert gu(mat(), up, h=0) == tb.TB_EINVAL
    assert gu(mat(), up, h=0x10000000) == tb.TB_EINVAL       # h overlaps up's codes


def test_gateup_x_validation(L):
    # tb_ffn_gateup_silu_x(wg, wu, x, m, qx, dqx, h): the x call checks what both of the
    # calls it replaces check, and that its three outputs overlap nothing
    wg, wu = mat(), mat(codes=0x10000000, scales=0x14000000)

    def gx(wg=wg, wu=wu, x=0x20000000, m=1, qx=0x30000000, dqx=0x34000000, h=0x38000000):
        return L.tb_ffn_gateup_silu_x(ctypes.byref(wg), ctypes.byref(wu), x, m, qx, dqx, h, None)
    assert gx(wu=mat(codes=0x10000000, scales=0x14000000, n=128)) == tb.TB_EINVAL
    assert gx(wu=mat(codes=0x10000000, scales=0x14000000, fmt=1)) == tb.TB_EINVAL
    assert gx(m=0) == tb.TB_EINVAL
    assert gx(m=9) == tb.TB_EINVAL
    for name in ("x", "qx", "dqx", "h"):
        assert gx(**{name: 0}) == tb.TB_EINVAL, name
    assert gx(x=0x20000004) == tb.TB_EALIGN
    assert gx(qx=0x30000008) == tb.TB_EALIGN
    assert gx(dqx=0x34000004) == tb.TB_EALIGN
    assert gx(h=0x38000004) == tb.TB_EALIGN
    assert gx(qx=0x20000000) == tb.TB_EINVAL                 # qx overlaps x
    assert gx(h=0x10000000) == tb.TB_EINVAL                  # h overlaps up's codes
    assert gx(dqx=0x30000000) == tb.TB_EINVAL                # dqx overlaps qx
    assert gx(h=0x34000000) == tb.TB_EINVAL                  # h overlaps dqx


def test_gemv_x_validation(L):
    # tb_gemv_ternary_x shares tb_ffn_down's checks
    w = mat()

    def gx(x=0x20000000, m=1, qx=0x30000000, dqx=0x34000000, y=0x38000000):
        return L.tb_gemv_ternary_x(ctypes.byref(w), x, m, qx, dqx, y, None)
    assert gx(m=0) == tb.TB_EINVAL
    assert gx(m=9) == tb.TB_EINVAL
    assert gx(qx=0) == tb.TB_EINVAL
    assert gx(x=0x20000004) == tb.TB_EALIGN
    assert gx(qx=0x20000000) == tb.TB_EINVAL                 # qx overlaps x
    assert gx(y=0x30000000) == tb.TB_EINVAL                  # y overlaps qx


def test_sign_interleave_validation(L):
    # tb_sign_interleave(w, codes_ri, scales_ri): a sign matrix with n % 4 == 0, aligned,
    # non-overlapping outputs
    def si(w, co=0x20000000, so=0x30000000):
        return L.tb_sign_interleave(ctypes.byref(w), co, so, None)
    assert si(mat(fmt=0)) == tb.TB_EINVAL                    # ternary
    assert si(mat(fmt=1, n=254)) == tb.TB_EINVAL             # n % 4
    assert si(mat(fmt=1), co=0) == tb.TB_EINVAL
    assert si(mat(fmt=1), co=0x20000004) == tb.TB_EALIGN
    assert si(mat(fmt=1), so=0x20000000) == tb.TB_EINVAL     # outputs overlap
    assert si(mat(fmt=1), co=ALIGNED) == tb.TB_EINVAL        # overwrites the codes
    assert si(mat(fmt=3)) == tb.TB_EINVAL                    # unknown format


def test_row_interleaved_layout_only_for_the_gemv(L):
    # the interleaved layout (fmt 2, n % 4 == 0) is checked like the others and refused by
    # the calls other than the GEMV and the block sums
    ri = mat(fmt=2)
    assert L.tb_gemv_ternary(ctypes.byref(mat(fmt=2, n=254)), ALIGNED3, ALIGNED4, 1,
                             0x20000000, None) == tb.TB_EINVAL
    h = 0x20000000
    assert L.tb_ffn_gateup_silu(ctypes.byref(ri), ctypes.byref(mat(fmt=2, codes=0x10000000,
                                scales=0x14000000)), ALIGNED3, ALIGNED4, 1, h,
                                None) == tb.TB_EUNSUPPORTED
    assert L.tb_ffn_down(ctypes.byref(mat(fmt=2, n=64, k=256)), 0x20000000, 1, 0x30000000,
                         0x34000000, 0x38000000, None) == tb.TB_EUNSUPPORTED
    assert L.tb_ffn_down_noalloc(ctypes.byref(mat(fmt=2, n=64, k=256)), 0x20000000, 1,
                                 0x38000000, None) == tb.TB_EUNSUPPORTED


def test_down_validation(L):
    wd = mat(n=5120, k=17408)

    def dn(w, h=0x20000000, qh=0x30000000, dqh=0x34000000, y=0x38000000, m=1):
        return L.tb_ffn_down(ctypes.byref(w), h, m, qh, dqh, y, None)
    assert dn(wd, m=9) == tb.TB_EINVAL
    assert dn(wd, qh=0) == tb.TB_EINVAL
    assert dn(wd, qh=0x20000000) == tb.TB_EINVAL             # workspace overlaps h
    assert dn(wd, y=0x30000000) == tb.TB_EINVAL              # y overlaps the workspace
    assert dn(wd, dqh=0x34000004) == tb.TB_EALIGN


def test_down_split_validation(L):
    wd = mat(n=5120, k=17408)
    need = tb.tb_ffn_down_split_workspace_bytes(MatrixRef(wd), 8)
    # float step partials [ceil(k/1024)][m][n] (ternary), [ceil(k/2048)][m][n] (sign)
    assert need == 17 * 8 * 5120 * 4
    assert tb.tb_ffn_down_split_workspace_bytes(MatrixRef(mat(n=5120, k=17408, fmt=1)), 3) == \
        9 * 3 * 5120 * 4
    assert tb.tb_ffn_down_split_workspace_bytes(MatrixRef(wd), 0) == 0
    assert tb.tb_ffn_down_split_workspace_bytes(MatrixRef(wd), 9) == 0
    assert tb.tb_ffn_down_split_workspace_bytes(MatrixRef(mat(fmt=2)), 1) == 0
    WS = 0x40000000

    def dn(w, h=0x20000000, qh=0x30000000, dqh=0x34000000, y=0x38000000, m=8, ws=WS, wsb=need):
        return L.tb_ffn_down_split(ctypes.byref(w), h, m, qh, dqh, y, ws, wsb, None)
    assert dn(wd, m=0) == tb.TB_EINVAL
    assert dn(wd, m=9) == tb.TB_EINVAL
    assert dn(wd, ws=0) == tb.TB_EINVAL
    assert dn(wd, wsb=need - 4) == tb.TB_EINVAL                    # workspace too small
    assert dn(wd, ws=WS + 4) == tb.TB_EALIGN
    assert dn(wd, qh=0x20000000) == tb.TB_EINVAL                   # qh overlaps h
    assert dn(wd, ws=0x38000000) == tb.TB_EINVAL                   # workspace overlaps y
    assert dn(mat(n=5120, k=17408, fmt=2)) == tb.TB_EUNSUPPORTED


def test_down_split_batch_validation(L):
    wd = mat(n=5120, k=17408)
    need = tb.tb_ffn_down_split_batch_workspace_bytes(MatrixRef(wd), 32)
    assert need == 17 * 32 * 5120 * 4
    assert tb.tb_ffn_down_split_batch_workspace_bytes(MatrixRef(wd), 8) == \
        tb.tb_ffn_down_split_workspace_bytes(MatrixRef(wd), 8)
    assert tb.tb_ffn_down_split_batch_workspace_bytes(MatrixRef(wd), 0) == 0
    assert tb.tb_ffn_down_split_batch_workspace_bytes(MatrixRef(wd), 33) == 0
    assert tb.tb_ffn_down_split_batch_workspace_bytes(MatrixRef(mat(fmt=2)), 16) == 0
    WS = 0x40000000

    def dn(w, h=0x20000000, qh=0x30000000, dqh=0x34000000, y=0x38000000, m=32, ws=WS, wsb=need):
        return L.tb_ffn_down_split_batch(ctypes.byref(w), h, m, qh, dqh, y, ws, wsb, None)
    assert dn(wd, m=0) == tb.TB_EINVAL
    assert dn(wd, m=33) == tb.TB_EINVAL
    assert dn(wd, ws=0) == tb.TB_EINVAL
    assert dn(wd, wsb=need - 4) == tb.TB_EINVAL                    # workspace too small
    assert dn(wd, ws=WS + 4) == tb.TB_EALIGN
    assert dn(wd, qh=0x20000000) == tb.TB_EINVAL                   # qh overlaps h
    assert dn(wd, ws=0x38000000) == tb.TB_EINVAL                   # workspace overlaps y
    assert dn(mat(n=5120, k=17408, fmt=2)) == tb.TB_EUNSUPPORTED


class MatrixRef:
    """A CMatrix in the shape the binding's workspace-size helper takes (.c)."""

    def __init__(self, c):
        self.c = c


def test_block_sums_validation(L):
    assert L.tb_gemv_block_sums(ctypes.byref(mat()), ALIGNED3, 0, ALIGNED4, None) == tb.TB_EINVAL
    assert L.tb_gemv_block_sums(ctypes.byref(mat()), ALIGNED3, 1, 0, None) == tb.TB_EINVAL
    assert L.tb_gemv_block_sums(ctypes.byref(mat()), ALIGNED3, 1, ALIGNED4 + 4,
                                None) == tb.TB_EALIGN


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(tb, "_lib", None)
    monkeypatch.setattr(tb, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="missing"):
        tb.lib()


def test_ffn_workspace_bytes(L):
    # sync words, then h [m][inter] f32, q_h [m][inter] i8, dq_h and sum q_h [m][inter/128]
    for m, inter in ((1, 384), (8, 17408), (3, 2176)):
        nb = tb.tb_ffn_workspace_bytes(m, 5120, inter)
        assert nb >= 4096 + m * inter * 5 + 2 * m * (inter // 128) * 4
        assert nb % 256 == 0
    assert tb.tb_ffn_workspace_bytes(0, 5120, 17408) == 0
    assert tb.tb_ffn_workspace_bytes(9, 5120, 17408) == 0
    assert tb.tb_ffn_workspace_bytes(1, 5120, 100) == 0


def test_ffn_workspace_init_validation(L):
    assert L.tb_ffn_workspace_init(None, 1 << 20, 0, None) == tb.TB_EINVAL
    assert L.tb_ffn_workspace_init(ALIGNED, 64, 0, None) == tb.TB_EINVAL       # below the sync words
    assert L.tb_ffn_workspace_init(ALIGNED + 4, 1 << 20, 0, None) == tb.TB_EALIGN
    err = ctypes.c_int(7)
    assert L.tb_ffn_workspace_error(None, ctypes.byref(err)) == tb.TB_EINVAL
    assert L.tb_ffn_workspace_error(ALIGNED, None) == tb.TB_EINVAL


def test_ffn_layers_validation(L):
    H, N = 512, 384
    base = 0x10000000

    def weights(i, n_gate=N, fmt=0, k_down=N):
        o = base + i * 0x100000
        return tb.CFfnWeights(mat(o, o + 0x20000, N if n_gate is None else n_gate, H, fmt),
                              mat(o + 0x40000, o + 0x60000, N, H, fmt),
                              mat(o + 0x80000, o + 0xA0000, H, k_down, fmt))
    arr = (tb.CFfnWeights * 2)(weights(0), weights(1))
    ws_bytes = tb.tb_ffn_workspace_bytes(1, H, N)
    X, Y, WS = 0x40000000, 0x48000000, 0x50000000

    def call(a=arr, n=2, x=X, m=1, flags=0, ws=WS, wsb=ws_bytes, y=Y):
        return L.tb_ffn_layers(a, n, x, m, flags, ws, wsb, y, None)
    assert call(n=0) == tb.TB_EINVAL
    assert call(a=None) == tb.TB_EINVAL
    assert call(m=9) == tb.TB_EINVAL
    assert call(flags=2) == tb.TB_EINVAL
    assert call(x=0) == tb.TB_EINVAL
    assert call(ws=0) == tb.TB_EINVAL
    assert call(wsb=ws_bytes - 256) == tb.TB_EINVAL                  # workspace too small
    assert call(x=X + 8) == tb.TB_EALIGN
    assert call(ws=WS + 4) == tb.TB_EALIGN
    assert call(y=X + 16) == tb.TB_EINVAL                             # y overlaps x
    assert call(ws=Y + 256) == tb.TB_EINVAL                           # workspace overlaps y
    assert call(y=base + 0x40) == tb.TB_EINVAL                        # y overlaps weights
    bad = (tb.CFfnWeights * 2)(weights(0), weights(1, n_gate=256))  # gate/up rows differ
    assert call(a=bad) == tb.TB_EINVAL
    bad = (tb.CFfnWeights * 2)(weights(0), weights(1, fmt=1))       # formats differ
    assert call(a=bad) == tb.TB_EINVAL
    bad = (tb.CFfnWeights * 2)(weights(0), weights(1, k_down=256))  # down does not match
    assert call(a=bad) == tb.TB_EINVAL


def test_valid_calls_without_a_device_return_ehip(L):
    # With no GPU present a valid call must fail with TB_EHIP, not crash. Where a device
    # exists the fake addresses would reach a kernel, so the test only runs without one.
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    w, w2 = mat(), mat(codes=ALIGNED + 0x100000, scales=ALIGNED2 + 0x100000)
    y = ALIGNED4 + 0x100000
    assert rq(L) == tb.TB_EHIP
    assert L.tb_gemv_ternary(ctypes.byref(w), ALIGNED3, ALIGNED4, 1, y, None) == tb.TB_EHIP
    assert L.tb_ffn_gateup_silu(ctypes.byref(w), ctypes.byref(w2), ALIGNED3, ALIGNED4, 1, y,
                                None) == tb.TB_EHIP
    assert L.tb_gemv_block_sums(ctypes.byref(w), ALIGNED3, 1, ALIGNED4, None) == tb.TB_EHIP
    assert L.tb_ffn_gateup_silu_x(ctypes.byref(w), ctypes.byref(w2), 0x20000000, 1, 0x30000000,
                                  0x34000000, 0x38000000, None) == tb.TB_EHIP
    assert L.tb_gemv_ternary_x(ctypes.byref(w), 0x20000000, 1, 0x30000000, 0x34000000,
                               0x38000000, None) == tb.TB_EHIP
    need = L.tb_ffn_down_split_workspace_bytes(ctypes.byref(w), 2)
    assert L.tb_ffn_down_split(ctypes.byref(w), 0x20000000, 2, 0x30000000, 0x34000000, 0x38000000,
                               0x40000000, need, None) == tb.TB_EHIP


def test_batch_calls_validate_rows_and_arguments(L):
    # the batch family takes 1..32 rows; everything else is checked as in the 1..8 calls
    assert L.tb_rotate_quant_i8_batch(ALIGNED, 0, 512, ALIGNED2, ALIGNED3, None) == tb.TB_EINVAL
    assert L.tb_rotate_quant_i8_batch(ALIGNED, 33, 512, ALIGNED2, ALIGNED3, None) == tb.TB_EINVAL
    assert L.tb_rotate_quant_i8_batch(ALIGNED, 32, 100, ALIGNED2, ALIGNED3, None) == tb.TB_EINVAL
    assert L.tb_rotate_quant_i8_batch(ALIGNED + 4, 16, 512, ALIGNED2, ALIGNED3, None) == tb.TB_EALIGN
    w = mat()
    y = ALIGNED4 + 0x100000
    for m in (0, 33):
        assert L.tb_gemv_ternary_batch(ctypes.byref(w), ALIGNED3, ALIGNED4, m, y, None) == tb.TB_EINVAL
        assert L.tb_ffn_gateup_silu_batch(ctypes.byref(w), ctypes.byref(w), ALIGNED3, ALIGNED4, m,
                                          y, None) == tb.TB_EINVAL
        assert L.tb_ffn_down_batch(ctypes.byref(mat(n=64, k=256)), ALIGNED3, m, ALIGNED4,
                                   ALIGNED4 + 0x10000, y, None) == tb.TB_EINVAL
        assert L.tb_gemv_block_sums_batch(ctypes.byref(w), ALIGNED3, m, y, None) == tb.TB_EINVAL
    assert L.tb_gemv_ternary_batch(ctypes.byref(mat(k=500)), ALIGNED3, ALIGNED4, 16, y,
                                   None) == tb.TB_EINVAL
    assert L.tb_gemv_ternary_batch(ctypes.byref(w), ALIGNED3 + 8, ALIGNED4, 16, y,
                                   None) == tb.TB_EALIGN
    # y overlapping q
    assert L.tb_gemv_ternary_batch(ctypes.byref(w), ALIGNED3, ALIGNED4, 16, ALIGNED3,
                                   None) == tb.TB_EINVAL
    # the 1..8 calls still reject 9 rows
    assert L.tb_gemv_ternary(ctypes.byref(w), ALIGNED3, ALIGNED4, 9, y, None) == tb.TB_EINVAL
