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
    assert L.tb_abi_version() == 1


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
    assert g(mat(fmt=2)) == tb.TB_EINVAL
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


def test_down_validation(L):
    wd = mat(n=5120, k=17408)

    def dn(w, h=0x20000000, qh=0x30000000, dqh=0x34000000, y=0x38000000, m=1):
        return L.tb_ffn_down(ctypes.byref(w), h, m, qh, dqh, y, None)
    assert dn(wd, m=9) == tb.TB_EINVAL
    assert dn(wd, qh=0) == tb.TB_EINVAL
    assert dn(wd, qh=0x20000000) == tb.TB_EINVAL             # workspace overlaps h
    assert dn(wd, y=0x30000000) == tb.TB_EINVAL              # y overlaps the workspace
    assert dn(wd, dqh=0x34000004) == tb.TB_EALIGN


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
