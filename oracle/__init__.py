"""CPU oracle for the ternary-weight int8 FFN path (ctypes over tb_oracle.c).

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP library and
its Python binding never import it, and the two share no code.

``Oracle`` wraps one compiled copy of tb_oracle.c. The module-level functions
use the default copy (``liboracle.so`` next to this file). The mutant tests
build other copies from edited sources. The C file cites the passages each
step follows.

Parity unpinned: the low-order fp32 bits of the GPU's y, h and dq beyond the
stated tolerances, and the particular reduction order the GPU uses.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "tb_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-tree-vectorize", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]

FMT_TERNARY2 = 0
FMT_SIGN1 = 1
BLOCK = 128


def build(src: str | None = None, out: str | None = None) -> str:
    """Compile tb_oracle.c (or another source) with gcc; always recompiles."""
    src = src or SRC
    out = out or LIB_PATH
    cmd = ["gcc", *CFLAGS, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "tbo_version": ([], _I),
    "tbo_half_to_double": ([ctypes.c_uint16], ctypes.c_double),
    "tbo_fwht128": ([_P], None),
    "tbo_dq_unit": ([], ctypes.c_float),
    "tbo_rotate_quant": ([_P, _I, _I, _P, _P], _I),
    "tbo_weight": ([_P, _I, _I], _I),
    "tbo_block_sums": ([_P, _I, _I, _I, _P, _I, _P], _I),
    "tbo_gemv_rows": ([_P, _P, _I, _I, _I, _P, _P, _I, _P, _I, _P, _P], _I),
    "tbo_gemv": ([_P, _P, _I, _I, _I, _P, _P, _I, _P, _P], _I),
    "tbo_gemv_unpacked": ([_P, _P, _I, _I, _I, _P, _P, _I, _P, _P], _I),
    "tbo_silu": ([ctypes.c_double], ctypes.c_double),
    "tbo_gateup_silu": ([_P, _P, _P, _P, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P], _I),
    "tbo_ffn_down_rows": ([_P, _P, _I, _I, _I, _P, _I, _P, _P, _P, _I, _P, _P], _I),
}


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags.c_contiguous
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad arguments (rc={rc})")


def _codes(w):
    return _c(w.codes, np.uint8), _c(w.scales, np.uint16)


class Oracle:
    """numpy front end of one compiled copy of tb_oracle.c."""

    def __init__(self, path: str):
        self.path = path
        self.L = ctypes.CDLL(path)
        for name, (args, res) in _SIGS.items():
            fn = getattr(self.L, name)
            fn.argtypes = args
            fn.restype = res

    # ------------------------------------------------------------ scalar pieces
    def half_to_double(self, bits: int) -> float:
        return self.L.tbo_half_to_double(int(bits) & 0xFFFF)

    def dq_unit(self) -> np.float32:
        return np.float32(self.L.tbo_dq_unit())

    def fwht128(self, v) -> np.ndarray:
        a = _c(v, np.float32).copy()
        assert a.shape == (BLOCK,)
        self.L.tbo_fwht128(_ptr(a))
        return a

    def silu(self, z: float) -> float:
        return self.L.tbo_silu(float(z))

    def weight(self, row_codes, fmt: int, i: int) -> int:
        r = _c(row_codes, np.uint8)
        return self.L.tbo_weight(_ptr(r), fmt, i)

    # ------------------------------------------------------------ array ops
    def rotate_quant(self, x) -> tuple[np.ndarray, np.ndarray]:
        """x float32 [m][k] -> (q int8 [m][k], dq float32 [m][k/128])."""
        x = _c(x, np.float32)
        if x.ndim == 1:
            x = x[None, :]
        m, k = x.shape
        q = np.empty((m, k), np.int8)
        dq = np.empty((m, k // BLOCK), np.float32)
        _check(self.L.tbo_rotate_quant(_ptr(x), m, k, _ptr(q), _ptr(dq)), "rotate_quant")
        return q, dq

    def block_sums(self, w, q) -> np.ndarray:
        """isum int32 [m][n][k/128] for a packed matrix w (synth.PackedMatrix)."""
        codes, _ = _codes(w)
        q = _c(q, np.int8)
        m = q.shape[0]
        out = np.empty((m, w.n, w.k // BLOCK), np.int32)
        _check(self.L.tbo_block_sums(_ptr(codes), w.fmt, w.n, w.k, _ptr(q), m, _ptr(out)),
               "block_sums")
        return out

    def gemv(self, w, q, dq, rows=None) -> tuple[np.ndarray, np.ndarray]:
        """(y, sabs), each float64 [m][len(rows) or n]."""
        codes, scales = _codes(w)
        q = _c(q, np.int8)
        dq = _c(dq, np.float32)
        m = q.shape[0]
        rows_a = None if rows is None else _c(rows, np.int32)
        cnt = w.n if rows_a is None else rows_a.size
        y = np.empty((m, cnt), np.float64)
        sabs = np.empty((m, cnt), np.float64)
        _check(self.L.tbo_gemv_rows(_ptr(codes), _ptr(scales), w.fmt, w.n, w.k, _ptr(q),
                                    _ptr(dq), m, _ptr(rows_a), cnt, _ptr(y), _ptr(sabs)), "gemv")
        return y, sabs

    def gemv_unpacked(self, wcodes, scales_f32, fmt, q, dq) -> tuple[np.ndarray, np.ndarray]:
        """GEMV from the codes before packing: (isum int32 [m][n][nb], y float64 [m][n])."""
        wcodes = _c(wcodes, np.uint8)
        scales_f32 = _c(scales_f32, np.float32)
        q = _c(q, np.int8)
        dq = _c(dq, np.float32)
        n, k = wcodes.shape
        m = q.shape[0]
        isum = np.empty((m, n, k // BLOCK), np.int32)
        y = np.empty((m, n), np.float64)
        _check(self.L.tbo_gemv_unpacked(_ptr(wcodes), _ptr(scales_f32), fmt, n, k, _ptr(q),
                                        _ptr(dq), m, _ptr(isum), _ptr(y)), "gemv_unpacked")
        return isum, y

    def gateup_silu(self, wg, wu, q, dq) -> dict:
        """g, u, h = silu(g)*u and the term sums sg, su, all float64 [m][n]."""
        gc, gs = _codes(wg)
        uc, us = _codes(wu)
        assert (wg.n, wg.k, wg.fmt) == (wu.n, wu.k, wu.fmt)
        q = _c(q, np.int8)
        dq = _c(dq, np.float32)
        m = q.shape[0]
        out = {key: np.empty((m, wg.n), np.float64) for key in ("g", "u", "h", "sg", "su")}
        _check(self.L.tbo_gateup_silu(_ptr(gc), _ptr(gs), _ptr(uc), _ptr(us), wg.fmt, wg.n,
                                      wg.k, _ptr(q), _ptr(dq), m, _ptr(out["g"]),
                                      _ptr(out["u"]), _ptr(out["h"]), _ptr(out["sg"]),
                                      _ptr(out["su"])), "gateup_silu")
        return out

    def ffn_down(self, wd, h, rows=None) -> dict:
        """Quantise fp32 h [m][k] like x, then GEMV. Returns qh, dqh, y, sabs."""
        codes, scales = _codes(wd)
        h = _c(h, np.float32)
        m, k = h.shape
        assert k == wd.k
        rows_a = None if rows is None else _c(rows, np.int32)
        cnt = wd.n if rows_a is None else rows_a.size
        qh = np.empty((m, k), np.int8)
        dqh = np.empty((m, k // BLOCK), np.float32)
        y = np.empty((m, cnt), np.float64)
        sabs = np.empty((m, cnt), np.float64)
        _check(self.L.tbo_ffn_down_rows(_ptr(codes), _ptr(scales), wd.fmt, wd.n, wd.k, _ptr(h),
                                        m, _ptr(qh), _ptr(dqh), _ptr(rows_a), cnt, _ptr(y),
                                        _ptr(sabs)), "ffn_down")
        return {"qh": qh, "dqh": dqh, "y": y, "sabs": sabs}

    def ffn(self, layer, x) -> dict:
        """Whole FFN layer from x: rotquant, gate/up + SiLU, h rounded to fp32, down."""
        q, dq = self.rotate_quant(x)
        gu = self.gateup_silu(layer.gate, layer.up, q, dq)
        h32 = gu["h"].astype(np.float32)
        dn = self.ffn_down(layer.down, h32)
        return {"q": q, "dq": dq, **gu, "h32": h32, **dn}


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from tb_oracle.c next to this file (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def __getattr__(name):
    # Module-level shortcuts: oracle.rotate_quant(...) == oracle.default().rotate_quant(...)
    if not name.startswith("_") and hasattr(Oracle, name):
        return getattr(default(), name)
    raise AttributeError(name)
