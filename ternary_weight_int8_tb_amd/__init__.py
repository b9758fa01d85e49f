"""Python binding of libtb.so: ternary-weight int8 FFN decode on MI355X (gfx950).

Argument marshalling only. Every step of the path runs in the HIP kernels of
``csrc/tb.hip`` behind the C ABI in ``include/tb.h``. The functions take the
ABI's names; torch tensors supply device memory and the stream. There is no
CPU fallback: if libtb.so is missing or cannot be loaded, every call raises.

Importing this package loads nothing. ``synth`` (the input generator) works
without a GPU.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtb.so")

TB_OK, TB_EINVAL, TB_EALIGN, TB_EUNSUPPORTED, TB_EHIP, TB_ESCRATCH = 0, -1, -2, -3, -4, -5
TB_FMT_TERNARY2, TB_FMT_SIGN1, TB_FMT_SIGN1_RI4 = 0, 1, 2
BLOCK = 128
MAX_ROWS = 8
MAX_BATCH_ROWS = 32
ABI_VERSION = 6

# every symbol include/tb.h declares
ABI_SYMBOLS = ("tb_rotate_quant_i8", "tb_gemv_ternary", "tb_gemv_ternary_x", "tb_ffn_gateup_silu",
               "tb_ffn_gateup_silu_x",
               "tb_ffn_down",
               "tb_gemv_block_sums", "tb_rotate_quant_i8_batch", "tb_gemv_ternary_batch",
               "tb_ffn_gateup_silu_batch", "tb_ffn_down_batch", "tb_gemv_block_sums_batch",
               "tb_ffn_down_noalloc", "tb_sign_interleave",
               "tb_ffn_down_split", "tb_ffn_down_split_workspace_bytes",
               "tb_ffn_down_split_batch", "tb_ffn_down_split_batch_workspace_bytes",
               "tb_ffn_workspace_bytes", "tb_ffn_workspace_init",
               "tb_ffn_layers", "tb_ffn_workspace_error", "tb_status_str", "tb_abi_version")
TB_FFN_CHAIN = 1


class TbError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({tb_status_str(status)})")


class CMatrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("fmt", ctypes.c_int32)]


class CFfnWeights(ctypes.Structure):
    _fields_ = [("gate", CMatrix), ("up", CMatrix), ("down", CMatrix)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_MP = ctypes.POINTER(CMatrix)
_SIGS = {
    "tb_rotate_quant_i8": ([_P, _I, _I, _P, _P, _P], _I),
    "tb_gemv_ternary": ([_MP, _P, _P, _I, _P, _P], _I),
    "tb_ffn_gateup_silu": ([_MP, _MP, _P, _P, _I, _P, _P], _I),
    "tb_ffn_gateup_silu_x": ([_MP, _MP, _P, _I, _P, _P, _P, _P], _I),
    "tb_gemv_ternary_x": ([_MP, _P, _I, _P, _P, _P, _P], _I),
    "tb_ffn_down": ([_MP, _P, _I, _P, _P, _P, _P], _I),
    "tb_gemv_block_sums": ([_MP, _P, _I, _P, _P], _I),
    "tb_rotate_quant_i8_batch": ([_P, _I, _I, _P, _P, _P], _I),
    "tb_gemv_ternary_batch": ([_MP, _P, _P, _I, _P, _P], _I),
    "tb_ffn_gateup_silu_batch": ([_MP, _MP, _P, _P, _I, _P, _P], _I),
    "tb_ffn_down_batch": ([_MP, _P, _I, _P, _P, _P, _P], _I),
    "tb_gemv_block_sums_batch": ([_MP, _P, _I, _P, _P], _I),
    "tb_ffn_down_noalloc": ([_MP, _P, _I, _P, _P], _I),
    "tb_sign_interleave": ([_MP, _P, _P, _P], _I),
    "tb_ffn_down_split": ([_MP, _P, _I, _P, _P, _P, _P, ctypes.c_size_t, _P], _I),
    "tb_ffn_down_split_workspace_bytes": ([_MP, _I], ctypes.c_size_t),
    "tb_ffn_down_split_batch": ([_MP, _P, _I, _P, _P, _P, _P, ctypes.c_size_t, _P], _I),
    "tb_ffn_down_split_batch_workspace_bytes": ([_MP, _I], ctypes.c_size_t),
    "tb_ffn_workspace_bytes": ([_I, _I, _I], ctypes.c_size_t),
    "tb_ffn_workspace_init": ([_P, ctypes.c_size_t, ctypes.c_uint32, _P], _I),
    "tb_ffn_layers": ([ctypes.POINTER(CFfnWeights), _I, _P, _I, ctypes.c_uint, _P, ctypes.c_size_t,
                       _P, _P], _I),
    "tb_ffn_workspace_error": ([_P, ctypes.POINTER(_I)], _I),
    "tb_status_str": ([_I], ctypes.c_char_p),
    "tb_abi_version": ([], _I),
}

_lib: ctypes.CDLL | None = None


def lib() -> ctypes.CDLL:
    """Load libtb.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def tb_status_str(status: int) -> str:
    return lib().tb_status_str(int(status)).decode()


def tb_abi_version() -> int:
    return lib().tb_abi_version()


class Matrix:
    """A weight matrix on the device: codes and scales tensors plus its shape and format."""

    def __init__(self, codes, scales, n: int, k: int, fmt: int):
        self.codes, self.scales = codes, scales
        self.n, self.k, self.fmt = int(n), int(k), int(fmt)
        self._c = CMatrix(codes.data_ptr(), scales.data_ptr(), self.n, self.k, self.fmt)

    @property
    def c(self) -> CMatrix:
        return self._c

    @property
    def nbytes(self) -> int:
        return self.codes.numel() * self.codes.element_size() + \
            self.scales.numel() * self.scales.element_size()

    @classmethod
    def upload(cls, packed, device="cuda") -> "Matrix":
        """Copy a host matrix (synth.PackedMatrix) to the device."""
        import torch
        codes = torch.from_numpy(packed.codes).to(device)
        scales = torch.from_numpy(packed.scales.view("int16")).to(device)
        return cls(codes, scales, packed.n, packed.k, packed.fmt)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _rows(t) -> int:
    return int(t.shape[0]) if t.dim() > 1 else 1


def _call(name: str, *args):
    rc = getattr(lib(), name)(*args)
    if rc != TB_OK:
        raise TbError(name, rc)


def tb_rotate_quant_i8(x, q, dq, stream=None) -> None:
    """x float32 [m][k] -> q int8 [m][k], dq float32 [m][k/128] (device tensors)."""
    m, k = _rows(x), int(x.shape[-1])
    _call("tb_rotate_quant_i8", x.data_ptr(), m, k, q.data_ptr(), dq.data_ptr(), _stream(stream))


def tb_gemv_ternary(w: Matrix, q, dq, y, stream=None) -> None:
    """y float32 [m][w.n] = GEMV of w against the int8 rows q with scales dq."""
    _call("tb_gemv_ternary", ctypes.byref(w.c), q.data_ptr(), dq.data_ptr(), _rows(q),
          y.data_ptr(), _stream(stream))


def tb_gemv_ternary_x(w: Matrix, x, qx, dqx, y, stream=None) -> None:
    """y = GEMV of w against rotquant(x), written to qx, dqx; one call."""
    _call("tb_gemv_ternary_x", ctypes.byref(w.c), x.data_ptr(), _rows(x), qx.data_ptr(),
          dqx.data_ptr(), y.data_ptr(), _stream(stream))


def tb_ffn_gateup_silu(wg: Matrix, wu: Matrix, q, dq, h, stream=None) -> None:
    """h float32 [m][wg.n] = silu(wg q) * (wu q), from one shared int8 copy."""
    _call("tb_ffn_gateup_silu", ctypes.byref(wg.c), ctypes.byref(wu.c), q.data_ptr(),
          dq.data_ptr(), _rows(q), h.data_ptr(), _stream(stream))


def tb_ffn_gateup_silu_x(wg: Matrix, wu: Matrix, x, qx, dqx, h, stream=None) -> None:
    """h = silu(wg q) * (wu q) with (q, dq) = rotquant(x), written to qx, dqx; one call."""
    _call("tb_ffn_gateup_silu_x", ctypes.byref(wg.c), ctypes.byref(wu.c), x.data_ptr(), _rows(x),
          qx.data_ptr(), dqx.data_ptr(), h.data_ptr(), _stream(stream))


def tb_ffn_down(wd: Matrix, h, qh_ws, dqh_ws, y, stream=None) -> None:
    """y float32 [m][wd.n] = down GEMV of rotquant(h); qh_ws/dqh_ws are the workspace."""
    _call("tb_ffn_down", ctypes.byref(wd.c), h.data_ptr(), _rows(h), qh_ws.data_ptr(),
          dqh_ws.data_ptr(), y.data_ptr(), _stream(stream))


def tb_gemv_block_sums(w: Matrix, q, isum, stream=None) -> None:
    """isum int32 [m][w.n][w.k/128]: the integer block sums before the scale fold."""
    _call("tb_gemv_block_sums", ctypes.byref(w.c), q.data_ptr(), _rows(q), isum.data_ptr(),
          _stream(stream))


def tb_rotate_quant_i8_batch(x, q, dq, stream=None) -> None:
    """tb_rotate_quant_i8 for up to 32 rows."""
    m, k = _rows(x), int(x.shape[-1])
    _call("tb_rotate_quant_i8_batch", x.data_ptr(), m, k, q.data_ptr(), dq.data_ptr(),
          _stream(stream))


def tb_gemv_ternary_batch(w: Matrix, q, dq, y, stream=None) -> None:
    """tb_gemv_ternary for up to 32 rows."""
    _call("tb_gemv_ternary_batch", ctypes.byref(w.c), q.data_ptr(), dq.data_ptr(), _rows(q),
          y.data_ptr(), _stream(stream))


def tb_ffn_gateup_silu_batch(wg: Matrix, wu: Matrix, q, dq, h, stream=None) -> None:
    """tb_ffn_gateup_silu for up to 32 rows."""
    _call("tb_ffn_gateup_silu_batch", ctypes.byref(wg.c), ctypes.byref(wu.c), q.data_ptr(),
          dq.data_ptr(), _rows(q), h.data_ptr(), _stream(stream))


def tb_ffn_down_batch(wd: Matrix, h, qh_ws, dqh_ws, y, stream=None) -> None:
    """tb_ffn_down for up to 32 rows."""
    _call("tb_ffn_down_batch", ctypes.byref(wd.c), h.data_ptr(), _rows(h), qh_ws.data_ptr(),
          dqh_ws.data_ptr(), y.data_ptr(), _stream(stream))


def tb_gemv_block_sums_batch(w: Matrix, q, isum, stream=None) -> None:
    """tb_gemv_block_sums for up to 32 rows."""
    _call("tb_gemv_block_sums_batch", ctypes.byref(w.c), q.data_ptr(), _rows(q), isum.data_ptr(),
          _stream(stream))


def tb_sign_interleave(w: Matrix, stream=None) -> Matrix:
    """The TB_FMT_SIGN1_RI4 copy of a sign matrix (rows interleaved by four), in new device
    tensors, for the lookup-table GEMV."""
    import torch
    codes = torch.empty_like(w.codes)
    scales = torch.empty_like(w.scales)
    _call("tb_sign_interleave", ctypes.byref(w.c), codes.data_ptr(), scales.data_ptr(),
          _stream(stream))
    return Matrix(codes, scales, w.n, w.k, TB_FMT_SIGN1_RI4)


def tb_ffn_down_noalloc(wd: Matrix, h, y, stream=None) -> None:
    """tb_ffn_down with the library's static scratch instead of a caller workspace."""
    _call("tb_ffn_down_noalloc", ctypes.byref(wd.c), h.data_ptr(), _rows(h), y.data_ptr(),
          _stream(stream))


def tb_ffn_down_split_workspace_bytes(wd: Matrix, m: int) -> int:
    """Bytes of device workspace tb_ffn_down_split needs for m rows (0 for bad arguments)."""
    return int(lib().tb_ffn_down_split_workspace_bytes(ctypes.byref(wd.c), int(m)))


def tb_ffn_down_split_batch_workspace_bytes(wd: Matrix, m: int) -> int:
    """Bytes of device workspace tb_ffn_down_split_batch needs for m rows (0 for bad arguments)."""
    return int(lib().tb_ffn_down_split_batch_workspace_bytes(ctypes.byref(wd.c), int(m)))


def tb_ffn_down_split_workspace(wd: Matrix, m: int, batch: bool = False):
    """A new tb_ffn_down_split (batch: tb_ffn_down_split_batch) workspace for m rows
    (uint8 device tensor; no initialisation)."""
    import torch
    name = "tb_ffn_down_split_batch_workspace_bytes" if batch else "tb_ffn_down_split_workspace_bytes"
    nbytes = int(getattr(lib(), name)(ctypes.byref(wd.c), int(m)))
    if nbytes == 0:
        raise TbError(name, TB_EINVAL)
    return torch.empty(nbytes, dtype=torch.uint8, device=wd.codes.device)


def tb_ffn_down_split(wd: Matrix, h, qh, dqh, y, ws, stream=None) -> None:
    """tb_ffn_down with a workspace for the split over k; y, qh, dqh are bit-identical."""
    _call("tb_ffn_down_split", ctypes.byref(wd.c), h.data_ptr(), _rows(h), qh.data_ptr(),
          dqh.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
          _stream(stream))


def tb_ffn_down_split_batch(wd: Matrix, h, qh, dqh, y, ws, stream=None) -> None:
    """tb_ffn_down_split for 1 ... 32 rows; each row bit-identical to tb_ffn_down alone."""
    _call("tb_ffn_down_split_batch", ctypes.byref(wd.c), h.data_ptr(), _rows(h), qh.data_ptr(),
          dqh.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
          _stream(stream))


def tb_ffn_workspace_bytes(m: int, hidden: int, inter: int) -> int:
    """Bytes of device workspace tb_ffn_layers needs for m rows (0 for bad arguments)."""
    return int(lib().tb_ffn_workspace_bytes(int(m), int(hidden), int(inter)))


def tb_ffn_workspace_init(ws, spin_ticks: int = 0, stream=None) -> None:
    """Initialise a workspace (uint8 device tensor); spin_ticks 0 = the default limit."""
    _call("tb_ffn_workspace_init", ws.data_ptr(), ws.numel() * ws.element_size(),
          int(spin_ticks), _stream(stream))


def tb_ffn_workspace_error(ws) -> int:
    """The sticky error word of a workspace (synchronises with the device)."""
    err = _I(0)
    _call("tb_ffn_workspace_error", ws.data_ptr(), ctypes.byref(err))
    return int(err.value)


class FfnLayers:
    """A host array of tb_ffn_weights for tb_ffn_layers, built once from (gate, up, down)."""

    def __init__(self, layers):
        self.layers = list(layers)
        self.arr = (CFfnWeights * len(self.layers))()
        for i, (g, u, d) in enumerate(self.layers):
            self.arr[i].gate, self.arr[i].up, self.arr[i].down = g.c, u.c, d.c

    def __len__(self) -> int:
        return len(self.layers)


def tb_ffn_layers(layers: FfnLayers, x, ws, y, chain: bool = False, stream=None) -> None:
    """Run len(layers) whole FFN layers (one launch per 32 layers).

    x float32 [L][m][hidden] (or [m][hidden] with chain=True: layer l+1 takes layer l's y),
    y float32 [L][m][hidden], ws an initialised uint8 workspace tensor."""
    if y.dim() != 3:
        raise ValueError("y must be [layers][m][hidden]")
    m = int(y.shape[1])
    _call("tb_ffn_layers", layers.arr, len(layers), x.data_ptr(), m,
          TB_FFN_CHAIN if chain else 0, ws.data_ptr(), ws.numel() * ws.element_size(),
          y.data_ptr(), _stream(stream))
