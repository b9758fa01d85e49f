"""Device-side helpers for the GPU tests: upload, poisoned outputs, calls through the C ABI.

Every output buffer is filled with a poison value before the call, so an
element the kernels never write shows up as a mismatch.
"""

from __future__ import annotations

import numpy as np
import torch

import ternary_weight_int8_tb_amd as tb

DEV = "cuda"
POISON_I8 = 0x5A
POISON_I32 = -0x7FFFFFF1


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f32_out(*shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


def i8_out(*shape):
    return torch.full(shape, POISON_I8, dtype=torch.int8, device=DEV)


def i32_out(*shape):
    return torch.full(shape, POISON_I32, dtype=torch.int32, device=DEV)


class GpuLayer:
    def __init__(self, layer):
        self.gate = tb.Matrix.upload(layer.gate, DEV)
        self.up = tb.Matrix.upload(layer.up, DEV)
        self.down = tb.Matrix.upload(layer.down, DEV)
        self.hidden = layer.gate.k
        self.inter = layer.gate.n


def rotquant(x: np.ndarray, stream=None):
    m, k = x.shape
    q, dq = i8_out(m, k), f32_out(m, k // 128)
    tb.tb_rotate_quant_i8(dev(x), q, dq, stream)
    return host(q), host(dq)


def gemv(w: tb.Matrix, q: np.ndarray, dq: np.ndarray):
    y = f32_out(q.shape[0], w.n)
    tb.tb_gemv_ternary(w, dev(q), dev(dq), y)
    return host(y)


def block_sums(w: tb.Matrix, q: np.ndarray):
    out = i32_out(q.shape[0], w.n, w.k // 128)
    tb.tb_gemv_block_sums(w, dev(q), out)
    return host(out)


def gateup(g: GpuLayer, q: np.ndarray, dq: np.ndarray):
    h = f32_out(q.shape[0], g.inter)
    tb.tb_ffn_gateup_silu(g.gate, g.up, dev(q), dev(dq), h)
    return host(h)


def down(wd: tb.Matrix, h: np.ndarray):
    m, k = h.shape
    qh, dqh, y = i8_out(m, k), f32_out(m, k // 128), f32_out(m, wd.n)
    tb.tb_ffn_down(wd, dev(h), qh, dqh, y)
    return host(qh), host(dqh), host(y)


class LayerRun:
    """Device buffers for one FFN layer call chain at m rows (poisoned before each run)."""

    def __init__(self, g: GpuLayer, m: int):
        self.g, self.m = g, m
        k, n = g.hidden, g.inter
        self.x = torch.empty(m, k, dtype=torch.float32, device=DEV)
        self.q, self.dq = i8_out(m, k), f32_out(m, k // 128)
        self.h = f32_out(m, n)
        self.qh, self.dqh = i8_out(m, n), f32_out(m, n // 128)
        self.y = f32_out(m, k)

    def poison(self):
        for t in (self.dq, self.h, self.dqh, self.y):
            t.fill_(float("nan"))
        self.q.fill_(POISON_I8)
        self.qh.fill_(POISON_I8)

    def launch(self, stream=None):
        g = self.g
        tb.tb_rotate_quant_i8(self.x, self.q, self.dq, stream)
        tb.tb_ffn_gateup_silu(g.gate, g.up, self.q, self.dq, self.h, stream)
        tb.tb_ffn_down(g.down, self.h, self.qh, self.dqh, self.y, stream)

    def run(self, x: np.ndarray, stream=None) -> dict:
        self.x.copy_(torch.from_numpy(np.ascontiguousarray(x)))
        self.poison()
        self.launch(stream)
        return self.fetch()

    def fetch(self) -> dict:
        torch.cuda.synchronize()
        return {name: getattr(self, name).cpu().numpy()
                for name in ("q", "dq", "h", "qh", "dqh", "y")}
