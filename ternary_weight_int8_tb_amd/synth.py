"""Seeded synthetic inputs for the ternary FFN path.

This module draws weights and activations and writes them in the packed
storage format. It holds none of the method's arithmetic: no rotation,
quantisation, decoding to +-1, dot products or scale folding. Both the HIP
path and the CPU oracle consume its bytes.

Streams
-------
Every tensor has its own numpy stream:
``np.random.default_rng(np.random.SeedSequence([seed, layer, tensor]))``.
Tensor ids are the ``T_*`` constants below.

Weight formats
--------------
The ternary format stores 128 weights per block in 32 bytes, plus one fp16
scale per block in a separate array. The sign format stores 16 bytes per
block plus the same scales.

* Ternary codes take the values 0, 1 and 2, i.i.d. uniform. Code ``c`` of
  weight ``i`` of a row sits in byte ``i >> 2`` of that row's codes, bits
  ``2*(i & 3)`` and ``2*(i & 3) + 1``, least significant bits first.
  Four i.i.d. uniform codes make each byte uniform over the 81 bytes with no
  field equal to 3. So the generator draws one integer ``d`` in ``[0, 81)``
  per byte and places the base-3 digits of ``d`` in the four fields. This is
  exact, and about 4x faster than drawing codes one by one.
* Sign bits are i.i.d. Bernoulli(1/2), so every code byte is uniform over
  all 256 values. Bit ``i`` sits in byte ``i >> 3``, bit ``i & 7``. The bytes
  are drawn as full-range uint32 words and read as little-endian bytes.
* Scales are ``lognormal(mu=-4, sigma=0.5)`` rounded to IEEE binary16 (round
  to nearest even) and stored as raw uint16 bit patterns.

The matrix layout is row-major and contiguous: ``codes[N][K/128][32]``
(ternary) or ``codes[N][K/128][16]`` (sign), and ``scales[N][K/128]``.

Activations
-----------
Activations are drawn in float64 and then rounded to float32. The draws are
i.i.d. N(0, 1), or Student-t with nu=3 plus outlier channels. An outlier
channel is one of ``floor(frac*K)`` fixed input indices, drawn once without
replacement and multiplied by 50.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BLOCK = 128

T_GATE = 0      # gate matrix, or the only matrix of a single GEMV
T_UP = 1
T_DOWN = 2
T_ACT = 3       # activation rows x
T_OUTLIER = 4   # outlier channel indices
T_HIDDEN = 5    # stand-alone hidden rows h, fed straight to the down stage

FMT_TERNARY2 = 0
FMT_SIGN1 = 1


def rng_for(seed: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, layer, tensor]))


def _digit_tables():
    """byte_of[d] places the base-3 digits of d in the 2-bit fields; trits[d] lists them."""
    d = np.arange(81)
    trits = np.stack([(d // 3**i) % 3 for i in range(4)], axis=1).astype(np.uint8)
    byte_of = np.zeros(81, np.uint8)
    for i in range(4):
        byte_of |= (trits[:, i] << (2 * i)).astype(np.uint8)
    return byte_of, trits


_BYTE_OF, _TRITS = _digit_tables()


@dataclass
class PackedMatrix:
    """One weight matrix in the packed storage format (host copy)."""
    codes: np.ndarray    # uint8 [n][nb][32] (ternary) or [n][nb][16] (sign)
    scales: np.ndarray   # uint16 [n][nb], binary16 bit patterns
    n: int
    k: int
    fmt: int
    draw: np.ndarray | None = None   # ternary: the per-byte draws d (uint16 [n][k/4])

    @property
    def nbytes(self) -> int:
        return self.codes.nbytes + self.scales.nbytes

    def codes_unpacked(self) -> np.ndarray:
        """Per-weight codes before packing: uint8 [n][k].

        Ternary gives the codes 0, 1, 2. Sign gives the bits 0, 1.
        """
        if self.fmt == FMT_TERNARY2:
            return _TRITS[self.draw.reshape(self.n, self.k // 4)].reshape(self.n, self.k)
        bits = np.unpackbits(self.codes.reshape(self.n, -1), axis=1, bitorder="little")
        return bits.reshape(self.n, self.k)

    def scales_f32(self) -> np.ndarray:
        return self.scales.view(np.float16).astype(np.float32)


def pack_ternary(codes: np.ndarray, scales: np.ndarray) -> PackedMatrix:
    """Pack per-weight codes (uint8 [n][k], values 0..3) into the ternary storage format.

    scales are binary16 bit patterns (uint16 [n][k/128]) or float values that are
    rounded to binary16.
    """
    codes = np.asarray(codes, np.uint8)
    n, k = codes.shape
    if k % BLOCK:
        raise ValueError("k must be a multiple of 128")
    c = codes.reshape(n, k // 4, 4)
    packed = (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)
    return PackedMatrix(packed.reshape(n, k // BLOCK, 32), _scale_bits(scales, n, k), n, k,
                        FMT_TERNARY2)


def pack_sign(bits: np.ndarray, scales: np.ndarray) -> PackedMatrix:
    """Pack per-weight sign bits (uint8 [n][k], values 0/1) into the sign storage format."""
    bits = np.asarray(bits, np.uint8)
    n, k = bits.shape
    if k % BLOCK:
        raise ValueError("k must be a multiple of 128")
    packed = np.packbits(bits, axis=1, bitorder="little")
    return PackedMatrix(packed.reshape(n, k // BLOCK, 16), _scale_bits(scales, n, k), n, k,
                        FMT_SIGN1)


def _scale_bits(scales, n: int, k: int) -> np.ndarray:
    s = np.asarray(scales)
    if s.dtype != np.uint16:
        s = s.astype(np.float16).view(np.uint16)
    return np.ascontiguousarray(s.reshape(n, k // BLOCK))


def _scales(rng: np.random.Generator, n: int, nb: int) -> np.ndarray:
    return rng.lognormal(-4.0, 0.5, n * nb).astype(np.float16).view(np.uint16).reshape(n, nb)


def ternary_matrix(n: int, k: int, seed: int, layer: int, tensor: int,
                   keep_draw: bool = False) -> PackedMatrix:
    if k % BLOCK:
        raise ValueError("k must be a multiple of 128")
    nb = k // BLOCK
    rng = rng_for(seed, layer, tensor)
    d = rng.integers(0, 81, n * k // 4, dtype=np.uint16)
    codes = _BYTE_OF[d].reshape(n, nb, 32)
    scales = _scales(rng, n, nb)
    return PackedMatrix(codes, scales, n, k, FMT_TERNARY2, d if keep_draw else None)


def sign_matrix(n: int, k: int, seed: int, layer: int, tensor: int) -> PackedMatrix:
    if k % BLOCK:
        raise ValueError("k must be a multiple of 128")
    nb = k // BLOCK
    rng = rng_for(seed, layer, tensor)
    # uniform bytes from full-range 32-bit draws, read as little-endian bytes
    words = rng.integers(0, 2 ** 32, n * k // 32, dtype=np.uint32)
    codes = words.astype("<u4").view(np.uint8).reshape(n, nb, 16)
    scales = _scales(rng, n, nb)
    return PackedMatrix(codes, scales, n, k, FMT_SIGN1)


def matrix(fmt: int, n: int, k: int, seed: int, layer: int, tensor: int,
           keep_draw: bool = False) -> PackedMatrix:
    if fmt == FMT_TERNARY2:
        return ternary_matrix(n, k, seed, layer, tensor, keep_draw)
    if fmt == FMT_SIGN1:
        return sign_matrix(n, k, seed, layer, tensor)
    raise ValueError(f"unknown format {fmt}")


def normal_rows(m: int, k: int, seed: int, layer: int, tensor: int = T_ACT) -> np.ndarray:
    """m i.i.d. N(0,1) rows of length k, drawn in float64 and rounded to float32."""
    return rng_for(seed, layer, tensor).standard_normal((m, k)).astype(np.float32)


def outlier_channels(k: int, seed: int, layer: int, frac: float = 0.01) -> np.ndarray:
    count = int(np.floor(frac * k))
    idx = rng_for(seed, layer, T_OUTLIER).choice(k, size=count, replace=False)
    return np.sort(idx)


def student_t_rows(m: int, k: int, seed: int, layer: int, nu: float = 3.0,
                   frac: float = 0.01, outlier_scale: float = 50.0) -> np.ndarray:
    """Student-t(nu) rows; a fixed set of input channels is scaled by outlier_scale."""
    x = rng_for(seed, layer, T_ACT).standard_t(nu, (m, k))
    x[:, outlier_channels(k, seed, layer, frac)] *= outlier_scale
    return x.astype(np.float32)


# ---------------------------------------------------------------------------
# Workloads: the FFN layer shapes (hidden 5120, intermediate 17408)
# ---------------------------------------------------------------------------

HIDDEN = 5120
INTER = 17408


@dataclass
class FfnLayer:
    gate: PackedMatrix   # [INTER x HIDDEN]
    up: PackedMatrix     # [INTER x HIDDEN]
    down: PackedMatrix   # [HIDDEN x INTER]

    @property
    def nbytes(self) -> int:
        return self.gate.nbytes + self.up.nbytes + self.down.nbytes


def ffn_layer(seed: int, layer: int, fmt: int = FMT_TERNARY2, hidden: int = HIDDEN,
              inter: int = INTER, keep_draw: bool = False, threads: int = 3) -> FfnLayer:
    jobs = [(inter, hidden, T_GATE), (inter, hidden, T_UP), (hidden, inter, T_DOWN)]
    with ThreadPoolExecutor(max(1, threads)) as ex:
        mats = list(ex.map(lambda a: matrix(fmt, a[0], a[1], seed, layer, a[2], keep_draw), jobs))
    return FfnLayer(*mats)


def ffn_stream(seed: int, layers: int, fmt: int = FMT_TERNARY2, threads: int = 8,
               hidden: int = HIDDEN, inter: int = INTER) -> list[FfnLayer]:
    """Independently seeded layers: layer l draws from streams (seed, l, tensor)."""
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda l: ffn_layer(seed, l, fmt, hidden, inter, threads=1),
                           range(layers)))


# ---------------------------------------------------------------------------
# Second workload: the projections of a full-attention layer of the same model
# (hidden 5120; head dim 256, 8:1 grouped-query attention with 2 key/value heads,
# so 16 query heads; gated queries). The input projection is one fused matrix of
# query (4096), gate (4096), key (512) and value (512) rows; the output projection
# maps the 4096 attention outputs back to the hidden size. Every 4th of the 64
# layers is a full-attention layer: 16 such layers.
# ---------------------------------------------------------------------------

HEAD_DIM = 256
Q_HEADS = 16
KV_HEADS = 2
ATTN_Q = Q_HEADS * HEAD_DIM                          # 4096
ATTN_QKVG = 2 * ATTN_Q + 2 * KV_HEADS * HEAD_DIM     # 9216: query, gate, key, value rows
ATTN_LAYERS = 16

T_QKVG = 6       # fused input projection [ATTN_QKVG x HIDDEN]
T_OPROJ = 7      # output projection [HIDDEN x ATTN_Q]
T_ATTN_OUT = 8   # stand-in rows for the attention output fed to the output projection


@dataclass
class AttnLayer:
    qkvg: PackedMatrix   # [ATTN_QKVG x HIDDEN]
    o: PackedMatrix      # [HIDDEN x ATTN_Q]

    @property
    def nbytes(self) -> int:
        return self.qkvg.nbytes + self.o.nbytes


def attn_layer(seed: int, layer: int, fmt: int = FMT_TERNARY2) -> AttnLayer:
    return AttnLayer(matrix(fmt, ATTN_QKVG, HIDDEN, seed, layer, T_QKVG),
                     matrix(fmt, HIDDEN, ATTN_Q, seed, layer, T_OPROJ))


def attn_stream(seed: int, layers: int = ATTN_LAYERS, fmt: int = FMT_TERNARY2,
                threads: int = 8) -> list[AttnLayer]:
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda l: attn_layer(seed, l, fmt), range(layers)))
