"""The seeded input generator (CPU only)."""

import hashlib

import numpy as np

from ternary_weight_int8_tb_amd import synth


def _sha(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    a = synth.ternary_matrix(256, 512, 0, 0, synth.T_GATE)
    b = synth.ternary_matrix(256, 512, 0, 0, synth.T_GATE)
    assert _sha(a.codes, a.scales) == _sha(b.codes, b.scales)
    c = synth.ternary_matrix(256, 512, 0, 1, synth.T_GATE)
    assert _sha(a.codes) != _sha(c.codes)
    x1 = synth.normal_rows(8, 5120, 1, 0)
    assert np.array_equal(x1[:2], synth.normal_rows(8, 5120, 1, 0)[:2])


def test_layout_and_sizes():
    w = synth.ternary_matrix(17408, 5120, 0, 0, synth.T_GATE)
    assert w.codes.shape == (17408, 40, 32) and w.codes.dtype == np.uint8
    assert w.scales.shape == (17408, 40) and w.scales.dtype == np.uint16
    assert w.nbytes == 23_674_880
    s = synth.sign_matrix(5120, 17408, 4, 0, synth.T_DOWN)
    assert s.codes.shape == (5120, 136, 16) and s.nbytes == 5120 * 136 * 18


def test_code_distribution():
    w = synth.ternary_matrix(1024, 4096, 5, 0, synth.T_GATE, keep_draw=True)
    c = w.codes_unpacked()
    n = c.size
    for v in range(3):
        f = (c == v).mean()
        assert abs(f - 1 / 3) < 5 * np.sqrt((1 / 3) * (2 / 3) / n), (v, f)
    assert not (c == 3).any()
    # no 2-bit field of any packed byte holds the unused code 3
    b = w.codes.reshape(-1)
    for sh in range(4):
        assert not (((b >> (2 * sh)) & 3) == 3).any()
    s = synth.sign_matrix(512, 4096, 5, 0, synth.T_GATE)
    bits = s.codes_unpacked()
    assert abs(bits.mean() - 0.5) < 5 * np.sqrt(0.25 / bits.size)


def test_scale_distribution():
    w = synth.ternary_matrix(4096, 5120, 6, 0, synth.T_GATE)
    ls = np.log(w.scales_f32().astype(np.float64))
    assert abs(ls.mean() + 4.0) < 0.01 and abs(ls.std() - 0.5) < 0.01


def test_student_t_outliers():
    k = 5120
    idx = synth.outlier_channels(k, 4, 0)
    assert idx.size == 51 and np.unique(idx).size == 51
    x = synth.student_t_rows(8, k, 4, 0)
    base = synth.rng_for(4, 0, synth.T_ACT).standard_t(3.0, (8, k))
    assert np.array_equal(x[:, idx], (base[:, idx] * 50).astype(np.float32))
    rest = np.setdiff1d(np.arange(k), idx)
    assert np.array_equal(x[:, rest], base[:, rest].astype(np.float32))
    # heavy tails: P(|t_3| > 5) is about 1.5%
    tail = (np.abs(base) > 5).mean()
    assert 0.008 < tail < 0.025


def test_pack_roundtrip():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 4, (7, 256)).astype(np.uint8)
    w = synth.pack_ternary(codes, np.ones((7, 2)))
    # unpack by reading the fields back (format reading, test side)
    b = w.codes.reshape(7, 64)
    back = np.stack([(b >> (2 * i)) & 3 for i in range(4)], axis=2).reshape(7, 256)
    assert np.array_equal(back, codes)
    bits = rng.integers(0, 2, (3, 384)).astype(np.uint8)
    s = synth.pack_sign(bits, np.ones((3, 3)))
    assert np.array_equal(s.codes_unpacked(), bits)
