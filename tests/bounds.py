"""Tolerances for comparing the HIP path with the oracle, derived from the arithmetic.

GEMV: the fp32 fold of nb terms, each term tau_b = (s*dq)*isum rounded twice, has an
error of at most (nb + 2) * 2^-24 * sum|tau|. That is 8.2e-6 relative at k = 17408,
and the required bar is 1e-4 * sum|tau|: every summation order passes, but a
dropped or doubled block does not.

h = silu(g) * u: the errors of g and u propagate through silu, whose slope
is at most 1.0998. Add 8 ulp for expf, the division and the product.

Chained FFN: h reaches the down quantiser with fp32 error, so a rotated value
lying close to a rounding boundary may land on either neighbouring int8 code.
``chain_bounds`` takes only oracle quantities and the h tolerance. It returns,
for every code of rotquant(h), the interval of values that an h within
tolerance can produce, the matching dq interval, and a bound on the down
output. No GPU value enters these bounds.
"""

from __future__ import annotations

import numpy as np
from scipy.special import expit

U = 2.0 ** -24
GEMV_REL = 1e-4          # |err| <= 1e-4 * sum|terms| per output, the stated parity bar
SILU_SLOPE = 1.0998


def sylvester(n: int = 128) -> np.ndarray:
    i = np.arange(n)
    pop = np.array([bin(v).count("1") for v in range(n)])
    return np.where(pop[i[:, None] & i[None, :]] % 2 == 0, 1.0, -1.0)


H = sylvester()


def nonzero_weights(w) -> np.ndarray:
    """|t| (0 or 1) of every weight of a packed matrix, read from its 2-bit fields."""
    if w.fmt == 1:
        return np.ones((w.n, w.k), np.uint8)
    b = w.codes.reshape(w.n, w.k // 4)
    fields = np.stack([(b >> (2 * i)) & 3 for i in range(4)], axis=2).reshape(w.n, w.k)
    return ((fields == 1) | (fields == 2)).astype(np.uint8)


def gemv_ok(y_gpu, y_ref, sabs, rel=GEMV_REL):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = rel * sabs
    ok = err <= tol
    worst = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    return bool(ok.all()), worst


def h_tolerance(g, u, sg, su):
    """Per-element bound on |h_gpu - h_ref| from the GEMV bar on g and u."""
    dg = GEMV_REL * sg
    du = GEMV_REL * su
    h = g * expit(g) * u
    return SILU_SLOPE * dg * (np.abs(u) + du) + np.abs(g * expit(g)) * du + 8 * U * np.abs(h)


def chain_bounds(h_ref, tol_h, qh_or, dqh_or, isum_or, t_abs, scales, unit):
    """Bounds for the down stage of a chained FFN.

    h_ref   float64 [m][k]       oracle h (double)
    tol_h   float64 [m][k]       h tolerance
    qh_or   int8 [m][k], dqh_or float32 [m][nb]: the oracle's rotquant(fp32(h_ref))
    isum_or int32 [m][n][nb]     the oracle's down block sums
    t_abs   uint8 [n][k]         |t| of the down weights (0 or 1)
    scales  float64 [n][nb]      down block scales
    unit    the fp32 dq unit
    Returns q_lo, q_hi (int [m][k]), dq_lo, dq_hi (float64 [m][nb]) and
    extra (float64 [m][n]): how far y may move beyond the fold bar.
    """
    m, k = h_ref.shape
    nb = k // 128
    h32 = h_ref.astype(np.float32).astype(np.float64)
    dev = tol_h + np.abs(h32 - h_ref)
    hb = h32.reshape(m, nb, 128)
    u = np.einsum("ij,rbj->rbi", H, hb)
    # both sides' fp32 transforms lie within 8U*sum|h| of the exact rotation
    T = dev.reshape(m, nb, 128).sum(axis=2) + 2 * 8 * U * np.abs(hb).sum(axis=2) + 1e-300
    amax = np.abs(u).max(axis=2)
    a_lo = np.maximum(amax - T, 1e-300)[:, :, None]
    a_hi = (amax + T)[:, :, None]
    Tb = T[:, :, None]
    cands = np.stack([(u - Tb) * 127 / a_lo, (u - Tb) * 127 / a_hi,
                      (u + Tb) * 127 / a_lo, (u + Tb) * 127 / a_hi])
    lo = cands.min(axis=0)
    hi = cands.max(axis=0)
    lo = lo - np.abs(lo) * 4 * U
    hi = hi + np.abs(hi) * 4 * U
    q_lo = np.clip(np.rint(lo), -127, 127).reshape(m, k)
    q_hi = np.clip(np.rint(hi), -127, 127).reshape(m, k)
    dq_lo = (amax - T) * unit * (1 - 3 * U)
    dq_hi = (amax + T) * unit * (1 + 3 * U)
    q_or = qh_or.astype(np.float64)
    assert np.all(q_lo <= q_or) and np.all(q_or <= q_hi), "oracle outside its own interval"
    # y: sum_b s*(|ddq|*|isum| + dq_hi * sum_i |t_i| * |dq_i|)
    d_dq = np.maximum(dq_hi - dqh_or, dqh_or - dq_lo)                   # [m][nb]
    extra = np.einsum("nb,rnb->rn", scales, np.abs(isum_or) * d_dq[:, None, :])
    wdev = np.maximum(q_hi - q_or, q_or - q_lo)                          # [m][k]
    # + sum over codes kk that may move: s[n][b] * dq_hi[r][b] * wdev[r][kk] * |t[n][kk]|,
    # one block b = kk // 128 at a time as a product over its 128 codes
    wb = wdev.reshape(m, nb, 128) * dq_hi[:, :, None]                   # [m][nb][128]
    for b in np.nonzero(wb.any(axis=(0, 2)))[0]:
        tb_ = t_abs[:, b * 128:(b + 1) * 128].astype(np.float64)         # [n][128]
        extra += (tb_ @ wb[:, b, :].T).T * scales[:, b][None, :]
    return q_lo, q_hi, dq_lo, dq_hi, extra
