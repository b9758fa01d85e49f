"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is tb_oracle.c with one plausible mistake in it: a dropped term, a
wrong sign or index, a transposed operand, a wrong rounding rule. It is built
into a temporary library, and at least one pin must fail against it.
"""

import pytest

import oracle
from tests import pins

MUTANTS = {
    "butterfly_sign": ("v[i + h] = a - b;", "v[i + h] = b - a;"),
    "fwht_last_stage_dropped": ("for (int h = 1; h < TBO_BLOCK; h <<= 1)",
                                "for (int h = 1; h < TBO_BLOCK / 2; h <<= 1)"),
    "code_map_swapped": ("return (c & 1) - (c >> 1);", "return (c >> 1) - (c & 1);"),
    "field_order_reversed": ("(row[i >> 2] >> (2 * (i & 3))) & 3",
                             "(row[i >> 2] >> (6 - 2 * (i & 3))) & 3"),
    "sign_inverted": ("& 1) ? 1 : -1;", "& 1) ? -1 : 1;"),
    "last_block_dropped": ("y[(size_t)r * count + slot] += term;",
                           "if (b + 1 < nb) y[(size_t)r * count + slot] += term;"),
    "scale_index_shifted": ("scales[(size_t)j * nb + b]);",
                            "scales[(size_t)j * nb + (b + 1 < nb ? b + 1 : b)]);"),
    "round_half_away": ("float t = rintf(u[i] * inv);", "float t = roundf(u[i] * inv);"),
    "round_truncate": ("float t = rintf(u[i] * inv);", "float t = truncf(u[i] * inv);"),
    "dq_unit_unnormalised": ("(float)(1.0 / (127.0 * sqrt(128.0)))", "(float)(1.0 / 127.0)"),
    "amax_signed": ("float a = fabsf(u[i]);", "float a = u[i];"),
    "half_exponent_bias": ("e - 25);", "e - 24);"),
    "half_subnormal": ("ldexp((double)f, -24);", "ldexp((double)f, -25);"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "activation_row_ignored": ("const int8_t *qb = q + (size_t)r * k + (size_t)b * TBO_BLOCK;",
                               "const int8_t *qb = q + (size_t)b * TBO_BLOCK;"),
    "dq_row_ignored": ("(double)dq[(size_t)r * nb + b] * (double)isum",
                       "(double)dq[b] * (double)isum"),
    "gate_up_swapped": ("h[i] = tbo_silu(g[i]) * u[i];", "h[i] = tbo_silu(u[i]) * g[i];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert old in src, f"mutant {name}: pattern no longer in tb_oracle.c"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(str(path), str(tmp_path / "libmutant.so"))
    o = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
