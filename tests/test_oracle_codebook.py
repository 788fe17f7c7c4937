"""Pins of the oracle's dynamic-tree codebooks and block quantiser.

What the pages fix ("8-bit Optimizers via Block-wise Quantization", method
bullets): blocks of 2048 elements, per-block absolute maximum as the
normaliser, non-linear 8-bit code found by binary search, decode by table
lookup times the block maximum.  What the code reading fixes (module header
of oracle.codebook): decimal exponent by leading zeros, linear fraction with
the upper end of each step, 256 ordered entries.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codebook
from oracle.adamw import BLOCK, quantize_blockwise, dequantize_blockwise

S, MS, U, MU = codebook.tables()


def f32bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


# ----------------------------------------------------------------------------- tables
def test_tables_shape_order_and_ends():
    for t in (S, U):
        assert t.dtype == np.float32 and t.shape == (256,)
        assert np.all(np.diff(t.astype(np.float64)) > 0), "codebook must be strictly increasing"
    assert S[0] == -1.0 and S[255] == 1.0 and S[codebook.SIGNED_ZERO_CODE] == 0.0
    assert U[0] == 0.0 and U[255] == 1.0 and codebook.UNSIGNED_ZERO_CODE == 0
    assert S.min() >= -1 and S.max() <= 1 and U.min() >= 0 and U.max() <= 1


def _levels_per_decade(values, top_decade):
    counts = {}
    for v in values:
        v = Fraction(abs(float(v)))
        if v == 0:
            continue
        e = 0
        # fp32 rounding can put a decade's top level a hair above 10^-E
        while v <= Fraction(1, 10 ** (e + 1)) * (1 + Fraction(1, 2 ** 22)):
            e += 1
        counts[e] = counts.get(e, 0) + 1
    return counts


def test_tree_bit_budget_per_decade():
    """Unsigned: decade E holds 2^(7-E) levels (E=0..7); signed: 2^(6-E) per sign (E=0..6)."""
    assert _levels_per_decade(U, 7) == {e: 2 ** (7 - e) for e in range(8)}
    neg = [x for x in S if x < 0]
    pos = [x for x in S if x > 0]
    assert _levels_per_decade(neg, 6) == {e: 2 ** (6 - e) for e in range(7)}
    # positive side: the same 127 levels plus the extra 1e-7 level (decade 7)
    want = {e: 2 ** (6 - e) for e in range(7)}
    want[7] = 1
    assert _levels_per_decade(pos, 7) == want


def test_decades_are_evenly_split_and_topped_by_powers_of_ten():
    for table, top in ((U, 7), (S[S > 0], 6)):
        for e in range(top + 1):
            lo, hi = 10.0 ** -(e + 1), 10.0 ** -e
            lv = np.array([float(x) for x in table if lo * (1 + 1e-6) < float(x) <= hi * (1 + 1e-6)])
            assert abs(lv[-1] - hi) <= hi * 2 ** -24, (e, lv[-1])
            if lv.size > 1:
                steps = np.diff(lv)
                want = 0.9 * hi / lv.size
                assert np.allclose(steps, want, rtol=1e-5, atol=hi * 2 ** -22), e
                # the lowest level sits one step above the decade floor (upper-end reading)
                assert abs(lv[0] - (lo + want)) <= hi * 2 ** -22


def test_signed_table_is_symmetric_apart_from_the_extra_level():
    for k in range(127):
        assert S[k] == -S[255 - k], k
    assert S[128] == np.float32(1e-7)


def test_spot_values_of_the_reading():
    """Hand-derived closed forms of the tree code reading (exact rationals, rounded to fp32)."""
    r = codebook.fraction_to_f32
    assert U[1] == r(Fraction(1, 10 ** 7))
    assert U[2] == r(Fraction(11, 2 * 10 ** 7))
    assert U[3] == r(Fraction(1, 10 ** 6))
    assert U[254] == r(Fraction(1271, 1280))
    assert S[1] == r(Fraction(-631, 640))
    assert S[126] == r(Fraction(-1, 10 ** 6))
    assert S[129] == r(Fraction(1, 10 ** 6))
    assert S[130] == r(Fraction(11, 2 * 10 ** 6))


def test_fraction_to_f32_is_nearest_with_ties_to_even():
    one = Fraction(1)
    ulp = Fraction(1, 2 ** 23)
    assert codebook.fraction_to_f32(one + ulp / 2) == np.float32(1.0)          # tie -> even
    assert codebook.fraction_to_f32(one + 3 * ulp / 2) == np.float32(1 + 2 * 2 ** -23)
    assert codebook.fraction_to_f32(one + ulp / 2 + Fraction(1, 2 ** 60)) == np.float32(1 + 2 ** -23)
    for v in (Fraction(1, 10), Fraction(-7, 3), Fraction(1, 10 ** 7)):
        got = Fraction(float(codebook.fraction_to_f32(v)))
        assert abs(got - v) <= abs(v) * Fraction(1, 2 ** 24)


def test_midpoints_sit_between_neighbours():
    for t, m in ((S, MS), (U, MU)):
        assert m.shape == (255,)
        for k in range(255):
            exact = (Fraction(float(t[k])) + Fraction(float(t[k + 1]))) / 2
            assert t[k] < m[k] < t[k + 1]
            assert abs(Fraction(float(m[k])) - exact) <= abs(exact) * Fraction(1, 2 ** 24)


# ----------------------------------------------------------------------------- quantiser
def _brute_nearest(table, n):
    """Nearest entry by exact distance, lower index on ties."""
    best, best_d = None, None
    nf = Fraction(float(n))
    for k in range(256):
        d = abs(Fraction(float(table[k])) - nf)
        if best is None or d < best_d:
            best, best_d = k, d
    return best


def _near_midpoint(table, n):
    nf = Fraction(float(n))
    for k in range(255):
        exact = (Fraction(float(table[k])) + Fraction(float(table[k + 1]))) / 2
        if abs(nf - exact) <= abs(exact) * Fraction(1, 2 ** 23):
            return True
    return False


def _adversarial_values(table, mid, rng):
    vals = [0.0, -0.0, 1.0, -1.0, 1e-7, -1e-7, 5e-8, 2.0 ** -140]
    vals += [float(x) for x in mid[rng.integers(0, 255, 6)]]           # exact midpoints
    vals += [float(x) for x in table[rng.integers(0, 256, 6)]]         # exact entries
    return vals


@pytest.mark.parametrize("signed", [True, False])
def test_quantizer_matches_brute_force_on_16_element_tensors(signed):
    table, mid = (S, MS) if signed else (U, MU)
    zero = codebook.SIGNED_ZERO_CODE if signed else codebook.UNSIGNED_ZERO_CODE
    rng = np.random.default_rng(1 if signed else 2)
    disagreements = 0
    checked = 0
    for trial in range(700):
        if trial % 7 == 0:
            x = np.array((_adversarial_values(table, mid, rng) * 3)[:16], dtype=np.float32)
        else:
            scale = 10.0 ** rng.uniform(-9, 2)
            x = (rng.standard_normal(16) * scale).astype(np.float32)
            x *= np.float32(10.0) ** rng.uniform(-4, 0, 16).astype(np.float32)
        if not signed:
            x = np.abs(x)
        codes, absmax = quantize_blockwise(x, mid, zero)
        a = np.max(np.abs(x))
        assert absmax.shape == (1,) and f32bits(absmax[0]) == f32bits(a)
        if a < 2.0 ** -126:
            assert np.all(codes == zero)
            continue
        inv = np.float32(1.0) / a
        for xi, c in zip(x, codes):
            n = np.float32(xi * inv)
            bf = _brute_nearest(table, n)
            checked += 1
            if bf != c:
                assert _near_midpoint(table, n), (float(xi), float(n), int(c), bf)
                assert abs(int(c) - bf) == 1
                disagreements += 1
    assert checked > 5000
    assert disagreements > 0        # the adversarial exact midpoints do reach the slack


def test_midpoint_ties_take_the_lower_code():
    for table, mid, zero in ((S, MS, 127), (U, MU, 0)):
        for k in (0, 7, 126, 127, 128, 200, 254):
            x = np.array([mid[k], 1.0], dtype=np.float32)     # absmax 1 -> normalised == x
            codes, _ = quantize_blockwise(x, mid, zero)
            assert codes[0] == k and codes[1] == 255


def test_a_zero_normalised_value_takes_the_zero_code():
    """n = +0 and n = -0 code to the zero code under the nearest-entry search and under
    stochastic rounding between neighbours (any random word): a block whose absmax is
    below 2^-126 (normaliser 0, so every n is +-0) stores the zero code either by that
    rule or by the explicit zero-code case, with the same bytes."""
    from oracle import state_sr
    zeros = np.array([0.0, -0.0], dtype=np.float32)
    assert np.all(np.searchsorted(MS, zeros, side="left") == codebook.SIGNED_ZERO_CODE)
    assert np.all(np.searchsorted(MU, zeros[:1], side="left") == codebook.UNSIGNED_ZERO_CODE)
    r16 = np.arange(0, 65536, 257, dtype=np.uint32)
    for table, zero, n in ((state_sr.signed_table(), codebook.SIGNED_ZERO_CODE, zeros),
                           (state_sr.unsigned_table(), codebook.UNSIGNED_ZERO_CODE, zeros[:1])):
        w = state_sr.gap_weights(table)
        for x in n:
            got = state_sr.sr_codes(np.full(r16.size, x, dtype=np.float32), table, w, r16)
            assert np.all(got == zero)


def test_error_within_half_local_gap():
    """|C[q] * A - x| <= half the gap of the bracketing entries * A (+ fp32 slack)."""
    rng = np.random.default_rng(3)
    for table, mid, zero, signed in ((S, MS, 127, True), (U, MU, 0, False)):
        x = (rng.standard_normal(BLOCK * 6 + 123) * 1e-3).astype(np.float32)
        x *= np.float32(10.0) ** rng.uniform(-5, 0, x.size).astype(np.float32)
        if not signed:
            x = x * x
        codes, absmax = quantize_blockwise(x, mid, zero)
        deq = dequantize_blockwise(codes, absmax, table).astype(np.float64)
        a = np.repeat(absmax.astype(np.float64), BLOCK)[: x.size]
        n = x.astype(np.float64) / a
        k = np.clip(np.searchsorted(table.astype(np.float64), n, side="right") - 1, 0, 254)
        gap = (table[k + 1].astype(np.float64) - table[k].astype(np.float64))
        bound = 0.5 * gap * a * (1 + 2.0 ** -20) + 2.0 ** -23 * a
        assert np.all(np.abs(deq - x.astype(np.float64)) <= bound)


def test_block_absmax_is_the_exact_block_max_and_partial_tail():
    rng = np.random.default_rng(4)
    n = BLOCK * 3 + 517
    x = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    x[BLOCK:2 * BLOCK] = 0.0                                    # an all-zero block
    x[2 * BLOCK:3 * BLOCK] = np.float32(2.0 ** -130)            # a subnormal block
    x[2 * BLOCK + 5] = np.float32(-(2.0 ** -128))
    codes, absmax = quantize_blockwise(x, MS, 127)
    assert absmax.shape == (4,)
    for b in range(4):
        seg = x[b * BLOCK: min(n, (b + 1) * BLOCK)]
        want = max(abs(float(v)) for v in seg)
        assert float(absmax[b]) == want
    assert np.all(codes[BLOCK:3 * BLOCK] == 127)
    assert float(absmax[2]) == 2.0 ** -128
    # the partial block's max ignores everything past the end of the tensor
    x2 = x.copy()
    codes2, absmax2 = quantize_blockwise(x2[: n - 17], MS, 127)
    seg = x[3 * BLOCK: n - 17]
    assert float(absmax2[3]) == max(abs(float(v)) for v in seg)


def test_dequantize_is_table_times_block_max():
    rng = np.random.default_rng(5)
    n = BLOCK + 300
    codes = rng.integers(0, 256, n, dtype=np.uint8)
    absmax = np.array([0.25, 3.0e-5], dtype=np.float32)
    got = dequantize_blockwise(codes, absmax, S)
    for i in range(0, n, 37):
        assert got[i] == np.float32(S[codes[i]] * absmax[i // BLOCK])
