"""Dynamic-tree 8-bit codebooks for the two Adam moments (oracle).

TEST INFRASTRUCTURE ONLY (see the package header).

Source.  "8-bit Optimizers via Block-wise Quantization": the list of the
paper's innovations (non-linear dynamic quantization that extends dynamic tree
quantization to unipolar data) and the method bullets (values are normalised
into the block, mapped to 8-bit indices by a binary search, and decoded by a
lookup table times the block maximum).  The page names the dynamic tree code
but does not spell it out, so the construction below is a reading:

  * A code is a bit string.  After an optional sign bit, the number E of
    leading zero bits is a decimal exponent, the first one bit that follows
    is an indicator, and the F bits after it are a linear fraction f.
  * The value is 10^-E * (1/10 + 9/10 * (f + 1) / 2^F): the F fraction bits
    cut the decade (10^-(E+1), 10^-E] into 2^F equal steps and the code takes
    the upper end of its step, so every decade tops out exactly at 10^-E.
  * Unsigned (second moment, which is never negative): all 8 bits are
    magnitude bits, E = 0..7 and F = 7 - E, which gives 255 levels; the
    all-zero string is 0.  That is 256 entries in [0, 1].
  * Signed (first moment): a sign bit and 7 magnitude bits, E = 0..6 and
    F = 6 - E, which gives 127 levels per sign plus 0 (positive sign, zero
    magnitude).  The remaining string (negative sign, zero magnitude) would be
    a second zero; it is given the value +1e-7, the decade the unsigned code
    has beyond the signed one, so the table has 256 distinct entries in
    [-1, 1].
  * Each level is the fp32 number nearest the exact rational value (ties to
    even).  The table is sorted ascending and a code IS its index in the
    sorted table, so codes order like their values.
  * Rounding to a code picks the nearest entry, using the 255 midpoints
    mid_k = fp32 nearest to (C_k + C_{k+1}) / 2: the code of n is the number
    of midpoints strictly below n, so a value exactly on a midpoint takes the
    lower code.

Parity: the invariants the pages fix (256 entries, monotone, ends at -1/0/+1)
and brute-force nearest-entry search are pinned by tests; the individual
level values against the original paper's own table are "parity unpinned",
because the pages do not print that table.
"""

from fractions import Fraction

import numpy as np

NUM_CODES = 256
SIGNED_ZERO_CODE = 127
UNSIGNED_ZERO_CODE = 0


def fraction_to_f32(value: Fraction) -> np.float32:
    """Nearest fp32 to an exact rational, ties to even (exact, no double rounding)."""
    guess = np.float32(float(value))
    below = np.nextafter(guess, np.float32(-np.inf), dtype=np.float32)
    above = np.nextafter(guess, np.float32(np.inf), dtype=np.float32)
    best = None
    best_err = None
    for cand in (below, guess, above):
        err = abs(Fraction(float(cand)) - value)
        if best is None or err < best_err:
            best, best_err = cand, err
        elif err == best_err:
            # tie: keep the candidate with an even last significand bit
            if int(np.array(cand, dtype=np.float32).view(np.uint32)) & 1 == 0:
                best = cand
    return np.float32(best)


def tree_magnitude(pattern: int, nbits: int) -> Fraction:
    """Exact value of an nbits-wide magnitude bit string under the tree code.

    pattern == 0 has no indicator bit and is the zero level.
    """
    if pattern == 0:
        return Fraction(0)
    # E = leading zeros of the nbits-wide string, then the indicator bit
    width = pattern.bit_length()
    zeros = nbits - width
    frac_bits = width - 1            # bits after the indicator
    frac = pattern - (1 << frac_bits)  # drop the indicator
    decade = Fraction(1, 10 ** zeros)
    return decade * (Fraction(1, 10) + Fraction(9, 10) * Fraction(frac + 1, 1 << frac_bits))


def unsigned_levels_exact():
    """256 exact values of the unsigned tree code (all 8 bits are magnitude)."""
    return [tree_magnitude(b, 8) for b in range(NUM_CODES)]


def signed_levels_exact():
    """256 exact values of the signed tree code (sign bit + 7 magnitude bits)."""
    out = []
    for b in range(NUM_CODES):
        sign = b >> 7
        mag = b & 0x7F
        if mag == 0:
            # +0, and the otherwise-unused "negative zero" string -> +1e-7
            out.append(Fraction(0) if sign == 0 else Fraction(1, 10 ** 7))
        else:
            v = tree_magnitude(mag, 7)
            out.append(-v if sign else v)
    return out


def _table(levels_exact):
    ordered = sorted(levels_exact)
    if len(set(ordered)) != NUM_CODES:
        raise AssertionError("codebook levels are not distinct")
    return np.array([fraction_to_f32(v) for v in ordered], dtype=np.float32)


def signed_codebook() -> np.ndarray:
    """fp32[256], ascending; index 127 is 0 (the zero code of the first moment)."""
    return _table(signed_levels_exact())


def unsigned_codebook() -> np.ndarray:
    """fp32[256], ascending; index 0 is 0 (the zero code of the second moment)."""
    return _table(unsigned_levels_exact())


def midpoints(table: np.ndarray) -> np.ndarray:
    """fp32[255]: nearest fp32 to the exact midpoint of neighbouring entries."""
    out = np.empty(NUM_CODES - 1, dtype=np.float32)
    for k in range(NUM_CODES - 1):
        exact = (Fraction(float(table[k])) + Fraction(float(table[k + 1]))) / 2
        out[k] = fraction_to_f32(exact)
    return out


_CACHE = {}


def tables():
    """(signed, signed_mid, unsigned, unsigned_mid), built once per process."""
    if not _CACHE:
        s = signed_codebook()
        u = unsigned_codebook()
        _CACHE["t"] = (s, midpoints(s), u, midpoints(u))
    return _CACHE["t"]
