"""The fast paths' exact pieces, checked on the GPU: correctly rounded square root and
division, and the code lookups of the requantisation.

The library reaches IEEE results with short sequences (opt8_exact.h): a square root
from the hardware reciprocal square root and one Newton step, a division from a
refined reciprocal and one residual correction, each valid on a stated input range
that the step kernels check per block.  tests/exact_math/exact_check.hip runs those
very functions against the compiler's IEEE sqrtf and '/' over:

  - every fp32 in [2^-96, FLT_MAX] and +0 (the square root's whole range);
  - 2^39 significand pairs of the division (2^16 dividends spread over [1, 2) times
    every divisor in [1, 2); the quotient's rounding depends on the significands only
    while no operand or residual leaves the normal range);
  - 2^32 random pairs with divisor exponents in [-60, 100], quotient exponents in
    [-99, 100] and dividends of magnitude at least 2^-89 (the ranges the step's check
    admits: a block with a smaller non-zero moment takes the plain path).

The device reference itself is confirmed on evenly spaced samples of each sweep against
numpy's float32 sqrt and division, which are IEEE operations on the host.

The requantisation's fast path finds a code with one bucket-LUT read and one comparison
(opt8_codes.h); the plain path binary-searches the sorted midpoints, or for stochastic state
rounding the sorted entries.  Over every fp32 n in (-2, 2) (signed codes) and [0, 2)
(unsigned codes), on the table image built by the library's own builder, the two agree; for
stochastic state rounding with a random 16-bit draw per n.  Samples of each sweep are checked
against the oracle's definitions: the count of midpoints below n (numpy searchsorted on the
oracle's midpoints) and the oracle's stochastic code rule.
"""

import ctypes
import os

import numpy as np
import pytest

from gpu_helpers import log

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exact_math", "libexact_check.so")
NSAMPLE = 1 << 16


@pytest.fixture(scope="module")
def L():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    fp = ctypes.POINTER(ctypes.c_float)
    lib.exact_check_sqrt.argtypes = [ctypes.c_uint32, ctypes.c_uint32, fp, ctypes.c_int]
    lib.exact_check_sqrt.restype = ctypes.c_int64
    lib.exact_check_div_significands.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, fp, ctypes.c_int]
    lib.exact_check_div_significands.restype = ctypes.c_int64
    lib.exact_check_div_random.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_ulonglong), fp, ctypes.c_int]
    lib.exact_check_div_random.restype = ctypes.c_int64
    lib.exact_check_codes.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64,
                                      ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
    lib.exact_check_codes.restype = ctypes.c_int64
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def test_sqrt_rn_on_its_whole_range(L):
    lo = np.float32(2.0 ** -96).view(np.uint32).item()
    hi = np.float32(np.finfo(np.float32).max).view(np.uint32).item()
    sample = np.zeros(2 * NSAMPLE, np.float32)
    bad = L.exact_check_sqrt(lo, hi, _ptr(sample), NSAMPLE)
    log(f"sqrt_rn: {bad} mismatches over {hi - lo + 1} inputs")
    assert bad == 0
    x, got = sample[0::2], sample[1::2]
    assert np.all(x > 0)
    assert np.array_equal(_bits(got), _bits(np.sqrt(x)))   # the device reference is IEEE
    # +0 stays +0 (the input floor keeps the reciprocal root finite)
    zero = np.zeros(2, np.float32)
    assert L.exact_check_sqrt(0, 0, _ptr(zero), 1) == 0
    assert _bits(zero[1]) == 0


def test_div_rn_on_significand_pairs(L):
    sample = np.zeros(3 * NSAMPLE, np.float32)
    # 2^16 dividend significands with stride 127 (odd, so all distinct mod 2^23)
    bad = L.exact_check_div_significands(12345, 127, 1 << 16, _ptr(sample), NSAMPLE)
    log(f"div_rn: {bad} mismatches over {1 << 39} significand pairs")
    assert bad == 0
    a, d, got = sample[0::3], sample[1::3], sample[2::3]
    assert np.all((a >= 1) & (a < 2) & (d >= 1) & (d < 2))
    assert np.array_equal(_bits(got), _bits(a / d))


def test_div_rn_on_the_steps_exponent_ranges(L):
    sample = np.zeros(3 * NSAMPLE, np.float32)
    checked = ctypes.c_ulonglong(0)
    count = 1 << 32
    bad = L.exact_check_div_random(20240917, count, -89, ctypes.byref(checked), _ptr(sample), NSAMPLE)
    log(f"div_rn: {bad} mismatches over {checked.value} random pairs in range")
    assert bad == 0
    assert checked.value > count // 3
    a, d, got = sample[0::3], sample[1::3], sample[2::3]
    used = d != 0                      # samples that fell outside the ranges stay zero
    assert used.sum() > NSAMPLE // 3
    with np.errstate(over="raise", under="raise"):
        want = a[used] / d[used]
    assert np.array_equal(_bits(got[used]), _bits(want))


def test_div_rn_range_bound_on_the_dividend_is_needed(L):
    """Below the bound the residual leaves the normal range and the sequence does miss:
    dividends of magnitude 2^-126 .. 2^-90 only (which the step's check keeps away)."""
    checked = ctypes.c_ulonglong(0)
    small = np.zeros(3, np.float32)
    bad_all = L.exact_check_div_random(20240917, 1 << 30, -126, ctypes.byref(checked), _ptr(small), 1)
    bad_ok = L.exact_check_div_random(20240917, 1 << 30, -89, ctypes.byref(checked), _ptr(small), 1)
    log(f"div_rn below 2^-89: {bad_all - bad_ok} mismatches")
    assert bad_ok == 0 and bad_all > 0


# fp32 bit ranges of the normalised moments the LUTs cover: +0 <= n < 2 and -0 >= n > -2
POSITIVE = (0x00000000, 0x3FFFFFFF)
NEGATIVE = (0x80000000, 0xBFFFFFFF)
WHICH = {"signed": 0, "unsigned": 1, "signed-sr": 2, "unsigned-sr": 3}


def _codes_sweep(L, which, lo, hi, seed=0):
    sample = np.zeros(3 * NSAMPLE, np.uint32)
    bad = L.exact_check_codes(WHICH[which], lo, hi, seed, sample.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                              NSAMPLE)
    log(f"code lookup {which} [{lo:#010x}, {hi:#010x}]: {bad} mismatches over {hi - lo + 1} values")
    n = sample[0::3].view(np.float32)
    return bad, n, sample[1::3], sample[2::3]


@pytest.mark.parametrize("which,ranges", [("signed", (POSITIVE, NEGATIVE)), ("unsigned", (POSITIVE,))])
def test_lut_codes_equal_the_binary_search_everywhere(L, which, ranges):
    import oracle
    s_tab, s_mid, u_tab, u_mid = oracle.codebook.tables()
    mid = s_mid if which == "signed" else u_mid
    for lo, hi in ranges:
        bad, n, _, got = _codes_sweep(L, which, lo, hi)
        assert bad == 0
        assert np.array_equal(got, np.searchsorted(mid, n, side="left"))   # the oracle's rule


@pytest.mark.parametrize("which,ranges", [("signed-sr", (POSITIVE, NEGATIVE)), ("unsigned-sr", (POSITIVE,))])
def test_stochastic_lut_codes_equal_the_search_everywhere(L, which, ranges):
    import oracle
    table = oracle.state_sr.signed_table() if which == "signed-sr" else oracle.state_sr.unsigned_table()
    weights = oracle.state_sr.gap_weights(table)
    for k, (lo, hi) in enumerate(ranges):
        bad, n, r16, got = _codes_sweep(L, which, lo, hi, seed=77 + k)
        assert bad == 0
        want = oracle.state_sr.sr_codes(n, table, weights, r16.astype(np.uint32))
        assert np.array_equal(got, want.astype(np.uint32))
