"""Pins of the oracle's bf16 rounding.

Stochastic rounding must be unbiased and leave bf16-representable values alone
("Stochastic rounding support for 8-bit optimizers", feature request: round up
or down with a chance set by the rounding error).  Round-to-nearest-even is
pinned against torch's float32 -> bfloat16 conversion (a library routine).
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import philox
from oracle.rounding import bf16_to_f32, f32_to_bf16_rne, f32_to_bf16_sr

ALL_R = np.arange(1 << 16, dtype=np.uint32)


def _sample_values(rng, n):
    mags = 10.0 ** rng.uniform(-40, 38, n)
    x = (rng.choice([-1.0, 1.0], n) * mags).astype(np.float32)
    extra = np.array([1.0, -1.0, 0.0, 2.0 ** -149, -(2.0 ** -140), 3.0e38, -3.3e38,
                      np.float32(1.0) + np.float32(2.0 ** -20), 65504.0], dtype=np.float32)
    return np.concatenate([x, extra])


def test_sr_mean_over_all_random_words_is_exact():
    rng = np.random.default_rng(11)
    for x in _sample_values(rng, 60):
        out = f32_to_bf16_sr(np.full(ALL_R.size, x, dtype=np.float32), ALL_R)
        vals = bf16_to_f32(out).astype(np.float64)
        if not np.all(np.isfinite(vals)):
            # the top of the range may round to inf; check the probability instead
            lo_bits = int(np.float32(x).view(np.uint32)) & 0xFFFF
            assert int(np.sum(~np.isfinite(vals))) == lo_bits
            continue
        uniq, counts = np.unique(vals, return_counts=True)
        mean = sum(Fraction(float(v)) * int(c) for v, c in zip(uniq, counts)) / ALL_R.size
        assert mean == Fraction(float(x)), float(x)
        assert uniq.size <= 2


def test_sr_fixes_bf16_values_and_moves_at_most_one_step():
    rng = np.random.default_rng(12)
    b = rng.integers(0, 1 << 16, 4000).astype(np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]                        # finite patterns
    x = bf16_to_f32(b)
    for r in (0, 1, 0x7FFF, 0x8000, 0xFFFF):
        assert np.array_equal(f32_to_bf16_sr(x, np.full(x.size, r, np.uint32)), b)
    y = _sample_values(rng, 2000)
    y = y[np.abs(y) < 3e38]
    lo = f32_to_bf16_sr(y, np.zeros(y.size, np.uint32))     # truncation toward zero
    hi = f32_to_bf16_sr(y, np.full(y.size, 0xFFFF, np.uint32))
    assert np.all(np.abs(bf16_to_f32(lo)) <= np.abs(y))
    assert np.all(np.abs(bf16_to_f32(hi)) >= np.abs(y))
    steps = (hi.astype(np.int64) & 0x7FFF) - (lo.astype(np.int64) & 0x7FFF)
    assert np.all((steps == 0) | (steps == 1))


def test_sr_monte_carlo_with_the_real_generator():
    """Mean of SR(x) over 10^5 Philox draws is within 3 sigma of x."""
    n = 100_000
    idx = np.arange(n, dtype=np.uint64)
    for k, x in enumerate([np.float32(1.0 - 3e-4), np.float32(-0.0123457), np.float32(3.3e-20)]):
        r = philox.sr_bits(2024, 5, k, idx, philox.STREAM_PARAM)
        out = bf16_to_f32(f32_to_bf16_sr(np.full(n, x, np.float32), r)).astype(np.float64)
        lo = float(bf16_to_f32(f32_to_bf16_sr(np.array([x]), np.array([0], np.uint32)))[0])
        hi = float(bf16_to_f32(f32_to_bf16_sr(np.array([x]), np.array([0xFFFF], np.uint32)))[0])
        q = (float(x) - lo) / (hi - lo)
        sigma = abs(hi - lo) * np.sqrt(q * (1 - q) / n)
        assert abs(out.mean() - float(x)) <= 3 * sigma, (float(x), out.mean(), sigma)


def test_rne_matches_torch_conversion():
    rng = np.random.default_rng(13)
    x = _sample_values(rng, 200_000)
    # exact ties: low half exactly 0x8000 with odd and even upper halves
    ties = (rng.integers(0, 1 << 15, 2000).astype(np.uint32) << 16) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_rne(x), want)


def test_nan_becomes_quiet_nan_with_sign():
    nan_bits = np.array([0x7FC00000, 0xFFC00001, 0x7F800001, 0xFFFFFFFF], dtype=np.uint32)
    x = nan_bits.view(np.float32)
    for out in (f32_to_bf16_sr(x, np.full(4, 0xFFFF, np.uint32)), f32_to_bf16_rne(x)):
        assert out.tolist() == [0x7FC0, 0xFFC0, 0x7FC0, 0xFFC0]
