"""Pins of the oracle's stochastic rounding of the 8-bit state between neighbouring entries.

References: the exact mean over every value of the 16 random bits, a float64
search for the neighbours, exact rational thresholds, and a decaying second
moment that nearest rounding freezes.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codebook
from oracle.adamw import BLOCK, Hparams, MODE_8BIT, step_tensor
from oracle.philox import sr_bits, STREAM_M
from oracle.state_sr import gap_weights, quantize_blockwise_sr, sr_codes
from workloads import gen

TABLES = {"signed": codebook.tables()[0], "unsigned": codebook.tables()[2]}
ALL_R = np.arange(65536, dtype=np.uint32)


def _samples(table, rng, n):
    """Normalised values over the table's range: uniform, log-spaced, exact entries, and
    the points just beside entries."""
    lo = float(table[0])
    u = rng.uniform(lo, 1.0, n).astype(np.float32)
    mag = (10.0 ** rng.uniform(-8, 0, n)).astype(np.float32)
    sgn = np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32) if lo < 0 else np.float32(1)
    ent = table.copy()
    near = np.concatenate([np.nextafter(table, np.float32(2)), np.nextafter(table, np.float32(-2))])
    x = np.concatenate([u, mag * sgn, ent, near]).astype(np.float32)
    return x[(x >= lo) & (x <= 1.0)]


@pytest.mark.parametrize("which", ["signed", "unsigned"])
def test_mean_over_all_random_words_is_the_value(which):
    """Averaged over all 65536 draws, the decoded entry equals n up to the 2^-16
    granularity of the gap and the rounding of f (a flipped comparison, a wrong gap
    weight or a wrong neighbour index would bias it by a whole fraction of a gap)."""
    table = TABLES[which]
    rng = np.random.default_rng(1)
    x = _samples(table, rng, 300)
    w = gap_weights(table)
    for n in x:
        codes = sr_codes(np.full(65536, n, np.float32), table, w, ALL_R)
        k = int(codes.min())
        assert codes.max() <= k + 1
        mean = float(np.mean(table[codes].astype(np.float64)))
        gap = float(table[min(k + 1, 255)]) - float(table[k])
        assert abs(mean - float(n)) <= gap * 2.0 ** -15 + abs(float(n)) * 2.0 ** -22, (n, k, mean)


@pytest.mark.parametrize("which", ["signed", "unsigned"])
def test_codes_are_the_two_neighbours_and_entries_stay(which):
    table = TABLES[which]
    t64 = table.astype(np.float64)
    rng = np.random.default_rng(2)
    x = _samples(table, rng, 5000)
    r = rng.integers(0, 65536, x.size).astype(np.uint32)
    codes = sr_codes(x, table, gap_weights(table), r).astype(np.int64)
    # float64 search: the entries at or around n
    k = np.array([max(0, min(254, int(np.searchsorted(t64, float(v), side="right")) - 1)) for v in x])
    assert np.all((codes == k) | (codes == k + 1))
    assert np.all(t64[codes] <= np.maximum(x.astype(np.float64), t64[k + 1]))
    # a value equal to an entry is stored as that entry whatever the draw, the draw 0 included
    ent = np.repeat(table, 64)
    rr = rng.integers(0, 65536, ent.size).astype(np.uint32)
    rr[::2] = 0
    assert np.array_equal(table[sr_codes(ent, table, gap_weights(table), rr)], ent)


def test_decision_matches_the_exact_rational_threshold():
    """Away from the threshold (|65536 P - r| > 1/4), up iff r < 65536 (n - C[k]) / (C[k+1] - C[k])
    computed exactly."""
    table = TABLES["signed"]
    rng = np.random.default_rng(3)
    x = _samples(table, rng, 3000)
    r = rng.integers(0, 65536, x.size).astype(np.uint32)
    codes = sr_codes(x, table, gap_weights(table), r).astype(np.int64)
    checked = 0
    for v, rv, c in zip(x, r, codes):
        k = max(0, min(254, int(np.searchsorted(table, v, side="right")) - 1))
        p = (Fraction(float(v)) - Fraction(float(table[k]))) / (Fraction(float(table[k + 1])) -
                                                                  Fraction(float(table[k])))
        t = 65536 * p
        if abs(t - int(rv)) <= Fraction(1, 4):
            continue
        assert (c == k + 1) == (int(rv) < t), (v, k, rv, float(t))
        checked += 1
    assert checked > 2900


def test_zero_block_non_finite_and_partial_tail():
    n = BLOCK * 3 + 100
    x = np.zeros(n, np.float32)
    x[BLOCK:] = np.float32(1e-3) * np.linspace(-1, 1, n - BLOCK, dtype=np.float32)
    x[BLOCK + 5] = np.nan      # NaN absmax: the block is not live, zero codes (as with nearest)
    x[2 * BLOCK + 7] = np.inf  # inf absmax: n = inf * 0 = NaN for that element (code 255), 0 elsewhere
    r = np.arange(n, dtype=np.uint32) & 0xFFFF
    codes, am = quantize_blockwise_sr(x, TABLES["signed"], codebook.SIGNED_ZERO_CODE, r)
    assert np.all(codes[:BLOCK] == codebook.SIGNED_ZERO_CODE)    # all-zero block, no draw
    assert am[0] == 0
    assert np.isnan(am[1]) and np.all(codes[BLOCK:2 * BLOCK] == codebook.SIGNED_ZERO_CODE)
    assert np.isinf(am[2]) and codes[2 * BLOCK + 7] == 255
    assert np.all(np.delete(codes[2 * BLOCK:3 * BLOCK], 7) == codebook.SIGNED_ZERO_CODE)
    assert am[3] == np.float32(np.max(np.abs(x[3 * BLOCK:])))     # tail: valid elements only


def test_unbiased_with_the_real_generator():
    """Monte-Carlo over 2^20 elements with Philox draws: the decoded block mean matches the
    fp32 values to within 4 standard deviations of the rounding noise."""
    table = TABLES["signed"]
    rng = np.random.default_rng(4)
    n = 1 << 20
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    r = sr_bits(7, 3, 11, np.arange(n, dtype=np.uint64), STREAM_M)
    codes, am = quantize_blockwise_sr(x, table, codebook.SIGNED_ZERO_CODE, r)
    dec = table[codes].astype(np.float64) * np.repeat(am.astype(np.float64), BLOCK)[:n]
    err = dec - x.astype(np.float64)
    # per element the error is a two-point variable within one gap: its sd is below gap / 2
    k = np.clip(np.searchsorted(table, x / np.repeat(am, BLOCK)[:n], side="right") - 1, 0, 254)
    gaps = (table[k + 1].astype(np.float64) - table[k]) * np.repeat(am, BLOCK)[:n]
    sd = np.sqrt(np.sum((gaps / 2) ** 2)) / n
    assert abs(err.mean()) < 4 * sd
    assert np.all(np.abs(err) <= gaps * (1 + 2.0 ** -20))


def test_decaying_second_moment_is_frozen_by_nearest_and_followed_by_stochastic():
    """v of an element with zero gradient decays by beta2 per step while the block absmax is
    held by an element with a steady large gradient: the relative change per step is far
    below half a code gap, so the nearest code never moves, while the stochastic code follows
    the decay on average."""
    n = BLOCK
    p = np.zeros(n, np.uint16)
    steps = 300
    hp0 = dict(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    g = np.zeros(n, np.float32)
    g[0] = 1.0
    g_bits = gen.to_bf16_bits(g)
    # start: v = 0.25 (of the absmax 1.0) everywhere but element 0
    cu = TABLES["unsigned"]
    code0 = int(np.argmin(np.abs(cu - 0.25)))
    results = {}
    for state_round in (0, 1):
        m = np.full(n, 127, np.uint8)
        v = np.full(n, code0, np.uint8)
        v[0] = 255
        am = np.zeros(1, np.float32)
        av = np.ones(1, np.float32)
        for t in range(1, steps + 1):
            hp = Hparams(step=t, seed=5, state_round=state_round, **hp0)
            _, m, v, am, av = step_tensor(MODE_8BIT, p, g_bits, m, v, am, av, hp, tensor_id=0)
        results[state_round] = cu[v[1:]].astype(np.float64) * float(av[0])
    # float64 reference of the decay (absmax: v of element 0 stays ~1 with g = 1)
    want = float(cu[code0]) * 0.999 ** steps
    assert np.all(results[0] == results[0][0]) and results[0][0] > 1.3 * want    # frozen
    assert abs(results[1].mean() - want) < 0.02 * want                            # followed
