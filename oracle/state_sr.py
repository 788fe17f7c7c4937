"""Stochastic rounding of the 8-bit state between neighbouring codebook entries (oracle).

TEST INFRASTRUCTURE ONLY (see the package header).

The pages suggest rounding the momenta stochastically as well as the
parameters ("[Feat]: Stochastic rounding of AdamW momentums", the comment
thread: fp32 arithmetic, the momenta cast back each step, possibly with
stochastic rounding); for bf16 momenta that is the bf16-state mode.  This
module carries the same idea to the 8-bit block-wise state: instead of the
nearest codebook entry, a normalised value n is stored as one of the two
entries around it, the upper one with a probability equal to the fraction of
the gap below n, so the decoded state is unbiased.  The pages do not define
it; the reading, shared with the library:

  * n = x * fp32(1 / absmax) exactly as for nearest rounding; a block whose
    absmax is below 2^-126 stores the zero code (no random draw).
  * k = (number of entries C[j] <= n) - 1, clamped to [0, 254]: the entry at
    or below n (the lowest entry for n below the table, the second highest
    for n at or above the top).
  * W[k] = fp32(65536 / (C[k+1] - C[k])), the difference and the quotient in
    double, rounded once to fp32 (W[255] = 0, unused).
  * f = fp32(fp32(n - C[k]) * W[k]), the position of n in the gap in units
    of 2^-16 of it.
  * the 16 random bits r of the element (the Philox slice of the parameter's
    stochastic rounding, on stream 1 for the first moment and 2 for the
    second) pick the upper entry iff f > r; code = k + 1 then, else k.
    P(upper) = min(ceil(f), 65536) / 65536 for f > 0, 0 for f <= 0.
  * n that is NaN stores code 255, as with nearest rounding.

Parity: pinned by the exact mean over all 65536 values of r (within the
2^-16 granularity of the gap and the rounding of f), by the neighbour
property against a float64 search, by exact entries never moving, by a
float64 rational comparison of the decision away from the threshold, and by
a decaying second moment that nearest rounding freezes and this rounding
follows on average.
"""

import numpy as np

from . import codebook
from .adamw import MIN_NORMAL_F32, _blocked, _f32

STATE_ROUND_NEAREST = 0
STATE_ROUND_STOCHASTIC = 1


def gap_weights(table: np.ndarray) -> np.ndarray:
    """W[k] = fp32(65536 / (C[k+1] - C[k])) in double, W[255] = 0."""
    c = np.asarray(table, dtype=np.float64)
    w = np.zeros(c.size, dtype=np.float32)
    w[:-1] = (65536.0 / (c[1:] - c[:-1])).astype(np.float32)
    return w


def sr_codes(n: np.ndarray, table: np.ndarray, weights: np.ndarray, r16: np.ndarray) -> np.ndarray:
    """Codes of normalised values n (fp32) with random 16-bit draws r16 (same shape)."""
    n = _f32(np.asarray(n, dtype=np.float32))
    count = np.searchsorted(table, n, side="right")          # #{C[j] <= n}; NaN -> 256
    k = np.clip(count.astype(np.int64) - 1, 0, table.size - 2)
    d = _f32(n - table[k])
    f = _f32(d * weights[k])
    up = f > np.asarray(r16, dtype=np.uint32).astype(np.float32)
    code = k + up.astype(np.int64)
    code = np.where(np.isnan(n), table.size - 1, code)
    return code.astype(np.uint8)


def quantize_blockwise_sr(x: np.ndarray, table: np.ndarray, zero_code: int, r16: np.ndarray):
    """Block absmax, normalise by fp32(1/absmax), stochastic code between neighbours.

    r16: uint32/uint16 random draws, one per element of x.  Returns (codes, absmax).
    """
    x = _f32(np.asarray(x, dtype=np.float32))
    rows = _blocked(x)
    rr = _blocked(np.asarray(r16, dtype=np.uint32))
    absmax = _f32(np.max(np.abs(rows), axis=1))
    codes = np.full(rows.shape, zero_code, dtype=np.uint8)
    live = absmax >= MIN_NORMAL_F32
    if live.any():
        inv = _f32(np.float32(1.0) / absmax[live])
        normed = _f32(rows[live] * inv[:, None])
        codes[live] = sr_codes(normed, table, gap_weights(table), rr[live])
    return codes.reshape(-1)[: x.size], absmax


def signed_table():
    return codebook.tables()[0]


def unsigned_table():
    return codebook.tables()[2]
