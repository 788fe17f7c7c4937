"""bf16 decode, stochastic rounding and round-to-nearest-even (oracle).

TEST INFRASTRUCTURE ONLY (see the package header).

bf16 is carried as uint16: the upper half of an fp32 bit pattern, so decoding
is exact (shift left by 16).

Stochastic rounding ("Stochastic rounding support for 8-bit optimizers",
feature request: round up or down with a chance set by the rounding error).
Reading: add a uniform 16-bit random word r to the low half of the fp32 bit
pattern and keep the upper half.  With the low half equal to d, the result
moves one bf16 step away from zero exactly when d + r >= 2^16, i.e. with
probability d / 2^16, which is the distance to the lower-magnitude neighbour
in units of the bf16 step: the expected result equals the fp32 input.  Values
that bf16 represents (d = 0) never move.  NaN maps to the quiet NaN with the
input's sign.  Finite values at the very top of the range round to +-inf with
their correct probability.

Round-to-nearest-even is the deterministic baseline the bitsandbytes thread
asks SR to be compared with ("Stochastic rounding support for 8-bit
optimizers", comment proposing nearest vs stochastic rounding against a
higher-precision reference).

Parity: exhaustive mean over all 2^16 random words, bf16-representable
fixed points and a Monte-Carlo check are pinned by tests; round-to-nearest is
pinned against torch's own float32 -> bfloat16 conversion.
"""

import numpy as np

_HI = np.uint32(0xFFFF0000)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _nan_fix(x: np.ndarray, out: np.ndarray, bits: np.ndarray) -> np.ndarray:
    nan = np.isnan(x)
    if nan.any():
        sign = ((bits >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16)
        out = np.where(nan, np.uint16(0x7FC0) | sign, out)
    return out.astype(np.uint16)


def f32_to_bf16_sr(x: np.ndarray, r16: np.ndarray) -> np.ndarray:
    """Stochastic rounding of float32 to bf16 with 16-bit random words r16."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    r = np.asarray(r16, dtype=np.uint32) & np.uint32(0xFFFF)
    s = bits + r  # uint32 wrap-around; only NaN patterns can wrap
    out = ((s & _HI) >> np.uint32(16)).astype(np.uint16)
    return _nan_fix(x, out, bits)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16, ties to even."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    s = bits + np.uint32(0x7FFF) + lsb
    out = ((s & _HI) >> np.uint32(16)).astype(np.uint16)
    return _nan_fix(x, out, bits)
