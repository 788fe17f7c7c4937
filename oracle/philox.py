"""Philox4x32-10 counter-based generator and the stochastic-rounding bit stream.

TEST INFRASTRUCTURE ONLY (see the package header).

Generator: Philox4x32 with 10 rounds, from J. K. Salmon, M. A. Moraes,
R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
A round multiplies counter words 0 and 2 by the two Philox multipliers, keeps
the 64-bit products, and produces

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0));

the key is bumped by the two Weyl constants before rounds 2..10.

Keying of the random bits that drive stochastic rounding.  The pages ask for
rounding up or down with a probability set by the rounding error ("Stochastic
rounding support for 8-bit optimizers", feature request) and for randomness
that all data-parallel replicas share ("Stochastic Rounding for LLM Training:
Theory and Practice", TL;DR: shared randomness in distributed settings).  The
reading used: the bits depend only on (seed, step, tensor id, global element
index, stream) and never on a rank or a launch shape.

  key     = (lo32(seed), hi32(seed))
  counter = (lo32(i // 8), hi32(i // 8) | stream << 30, lo32(step), tensor_id)
  element i uses the 16-bit half (i % 8) & 1 (low half first) of output word
  (i % 8) >> 1.
  streams: 0 = parameter, 1 = first moment, 2 = second moment.

Parity: the generator is pinned against rocRAND's host-side Philox4x32-10
(a library routine, test side only); the keying above is a definition of this
library (the pages fix none).
"""

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = 0xFFFFFFFF

STREAM_PARAM = 0
STREAM_M = 1
STREAM_V = 2


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox rounds over arrays of counter words; returns 4 uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = int(k0) & _MASK
    k1 = int(k1) & _MASK
    m0 = np.uint64(M0)
    m1 = np.uint64(M1)
    sh = np.uint64(32)
    lo = np.uint64(_MASK)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & _MASK
            k1 = (k1 + W1) & _MASK
        p0 = m0 * c0  # < 2^64: both factors < 2^32
        p1 = m1 * c2
        c0, c1, c2, c3 = (
            (p1 >> sh) ^ c1 ^ np.uint64(k0),
            p1 & lo,
            (p0 >> sh) ^ c3 ^ np.uint64(k1),
            p0 & lo,
        )
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def sr_bits(seed: int, step: int, tensor_id: int, index, stream: int) -> np.ndarray:
    """uint32[n] of 16-bit random words (0..65535), one per global element index."""
    index = np.asarray(index, dtype=np.uint64).reshape(-1)
    group = index >> np.uint64(3)
    # one Philox call per distinct group of 8 consecutive indices
    if index.size and np.array_equal(index, np.arange(int(index[0]), int(index[0]) + index.size,
                                                      dtype=np.uint64)):
        first = int(group[0])
        groups = np.arange(first, int(group[-1]) + 1, dtype=np.uint64)
        which = (group - np.uint64(first)).astype(np.int64)
    else:
        groups, which = np.unique(group, return_inverse=True)
    c0 = groups & np.uint64(_MASK)
    c1 = (groups >> np.uint64(32)) | np.uint64((stream & 3) << 30)
    c2 = np.full(groups.shape, step & _MASK, dtype=np.uint64)
    c3 = np.full(groups.shape, tensor_id & _MASK, dtype=np.uint64)
    words = np.stack(philox4x32_10(c0, c1, c2, c3, seed & _MASK, (seed >> 32) & _MASK))
    lane = (index & np.uint64(7)).astype(np.int64)
    word = words[lane >> 1, which]
    shift = ((lane & 1) * 16).astype(np.uint32)
    return (word >> shift) & np.uint32(0xFFFF)
