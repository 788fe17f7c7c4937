"""Pins of the oracle's Philox4x32-10 and of the stochastic-rounding bit layout.

The generator is compared with rocRAND's host-side philox4x32_10 engine
(a library routine, compiled here from its header for the CPU only).
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))
ROCRAND_HDR = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


def build_ref(dirpath):
    """Compile the rocRAND host reference into dirpath; None if the toolchain is missing."""
    if not os.path.exists(ROCRAND_HDR) or shutil.which("g++") is None:
        return None
    exe = os.path.join(str(dirpath), "philox_ref")
    subprocess.run(["g++", "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(HERE, "rocrand_philox_ref.cpp"), "-o", exe], check=True)

    def run(rows):
        text = "".join("%x %x %x %x %x\n" % r for r in rows)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [tuple(int(w, 16) for w in line.split()) for line in out.strip().splitlines()]
    return run


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    ref = build_ref(tmp_path_factory.mktemp("rr"))
    if ref is None:
        pytest.skip("rocRAND header or g++ not available")
    return ref


def check_philox(rocrand_ref, fn):
    rng = np.random.default_rng(7)
    rows = []
    # zeros, all-ones and random keys / counters, high bits in every word
    rows.append((0, 0, 0, 0, 0))
    rows.append((0xFFFFFFFFFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF))
    for _ in range(200):
        key = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        c = [int(x) for x in rng.integers(0, 2**32, 4, dtype=np.uint64)]
        rows.append((key, *c))
    ref = rocrand_ref(rows)
    for (key, c0, c1, c2, c3), want in zip(rows, ref):
        got = fn([c0], [c1], [c2], [c3], key & 0xFFFFFFFF, key >> 32)
        assert tuple(int(x[0]) for x in got) == want, (hex(key), c0, c1, c2, c3)


def test_philox_matches_rocrand(rocrand_ref):
    check_philox(rocrand_ref, philox.philox4x32_10)


def test_sr_bits_layout_against_rocrand(rocrand_ref):
    """Element i takes 16-bit half (i%8)&1 of word (i%8)>>1 of the block for i//8."""
    seed, step, tid = 0x0123456789ABCDEF, 77, 5
    base = (1 << 33) * 8 + 16          # group index above 2^32 exercises counter word 1
    for stream in (0, 1, 2):
        idx = np.arange(base, base + 24, dtype=np.uint64)
        bits = philox.sr_bits(seed, step, tid, idx, stream)
        rows = []
        for grp in range(base // 8, base // 8 + 3):
            rows.append((seed, grp & 0xFFFFFFFF, (grp >> 32) | (stream << 30), step, tid))
        words = rocrand_ref(rows)
        want = []
        for w4 in words:
            for j in range(8):
                want.append((w4[j >> 1] >> (16 * (j & 1))) & 0xFFFF)
        assert bits.tolist() == want


def test_sr_bits_streams_and_steps_differ():
    idx = np.arange(4096, dtype=np.uint64)
    a = philox.sr_bits(1, 1, 0, idx, 0)
    assert not np.array_equal(a, philox.sr_bits(1, 1, 0, idx, 1))
    assert not np.array_equal(a, philox.sr_bits(1, 2, 0, idx, 0))
    assert not np.array_equal(a, philox.sr_bits(1, 1, 1, idx, 0))
    assert not np.array_equal(a, philox.sr_bits(2, 1, 0, idx, 0))
    assert np.array_equal(a, philox.sr_bits(1, 1, 0, idx, 0))


def test_sr_bits_uniform_chi2():
    """16-bit words are uniform: chi-square over 256 bins of the top byte."""
    idx = np.arange(1 << 18, dtype=np.uint64)
    bits = philox.sr_bits(99, 3, 11, idx, 0)
    assert bits.max() <= 0xFFFF
    counts = np.bincount((bits >> 8).astype(np.int64), minlength=256)
    exp = idx.size / 256
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    # 255 degrees of freedom: mean 255, sd ~22.6; 6 sd either side
    assert 120 < chi2 < 390, chi2
    low = np.bincount((bits & 0xFF).astype(np.int64), minlength=256)
    chi2l = float(((low - exp) ** 2 / exp).sum())
    assert 120 < chi2l < 390, chi2l
