"""Exact ties of the requantisation, on the GPU.

Rounding a normalised moment to a code ("8-bit Optimizers via Block-wise
Quantization", method bullets: the 8-bit index is found by binary search in
the codebook) has one boundary case random inputs never reach: a value that
lands exactly on the midpoint of two neighbouring entries.  The reading both
sides implement sends it to the LOWER code.  With stochastic rounding of the
state the boundary is f == r (the value's position in its gap, in units of
2^-16, equal to the element's random draw), which also keeps the lower entry.

The inputs are built on the host so that these ties happen on purpose:
beta1 = beta2 = 1/2 and a block absmax of exactly 1.0 (the first element of
every block is g = 1 with codes 255, so max|m2| = max v2 = 1 and the
normalised value is the moment itself), and each other element takes a state
code q and a bf16 gradient g with

    m2 = fl(fl(S[q]/2) + fl(g/2))          equal to a signed midpoint, or
    v2 = fl(fl(U[q]/2) + fl(g*g/2))        equal to an unsigned midpoint,

found by exhaustive search over q and every bf16 g in [-1, 1].  182 of the
255 signed and 140 of the 255 unsigned midpoints are reachable this way.  For
stochastic state rounding, the elements whose random draw (known from the
oracle's Philox) equals an integer-valued f that some (q, g) produces get that
(q, g).  The GPU must give the lower code at every tie, with no allowance,
and equal the oracle everywhere, on the fast path (LUT + one midpoint
comparison) and on the plain path (binary search; eps below 2^-60 sends every
block there), in full blocks and in a partial last block.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DevTensorSet, gpu_step, log
from oracle import codebook, philox, state_sr
from precision_optimizer_step_amd import opt8

pytestmark = pytest.mark.gpu

F32 = np.float32
HALF = F32(0.5)
EPS_FAST = 1e-8
EPS_PLAIN = 2.0 ** -62          # below the fast sequences' eps range: every block takes the plain path
TINY = F32(2.0 ** -80)          # keeps every non-zero moment inside the fast path's range


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


def _bf16_grid():
    """Every non-negative bf16 value up to 1.0 (as float32), and the signed set."""
    bits = np.arange(0x0000, 0x3F81, dtype=np.uint32)
    pos = (bits << 16).view(np.float32)
    pos = pos[(pos == 0) | (pos >= TINY)]
    return pos, np.concatenate([pos, -pos[1:]])


def _moments(table, q, g, squared):
    x = (g * g).astype(np.float32) if squared else g
    return (F32(HALF * table[q]) + (HALF * x).astype(np.float32)).astype(np.float32)


@functools.lru_cache(maxsize=None)
def midpoint_hits(signed: bool, per_mid: int = 6):
    """{k: [(q, g), ...]}: state code q and gradient g whose moment is exactly midpoint k."""
    s, ms, u, mu = codebook.tables()
    table, mid = (s, ms) if signed else (u, mu)
    pos, both = _bf16_grid()
    grid = both if signed else pos
    found = {}
    for q in range(256):
        n = _moments(table, q, grid, not signed)
        hit = np.isin(n.view(np.uint32), mid.view(np.uint32))
        for g, x in zip(grid[hit], n[hit]):
            k = int(np.searchsorted(mid, x))
            assert mid[k] == x
            lst = found.setdefault(k, [])
            if len(lst) < per_mid:
                lst.append((q, float(g)))
    return found


@functools.lru_cache(maxsize=None)
def sr_tie_cover(signed: bool):
    """{r: (q, g)} for every integer r in [1, 65535] that f = fl(fl(n - C[k]) W[k]) reaches."""
    s, _, u, _ = codebook.tables()
    table = s if signed else u
    w = state_sr.gap_weights(table)
    pos, both = _bf16_grid()
    grid = both if signed else pos
    cover = {}
    for q in range(256):
        n = _moments(table, q, grid, not signed)
        k = np.clip(np.searchsorted(table, n, side="right").astype(np.int64) - 1, 0, 254)
        f = ((n - table[k]).astype(np.float32) * w[k]).astype(np.float32)
        ok = (f == np.floor(f)) & (f >= 1) & (f < 65536)
        for fv, g in zip(f[ok].astype(np.int64), grid[ok]):
            cover.setdefault(int(fv), (q, float(g)))
    return cover


def _to_bf16(g):
    b = np.asarray(g, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "gradients must be bf16 values"
    return (b >> 16).astype(np.uint16)


def _assemble(items, n_total=None):
    """Lay (qm, qv, g) items out in blocks of 2048 whose first element is the max element."""
    body = list(items)
    qm, qv, g = [], [], []
    while body or (n_total is not None and len(g) < n_total):
        if len(g) % oracle.BLOCK == 0:
            qm.append(255)
            qv.append(255)
            g.append(1.0)
            continue
        x = body.pop(0) if body else (127, 255, 0.25)
        qm.append(x[0])
        qv.append(x[1])
        g.append(x[2])
        if n_total is not None and len(g) >= n_total:
            break
    n = len(g)
    nb = (n + oracle.BLOCK - 1) // oracle.BLOCK
    return (np.array(qm, np.uint8), np.array(qv, np.uint8), _to_bf16(np.array(g, np.float32)),
            np.ones(nb, np.float32), np.ones(nb, np.float32))


def _param(n, seed):
    rng = np.random.default_rng(seed)
    from workloads import gen
    return gen.to_bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))


def _run(qm, qv, g, am, av, hp, tensor_id, algo=0):
    p = _param(g.size, 11 + tensor_id)
    s = DevTensorSet(oracle.MODE_8BIT, p, g, qm.copy(), None if algo else qv.copy(), am.copy(),
                     None if algo else av.copy(), tensor_id=tensor_id)
    gpu_step([s], hp, algo)
    got = s.read()
    if algo:
        want = oracle.step_tensor_1state(algo, oracle.MODE_8BIT, p, g, qm, am, hp, tensor_id)
        want = [want[0], want[1], None, want[2], None]
    else:
        want = oracle.step_tensor(oracle.MODE_8BIT, p, g, qm, qv, am, av, hp, tensor_id)
    return got, want


def _exact(name, got, want):
    for part, x, y in zip(("param", "m", "v", "absmax_m", "absmax_v"), got, want):
        if y is None:
            continue
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)), \
            f"{name}: {part} differs from the oracle at {np.flatnonzero(np.asarray(x) != np.asarray(y))[:5]}"


@pytest.mark.parametrize("path", ["fast", "plain"])
def test_midpoint_ties_take_the_lower_code(path):
    hs, hu = midpoint_hits(True), midpoint_hits(False)
    assert len(hs) >= 150 and len(hu) >= 120
    items, expect = [], []
    for k, lst in sorted(hs.items()):
        for q, g in lst:
            items.append((q, 255, g))         # v2 = (1 + g^2)/2 stays in the fast range
            expect.append(("m", k))
    for k, lst in sorted(hu.items()):
        for q, g in lst:
            items.append((127, q, g))         # m2 = g/2
            expect.append(("v", k))
    order = np.random.default_rng(3).permutation(len(items))
    items3 = [items[i] for i in order] * 3      # three copies: full blocks and a partial last block
    exp3 = [expect[i] for i in order] * 3
    qm, qv, g, am, av = _assemble(items3)
    assert g.size % oracle.BLOCK != 0
    eps = EPS_FAST if path == "fast" else EPS_PLAIN
    hp = oracle.Hparams(lr=1e-3, beta1=0.5, beta2=0.5, eps=eps, weight_decay=0.01, step=3, seed=5)
    # where each item landed: every block starts with one max element
    pos = [i for i in range(g.size) if i % oracle.BLOCK != 0][:len(items3)]
    s, ms, u, mu = codebook.tables()
    if path == "fast":    # every non-zero moment inside the fast path's range: no block leaves it
        m2 = _moments(s, qm, (g.astype(np.uint32) << 16).view(np.float32), False)
        v2 = _moments(u, qv, (g.astype(np.uint32) << 16).view(np.float32), True)
        nz = np.concatenate([np.abs(m2[m2 != 0]), v2[v2 != 0]])
        assert nz.min() >= F32(2.0 ** -88) and m2.max() == 1 and v2.max() == 1
    got, want = _run(qm, qv, g, am, av, hp, tensor_id=7)
    _exact(f"ties/{path}", got, want)
    gm, gv = got[1], got[2]
    for i, (which, k) in zip(pos, exp3):
        c = int(gm[i] if which == "m" else gv[i])
        assert c == k, f"{path}: element {i} on {which} midpoint {k} got code {c} (lower code is {k})"
    log(f"ties/{path}: {sum(1 for e in exp3 if e[0] == 'm')} signed and "
        f"{sum(1 for e in exp3 if e[0] == 'v')} unsigned exact midpoints, all on the lower code")


@pytest.mark.parametrize("path", ["fast", "plain"])
def test_stochastic_state_ties_keep_the_lower_entry(path):
    """state_round = 1: where f == r exactly, the code stays k (the comparison is f > r)."""
    step, seed, n = 4, 77, 32 * oracle.BLOCK + 100
    cs, cu = sr_tie_cover(True), sr_tie_cover(False)
    assert len(cs) > 1500 and len(cu) > 250
    s, _, u, _ = codebook.tables()
    results = {}
    for which, tid, cover in (("m", 3, cs), ("v", 4, cu)):
        r16 = philox.sr_bits(seed, step, tid, np.arange(n, dtype=np.uint64), 1 if which == "m" else 2)
        qm = np.full(n, 127, np.uint8)
        qv = np.full(n, 255, np.uint8)
        gf = np.full(n, 0.25, np.float32)
        ties = []
        for i in range(n):
            if i % oracle.BLOCK == 0:
                qm[i], qv[i], gf[i] = 255, 255, 1.0
                continue
            hit = cover.get(int(r16[i]))
            if hit is not None:
                if which == "m":
                    qm[i], gf[i] = hit[0], hit[1]
                else:
                    qm[i], qv[i], gf[i] = 127, hit[0], hit[1]
                ties.append(i)
        g = _to_bf16(gf)
        am = np.ones((n + 2047) // 2048, np.float32)
        av = am.copy()
        eps = EPS_FAST if path == "fast" else EPS_PLAIN
        hp = oracle.Hparams(lr=1e-3, beta1=0.5, beta2=0.5, eps=eps, weight_decay=0.01, step=step, seed=seed,
                            state_round=1)
        got, want = _run(qm, qv, g, am, av, hp, tensor_id=tid)
        _exact(f"sr-ties/{path}/{which}", got, want)
        table = s if which == "m" else u
        x = _moments(table, qm if which == "m" else qv, gf, which == "v")
        k = np.clip(np.searchsorted(table, x, side="right").astype(np.int64) - 1, 0, 254)
        codes = got[1] if which == "m" else got[2]
        bad = [i for i in ties if int(codes[i]) != int(k[i])]
        assert not bad, f"{path}/{which}: f == r at {bad[:5]} moved up"
        results[which] = len(ties)
    assert results["m"] > 500 and results["v"] > 50
    log(f"sr-ties/{path}: {results['m']} signed and {results['v']} unsigned exact f == r ties kept the lower entry")


def test_lion_midpoint_ties_take_the_lower_code():
    """Lion's moment with beta2 = 1/2 is the same construction (m2 = S[q]/2 + g/2)."""
    hs = midpoint_hits(True)
    items, expect = [], []
    for k, lst in sorted(hs.items()):
        for q, g in lst:
            items.append((q, 255, g))
            expect.append(k)
    qm, qv, g, am, av = _assemble(items * 2)
    hp = oracle.Hparams(lr=1e-4, beta1=0.9, beta2=0.5, weight_decay=0.01, step=2, seed=6)
    got, want = _run(qm, qv, g, am, av, hp, tensor_id=9, algo=oracle.ALGO_LION)
    _exact("lion-ties", got, want)
    pos = [i for i in range(g.size) if i % oracle.BLOCK != 0][:len(items) * 2]
    for i, k in zip(pos, expect * 2):
        assert int(got[1][i]) == k
