"""GPU parity of the short last blocks.

A tensor whose last block holds at most 64 elements ("8-bit Optimizers via Block-wise
Quantization", method bullets: the last block of a tensor covers what is left of it) has that
block stepped by the short-block kernel, which packs eight such blocks into one wave (an
8-lane run each, the block maximum reduced within the run), under AdamW, Lion and SGD with
momentum.  A run that fails the fast path's check -- a non-finite value in its block, or (for
AdamW) hyperparameters outside the fast range for the whole launch -- has its block stepped
afterwards by the whole wave on the plain path, while the other runs of the wave keep their
fast results.  Every case here is compared with the oracle element by element, the mismatch
count required to be zero.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DevTensorSet, compare_state, gpu_step, log, oracle_step
from precision_optimizer_step_amd import opt8
from workloads import gen

pytestmark = pytest.mark.gpu

M8 = oracle.MODE_8BIT


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


def _bf16(rng, n, sigma):
    return gen.to_bf16_bits((rng.standard_normal(n) * sigma).astype(np.float32))


def _list(seed, lengths, zero_state=False, one_state=False):
    """One 8-bit tensor per tail length, with 0 or 1 full blocks before the tail (no second
    moment under the one-state rules)."""
    rng = np.random.default_rng(seed)
    sets, states = [], []
    for k, tail in enumerate(lengths):
        n = 2048 * (k % 2) + tail
        p, g = _bf16(rng, n, 0.02), _bf16(rng, n, 1e-3)
        if zero_state:
            nb = (n + 2047) // 2048
            m, v = np.full(n, 127, np.uint8), np.zeros(n, np.uint8)
            am, av = np.zeros(nb, np.float32), np.zeros(nb, np.float32)
        else:
            m, v, am, av = gen.random_state_8bit(seed, 40 + k, n)
        if one_state:
            v = av = None
        sets.append(DevTensorSet(M8, p, g, m, v, am, av, tensor_id=40 + k))
        states.append([p, m, v, am, av])
    return sets, states


def _step_and_compare(sets, states, hp, label, algo=0):
    gpu_step(sets, hp, algo)
    stats = {}
    for s, st in zip(sets, states):
        want = oracle_step(s, st, hp, algo)
        compare_state(f"{label}/t{s.tensor_id}", s.read(), want, M8, stats)
    mism = sum(stats.values())
    log(f"{label}: {len(sets)} tensors, mismatching elements {mism}")
    assert mism == 0


# every short length, the 65-element one that is not short, and a count of short blocks
# that leaves the last wave's runs partly empty (64 + 3 = 67 short blocks)
LENGTHS = list(range(1, 65)) + [65, 1, 7, 64]


@pytest.mark.parametrize("param_round,state_round", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_every_short_length(param_round, state_round):
    sets, states = _list(3 + param_round + 2 * state_round, LENGTHS)
    hp = oracle.Hparams(lr=1e-3, weight_decay=0.1, step=4, seed=1234, param_round=param_round,
                        state_round=state_round)
    _step_and_compare(sets, states, hp, f"short tails pr={param_round} sr={state_round}")


def test_zero_state_and_zero_gradients():
    """The zero state's first step, and blocks whose gradients are all zero (absmax 0 after
    the step: the zero code)."""
    sets, states = _list(11, LENGTHS, zero_state=True)
    for s in sets[::3]:
        s.set_grad(np.zeros_like(s.host[1]))
    hp = oracle.Hparams(lr=1e-3, weight_decay=0.01, step=1, seed=9)
    _step_and_compare(sets, states, hp, "short tails, zero state")


def test_non_finite_values_send_only_their_runs_to_the_plain_path():
    """A NaN gradient in one short block and an infinite one in another: those two runs take
    the plain path (NaN compared as NaN), every other run of the same waves keeps the fast
    path's result, all equal to the oracle's."""
    sets, states = _list(17, LENGTHS)
    bad = {5: 0x7FC0, 22: 0x7F80}   # tensor index -> gradient bits in its last block
    for k, bits in bad.items():
        g = sets[k].host[1].copy()
        g[-1] = bits
        sets[k].set_grad(g)
    hp = oracle.Hparams(lr=1e-3, weight_decay=0.01, step=3, seed=21)
    gpu_step(sets, hp)
    stats = {}
    for k, (s, st) in enumerate(zip(sets, states)):
        want = oracle_step(s, st, hp)
        got = s.read()
        if k not in bad:
            compare_state(f"t{s.tensor_id}", got, want, M8, stats)
            continue
        wp = oracle.rounding.bf16_to_f32(want[0])
        gp_ = oracle.rounding.bf16_to_f32(got[0])
        assert np.array_equal(np.isnan(wp), np.isnan(gp_))
        assert np.isnan(gp_).any(), "the non-finite gradient must reach the parameter"
        fin = ~np.isnan(wp)
        assert np.array_equal(got[0][fin], want[0][fin])
        for i in (1, 2):
            assert np.array_equal(got[i], want[i])
        for i in (3, 4):
            w, h = want[i], got[i]
            assert np.array_equal(np.isnan(w), np.isnan(h))
            assert np.array_equal(h[~np.isnan(w)], w[~np.isnan(w)])
    mism = sum(stats.values())
    log(f"short tails with non-finite gradients: mismatching elements elsewhere {mism}")
    assert mism == 0


def test_hyperparameters_outside_the_fast_range():
    """eps below 2^-60 switches the fast sequences off for the launch: every short block is
    stepped by the whole wave on the plain path."""
    sets, states = _list(29, LENGTHS)
    hp = oracle.Hparams(lr=1e-3, eps=1e-20, weight_decay=0.01, step=2, seed=3)
    _step_and_compare(sets, states, hp, "short tails, eps 1e-20")


@pytest.mark.parametrize("algo", [oracle.ALGO_LION, oracle.ALGO_MOMENTUM])
@pytest.mark.parametrize("param_round,state_round", [(0, 0), (1, 1)])
def test_one_state_rules(algo, param_round, state_round):
    sets, states = _list(41 + algo + param_round, LENGTHS, one_state=True)
    lr = 1e-4 if algo == oracle.ALGO_LION else 1e-3
    hp = oracle.Hparams(lr=lr, beta2=0.99 if algo == oracle.ALGO_LION else 0.999, weight_decay=0.01, step=3,
                        seed=77, param_round=param_round, state_round=state_round)
    _step_and_compare(sets, states, hp, f"short tails algo={algo} pr={param_round} sr={state_round}", algo)


@pytest.mark.parametrize("algo", [oracle.ALGO_LION, oracle.ALGO_MOMENTUM])
def test_one_state_non_finite_run(algo):
    """An infinite gradient in one short block: under Lion the parameter moves by lr at most
    and the moment becomes infinite (the run takes the plain path); the other runs keep the
    fast path; everything equals the oracle (NaN compared as NaN)."""
    sets, states = _list(53 + algo, LENGTHS, one_state=True)
    g = sets[9].host[1].copy()
    g[-1] = 0x7F80
    sets[9].set_grad(g)
    hp = oracle.Hparams(lr=1e-4, beta2=0.99, weight_decay=0.01, step=2, seed=3)
    gpu_step(sets, hp, algo)
    stats = {}
    for k, (s, st) in enumerate(zip(sets, states)):
        want = oracle_step(s, st, hp, algo)
        got = s.read()
        if k != 9:
            compare_state(f"t{s.tensor_id}", got, want, M8, stats)
            continue
        wp = oracle.rounding.bf16_to_f32(want[0])
        gp_ = oracle.rounding.bf16_to_f32(got[0])
        assert np.array_equal(np.isnan(wp), np.isnan(gp_))
        fin = ~np.isnan(wp)
        assert np.array_equal(got[0][fin], want[0][fin])
        assert np.array_equal(got[1], want[1])
        w, h = want[3], got[3]
        assert np.array_equal(np.isnan(w), np.isnan(h))
        assert np.array_equal(h[~np.isnan(w)], w[~np.isnan(w)])
    mism = sum(stats.values())
    log(f"one-state short tails with an infinite gradient (algo {algo}): mismatching elements elsewhere {mism}")
    assert mism == 0
