"""Pins of the oracle's one-state optimizers (Lion, SGD with momentum).

References: closed forms, the sign invariant of Lion, float64 trajectories,
and torch.optim.SGD (CPU fp32, a library routine) for momentum.
"""

import numpy as np
import pytest
import torch

from oracle.adamw import BLOCK, Hparams, MODE_8BIT, MODE_BF16_SR, MODE_FP32, ROUND_NEAREST
from oracle.onestate import (ALGO_LION, ALGO_MOMENTUM, host_scalars_1state, lion_update,
                             momentum_update, step_tensor_1state)
from oracle.rounding import bf16_to_f32
from workloads import gen


def bf16_rand(rng, n, sigma):
    return gen.to_bf16_bits((rng.standard_normal(n) * sigma).astype(np.float32))


def ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(np.maximum(x, np.float32(2.0 ** -126))).astype(np.float64)


def _lion64(p, grads, lr, b1, b2, wd):
    p = p.astype(np.float64).copy()
    m = np.zeros_like(p)
    for g in grads:
        g = g.astype(np.float64)
        c = b1 * m + (1 - b1) * g
        p = p - lr * wd * p - lr * np.sign(c)
        m = b2 * m + (1 - b2) * g
    return p


def _momentum64(p, grads, lr, b, wd):
    p = p.astype(np.float64).copy()
    m = np.zeros_like(p)
    for g in grads:
        m = b * m + g.astype(np.float64)
        p = p - lr * wd * p - lr * m
    return p


def test_lion_step1_closed_form():
    rng = np.random.default_rng(1)
    n = 5000
    p = bf16_to_f32(bf16_rand(rng, n, 0.02))
    g = bf16_to_f32(bf16_rand(rng, n, 1e-3))
    g[:7] = 0.0
    hp = Hparams(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.1, step=1)
    s = host_scalars_1state(hp)
    m2, pn = lion_update(p, g, np.zeros(n, np.float32), s)
    assert np.array_equal(m2, (s.w2 * g).astype(np.float32))
    want = p.astype(np.float64) * (1 - 1e-4 * 0.1) - 1e-4 * np.sign(g)
    assert np.all(np.abs(pn - want) <= 2 * ulp32(p) + 2 * ulp32(pn))
    # the step is exactly +-lr (or 0) away from the decayed parameter
    x = (p - s.lrwd * p).astype(np.float32)
    step = (x.astype(np.float64) - pn)
    nz = g != 0
    tol = ulp32(np.maximum(np.abs(x), np.abs(pn)))
    assert np.all(np.abs(np.abs(step[nz]) - float(s.lr)) <= tol[nz])
    assert np.array_equal(pn[~nz], x[~nz])


def test_lion_uses_the_old_moment_for_the_direction():
    """Step 2 with m1 and g of opposite sign: c and m2 can have different signs, and a
    direction formed from the NEW moment would flip the last pair."""
    s = host_scalars_1state(Hparams(lr=1e-3, beta1=0.9, beta2=0.99, step=2))
    p = np.zeros(4, np.float32)
    m1 = np.array([1.0, -1.0, 1.0, -1.0], np.float32)
    g = np.array([-20.0, 20.0, -8.5, 8.5], np.float32)
    # c = 0.9 m1 + 0.1 g = (-1.1, 1.1, 0.05, -0.05); m2 = 0.99 m1 + 0.01 g keeps m1's sign;
    # 0.9 m2 + 0.1 g would be (.., .., -0.0355, 0.0355)
    m2, pn = lion_update(p, g, m1, s)
    assert np.array_equal(np.sign(m2), np.sign(m1))
    lr = np.float32(1e-3)
    assert np.array_equal(pn, np.array([lr, -lr, -lr, lr], np.float32))


@pytest.mark.parametrize("wd", [0.0])
def test_momentum_matches_torch_sgd(wd):
    rng = np.random.default_rng(2)
    n = 4000
    p = bf16_to_f32(bf16_rand(rng, n, 0.02))
    m1 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g = bf16_to_f32(bf16_rand(rng, n, 1e-3))
    hp = Hparams(lr=1e-2, beta1=0.9, weight_decay=wd, step=3)
    m2, pn = momentum_update(p, g, m1, host_scalars_1state(hp))
    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.SGD([tp], lr=1e-2, momentum=0.9, dampening=0.0, weight_decay=0.0,
                          foreach=False)
    opt.state[tp]["momentum_buffer"] = torch.from_numpy(m1.copy())
    tp.grad = torch.from_numpy(g.copy())
    opt.step()
    tm = opt.state[tp]["momentum_buffer"].numpy().astype(np.float64)
    tpn = tp.detach().numpy().astype(np.float64)
    assert np.all(np.abs(m2 - tm) <= 2 * ulp32(np.maximum(np.abs(0.9 * m1), np.abs(g))))
    assert np.all(np.abs(pn - tpn) <= 2 * ulp32(p) + 1e-2 * 4 * ulp32(m2))


def test_momentum_decoupled_decay_and_zero_gradient():
    s = host_scalars_1state(Hparams(lr=1e-2, beta1=0.9, weight_decay=0.5, step=1))
    p = np.array([1.0, -2.0, 0.5], np.float32)
    m2, pn = momentum_update(p, np.zeros(3, np.float32), np.zeros(3, np.float32), s)
    assert not m2.any()
    assert np.array_equal(pn, (p - s.lrwd * p).astype(np.float32))


@pytest.mark.parametrize("algo", [ALGO_LION, ALGO_MOMENTUM])
@pytest.mark.parametrize("mode", [MODE_FP32, MODE_8BIT])
def test_trajectory_tracks_float64(algo, mode):
    rng = np.random.default_rng(3)
    n = 1 << 15
    p_bits = bf16_rand(rng, n, 0.02)
    grads = [bf16_rand(rng, n, 1e-3) for _ in range(12)]
    nb = n // BLOCK
    lr = 1e-4 if algo == ALGO_LION else 1e-1
    b1, b2, wd = 0.9, 0.99, 0.1
    m = np.full(n, 127, np.uint8) if mode == MODE_8BIT else np.zeros(n, np.float32)
    am = np.zeros(nb, np.float32) if mode == MODE_8BIT else None
    p = p_bits
    for t, g in enumerate(grads, start=1):
        hp = Hparams(lr=lr, beta1=b1, beta2=b2, weight_decay=wd, step=t, seed=5)
        p, m, am = step_tensor_1state(algo, mode, p, g, m, am, hp, tensor_id=0)
    gf = [bf16_to_f32(g) for g in grads]
    p0 = bf16_to_f32(p_bits)
    ref = _lion64(p0, gf, lr, b1, b2, wd) if algo == ALGO_LION else _momentum64(p0, gf, lr, b1, wd)
    got = bf16_to_f32(p).astype(np.float64)
    moved = np.abs(ref - p0).mean()
    err = got - ref
    assert np.sqrt(np.mean(err ** 2)) < (0.25 if mode == MODE_8BIT else 0.05) * moved + 2e-4
    assert abs(err.mean()) < 0.02 * moved + 2e-6


@pytest.mark.parametrize("algo", [ALGO_LION, ALGO_MOMENTUM])
@pytest.mark.parametrize("mode", [MODE_8BIT, MODE_BF16_SR, MODE_FP32])
def test_shard_equivalence_and_zero_lr(algo, mode):
    rng = np.random.default_rng(4)
    n = BLOCK * 3 + 77
    p = bf16_rand(rng, n, 0.02)
    g = bf16_rand(rng, n, 1e-3)
    if mode == MODE_8BIT:
        m, _, am, _ = gen.random_state_8bit(3, 0, n)
    elif mode == MODE_BF16_SR:
        m, am = gen.random_state_bf16(3, 0, n)[0], None
    else:
        m, am = gen.random_state_f32(3, 0, n)[0], None
    hp = Hparams(lr=1e-3, beta1=0.9, beta2=0.99, weight_decay=0.1, step=4, seed=9)
    whole = step_tensor_1state(algo, mode, p, g, m, am, hp, 3)
    cut = 2 * BLOCK
    a = step_tensor_1state(algo, mode, p[:cut], g[:cut], m[:cut], None if am is None else am[:2], hp, 3, 0)
    b = step_tensor_1state(algo, mode, p[cut:], g[cut:], m[cut:], None if am is None else am[2:], hp, 3, cut)
    for k in range(2):
        assert np.array_equal(whole[k], np.concatenate([a[k], b[k]]))
    zero = Hparams(lr=0.0, beta1=0.9, beta2=0.99, weight_decay=0.0, step=4, seed=9)
    for rnd in (0, ROUND_NEAREST):
        zero.param_round = rnd
        out = step_tensor_1state(algo, mode, p, g, m, am, zero, 3)
        assert np.array_equal(out[0], p)
