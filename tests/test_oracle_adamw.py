"""Pins of the oracle's AdamW step (host scalars, fp32 update, modes, rounding).

Independent references used here: torch.optim.AdamW on CPU fp32 (a library
routine), closed forms at step 1, a float64 AdamW trajectory, and invariants
(zero lr and wd, shard equivalence, stalled nearest rounding vs stochastic
rounding under decoupled weight decay).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import codebook
from oracle.adamw import (BLOCK, Hparams, MODE_8BIT, MODE_BF16_SR, MODE_FP32, ROUND_NEAREST,
                          adamw_param_update, host_scalars, step_tensor)
from oracle.rounding import bf16_to_f32
from workloads import gen, shapes

S, MS, U, MU = codebook.tables()


def ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(np.maximum(x, np.float32(2.0 ** -126))).astype(np.float64)


def bf16_rand(rng, n, sigma):
    return gen.to_bf16_bits((rng.standard_normal(n) * sigma).astype(np.float32))


# ----------------------------------------------------------------------------- scalars
@pytest.mark.parametrize("t", [1, 2, 3, 10, 1000, 50_000])
def test_host_scalars_against_pow(t):
    hp = Hparams(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=t)
    s = host_scalars(hp)
    bc1 = 1 - 0.9 ** t
    bc2 = 1 - 0.999 ** t
    for got, want in ((s.step_size, 3e-4 / bc1), (s.rbc2, 1 / math.sqrt(bc2))):
        assert got.dtype == np.float32
        assert abs(float(got) - want) <= float(ulp32(want)), (t, float(got), want)
    assert s.w1 == np.float32(0.1) and s.w2 == np.float32(1 - 0.999)
    assert s.lrwd == np.float32(3e-4 * 0.1)
    if t == 1:
        assert s.step_size == np.float32(3e-4 / (1 - 0.9))


# ----------------------------------------------------------------------------- fp32 update
@pytest.mark.parametrize("t,eps,wd", [(1, 1e-8, 0.01), (4, 1e-8, 0.1), (7, 1e-3, 0.0), (30, 1e-6, 0.5)])
def test_fp32_update_matches_torch_adamw(t, eps, wd):
    rng = np.random.default_rng(100 + t)
    n = 5000
    p_bits = bf16_rand(rng, n, 0.02)
    g_bits = bf16_rand(rng, n, 1e-3)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(n) * 1e-3) ** 2).astype(np.float32)
    v[:50] = 0.0
    lr = 1e-3
    hp = Hparams(lr=lr, beta1=0.9, beta2=0.999, eps=eps, weight_decay=wd, step=t)
    p = bf16_to_f32(p_bits)
    g = bf16_to_f32(g_bits)
    m2, v2, pn = adamw_param_update(p, g, m, v, host_scalars(hp))

    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(0.9, 0.999), eps=eps, weight_decay=wd,
                            foreach=False, fused=False)
    st = opt.state[tp]
    st["step"] = torch.tensor(float(t - 1))
    st["exp_avg"] = torch.from_numpy(m.copy())
    st["exp_avg_sq"] = torch.from_numpy(v.copy())
    tp.grad = torch.from_numpy(g.copy())
    opt.step()
    tm = st["exp_avg"].numpy().astype(np.float64)
    tv = st["exp_avg_sq"].numpy().astype(np.float64)
    tpn = tp.detach().numpy().astype(np.float64)

    tol_m = 4 * ulp32(np.maximum(np.abs(0.9 * m), np.abs(0.1 * g)))
    assert np.all(np.abs(m2 - tm) <= tol_m)
    assert np.all(np.abs(v2 - tv) <= 4 * ulp32(v2))
    s = host_scalars(hp)
    den = np.sqrt(v2.astype(np.float64)) * float(s.rbc2) + eps
    u = np.abs(m2.astype(np.float64)) / den
    tol_p = 4 * ulp32(p) + float(s.step_size) * (tol_m / den + u * 2.0 ** -20) + 2 * ulp32(pn)
    assert np.all(np.abs(pn - tpn) <= tol_p)


def test_step1_closed_form_from_zero_8bit_state():
    """At t=1 from zero state: m = (1-b1) g, v = (1-b2) g^2, p' = p(1-lr wd) - lr g/(|g|+eps)."""
    rng = np.random.default_rng(7)
    n = BLOCK * 2 + 100
    p_bits = bf16_rand(rng, n, 0.02)
    g_bits = bf16_rand(rng, n, 1e-3)
    g_bits[:10] = 0
    hp = Hparams(lr=1e-3, weight_decay=0.01, step=1, seed=5)
    s = host_scalars(hp)
    zq_m = np.full(n, 127, np.uint8)
    zq_v = np.zeros(n, np.uint8)
    za = np.zeros(2 + 1, np.float32)
    m1 = oracle.dequantize_blockwise(zq_m, za, S)
    v1 = oracle.dequantize_blockwise(zq_v, za, U)
    assert not m1.any() and not v1.any()
    p = bf16_to_f32(p_bits)
    g = bf16_to_f32(g_bits)
    m2, v2, pn = adamw_param_update(p, g, m1, v1, s)
    assert np.array_equal(m2, (s.w1 * g).astype(np.float32))
    assert np.array_equal(v2, (s.w2 * (g * g)).astype(np.float32))
    g64 = g.astype(np.float64)
    want = p.astype(np.float64) * (1 - 1e-3 * 0.01) - 1e-3 * g64 / (np.abs(g64) + 1e-8)
    assert np.all(np.abs(pn - want) <= 4 * ulp32(p) + 1e-3 * 1e-5 + 2 * ulp32(pn))
    # the whole step: the bf16 write lands on a neighbour of the fp32 value
    out = step_tensor(MODE_8BIT, p_bits, g_bits, zq_m, zq_v, za, za, hp, tensor_id=3)
    q = bf16_to_f32(out[0]).astype(np.float64)
    bf16_step = np.spacing(np.abs(pn)).astype(np.float64) * 65536
    assert np.all(np.abs(q - pn) < bf16_step)


@pytest.mark.parametrize("mode", [MODE_8BIT, MODE_BF16_SR, MODE_FP32])
def test_zero_lr_and_wd_leave_params_untouched(mode):
    rng = np.random.default_rng(9)
    n = BLOCK * 2 + 777
    p_bits = bf16_rand(rng, n, 0.02)
    g_bits = bf16_rand(rng, n, 1e-3)
    if mode == MODE_8BIT:
        m, v, am, av = gen.random_state_8bit(1, 0, n)
    elif mode == MODE_BF16_SR:
        (m, v), am, av = gen.random_state_bf16(1, 0, n), None, None
    else:
        (m, v), am, av = gen.random_state_f32(1, 0, n), None, None
    for rnd in (0, ROUND_NEAREST):
        hp = Hparams(lr=0.0, weight_decay=0.0, step=3, seed=11, param_round=rnd)
        out = step_tensor(mode, p_bits, g_bits, m, v, am, av, hp, tensor_id=2)
        assert np.array_equal(out[0], p_bits)
        assert not np.array_equal(out[1], m)          # the moments still move


# ----------------------------------------------------------------------------- trajectories
def _float64_adamw(p, grads, lr, b1, b2, eps, wd):
    """Textbook AdamW in float64; returns (final params, path length sum |step|, max |p|)."""
    p = p.astype(np.float64).copy()
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    path = np.zeros_like(p)
    top = np.abs(p)
    for t, g in enumerate(grads, start=1):
        g = g.astype(np.float64)
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * g * g
        mh = m / (1 - b1 ** t)
        vh = v / (1 - b2 ** t)
        new = p - lr * wd * p - lr * mh / (np.sqrt(vh) + eps)
        path += np.abs(new - p)
        p = new
        top = np.maximum(top, np.abs(p))
    return p, path, top


@pytest.mark.parametrize("mode", [MODE_8BIT, MODE_FP32, MODE_BF16_SR])
def test_accumulated_updates_track_float64_adamw(mode):
    """Ten steps on a 64K tensor: error vs a float64 AdamW stays at the rounding scale, unbiased."""
    w = shapes.single_tensor()
    rng = np.random.default_rng(21)
    n = 1 << 16
    p_bits = bf16_rand(rng, n, 0.02)
    grads = [gen.to_bf16_bits(gen.grad_values(w, t, 0)[:n]) for t in range(1, 11)]
    nb = (n + BLOCK - 1) // BLOCK
    if mode == MODE_8BIT:
        m, v, am, av = np.full(n, 127, np.uint8), np.zeros(n, np.uint8), \
            np.zeros(nb, np.float32), np.zeros(nb, np.float32)
    elif mode == MODE_FP32:
        m, v, am, av = np.zeros(n, np.float32), np.zeros(n, np.float32), None, None
    else:
        m, v, am, av = np.zeros(n, np.uint16), np.zeros(n, np.uint16), None, None
    p = p_bits
    for t in range(1, 11):
        hp = Hparams(lr=1e-3, weight_decay=0.01, step=t, seed=0)
        p, m, v, am, av = step_tensor(mode, p, grads[t - 1], m, v, am, av, hp, tensor_id=0)
    ref, path, top = _float64_adamw(bf16_to_f32(p_bits), [bf16_to_f32(g) for g in grads],
                                    1e-3, 0.9, 0.999, 1e-8, 0.01)
    got = bf16_to_f32(p).astype(np.float64)
    err = got - ref
    ulp_bf16 = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) * 65536
    ulp_top = np.spacing(top.astype(np.float32)).astype(np.float64) * 65536
    # per element: a few bf16 steps of SR noise at the largest magnitude visited, plus a
    # fraction of the path length for the state's own rounding.  8-bit state next to a
    # x100 outlier loses small moments entirely, so its worst case is a whole path length.
    excess = (np.abs(err) - 6 * ulp_top) / path
    if mode == MODE_8BIT:
        assert np.quantile(excess, 0.999) <= 0.2 and excess.max() <= 1.5
    else:
        assert excess.max() <= 0.02
    # unbiased on average: mean error well below one bf16 step of a typical element
    assert abs(err.mean()) < (0.05 if mode == MODE_8BIT else 0.02) * np.median(ulp_bf16)
    assert np.median(np.abs(err)) < (3.0 if mode == MODE_8BIT else 1.0) * np.median(ulp_bf16)


def test_decay_survives_with_sr_and_stalls_with_nearest():
    """LayerNorm-like weights at 1.0, zero grads: decay lr*wd*p << bf16 step.

    Nearest rounding never moves; stochastic rounding follows (1 - lr wd)^t on average.
    """
    n = 8192
    p0 = np.full(n, 0x3F80, np.uint16)        # 1.0
    g = np.zeros(n, np.uint16)
    lr, wd, T = 1e-3, 0.1, 300
    res = {}
    for rnd in (0, ROUND_NEAREST):
        p, m, v = p0, np.zeros(n, np.float32), np.zeros(n, np.float32)
        for t in range(1, T + 1):
            hp = Hparams(lr=lr, weight_decay=wd, step=t, seed=3, param_round=rnd)
            p, m, v, _, _ = step_tensor(MODE_FP32, p, g, m, v, None, None, hp, tensor_id=1)
        res[rnd] = bf16_to_f32(p).astype(np.float64)
    assert np.all(res[ROUND_NEAREST] == 1.0)
    want = (1 - lr * wd) ** T
    got = res[0].mean()
    sd = math.sqrt(T) * (2.0 ** -8) / 2 / math.sqrt(n)
    assert abs(got - want) <= 4 * sd, (got, want, sd)


@pytest.mark.parametrize("mode", [MODE_8BIT, MODE_BF16_SR, MODE_FP32])
def test_shard_equivalence(mode):
    """Stepping a tensor whole equals stepping block-aligned shards with their global index base."""
    rng = np.random.default_rng(31)
    n = BLOCK * 3 + 1234
    p_bits = bf16_rand(rng, n, 0.02)
    g_bits = bf16_rand(rng, n, 1e-3)
    if mode == MODE_8BIT:
        m, v, am, av = gen.random_state_8bit(4, 0, n)
    elif mode == MODE_BF16_SR:
        (m, v), am, av = gen.random_state_bf16(4, 0, n), None, None
    else:
        (m, v), am, av = gen.random_state_f32(4, 0, n), None, None
    hp = Hparams(lr=1e-3, weight_decay=0.1, step=2, seed=77)
    whole = step_tensor(mode, p_bits, g_bits, m, v, am, av, hp, tensor_id=9)
    cut = 2 * BLOCK
    a = step_tensor(mode, p_bits[:cut], g_bits[:cut], m[:cut], v[:cut],
                    None if am is None else am[:2], None if av is None else av[:2], hp, 9, 0)
    b = step_tensor(mode, p_bits[cut:], g_bits[cut:], m[cut:], v[cut:],
                    None if am is None else am[2:], None if av is None else av[2:], hp, 9, cut)
    for k in range(3):
        assert np.array_equal(whole[k], np.concatenate([a[k], b[k]]))
    if mode == MODE_8BIT:
        assert np.array_equal(whole[3], np.concatenate([a[3], b[3]]))
        assert np.array_equal(whole[4], np.concatenate([a[4], b[4]]))


def test_bf16_state_writes_are_stochastic_neighbours():
    rng = np.random.default_rng(41)
    n = 20000
    p_bits = bf16_rand(rng, n, 0.02)
    g_bits = bf16_rand(rng, n, 1e-3)
    m, v = gen.random_state_bf16(6, 0, n)
    hp = Hparams(lr=1e-3, weight_decay=0.1, step=5, seed=8)
    s = host_scalars(hp)
    m2, v2, _ = adamw_param_update(bf16_to_f32(p_bits), bf16_to_f32(g_bits),
                                   bf16_to_f32(m), bf16_to_f32(v), s)
    out = step_tensor(MODE_BF16_SR, p_bits, g_bits, m, v, None, None, hp, tensor_id=4)
    for new, exact in ((out[1], m2), (out[2], v2)):
        got = bf16_to_f32(new).astype(np.float64)
        step = np.spacing(np.abs(exact)).astype(np.float64) * 65536
        assert np.all(np.abs(got - exact) < step)
        frac_up = np.mean(np.abs(got) > np.abs(exact))
        want_up = np.mean((exact.view(np.uint32) & 0xFFFF) / 65536.0)
        assert abs(frac_up - want_up) < 0.02
    assert np.all(bf16_to_f32(out[2]) >= 0)


def test_default_mode_threshold():
    assert oracle.default_mode(4095) == MODE_FP32
    assert oracle.default_mode(1) == MODE_FP32
    assert oracle.default_mode(4096) == MODE_8BIT
