"""GPU parity of stochastic rounding of the 8-bit state (state_round = 1) against the oracle.

Every update rule, both parameter roundings, ragged lists mixing the three
state modes, a free-running tensor, degenerate and non-finite blocks, the
full 6.7B-shaped list on sampled blocks in one launch, and the decaying
second moment that nearest rounding freezes and this rounding follows.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (ALGO_ADAMW, DevTensorSet, build_list, compare_state, descriptors, gpu_step, log,
                         oracle_step, sample_blocks, snapshot, to_dev)
from precision_optimizer_step_amd import opt8
from workloads import gen, shapes

pytestmark = pytest.mark.gpu

M8, MB, MF = oracle.MODE_8BIT, oracle.MODE_BF16_SR, oracle.MODE_FP32
SS = oracle.STATE_ROUND_STOCHASTIC
ALGOS = [ALGO_ADAMW, oracle.ALGO_LION, oracle.ALGO_MOMENTUM]
NAMES = {ALGO_ADAMW: "adamw", oracle.ALGO_LION: "lion", oracle.ALGO_MOMENTUM: "momentum"}


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


def _hp(algo, step, seed=0xC0DE, param_round=oracle.ROUND_STOCHASTIC, lr=None, wd=0.1):
    if lr is None:
        lr = {ALGO_ADAMW: 1e-3, oracle.ALGO_LION: 1e-4, oracle.ALGO_MOMENTUM: 1e-2}[algo]
    return oracle.Hparams(lr=lr, beta1=0.9, beta2=0.99 if algo == oracle.ALGO_LION else 0.999, eps=1e-8,
                          weight_decay=wd, step=step, seed=seed, param_round=param_round, state_round=SS)


def _rand_bf16(rng, n, sigma):
    return gen.to_bf16_bits((rng.standard_normal(n) * sigma).astype(np.float32))


def _state(mode, n, seed, tid, two):
    if mode == M8:
        m, v, am, av = gen.random_state_8bit(seed, tid, n)
    elif mode == MB:
        (m, v), am, av = gen.random_state_bf16(seed, tid, n), None, None
    else:
        (m, v), am, av = gen.random_state_f32(seed, tid, n), None, None
    return (m, v, am, av) if two else (m, None, am, None)


def _step_compare(algo, sets, states, hp, label, stats):
    gpu_step(sets, hp, algo)
    nxt = []
    for s, st in zip(sets, states):
        want = oracle_step(s, st, hp, algo)
        compare_state(f"{label}/t{s.tensor_id}", s.read(), want, s.mode, stats)
        nxt.append(want)
    return nxt


def _force(sets, states):
    for s, (p, m, v, am, av) in zip(sets, states):
        s.P.copy_(to_dev(p))
        s.M.copy_(to_dev(m))
        if s.V is not None:
            s.V.copy_(to_dev(v))
        if s.AM is not None:
            s.AM.copy_(to_dev(am))
        if s.AV is not None:
            s.AV.copy_(to_dev(av))


@pytest.mark.parametrize("param_round", [oracle.ROUND_STOCHASTIC, oracle.ROUND_NEAREST])
@pytest.mark.parametrize("algo", ALGOS)
def test_mixed_list_ragged_sizes(algo, param_round):
    rng = np.random.default_rng(60 + algo + 5 * param_round)
    two = algo == ALGO_ADAMW
    sizes = [1, 7, 100, 2047, 2048, 2049, 4095, 4096, 6149, 20000, 3 * 2048 + 1024]
    sets, states = [], []
    tid = 0
    for n in sizes:
        for mode in (opt8.opt8_default_mode(n), M8, MB):
            if mode == MF and n >= 4096:
                continue
            p, g = _rand_bf16(rng, n, 0.02), _rand_bf16(rng, n, 1e-3)
            m, v, am, av = _state(mode, n, 21, tid, two)
            base = 2048 * int(rng.integers(0, 1000)) if tid % 3 == 0 else 0
            sets.append(DevTensorSet(mode, p, g, m, v, am, av, tensor_id=700 + tid, index_base=base))
            states.append([p, m, v, am, av])
            tid += 1
    stats = {}
    for t in (1, 2, 9):
        for s in sets:
            s.set_grad(_rand_bf16(rng, s.host[0].size, 1e-3))
        states = _step_compare(algo, sets, states, _hp(algo, t, param_round=param_round),
                               f"{NAMES[algo]} ss mixed step {t}", stats)
        _force(sets, states)
    log(f"{NAMES[algo]} stochastic-state mixed list ({len(sets)} tensors): mismatches {sum(stats.values())}")


@pytest.mark.parametrize("algo", ALGOS)
def test_single_tensor_free_running(algo):
    """1,048,576 elements from a zero 8-bit state, 10 steps, never forced: the two trajectories
    stay identical."""
    w = shapes.single_tensor()
    p = gen.param_init(w, 0)
    n = p.size
    two = algo == ALGO_ADAMW
    m = np.full(n, 127, np.uint8)
    v = np.zeros(n, np.uint8) if two else None
    am = np.zeros(n // 2048, np.float32)
    av = np.zeros(n // 2048, np.float32) if two else None
    s = DevTensorSet(M8, p, gen.grad_init(w, 1, 0), m, v, am, av, tensor_id=0)
    state = [p, m, v, am, av]
    stats = {}
    for t in range(1, 11):
        s.set_grad(gen.grad_init(w, t, 0))
        state = _step_compare(algo, [s], [state], _hp(algo, t, seed=w.seed), f"{NAMES[algo]} ss 1M step {t}",
                              stats)[0]
    log(f"{NAMES[algo]} stochastic-state free-running 1M: mismatches {sum(stats.values())}")
    assert sum(stats.values()) == 0, stats


@pytest.mark.parametrize("algo", ALGOS)
def test_degenerate_and_non_finite_blocks(algo):
    """Zero and subnormal blocks (zero codes, no draw), zero gradients in a live block,
    gradients near the bf16 maximum, and a block with an infinite gradient (NaN parameter,
    infinite absmax, code 255 where the normalised value is NaN)."""
    rng = np.random.default_rng(88 + algo)
    two = algo == ALGO_ADAMW
    n = 2048 * 6 + 333
    p, g = _rand_bf16(rng, n, 0.02), _rand_bf16(rng, n, 1e-3)
    m, v, am, av = _state(M8, n, 22, 0, two)
    g[:2048] = 0
    m[:2048] = 127
    am[0] = 0.0
    if two:
        v[:2048] = 0
        av[0] = 0.0
    g[2048:4096] = _rand_bf16(rng, 2048, 1e-39)
    am[1] = 0.0
    if two:
        av[1] = 0.0
    g[4096:4096 + 700] = 0
    g[6144:6144 + 16] = gen.to_bf16_bits(np.float32([3.0e38, -3.0e38] * 8))
    g[8192 + 3] = 0x7F80
    s = DevTensorSet(M8, p, g, m, v, am, av, tensor_id=4)
    hp = _hp(algo, 3)
    gpu_step([s], hp, algo)
    got = s.read()
    want = oracle_step(s, [p, m, v, am, av], hp, algo)
    wp, gp = oracle.rounding.bf16_to_f32(want[0]), oracle.rounding.bf16_to_f32(got[0])
    assert np.array_equal(np.isnan(wp), np.isnan(gp))
    assert np.array_equal(got[0][~np.isnan(wp)], want[0][~np.isnan(wp)])
    for k in (1, 2) if two else (1,):
        assert np.array_equal(got[k], want[k]), k
    for k in (3, 4) if two else (3,):
        assert np.array_equal(np.isnan(got[k]), np.isnan(want[k]))
        ok = ~np.isnan(want[k])
        assert np.array_equal(got[k][ok], want[k][ok])
    assert np.all(got[1][:4096] == 127)


def test_full_size_6p7b_sampled_blocks():
    """The 6.7B-shaped list in one call with stochastic state rounding (AdamW), checked on two
    random blocks plus the first and last block of every tensor."""
    w = shapes.get("gptneo-6.7b")
    log(f"building {len(w.tensors)} tensors, {w.numel} elements on the device")
    lst = build_list(w)
    torch.cuda.synchronize()
    blocks = sample_blocks(lst, 2, np.random.default_rng(3))
    before = snapshot(lst, blocks)
    hp = _hp(ALGO_ADAMW, 2, seed=w.seed, lr=w.lr)
    arr = descriptors(lst)
    opt8.opt8_adamw_step(arr, opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step,
                                                hp.seed, hp.param_round, hp.state_round))
    torch.cuda.synchronize()
    after = snapshot(lst, blocks)
    stats = {}
    for (i, b), x, y in zip(blocks, before, after):
        t = lst[i]
        want = oracle.step_tensor(t["mode"], x["p"], x["g"], x["m"], x["v"], x["am"], x["av"], hp,
                                  tensor_id=t["tid"], index_base=b * 2048)
        compare_state(f"ss/t{t['tid']}/b{b}", [y["p"], y["m"], y["v"], y["am"], y["av"]], want, t["mode"], stats)
    log(f"stochastic-state 6.7B: {len(blocks)} sampled blocks, mismatches {sum(stats.values())}")
    del lst, arr
    torch.cuda.empty_cache()


def test_decaying_second_moment_follows_on_the_gpu():
    """A block whose absmax is held by one element with a steady gradient while the others'
    second moments decay by beta2 per step: nearest codes stay frozen, stochastic codes follow
    the float64 decay on average (AdamW, 300 steps, 64 blocks)."""
    n = 2048 * 64
    dev = torch.device("cuda:0")
    cu = oracle.codebook.tables()[2]
    code0 = int(np.argmin(np.abs(cu - 0.25)))
    g = np.zeros(n, np.float32)
    g[::2048] = 1.0
    G = to_dev(gen.to_bf16_bits(g))
    out = {}
    for sr in (oracle.STATE_ROUND_NEAREST, SS):
        P = torch.zeros(n, dtype=torch.bfloat16, device=dev)
        M = torch.full((n,), 127, dtype=torch.uint8, device=dev)
        V = torch.full((n,), code0, dtype=torch.uint8, device=dev)
        V[::2048] = 255
        AM = torch.zeros(n // 2048, dtype=torch.float32, device=dev)
        AV = torch.ones(n // 2048, dtype=torch.float32, device=dev)
        arr = opt8.tensor_array([opt8.make_tensor(P, G, M, V, AM, AV, tensor_id=0)])
        for t in range(1, 301):
            opt8.opt8_adamw_step(arr, opt8.make_hparams(0.0, 0.9, 0.999, 1e-8, 0.0, t, 5, state_round=sr))
        torch.cuda.synchronize()
        vals = cu[V.cpu().numpy()].astype(np.float64) * np.repeat(AV.cpu().numpy().astype(np.float64), 2048)
        out[sr] = np.delete(vals, np.arange(0, n, 2048))
    want = float(cu[code0]) * 0.999 ** 300
    log(f"decay: want {want:.5f}, nearest {out[0].mean():.5f}, stochastic {out[SS].mean():.5f}")
    assert np.all(out[0] == out[0][0]) and out[0][0] > 1.3 * want
    assert abs(out[SS].mean() - want) < 0.01 * want
