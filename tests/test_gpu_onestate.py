"""GPU parity of the one-state rules (8-bit Lion, 8-bit SGD with momentum) against the oracle.

Same bar and the same structure as the AdamW parity tests: ragged mixed lists,
a free-running single tensor, degenerate blocks, non-finite inputs, and the
full 6.7B-shaped list on sampled blocks in the launch the benchmark times.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DevTensorSet, build_list, compare_state, descriptors, gpu_step, log,
                         oracle_step, sample_blocks, snapshot, to_dev)
from precision_optimizer_step_amd import opt8
from workloads import gen, shapes

pytestmark = pytest.mark.gpu

M8, MB, MF = oracle.MODE_8BIT, oracle.MODE_BF16_SR, oracle.MODE_FP32
LION, MOM = oracle.ALGO_LION, oracle.ALGO_MOMENTUM
ALGOS = [LION, MOM]
NAMES = {LION: "lion", MOM: "momentum"}


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


def _hp(algo, step, seed=0x5EED, param_round=oracle.ROUND_STOCHASTIC, lr=None, wd=0.1, state_round=0):
    if lr is None:
        lr = 1e-4 if algo == LION else 1e-2
    return oracle.Hparams(lr=lr, beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=wd, step=step,
                          seed=seed, param_round=param_round, state_round=state_round)


def _rand_bf16(rng, n, sigma):
    return gen.to_bf16_bits((rng.standard_normal(n) * sigma).astype(np.float32))


def _rand_state(mode, n, seed, tid):
    """(m, absmax_m) of a random non-trivial state."""
    if mode == M8:
        qm, _, am, _ = gen.random_state_8bit(seed, tid, n)
        return qm, am
    if mode == MB:
        return gen.random_state_bf16(seed, tid, n)[0], None
    return gen.random_state_f32(seed, tid, n)[0], None


def _set(mode, p, g, m, am, tid, base=0):
    return DevTensorSet(mode, p, g, m, None, am, None, tensor_id=tid, index_base=base)


def _step_and_compare(algo, sets, states, hp, label, stats):
    gpu_step(sets, hp, algo)
    nxt = []
    for s, st in zip(sets, states):
        want = oracle_step(s, st, hp, algo)
        compare_state(f"{label}/t{s.tensor_id}", s.read(), want, s.mode, stats)
        nxt.append(want)
    return nxt


def _force(sets, states):
    for s, (p, m, _v, am, _av) in zip(sets, states):
        s.P.copy_(to_dev(p))
        s.M.copy_(to_dev(m))
        if s.AM is not None:
            s.AM.copy_(to_dev(am))


@pytest.mark.parametrize("param_round", [oracle.ROUND_STOCHASTIC, oracle.ROUND_NEAREST])
@pytest.mark.parametrize("algo", ALGOS)
def test_mixed_list_ragged_sizes(algo, param_round):
    """Tiny, ragged and multi-block tensors of all three state modes in one list."""
    rng = np.random.default_rng(40 + algo + 3 * param_round)
    sizes = [1, 7, 8, 100, 2047, 2048, 2049, 4095, 4096, 6149, 20000, 3 * 2048 + 1024]
    sets, states = [], []
    tid = 0
    for n in sizes:
        for mode in (opt8.opt8_default_mode(n), M8, MB):
            if mode == MF and n >= 4096:
                continue
            p = _rand_bf16(rng, n, 0.02)
            g = _rand_bf16(rng, n, 1e-3)
            m, am = _rand_state(mode, n, 11, tid)
            base = 2048 * int(rng.integers(0, 1000)) if tid % 3 == 0 else 0
            sets.append(_set(mode, p, g, m, am, 500 + tid, base))
            states.append([p, m, None, am, None])
            tid += 1
    stats = {}
    for t in (1, 2, 7):
        for s in sets:
            s.set_grad(_rand_bf16(rng, s.host[0].size, 1e-3))
        hp = _hp(algo, t, seed=0x0123456789ABCDEF, param_round=param_round)
        states = _step_and_compare(algo, sets, states, hp, f"{NAMES[algo]} mixed step {t}", stats)
        _force(sets, states)
    log(f"{NAMES[algo]} mixed list ({len(sets)} tensors) mismatches: {sum(stats.values())}")


@pytest.mark.parametrize("algo", ALGOS)
def test_single_tensor_free_running(algo):
    """1,048,576 elements from a zero 8-bit state, fresh outlier gradients, 10 steps, never forced."""
    w = shapes.single_tensor()
    p = gen.param_init(w, 0)
    n = p.size
    m = np.full(n, 127, np.uint8)
    am = np.zeros(n // 2048, np.float32)
    s = _set(M8, p, gen.grad_init(w, 1, 0), m, am, 0)
    state = [p, m, None, am, None]
    stats = {}
    for t in range(1, 11):
        s.set_grad(gen.grad_init(w, t, 0))
        state = _step_and_compare(algo, [s], [state], _hp(algo, t, seed=w.seed), f"{NAMES[algo]} 1M step {t}",
                                  stats)[0]
    log(f"{NAMES[algo]} free-running 1M: mismatches {sum(stats.values())}")
    assert sum(stats.values()) == 0, stats


@pytest.mark.parametrize("algo", ALGOS)
def test_degenerate_blocks(algo):
    """Blocks that stress the special cases: all-zero, subnormal-only moments (stored as
    the zero code), zero gradients inside a live block (Lion's sign(0) = 0), gradients near
    the bf16 maximum, and lr = 0 / wd = 0 (parameters bit-identical)."""
    rng = np.random.default_rng(77 + algo)
    n = 2048 * 5 + 333
    p = _rand_bf16(rng, n, 0.02)
    g = _rand_bf16(rng, n, 1e-3)
    m, am = _rand_state(M8, n, 12, 0)
    g[:2048] = 0                                         # block 0: zero grad, zero state
    m[:2048] = 127
    am[0] = 0.0
    g[2048:4096] = _rand_bf16(rng, 2048, 1e-39)          # block 1: subnormal gradients only
    am[1] = 0.0
    g[4096:4096 + 700] = 0                               # block 2: zero grads in a live block
    g[6144:6144 + 16] = gen.to_bf16_bits(np.float32([3.0e38, -3.0e38] * 8))   # block 3: huge
    for rnd in (oracle.ROUND_STOCHASTIC, oracle.ROUND_NEAREST):
        for lr, wd in ((None, 0.1), (0.0, 0.0)):
            s = _set(M8, p, g, m, am, 3)
            hp = _hp(algo, 3, param_round=rnd, lr=lr, wd=wd)
            got = _step_and_compare(algo, [s], [[p, m, None, am, None]], hp,
                                    f"{NAMES[algo]} degenerate rnd={rnd} lr={lr}", {})[0]
            if lr == 0.0:
                assert np.array_equal(got[0], p)
            assert not np.any(got[3][:2] > 2.0 ** -126)   # blocks 0 and 1 below the normal range
            assert np.all(got[1][:4096] == 127)


@pytest.mark.parametrize("algo", ALGOS)
def test_non_finite_gradients(algo):
    """NaN and infinite gradients: parameters and block absmax NaN where the oracle's are
    (compared as NaN: the sign of a generated NaN differs between CPU and GPU), all other
    values bit-exact."""
    rng = np.random.default_rng(90 + algo)
    n = 2048 * 3
    p = _rand_bf16(rng, n, 0.02)
    g = _rand_bf16(rng, n, 1e-3)
    g[5] = 0x7FC0
    g[2048 + 9] = 0x7F80
    g[2048 + 700] = 0xFF80
    m, am = _rand_state(M8, n, 13, 0)
    s = _set(M8, p, g, m, am, 1)
    hp = _hp(algo, 2)
    gpu_step([s], hp, algo)
    got = s.read()
    want = oracle_step(s, [p, m, None, am, None], hp, algo)
    wp = oracle.rounding.bf16_to_f32(want[0])
    gp = oracle.rounding.bf16_to_f32(got[0])
    assert np.array_equal(np.isnan(wp), np.isnan(gp))
    fin = ~np.isnan(wp)
    assert np.array_equal(got[0][fin], want[0][fin])
    assert np.array_equal(got[1], want[1])
    assert np.array_equal(np.isnan(got[3]), np.isnan(want[3]))
    ok = ~np.isnan(want[3])
    assert np.array_equal(got[3][ok], want[3][ok])
    assert np.array_equal(got[0][4096:], want[0][4096:])


@pytest.mark.parametrize("state_round", [0, 1])
@pytest.mark.parametrize("algo", ALGOS)
def test_full_size_6p7b_sampled_blocks(algo, state_round):
    """The 6.7B-shaped list (388 tensors, 6,658,404,352 elements, one 8-bit state) stepped in
    one call, with the state rounded to nearest or stochastically (each rule and rounding has
    its own launch size at this length), checked on two random blocks plus the first and last
    block of every tensor."""
    w = shapes.get("gptneo-6.7b")
    log(f"{NAMES[algo]}: building {len(w.tensors)} tensors, {w.numel} elements on the device")
    lst = build_list(w, one_state=True)
    torch.cuda.synchronize()
    blocks = sample_blocks(lst, 2, np.random.default_rng(2))
    before = snapshot(lst, blocks)
    hp = _hp(algo, 2, seed=w.seed, state_round=state_round)
    arr = descriptors(lst)
    fn = opt8.opt8_lion_step if algo == LION else opt8.opt8_momentum_step
    fn(arr, opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step, hp.seed,
                              hp.param_round, hp.state_round))
    torch.cuda.synchronize()
    after = snapshot(lst, blocks)
    stats = {}
    for (i, b), x, y in zip(blocks, before, after):
        t = lst[i]
        want = oracle.step_tensor_1state(algo, t["mode"], x["p"], x["g"], x["m"], x["am"], hp,
                                         tensor_id=t["tid"], index_base=b * 2048)
        compare_state(f"{NAMES[algo]}/t{t['tid']}/b{b}", [y["p"], y["m"], None, y["am"], None],
                      [want[0], want[1], None, want[2], None], t["mode"], stats)
    log(f"{NAMES[algo]} 6.7B, state rounding {state_round}: {len(blocks)} sampled blocks, "
        f"mismatches {sum(stats.values())}")
    del lst, arr
    torch.cuda.empty_cache()
