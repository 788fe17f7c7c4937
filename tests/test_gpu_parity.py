"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Sizes are chosen so the oracle finishes in seconds while spanning many blocks
and ragged tails; the full-size 6.7B-shaped list is covered by sampled blocks
in test_gpu_fullsize.py.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DevTensorSet, compare_state, gpu_step, log, oracle_step, to_dev
from precision_optimizer_step_amd import opt8
from workloads import gen, shapes

pytestmark = pytest.mark.gpu

M8, MB, MF = oracle.MODE_8BIT, oracle.MODE_BF16_SR, oracle.MODE_FP32


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()
    log(f"device: {torch.cuda.get_device_name(0)}")


def _rand_bf16(rng, n, sigma):
    return gen.to_bf16_bits((rng.standard_normal(n) * sigma).astype(np.float32))


def _zero_state(mode, n):
    nb = (n + 2047) // 2048
    if mode == M8:
        return np.full(n, 127, np.uint8), np.zeros(n, np.uint8), np.zeros(nb, np.float32), np.zeros(nb, np.float32)
    if mode == MB:
        return np.zeros(n, np.uint16), np.zeros(n, np.uint16), None, None
    return np.zeros(n, np.float32), np.zeros(n, np.float32), None, None


def _rand_state(mode, n, seed, tid):
    if mode == M8:
        return gen.random_state_8bit(seed, tid, n)
    if mode == MB:
        return (*gen.random_state_bf16(seed, tid, n), None, None)
    return (*gen.random_state_f32(seed, tid, n), None, None)


def _run_and_compare(sets, states, hp, label, stats=None):
    """One GPU step over the list vs the oracle per tensor; returns the oracle's states."""
    gpu_step(sets, hp)
    nxt = []
    for s, st in zip(sets, states):
        want = oracle_step(s, st, hp)
        compare_state(f"{label}/t{s.tensor_id}", s.read(), want, s.mode, stats)
        nxt.append(want)
    return nxt


def _force(sets, states):
    """Overwrite the device state with the oracle's (keeps steps independent)."""
    for s, (p, m, v, am, av) in zip(sets, states):
        s.P.copy_(to_dev(p))
        s.M.copy_(to_dev(m))
        s.V.copy_(to_dev(v))
        if s.AM is not None:
            s.AM.copy_(to_dev(am))
            s.AV.copy_(to_dev(av))


# ----------------------------------------------------------------------------- workloads
def test_single_tensor_1m_ten_steps():
    """1,048,576 elements (512 blocks), zero state, fresh grads with 0.1% x100 outliers, 10 steps."""
    w = shapes.single_tensor()
    p = gen.param_init(w, 0)
    m, v, am, av = _zero_state(M8, p.size)
    s = DevTensorSet(M8, p, gen.grad_init(w, 1, 0), m, v, am, av, tensor_id=0)
    state = [p, m, v, am, av]
    stats = {}
    for t in range(1, w.steps + 1):
        s.set_grad(gen.grad_init(w, t, 0))
        hp = oracle.Hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                            weight_decay=w.weight_decay, step=t, seed=w.seed)
        state = _run_and_compare([s], [state], hp, f"single-1M step {t}", stats)[0]
        log(f"single-1M step {t}: mismatches so far {sum(stats.values())}")
    # the free-running trajectories also agree: nothing was forced above
    assert sum(stats.values()) == 0, stats


@pytest.mark.parametrize("param_round", [oracle.ROUND_STOCHASTIC, oracle.ROUND_NEAREST])
def test_mixed_list_ragged_sizes(param_round):
    """Tiny, ragged and multi-block tensors of all three modes in one list, random state."""
    rng = np.random.default_rng(5 + param_round)
    sizes = [1, 7, 8, 100, 2047, 2048, 2049, 4095, 4096, 6149, 20000, 3 * 2048 + 1024]
    sets, states = [], []
    tid = 0
    for n in sizes:
        for mode in (opt8.opt8_default_mode(n), M8, MB):
            if mode == MF and n >= 4096:
                continue
            p = _rand_bf16(rng, n, 0.02)
            g = _rand_bf16(rng, n, 1e-3)
            m, v, am, av = _rand_state(mode, n, 9, tid)
            base = 2048 * int(rng.integers(0, 1000)) if tid % 3 == 0 else 0
            sets.append(DevTensorSet(mode, p, g, m, v, am, av, tensor_id=1000 + tid, index_base=base))
            states.append([p, m, v, am, av])
            tid += 1
    log(f"mixed list: {len(sets)} tensors")
    stats = {}
    for t in (1, 2, 7):
        for s in sets:
            s.set_grad(_rand_bf16(rng, s.host[0].size, 1e-3))
        hp = oracle.Hparams(lr=1e-3, weight_decay=0.1, step=t, seed=0xABCDEF0123456789,
                            param_round=param_round)
        states = _run_and_compare(sets, states, hp, f"mixed step {t}", stats)
        _force(sets, states)
    log(f"mixed list mismatches: {sum(stats.values())}")


def test_gpt2_350m_first_last_layers_three_steps():
    """GPT-2 350M list: wpe, every tensor of layers 0 and 23 and ln_f (fp32 state under 4096)."""
    w = shapes.gpt2_350m()
    keep = [i for i in shapes.subset_for_sampling(w) if w.tensors[i].name != "wte"]
    sets, states = [], []
    for tid in keep:
        spec = w.tensors[tid]
        mode = opt8.opt8_default_mode(spec.numel)
        p = gen.param_init(w, tid)
        m, v, am, av = _zero_state(mode, spec.numel)
        sets.append(DevTensorSet(mode, p, gen.grad_init(w, 1, tid), m, v, am, av, tensor_id=tid))
        states.append([p, m, v, am, av])
    log(f"gpt2-350m subset: {len(sets)} tensors, {sum(s.host[0].size for s in sets)} elements")
    stats = {}
    for t in range(1, w.steps + 1):
        for s in sets:
            s.set_grad(gen.grad_init(w, t, s.tensor_id))
        hp = oracle.Hparams(lr=w.lr, weight_decay=w.weight_decay, step=t, seed=w.seed)
        states = _run_and_compare(sets, states, hp, f"gpt2 step {t}", stats)
    log(f"gpt2 subset mismatches: {sum(stats.values())}")


def test_lm_1p5b_nonuniform_grads():
    """1.5B-shaped layer-0 tensors + a 2,000-row slice of the embedding with the sparse-row recipe."""
    w = shapes.lm_1p5b()
    sets, states = [], []
    for tid, spec in enumerate(w.tensors):
        if not spec.name.startswith("h0.") and spec.name not in ("ln_f.w", "ln_f.b"):
            continue
        mode = opt8.opt8_default_mode(spec.numel)
        p = gen.param_init(w, tid)
        m, v, am, av = _zero_state(mode, spec.numel)
        sets.append(DevTensorSet(mode, p, gen.grad_init(w, 1, tid), m, v, am, av, tensor_id=tid))
        states.append([p, m, v, am, av])
    # sparse embedding rows: 5% of rows carry N(0, 1e-2) grads, the rest are exactly zero
    rows, width = 2000, 1600
    rng = np.random.default_rng(77)
    emb = _rand_bf16(rng, rows * width, 0.02)
    m, v, am, av = _zero_state(M8, rows * width)
    sets.append(DevTensorSet(M8, emb, np.zeros(rows * width, np.uint16), m, v, am, av, tensor_id=0))
    states.append([emb, m, v, am, av])
    stats = {}
    for t in range(1, w.steps + 1):
        for s in sets[:-1]:
            s.set_grad(gen.grad_init(w, t, s.tensor_id))
        g = np.zeros((rows, width), np.float32)
        pick = rng.choice(rows, 100, replace=False)
        g[pick] = rng.standard_normal((100, width)).astype(np.float32) * np.float32(1e-2)
        sets[-1].set_grad(gen.to_bf16_bits(g.reshape(-1)))
        hp = oracle.Hparams(lr=w.lr, weight_decay=w.weight_decay, step=t, seed=w.seed)
        states = _run_and_compare(sets, states, hp, f"lm-1.5b step {t}", stats)
    log(f"lm-1.5b subset mismatches: {sum(stats.values())}")


def test_gptneo_2p7b_bf16_state_mode():
    """BF16-AdamW-SR: every tensor in bf16 state (layer 0 of the 2.7B list), 3 steps."""
    w = shapes.gptneo_2p7b("bf16")
    sets, states = [], []
    for tid, spec in enumerate(w.tensors):
        if not spec.name.startswith("h0."):
            continue
        p = gen.param_init(w, tid)
        m, v, am, av = _zero_state(MB, spec.numel)
        sets.append(DevTensorSet(MB, p, gen.grad_init(w, 1, tid), m, v, am, av, tensor_id=tid))
        states.append([p, m, v, am, av])
    stats = {}
    for t in range(1, w.steps + 1):
        for s in sets:
            s.set_grad(gen.grad_init(w, t, s.tensor_id))
        hp = oracle.Hparams(lr=w.lr, weight_decay=w.weight_decay, step=t, seed=w.seed)
        states = _run_and_compare(sets, states, hp, f"bf16 step {t}", stats)
    log(f"bf16-state mismatches: {sum(stats.values())}")


# ----------------------------------------------------------------------------- edge cases
def test_degenerate_blocks():
    """All-zero grads and state, subnormal and huge grads, zero lr/wd, a lone element."""
    rng = np.random.default_rng(3)
    n = 2048 * 2 + 33
    cases = []
    p = _rand_bf16(rng, n, 0.02)
    cases.append(("zero grads, zero state", p, np.zeros(n, np.uint16), _zero_state(M8, n)))
    sub = (rng.integers(1, 0x7F, n) | (rng.integers(0, 2, n) << 15)).astype(np.uint16)  # bf16 subnormals
    cases.append(("subnormal grads", p, sub, _zero_state(M8, n)))
    big = _rand_bf16(rng, n, 1e3)
    cases.append(("huge grads", p, big, _rand_state(M8, n, 3, 1)))
    tiny_state = list(_rand_state(M8, n, 4, 2))
    tiny_state[2] = np.full_like(tiny_state[2], 1e-39)        # subnormal absmax
    cases.append(("subnormal absmax", p, _rand_bf16(rng, n, 1e-30), tuple(tiny_state)))
    cases.append(("lone element", _rand_bf16(rng, 1, 0.5), _rand_bf16(rng, 1, 1e-3), _zero_state(M8, 1)))
    for k, (label, pp, gg, st) in enumerate(cases):
        s = DevTensorSet(M8, pp, gg, *st, tensor_id=k)
        for hp in (oracle.Hparams(lr=1e-3, weight_decay=0.1, step=1, seed=1),
                   oracle.Hparams(lr=0.0, weight_decay=0.0, step=4, seed=1)):
            want = oracle_step(s, [pp, *st], hp)
            s2 = DevTensorSet(M8, pp, gg, *st, tensor_id=k)
            gpu_step([s2], hp)
            compare_state(label, s2.read(), want, M8)
            if hp.lr == 0.0:
                assert np.array_equal(s2.read()[0], pp), "zero lr and wd must leave params untouched"
        log(f"degenerate case ok: {label}")


def test_determinism_list_independence_and_resume():
    rng = np.random.default_rng(8)
    n = 2048 * 5 + 77
    p = _rand_bf16(rng, n, 0.02)
    grads = [_rand_bf16(rng, n, 1e-3) for _ in range(4)]
    st = _zero_state(M8, n)
    other_p = _rand_bf16(rng, 3000, 0.02)

    def run(with_other, split):
        s = DevTensorSet(M8, p, grads[0], *st, tensor_id=3)
        o = DevTensorSet(MF, other_p, _rand_bf16(np.random.default_rng(1), 3000, 1e-3),
                         *_zero_state(MF, 3000), tensor_id=4)
        for t in range(1, 5):
            s.set_grad(grads[t - 1])
            hp = oracle.Hparams(lr=1e-3, weight_decay=0.01, step=t, seed=99)
            gpu_step([s, o] if with_other else [s], hp)
            if split and t == 2:          # checkpoint: state to host and back into fresh buffers
                cur = s.read()
                s = DevTensorSet(M8, cur[0], grads[t - 1], cur[1], cur[2], cur[3], cur[4], tensor_id=3)
        return s.read()

    a = run(False, False)
    b = run(False, False)
    c = run(True, False)
    d = run(False, True)
    for x in (b, c, d):
        for u, w in zip(a, x):
            assert np.array_equal(u, w)


def test_index_base_equals_shard_of_a_larger_tensor():
    """A shard stepped with its global index base equals that slice of the whole tensor."""
    rng = np.random.default_rng(12)
    n = 2048 * 8 + 500
    p = _rand_bf16(rng, n, 0.02)
    g = _rand_bf16(rng, n, 1e-3)
    st = _rand_state(M8, n, 5, 5)
    hp = oracle.Hparams(lr=1e-3, weight_decay=0.01, step=3, seed=5)
    whole = DevTensorSet(M8, p, g, *st, tensor_id=11)
    gpu_step([whole], hp)
    cut = 2048 * 3
    qm, qv, am, av = st
    shard = DevTensorSet(M8, p[cut:], g[cut:], qm[cut:], qv[cut:], am[3:], av[3:],
                         tensor_id=11, index_base=cut)
    gpu_step([shard], hp)
    w = whole.read()
    s = shard.read()
    assert np.array_equal(w[0][cut:], s[0])
    assert np.array_equal(w[1][cut:], s[1]) and np.array_equal(w[2][cut:], s[2])
    assert np.array_equal(w[3][3:], s[3]) and np.array_equal(w[4][3:], s[4])


def test_non_finite_inputs():
    """NaN and infinite gradients: the parameter becomes NaN where the oracle's does, the
    block absmax follows NaN propagation, codes match.  (The sign of a NaN produced by an
    invalid operation differs between the CPU and the GPU, so NaN is compared as NaN.)"""
    rng = np.random.default_rng(21)
    n = 2048 * 3
    p = _rand_bf16(rng, n, 0.02)
    g = _rand_bf16(rng, n, 1e-3)
    g[5] = 0x7FC0            # NaN in block 0
    g[2048 + 9] = 0x7F80     # +inf in block 1
    g[2048 + 700] = 0xFF80   # -inf in block 1
    st = _rand_state(M8, n, 6, 6)
    hp = oracle.Hparams(lr=1e-3, weight_decay=0.01, step=2, seed=3)
    want = oracle_step(DevTensorSet(M8, p, g, *st, tensor_id=1), [p, *st], hp)
    s = DevTensorSet(M8, p, g, *st, tensor_id=1)
    gpu_step([s], hp)
    got = s.read()
    wp = oracle.rounding.bf16_to_f32(want[0])
    gp_ = oracle.rounding.bf16_to_f32(got[0])
    assert np.array_equal(np.isnan(wp), np.isnan(gp_))
    fin = ~np.isnan(wp)
    assert np.array_equal(got[0][fin], want[0][fin])
    for k in (1, 2):
        assert np.array_equal(got[k], want[k])
    for k in (3, 4):
        assert np.array_equal(np.isnan(got[k]), np.isnan(want[k]))
        ok = ~np.isnan(want[k])
        assert np.array_equal(got[k][ok], want[k][ok])
    # the third block is untouched by the bad values and matches bit for bit
    assert np.array_equal(got[0][4096:], want[0][4096:])


@pytest.mark.parametrize("algo,mode", [(0, M8), (0, MB), (oracle.ALGO_LION, M8), (oracle.ALGO_MOMENTUM, M8)])
def test_non_finite_in_a_partial_block(algo, mode):
    """A NaN and an infinite gradient inside the partial last block of a tensor: the partial
    block leaves its fast path for the plain one, and the results follow the oracle (NaN
    compared as NaN); the full block before it matches bit for bit."""
    rng = np.random.default_rng(22 + algo + 10 * mode)
    n = 2048 + 100
    p = _rand_bf16(rng, n, 0.02)
    g = _rand_bf16(rng, n, 1e-3)
    g[2048 + 50] = 0x7FC0
    g[2048 + 60] = 0x7F80
    m, v, am, av = _rand_state(mode, n, 7, 3)
    if algo != 0:
        v = av = None
    hp = oracle.Hparams(lr=1e-3, beta2=0.99 if algo else 0.999, weight_decay=0.01, step=2, seed=5)
    want = oracle_step(DevTensorSet(mode, p, g, m, v, am, av, tensor_id=2), [p, m, v, am, av], hp, algo)
    s = DevTensorSet(mode, p, g, m, v, am, av, tensor_id=2)
    gpu_step([s], hp, algo)
    got = s.read()
    wp = oracle.rounding.bf16_to_f32(want[0])
    gp_ = oracle.rounding.bf16_to_f32(got[0])
    assert np.array_equal(np.isnan(wp), np.isnan(gp_))
    assert np.isnan(gp_).any(), "the NaN gradient must reach the parameter"
    fin = ~np.isnan(wp)
    assert np.array_equal(got[0][fin], want[0][fin])
    for k in range(1, 5):
        if want[k] is None:
            continue
        if want[k].dtype == np.uint8:
            assert np.array_equal(got[k], want[k])
        else:
            w = want[k].view(np.float32) if want[k].dtype == np.float32 else oracle.rounding.bf16_to_f32(want[k])
            h = got[k].view(np.float32) if got[k].dtype == np.float32 else oracle.rounding.bf16_to_f32(got[k])
            assert np.array_equal(np.isnan(h), np.isnan(w))
            ok = ~np.isnan(w)
            assert np.array_equal(h[ok], w[ok])
    assert np.array_equal(got[0][:2048], want[0][:2048])


@pytest.mark.parametrize("label,hp_kw", [
    ("eps below 2^-60", dict(eps=1e-20)),
    ("eps above 2^60", dict(eps=1e20)),
    ("lr*wd above 1", dict(lr=0.5, weight_decay=4.0)),
    ("huge step size", dict(lr=1e9)),
])
def test_hyperparameters_outside_the_fast_range(label, hp_kw):
    """Hyperparameters that switch the fast AdamW sequences off for the whole launch (every
    block then takes the plain path) on a list of all three modes: still equal to the oracle."""
    rng = np.random.default_rng(31)
    sets, states = [], []
    for tid, (n, mode) in enumerate([(2048 * 5 + 19, M8), (2048 * 3, MB), (1000, MF), (4096, M8)]):
        p, g = _rand_bf16(rng, n, 0.02), _rand_bf16(rng, n, 1e-3)
        st = _rand_state(mode, n, 40, tid)
        sets.append(DevTensorSet(mode, p, g, *st, tensor_id=tid))
        states.append([p, *st])
    kw = dict(lr=1e-3, weight_decay=0.01, step=3, seed=5)
    kw.update(hp_kw)
    hp = oracle.Hparams(**kw)
    stats = {}
    _run_and_compare(sets, states, hp, label, stats)
    log(f"{label}: mismatches {sum(stats.values())}")


def test_negative_second_moment_state():
    """Invalid but defined: a negative absmax_v (8-bit) or negative bf16 v makes v2 negative,
    its square root NaN and the parameter NaN, as in the oracle; the fast paths must hand
    such blocks to the plain path.  NaN is compared as NaN, everything else bit for bit."""
    rng = np.random.default_rng(41)
    n = 2048 * 3
    p, g = _rand_bf16(rng, n, 0.02), _rand_bf16(rng, n, 1e-4)
    m8, v8, am8, av8 = _rand_state(M8, n, 42, 0)
    av8 = av8.copy()
    av8[1] = -av8[1] - 1e-6                       # block 1: negative second-moment scale
    mb, vb, _, _ = _rand_state(MB, n, 43, 1)
    vb = vb.copy()
    vb[2048 + 5] = gen.to_bf16_bits(np.float32([-1e-2]))[0]   # one negative bf16 v in block 1
    hp = oracle.Hparams(lr=1e-3, weight_decay=0.01, step=2, seed=7)
    for mode, st in ((M8, (m8, v8, am8, av8)), (MB, (mb, vb, None, None))):
        want = oracle_step(DevTensorSet(mode, p, g, *st, tensor_id=3), [p, *st], hp)
        s = DevTensorSet(mode, p, g, *st, tensor_id=3)
        gpu_step([s], hp)
        got = s.read()
        wp, gp = oracle.rounding.bf16_to_f32(want[0]), oracle.rounding.bf16_to_f32(got[0])
        assert np.isnan(wp).any(), "the case must produce NaN parameters"
        assert np.array_equal(np.isnan(wp), np.isnan(gp))
        assert np.array_equal(got[0][~np.isnan(wp)], want[0][~np.isnan(wp)])
        for k in (1, 2):
            if mode == MB:
                wk = oracle.rounding.bf16_to_f32(want[k])
                gk = oracle.rounding.bf16_to_f32(got[k])
                assert np.array_equal(np.isnan(wk), np.isnan(gk))
                assert np.array_equal(got[k][~np.isnan(wk)], want[k][~np.isnan(wk)])
            else:
                assert np.array_equal(got[k], want[k])
        if mode == M8:
            for k in (3, 4):
                assert np.array_equal(np.isnan(got[k]), np.isnan(want[k]))
                ok = ~np.isnan(want[k])
                assert np.array_equal(got[k][ok], want[k][ok])



def _edge(cond):
    """Smallest bf16 magnitude pattern h (a positive bf16 value g) with cond(g) true, for a
    condition that is false below some magnitude and true from there on."""
    h = np.arange(1, 0x7F80, dtype=np.uint32)
    with np.errstate(over="ignore", invalid="ignore"):
        ok = cond((h << 16).view(np.float32))
    assert ok.any() and ok[-1]
    return int(h[np.argmax(ok)])


def _frexp_e(x):
    return np.frexp(np.asarray(x, np.float32))[1]


@pytest.mark.parametrize("betas", [(0.9, 0.999), (0.0, 0.5), (0.99, 0.0)])
def test_fast_path_range_edges(betas):
    """Blocks on both sides of each bound of the 8-bit AdamW fast path's range check, found
    with the oracle's fp32 arithmetic at step 1: a lone gradient whose v2 or m2 sits at the
    smallest admitted exponent (2^-89) and one bf16 pattern below it, of either sign; a small
    m2 against a large denominator at the quotient bound (e(m2) >= e(den) - 98); a tiny
    absmax_m with zero gradients; and, with eps = 1e-18, the largest moment at the
    max|m2| / eps bound.  Every block must equal the oracle bit for bit, whichever path it
    takes."""
    rng = np.random.default_rng(57)
    kw = dict(lr=1e-3, beta1=betas[0], beta2=betas[1], weight_decay=0.01, seed=9)
    s1 = oracle.adamw.host_scalars(oracle.Hparams(step=1, **kw))
    w1, w2, rbc2, eps = s1.w1, s1.w2, s1.rbc2, s1.eps
    f = np.float32
    nb = 14
    n = 2048 * nb
    blk = [slice(2048 * b, 2048 * (b + 1)) for b in range(nb)]
    p = _rand_bf16(rng, n, 0.02)
    g = _rand_bf16(rng, n, 1e-3)
    qm, qv, am, av = (a.copy() for a in gen.random_state_8bit(58, 0, n))

    def zero_state(b):
        qm[blk[b]], qv[blk[b]], am[b], av[b] = 127, 0, 0.0, 0.0

    def lone(b, h, at=5):
        g[2048 * b + at] = np.uint16(h)

    # v2 = w2 * g^2 at the 2^-89 floor (zero state: m2 = w1 g, v2 = w2 g^2)
    lim = f(2.0 ** -89)
    if w2 != 0:
        hv = _edge(lambda x: (w2 * (x * x) >= lim) & (np.abs(w1 * x) >= lim))
        for b, h in ((0, hv), (1, hv - 1), (2, hv | 0x8000), (3, (hv - 1) | 0x8000)):
            zero_state(b)
            lone(b, h)
    # m2 = w1 * g at the floor; v2 held up by a non-zero second-moment state
    if w1 != 0:
        hm = _edge(lambda x: np.abs(w1 * x) >= lim)
        for b, h in ((4, hm), (5, hm - 1), (6, (hm - 1) | 0x8000)):
            qm[blk[b]], am[b], av[b] = 127, 1.0, 1e-6
            qv[blk[b]] = np.maximum(qv[blk[b]], 1)
            lone(b, h)
    # quotient bound: one large gradient sets den, a small m2 sits at e(den) - 98
    for b, side in ((7, 0), (8, 1)):
        qm[blk[b]], am[b], av[b] = 127, 1.0, 1e-6
        qv[blk[b]] = np.maximum(qv[blk[b]], 1)
        g[2048 * b] = gen.to_bf16_bits(f([3e4]))[0]
        gb = oracle.rounding.bf16_to_f32(g[blk[b]])
        v1 = oracle.codebook.tables()[2][qv[blk[b]]] * f(av[b])
        v2 = s1.beta2 * v1 + w2 * (gb * gb)
        e_den = _frexp_e(np.sqrt(np.max(v2)) * rbc2 + eps)
        if w1 != 0:
            h = _edge(lambda x: _frexp_e(w1 * x) >= e_den - 98)
            lone(b, h - side, at=9)
    # tiny absmax_m: m1 = Cs[q] * am far below the floor where the gradient is zero
    for b, a in ((9, 2.0 ** -80), (10, 2.0 ** -60)):
        am[b] = a
        g[blk[b]][::5] = 0
    stats = {}
    for step in (1, 3):
        hp = oracle.Hparams(step=step, **kw)
        sets = [DevTensorSet(M8, p, g, qm, qv, am, av, tensor_id=2)]
        _run_and_compare(sets, [[p, qm, qv, am, av]], hp, f"edges {betas} step {step}", stats)
    # max|m2| / eps at 2^100: eps = 1e-18, zero state, one large gradient per block
    kw_e = dict(kw, eps=1e-18)
    se = oracle.adamw.host_scalars(oracle.Hparams(step=1, **kw_e))
    if se.w1 != 0:
        e_eps = _frexp_e(se.eps)
        h = _edge(lambda x: _frexp_e(se.w1 * x) - e_eps > 100)
        g2 = g.copy()
        for b, hh in ((11, h), (12, h - 1), (13, (h - 1) | 0x8000)):
            zero_state(b)
            g2[2048 * b + 3] = np.uint16(hh)
        sets = [DevTensorSet(M8, p, g2, qm, qv, am, av, tensor_id=2)]
        _run_and_compare(sets, [[p, qm, qv, am, av]], oracle.Hparams(step=1, **kw_e),
                         f"edges {betas} eps 1e-18", stats)
    log(f"range edges {betas}: mismatches {sum(stats.values())}")
    assert sum(stats.values()) == 0

