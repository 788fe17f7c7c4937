"""Every full-size parameter list, run as its configuration states, checked
against the oracle after every step.

  gptneo-6.7b       8-bit state, 5 steps, lr 1.2e-4, wd 0.1, seed 1234,
                    gradients N(0, 1e-3) with 0.01% of them x100 (~40 GB on the device)
  lm-1.5b           3 steps, lr 1.5e-4, wd 0.01: embedding rows 95% zero and 5%
                    N(0, 1e-2), LayerNorm gradients N(0, 1e-4), the rest N(0, 1e-3)
                    with 0.01% x1000 (whole zero blocks: the zero-absmax path)
  gptneo-2.7b       3 steps, lr 3.2e-4, wd 0.1, 8-bit state (fp32 under 4096 elements)
  gptneo-2.7b-bf16  the same list with bf16 state written by stochastic rounding
  gpt2-350m         3 steps, lr 6e-4, wd 0.1, gradients N(0, 1e-3/sqrt(fan_in)):
                    EVERY element of every tensor, the embedding included
and the same protocol for the rules built on the same machinery, on the 6.7B
list: 8-bit Lion (lr 1.2e-5, betas 0.9 / 0.99), 8-bit SGD with momentum (0.9)
and AdamW with the 8-bit state rounded stochastically.

Each list starts from the zero state (absmax 0 and zero codes, or zero bf16 /
fp32 moments) with its parameter recipe, and gets fresh gradients at every
step, generated on the device from (seed, step, tensor id).  The whole list is
stepped in one call, the launch the benchmark times.  The sampled blocks --
every tensor's first and last block and 64 others drawn at random (every
block of gpt2-350m) -- are copied to the host before the first step, and the
oracle carries its own state for them from there: after every step, the
zero-state first step included, the GPU's parameters, codes and absmax
values for those blocks must match the oracle's within the comparison bar.
The oracle steps each run of consecutive sampled blocks alone, which is exact
because blocks are independent; it runs in worker processes.
"""

import time

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BLOCK, _np, compare_state, log
from oracle_pool import OraclePool, hp_fields, runs, split_runs
from precision_optimizer_step_amd import opt8
from workloads import gen, shapes

pytestmark = pytest.mark.gpu

SAMPLES_PER_TENSOR = 64


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


@pytest.fixture(scope="module")
def pool():
    p = OraclePool()
    yield p
    p.close()


def _mode_of(w, spec):
    if w.state_mode == "bf16":
        return oracle.MODE_BF16_SR
    return opt8.opt8_default_mode(spec.numel)


def _state_dtype(mode):
    return {oracle.MODE_8BIT: np.uint8, oracle.MODE_BF16_SR: np.uint16, oracle.MODE_FP32: np.float32}[mode]


class Sampled:
    """One tensor on the device, and the blocks of it the oracle follows."""

    def __init__(self, w, tid, blocks_per_tensor, rng, dev, one_state=False):
        spec = w.tensors[tid]
        self.tid, self.spec, self.n = tid, spec, spec.numel
        self.mode = _mode_of(w, spec)
        n = self.n
        nb = (n + BLOCK - 1) // BLOCK
        self.P = torch.empty(n, dtype=torch.bfloat16, device=dev)
        gen.param_init_device(spec, w, tid, self.P)
        self.G = torch.empty(n, dtype=torch.bfloat16, device=dev)
        self.AM = self.AV = None
        if self.mode == oracle.MODE_8BIT:
            self.M = torch.full((n,), 127, dtype=torch.uint8, device=dev)
            self.V = torch.zeros(n, dtype=torch.uint8, device=dev)
            self.AM = torch.zeros(nb, dtype=torch.float32, device=dev)
            self.AV = torch.zeros(nb, dtype=torch.float32, device=dev)
        else:
            dt = torch.bfloat16 if self.mode == oracle.MODE_BF16_SR else torch.float32
            self.M = torch.zeros(n, dtype=dt, device=dev)
            self.V = torch.zeros(n, dtype=dt, device=dev)
        if one_state:
            self.V = self.AV = None
        if blocks_per_tensor is None or nb <= blocks_per_tensor + 2:
            blocks = list(range(nb))
        else:
            inner = rng.choice(np.arange(1, nb - 1), size=blocks_per_tensor, replace=False)
            blocks = sorted({0, nb - 1} | set(int(b) for b in inner))
        self.whole = len(blocks) == nb
        self.blocks = blocks
        if self.whole:
            self.eidx = self.bidx = None
        else:
            self.eidx = torch.cat([torch.arange(b * BLOCK, min(n, (b + 1) * BLOCK), device=dev) for b in blocks])
            self.bidx = torch.tensor(blocks, dtype=torch.int64, device=dev)
        # pieces: (first block, block count, element range and block range in the gathered arrays)
        self.pieces = []
        pos_b = {b: i for i, b in enumerate(blocks)}
        for a, c in split_runs(runs(blocks), 2048):
            e0 = pos_b[a] * BLOCK
            e1 = e0 + min(n, (a + c) * BLOCK) - a * BLOCK
            self.pieces.append((a, c, e0, e1, pos_b[a], pos_b[a] + c))

    def desc(self):
        return opt8.make_tensor(self.P, self.G, self.M, self.V, self.AM, self.AV, tensor_id=self.tid,
                                mode=self.mode)

    def gather(self, t, per_block, dtype):
        if t is None:
            return None
        if not self.whole:
            t = t[self.bidx if per_block else self.eidx]
        return _np(t, dtype)

    def read(self):
        sd = _state_dtype(self.mode)
        return [self.gather(self.P, False, np.uint16), self.gather(self.M, False, sd),
                self.gather(self.V, False, sd), self.gather(self.AM, True, np.float32),
                self.gather(self.AV, True, np.float32)]


def _oracle_items(samples, carried, grads, hp, algo=0):
    items, where = [], []
    fields = hp_fields(hp)
    for s, (p, m, v, am, av), g in zip(samples, carried, grads):
        for a, c, e0, e1, b0, b1 in s.pieces:
            items.append((algo, s.mode, fields, p[e0:e1], g[e0:e1], m[e0:e1], None if v is None else v[e0:e1],
                          None if am is None else am[b0:b1], None if av is None else av[b0:b1],
                          s.tid, a * BLOCK))
            where.append(s)
    return items, where


def _assemble(samples, where, results):
    out = {}
    for s, r in zip(where, results):
        out.setdefault(s.tid, []).append(r)
    assembled = []
    for s in samples:
        parts = out[s.tid]
        cat = [None if parts[0][k] is None else np.concatenate([x[k] for x in parts]) for k in range(5)]
        assembled.append(cat)
    return assembled


ADAMW, LION, MOMENTUM = 0, oracle.ALGO_LION, oracle.ALGO_MOMENTUM
STEP_FN = {ADAMW: "opt8_adamw_step", LION: "opt8_lion_step", MOMENTUM: "opt8_momentum_step"}
# (list, sampled blocks per tensor (None: all), update rule, state rounding)
CONFIGS = [("gptneo-6.7b", SAMPLES_PER_TENSOR, ADAMW, 0), ("lm-1.5b", SAMPLES_PER_TENSOR, ADAMW, 0),
           ("gptneo-2.7b", SAMPLES_PER_TENSOR, ADAMW, 0), ("gptneo-2.7b-bf16", SAMPLES_PER_TENSOR, ADAMW, 0),
           ("gpt2-350m", None, ADAMW, 0),
           ("gptneo-6.7b", SAMPLES_PER_TENSOR, LION, 0), ("gptneo-6.7b", SAMPLES_PER_TENSOR, MOMENTUM, 0),
           ("gptneo-6.7b", SAMPLES_PER_TENSOR, ADAMW, 1)]
RULE_NAMES = {ADAMW: "adamw", LION: "lion", MOMENTUM: "momentum"}


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name,per_tensor,algo,state_round", CONFIGS,
                         ids=[f"{c[0]}-{RULE_NAMES[c[2]]}" + ("-sr-state" if c[3] else "") for c in CONFIGS])
def test_full_size_list_as_configured(name, per_tensor, algo, state_round, pool):
    w = shapes.get(name)
    # Lion at a tenth of the list's learning rate with beta2 0.99 (its usual setting)
    lr = w.lr / 10 if algo == LION else w.lr
    beta2 = 0.99 if algo == LION else w.beta2
    label = f"{name}/{RULE_NAMES[algo]}" + ("/sr-state" if state_round else "")
    dev = torch.device("cuda:0")
    t0 = time.time()
    rng = np.random.default_rng(2024)
    samples = [Sampled(w, tid, per_tensor, rng, dev, one_state=algo != ADAMW) for tid in range(len(w.tensors))]
    arr = opt8.tensor_array(s.desc() for s in samples)
    torch.cuda.synchronize()
    checked_elems = sum(p[3] - p[2] for s in samples for p in s.pieces)
    log(f"{label}: {len(samples)} tensors, {w.numel} elements from the zero state, {w.steps} steps; "
        f"the oracle follows {sum(len(s.blocks) for s in samples)} blocks ({checked_elems} elements); "
        f"built in {time.time() - t0:.1f}s")
    carried = [s.read() for s in samples]        # the parameters and the zero state, as the oracle starts
    per_step = []
    for step in range(1, w.steps + 1):
        t1 = time.time()
        for s in samples:
            gen.grad_init_device(s.spec, w, step, s.tid, s.G)
        grads = [s.gather(s.G, False, np.uint16) for s in samples]
        hp = oracle.Hparams(lr=lr, beta1=w.beta1, beta2=beta2, eps=w.eps, weight_decay=w.weight_decay,
                            step=step, seed=w.seed, state_round=state_round)
        getattr(opt8, STEP_FN[algo])(arr, opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                                                            hp.step, hp.seed, hp.param_round, hp.state_round))
        torch.cuda.synchronize()
        got = [s.read() for s in samples]
        items, where = _oracle_items(samples, carried, grads, hp, algo)
        want = _assemble(samples, where, pool.step(items))
        stats = {}
        for s, x, y in zip(samples, got, want):
            compare_state(f"{label}/step{step}/t{s.tid}", x, y, s.mode, stats)
        zero_blocks = sum(int(np.count_nonzero(y[3] == 0)) for y in want if y[3] is not None)
        mism = sum(stats.values())
        per_step.append(mism)
        log(f"{label}: step {step}: {checked_elems} elements checked, {mism} differ from the oracle "
            f"({zero_blocks} sampled blocks with a zero first-moment absmax); {time.time() - t1:.1f}s")
        carried = want
    log(f"{label}: mismatching elements per step {per_step}")
    del samples, arr
    torch.cuda.empty_cache()
