"""GPU parity over randomly drawn hyperparameters and rounding modes.

Each case draws an update rule (AdamW, Lion, momentum), beta1, beta2, eps, lr, weight decay,
a step number, a seed and both rounding choices, and runs three steps over a list holding an
8-bit tensor (0-3 full blocks and a last block of 1-2047 elements, drawn per case), a
bf16-state tensor and an fp32-state tensor (lengths drawn per case), each started from a
random state.  Every result is compared with the oracle, which carries its
state from step to step independently of the GPU.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import ALGO_ADAMW, DevTensorSet, compare_state, gpu_step, log, oracle_step
from precision_optimizer_step_amd import opt8
from workloads import gen

pytestmark = pytest.mark.gpu

M8, MB, MF = oracle.MODE_8BIT, oracle.MODE_BF16_SR, oracle.MODE_FP32
ALGOS = [ALGO_ADAMW, oracle.ALGO_LION, oracle.ALGO_MOMENTUM]


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


def _draw(rng):
    algo = ALGOS[int(rng.integers(0, 3))]
    hp = dict(lr=float(10.0 ** rng.uniform(-6, -1)),
              beta1=0.0 if rng.random() < 0.2 else float(rng.uniform(0.5, 0.99)),
              beta2=float(rng.choice([0.0, 0.9, 0.99, 0.999, 0.9999])),
              eps=float(10.0 ** rng.uniform(-12, -3)),
              weight_decay=0.0 if rng.random() < 0.2 else float(rng.uniform(0.0, 0.5)),
              step=int(rng.integers(1, 2000)), seed=int(rng.integers(0, 2 ** 63)),
              param_round=int(rng.integers(0, 2)), state_round=int(rng.integers(0, 2)))
    return algo, hp


@pytest.mark.parametrize("case", range(24))
def test_random_hyperparameters(case):
    rng = np.random.default_rng(1000 + case)
    algo, kw = _draw(rng)
    one = algo != ALGO_ADAMW
    gsig = float(10.0 ** rng.uniform(-5, -1))
    sets, states = [], []
    n8 = 2048 * int(rng.integers(0, 4)) + int(rng.integers(1, 2048))
    for tid, (n, mode) in enumerate([(n8, M8), (int(rng.integers(1, 5000)), MB), (int(rng.integers(1, 4096)), MF)]):
        p = gen.to_bf16_bits((rng.standard_normal(n) * 0.05).astype(np.float32))
        g = gen.to_bf16_bits((rng.standard_normal(n) * gsig).astype(np.float32))
        if mode == M8:
            m, v, am, av = gen.random_state_8bit(77 + case, tid, n, scale=gsig)
        elif mode == MB:
            (m, v), am, av = gen.random_state_bf16(77 + case, tid, n, scale=gsig), None, None
        else:
            (m, v), am, av = gen.random_state_f32(77 + case, tid, n, scale=gsig), None, None
        if one:
            v = av = None
        sets.append(DevTensorSet(mode, p, g, m, v, am, av, tensor_id=7 * tid + case))
        states.append([p, m, v, am, av])
    log(f"case {case}: algo {algo} {kw} grad sigma {gsig:.2e}")
    stats = {}
    for k in range(3):
        hp = oracle.Hparams(**dict(kw, step=kw["step"] + k))
        gpu_step(sets, hp, algo)
        for i, s in enumerate(sets):
            want = oracle_step(s, states[i], hp, algo)
            compare_state(f"case {case} step {k}/t{s.tensor_id}", s.read(), want, s.mode, stats)
            states[i] = want
    log(f"case {case}: mismatches {sum(stats.values())}")
