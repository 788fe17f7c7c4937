"""opt8_adamw_step_noalloc: the AdamW step with its descriptor lists in the
library's fixed device array instead of allocated buffers.

Called through the C ABI and compared with opt8_adamw_step on copies of the
same inputs, bit for bit, on two calls in a row (the second with a smaller
list), and with the oracle.  A list over the array's limit is refused with
nothing modified.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DevTensorSet, compare_state, log
from precision_optimizer_step_amd import opt8
from workloads import gen

pytestmark = pytest.mark.gpu

M8, BF, F32 = oracle.MODE_8BIT, oracle.MODE_BF16_SR, oracle.MODE_FP32


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


def host_inputs(sizes_modes, seed):
    out = []
    for tid, (n, mode) in enumerate(sizes_modes):
        rng = np.random.default_rng(seed + tid)
        p = gen.to_bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
        g = gen.to_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
        if mode == M8:
            qm, qv, am, av = gen.random_state_8bit(seed, tid, n)
            out.append((mode, p, g, qm, qv, am, av, tid))
        elif mode == BF:
            m, v = gen.random_state_bf16(seed, tid, n)
            out.append((mode, p, g, m, v, None, None, tid))
        else:
            m, v = gen.random_state_f32(seed, tid, n)
            out.append((mode, p, g, m, v, None, None, tid))
    return out


def sets_of(inputs):
    return [DevTensorSet(mode, p, g, m, v, am, av, tensor_id=tid) for mode, p, g, m, v, am, av, tid in inputs]


def same_bytes(a, b):
    return a is None and b is None or np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


@pytest.mark.parametrize("param_round", [opt8.OPT8_ROUND_STOCHASTIC, opt8.OPT8_ROUND_NEAREST])
def test_noalloc_equals_allocating_entry_point_on_two_calls(param_round):
    calls = [
        # first call: every kernel kind (8-bit full blocks and partial tails, bf16 and fp32 state)
        [(5 * 2048 + 777, M8), (2048 * 3, M8), (3000, F32), (4 * 2048 + 5, BF), (40000, M8), (17, F32)],
        # second call: a smaller list of smaller tensors, so the array keeps stale entries past its end
        [(2048 + 1, M8), (100, F32)],
    ]
    for k, spec in enumerate(calls):
        hp = oracle.Hparams(lr=1e-3, weight_decay=0.01, step=k + 2, seed=99, param_round=param_round)
        inputs = host_inputs(spec, seed=10 * k + 1)
        a, b = sets_of(inputs), sets_of(inputs)
        php = opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step, hp.seed,
                                hp.param_round, hp.state_round)
        log(f"no-alloc call {k + 1}: {len(spec)} tensors, param_round {param_round}")
        opt8.opt8_adamw_step([s.desc() for s in a], php)
        opt8.opt8_adamw_step_noalloc([s.desc() for s in b], php)
        torch.cuda.synchronize()
        for sa, sb, (mode, p, g, m, v, am, av, tid) in zip(a, b, inputs):
            ga, gb = sa.read(), sb.read()
            for x, y in zip(ga, gb):
                assert same_bytes(x, y), f"call {k + 1}, tensor {tid}: the two entry points differ"
            want = oracle.step_tensor(mode, p, g, m, v, am, av, hp, tid)
            compare_state(f"noalloc{k + 1}/t{tid}", gb, want, mode)


def test_noalloc_refuses_a_list_over_its_limit():
    n = 2048 + 3
    inputs = host_inputs([(n, M8)], seed=5)
    s = sets_of(inputs)[0]
    before = s.read()
    d = s.desc()
    descs = []
    for i in range(4097):           # only the count is looked at: refused before any other check
        x = opt8.opt8_tensor.from_buffer_copy(d)
        x.tensor_id = i
        descs.append(x)
    php = opt8.make_hparams(1e-3, step=2)
    rc = opt8.opt8_adamw_step_noalloc(descs, php, check=False)
    assert rc == opt8.OPT8_E_SIZE
    assert "at most 4096" in opt8.opt8_last_error()
    torch.cuda.synchronize()
    for x, y in zip(before, s.read()):
        assert same_bytes(x, y)
    # the array is still usable afterwards
    hp = oracle.Hparams(lr=1e-3, step=2)
    opt8.opt8_adamw_step_noalloc([s.desc()], php)
    torch.cuda.synchronize()
    mode, p, g, m, v, am, av, tid = inputs[0]
    compare_state("noalloc/after-refusal", s.read(), oracle.step_tensor(mode, p, g, m, v, am, av, hp, tid), mode)
