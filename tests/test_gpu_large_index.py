"""GPU parity where element indices leave 32 bits.

The random bits of element j come from Philox with the 64-bit group index j/8
split over two counter words (its high word shares a word with the stream
number), so a tensor whose global index passes 2^35 exercises the high word,
and one straddling j = 2^35 sees the low word wrap inside a block.  A single
tensor of more than 2^31 elements exercises 64-bit element and byte offsets in
the step kernels (4 GiB of bf16 per array).  Both are checked against the
oracle element by element.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BLOCK, DevTensorSet, compare_state, gpu_step, log, oracle_step, snapshot, to_dev
from precision_optimizer_step_amd import opt8
from workloads import gen

pytestmark = pytest.mark.gpu

M8, MB, MF = oracle.MODE_8BIT, oracle.MODE_BF16_SR, oracle.MODE_FP32


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


def _bf16(rng, n, sigma):
    return gen.to_bf16_bits((rng.standard_normal(n) * sigma).astype(np.float32))


def _state(mode, n, tid, one_state):
    if mode == M8:
        m, v, am, av = gen.random_state_8bit(31, tid, n)
    elif mode == MB:
        m, v = gen.random_state_bf16(31, tid, n)
        am = av = None
    else:
        m, v = gen.random_state_f32(31, tid, n)
        am = av = None
    if one_state:
        v = av = None
    return m, v, am, av


# index bases: the group counter's low word wraps inside the second block
# (j/8 passes 2^32 at j = 2^35), a base far above it, and the largest base the
# library accepts
BASES = [(1 << 35) - 2048, (1 << 40) + 5 * 2048, 1 << 60]


@pytest.mark.parametrize("algo,state_round", [(0, 0), (0, 1), (oracle.ALGO_LION, 1),
                                              (oracle.ALGO_MOMENTUM, 0)])
def test_group_counter_above_32_bits(algo, state_round):
    rng = np.random.default_rng(40 + 3 * algo + state_round)
    one_state = algo != 0
    sets, states = [], []
    tid = 0
    for base in BASES:
        for mode, n in ((M8, 3 * 2048 + 100), (M8, 2048 + 40), (MB, 2 * 2048 + 9), (MF, 1000)):
            p, g = _bf16(rng, n, 0.02), _bf16(rng, n, 1e-3)
            m, v, am, av = _state(mode, n, tid, one_state)
            sets.append(DevTensorSet(mode, p, g, m, v, am, av, tensor_id=500 + tid, index_base=base))
            states.append([p, m, v, am, av])
            tid += 1
    stats = {}
    for param_round in (oracle.ROUND_STOCHASTIC, oracle.ROUND_NEAREST):
        hp = oracle.Hparams(lr=1e-3, beta2=0.99 if one_state else 0.999, weight_decay=0.1, step=5,
                            seed=0x0123456789ABCDEF, param_round=param_round, state_round=state_round)
        log(f"large index bases: algo {algo} state_round {state_round} param_round {param_round}, "
            f"{len(sets)} tensors")
        gpu_step(sets, hp, algo)
        for s, st in zip(sets, states):
            want = oracle_step(s, st, hp, algo)
            compare_state(f"base {s.index_base}/t{s.tensor_id}", s.read(), want, s.mode, stats)
        # restore the inputs so both roundings start from the same state
        for s, (p, m, v, am, av) in zip(sets, states):
            for dst, src in ((s.P, p), (s.M, m), (s.V, v), (s.AM, am), (s.AV, av)):
                if dst is not None:
                    dst.copy_(to_dev(src))
    log(f"large index bases: mismatching elements {sum(stats.values())}")


@pytest.mark.parametrize("mode", [M8, MB])
def test_tensor_beyond_2_to_31_elements(mode):
    n = (1 << 31) + 2 * BLOCK + 777
    nb = (n + BLOCK - 1) // BLOCK
    dev = torch.device("cuda:0")
    log(f"tensor of {n} elements, mode {mode}: building on the device")
    gsd = torch.Generator(device=dev)
    gsd.manual_seed(20261202 + mode)
    P = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_(0, 0.02, generator=gsd)
    G = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_(0, 1e-3, generator=gsd)
    AM = AV = None
    if mode == M8:
        M = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev, generator=gsd)
        V = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev, generator=gsd)
        AM = torch.empty(nb, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=gsd).abs_()
        AV = torch.empty(nb, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=gsd).square_()
    else:
        M = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_(0, 1e-3, generator=gsd)
        V = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_(0, 1e-3, generator=gsd).square_()
    lst = [dict(tid=3, mode=mode, n=n, P=P, G=G, M=M, V=V, AM=AM, AV=AV)]
    # blocks on both sides of element 2^31 (block 2^20), the last full block and the tail
    half = (1 << 31) // BLOCK
    blocks = [(0, b) for b in (0, 1, half - 1, half, half + 1, nb - 2, nb - 1)]
    before = snapshot(lst, blocks)
    hp = oracle.Hparams(lr=1e-3, weight_decay=0.1, step=4, seed=99)
    arr = opt8.tensor_array([opt8.make_tensor(P, G, M, V, AM, AV, tensor_id=3, mode=mode)])
    opt8.opt8_adamw_step(arr, opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                                                hp.step, hp.seed))
    torch.cuda.synchronize()
    after = snapshot(lst, blocks)
    log(f"tensor of {n} elements: stepped; checking blocks {[b for _, b in blocks]}")
    stats = {}
    for (_, b), x, y in zip(blocks, before, after):
        want = oracle.step_tensor(mode, x["p"], x["g"], x["m"], x["v"], x["am"], x["av"], hp,
                                  tensor_id=3, index_base=b * BLOCK)
        compare_state(f"2^31+/b{b}", [y["p"], y["m"], y["v"], y["am"], y["av"]], want, mode, stats)
    log(f"tensor of {n} elements: mismatching elements {sum(stats.values())}")
    del P, G, M, V, AM, AV, lst, arr
    torch.cuda.empty_cache()
