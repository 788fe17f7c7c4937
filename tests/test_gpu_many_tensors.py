"""GPU parity on a list of many small tensors.

Each wave of the grid strides over thousands of blocks at a time, so on a
list of small tensors every stride crosses many tensor descriptors; the
kernels find the tensor holding a block with a wave-parallel search.  This
test steps 20,000 small 8-bit tensors (most with a partial last block, so the
partial-block launch holds thousands of entries too) in one call and checks
sampled tensors, whole, against the oracle.
"""

import time

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BLOCK, compare_state, log
from precision_optimizer_step_amd import opt8

pytestmark = pytest.mark.gpu

M8 = oracle.MODE_8BIT


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


def _host(t, dtype):
    h = t.detach().cpu()
    if h.dtype == torch.bfloat16:
        h = h.view(torch.int16)
    return h.numpy().view(dtype).copy()


def test_many_small_tensors_in_one_list():
    rng = np.random.default_rng(21)
    n_t = 20000
    sizes = rng.choice([2048, 4096, 4097, 6151, 10000], size=n_t).astype(np.int64)
    # tensors carved from flat buffers at 16-element (16-byte for the codes) aligned offsets
    offs = np.zeros(n_t, np.int64)
    offs[1:] = np.cumsum((sizes[:-1] + 15) // 16 * 16)
    total = int(offs[-1] + sizes[-1])
    nblk = (sizes + BLOCK - 1) // BLOCK
    boffs = np.zeros(n_t, np.int64)
    boffs[1:] = np.cumsum(nblk[:-1])
    dev = torch.device("cuda:0")
    gsd = torch.Generator(device=dev)
    gsd.manual_seed(2112)
    P = torch.empty(total, dtype=torch.bfloat16, device=dev).normal_(0, 0.02, generator=gsd)
    G = torch.empty(total, dtype=torch.bfloat16, device=dev).normal_(0, 1e-3, generator=gsd)
    M = torch.randint(0, 256, (total,), dtype=torch.uint8, device=dev, generator=gsd)
    V = torch.randint(0, 256, (total,), dtype=torch.uint8, device=dev, generator=gsd)
    nb_all = int(nblk.sum())
    AM = torch.empty(nb_all, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=gsd).abs_()
    AV = torch.empty(nb_all, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=gsd).square_()
    descs = [opt8.make_tensor(P.data_ptr() + 2 * int(o), G.data_ptr() + 2 * int(o), M.data_ptr() + int(o),
                              V.data_ptr() + int(o), AM.data_ptr() + 4 * int(bo), AV.data_ptr() + 4 * int(bo),
                              tensor_id=i, mode=M8, numel=int(n))
             for i, (o, bo, n) in enumerate(zip(offs, boffs, sizes))]
    arr = opt8.tensor_array(descs)
    picks = sorted(set([0, n_t - 1] + [int(x) for x in rng.integers(0, n_t, 40)]))

    def state(i):
        o, bo, n, nb = int(offs[i]), int(boffs[i]), int(sizes[i]), int(nblk[i])
        return [_host(P[o:o + n], np.uint16), _host(M[o:o + n], np.uint8), _host(V[o:o + n], np.uint8),
                _host(AM[bo:bo + nb], np.float32), _host(AV[bo:bo + nb], np.float32)]

    before = {i: state(i) for i in picks}
    grads = {i: _host(G[int(offs[i]):int(offs[i]) + int(sizes[i])], np.uint16) for i in picks}
    hp = oracle.Hparams(lr=1e-3, weight_decay=0.1, step=6, seed=31337)
    log(f"many small tensors: {n_t} tensors, {total} elements, {nb_all} blocks")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    opt8.opt8_adamw_step(arr, opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step,
                                                hp.seed))
    torch.cuda.synchronize()
    log(f"many small tensors: stepped in {1000 * (time.perf_counter() - t0):.2f} ms (first call, with upload)")
    stats = {}
    for i in picks:
        p, m, v, am, av = before[i]
        want = oracle.step_tensor(M8, p, grads[i], m, v, am, av, hp, tensor_id=i)
        compare_state(f"many/t{i}", state(i), want, M8, stats)
    log(f"many small tensors: {len(picks)} tensors checked, mismatching elements {sum(stats.values())}")
    del P, G, M, V, AM, AV, arr
    torch.cuda.empty_cache()
