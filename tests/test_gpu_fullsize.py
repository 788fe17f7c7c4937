"""Full-size parameter lists on the GPU, checked on sampled blocks.

The whole list (up to the 6.7B-shaped one, ~40 GB resident) is stepped in one
call, the launch the benchmark times.  The inputs of sampled blocks are copied
to the host before the step; the oracle then steps each sampled block alone
(blocks are independent: the block absmax never crosses a block and the random
bits depend on the global element index), and its outputs are compared with
the GPU's for those blocks.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import compare_state, log
from precision_optimizer_step_amd import opt8
from workloads import gen, shapes

pytestmark = pytest.mark.gpu

BLOCK = 2048


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


def _mode_of(w, spec):
    if w.state_mode == "bf16":
        return oracle.MODE_BF16_SR
    return opt8.opt8_default_mode(spec.numel)


def build_list(w, step=1, state_seed=7):
    """Device tensors of workload w: params, step-`step` grads and a random non-zero state."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    out = []
    for tid, spec in enumerate(w.tensors):
        n = spec.numel
        mode = _mode_of(w, spec)
        P = torch.empty(n, dtype=torch.bfloat16, device=dev)
        G = torch.empty(n, dtype=torch.bfloat16, device=dev)
        gen.param_init_device(spec, w, tid, P)
        gen.grad_init_device(spec, w, step, tid, G)
        g.manual_seed(gen.derived_seed(state_seed, 0, tid, gen.P_STATE_M))
        AM = AV = None
        if mode == oracle.MODE_8BIT:
            M = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev, generator=g)
            V = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev, generator=g)
            nb = (n + BLOCK - 1) // BLOCK
            AM = torch.empty(nb, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=g).abs_()
            AV = torch.empty(nb, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=g).square_()
        elif mode == oracle.MODE_BF16_SR:
            M = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_(0, 1e-3, generator=g)
            V = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_(0, 1e-3, generator=g).square_()
        else:
            M = torch.empty(n, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=g)
            V = torch.empty(n, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=g).square_()
        out.append(dict(tid=tid, mode=mode, n=n, P=P, G=G, M=M, V=V, AM=AM, AV=AV))
    return out


def descriptors(lst):
    return opt8.tensor_array(opt8.make_tensor(t["P"], t["G"], t["M"], t["V"], t["AM"], t["AV"],
                                              tensor_id=t["tid"], mode=t["mode"]) for t in lst)


def sample_blocks(lst, per_tensor, rng):
    pick = []
    for i, t in enumerate(lst):
        nb = (t["n"] + BLOCK - 1) // BLOCK
        cand = {0, nb - 1}
        if nb > 2:
            cand |= set(int(x) for x in rng.integers(1, nb - 1, min(per_tensor, nb - 2)))
        pick += [(i, b) for b in sorted(cand)]
    return pick


def _np(t, dtype):
    h = t.detach().cpu()
    if h.dtype == torch.bfloat16:
        h = h.view(torch.int16)
    return h.numpy().view(dtype).copy()


def snapshot(lst, blocks):
    snap = []
    for i, b in blocks:
        t = lst[i]
        lo, hi = b * BLOCK, min(t["n"], (b + 1) * BLOCK)
        sd = np.uint8 if t["mode"] == oracle.MODE_8BIT else np.uint16 if t["mode"] == oracle.MODE_BF16_SR \
            else np.float32
        item = dict(p=_np(t["P"][lo:hi], np.uint16), g=_np(t["G"][lo:hi], np.uint16),
                    m=_np(t["M"][lo:hi], sd), v=_np(t["V"][lo:hi], sd), am=None, av=None)
        if t["AM"] is not None:
            item["am"] = _np(t["AM"][b:b + 1], np.float32)
            item["av"] = _np(t["AV"][b:b + 1], np.float32)
        snap.append(item)
    return snap


@pytest.mark.parametrize("name", ["gptneo-6.7b", "gptneo-2.7b", "gptneo-2.7b-bf16", "lm-1.5b", "gpt2-350m"])
def test_full_size_list_on_sampled_blocks(name):
    w = shapes.get(name)
    log(f"{name}: building {len(w.tensors)} tensors, {w.numel} elements on the device")
    lst = build_list(w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    blocks = sample_blocks(lst, 2, rng)
    before = snapshot(lst, blocks)
    hp = oracle.Hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                        weight_decay=w.weight_decay, step=2, seed=w.seed)
    arr = descriptors(lst)
    opt8.opt8_adamw_step(arr, opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                                                hp.step, hp.seed))
    torch.cuda.synchronize()
    after = snapshot(lst, blocks)
    log(f"{name}: stepped; checking {len(blocks)} sampled blocks against the oracle")
    stats = {}
    for (i, b), x, y in zip(blocks, before, after):
        t = lst[i]
        want = oracle.step_tensor(t["mode"], x["p"], x["g"], x["m"], x["v"], x["am"], x["av"], hp,
                                  tensor_id=t["tid"], index_base=b * BLOCK)
        got = [y["p"], y["m"], y["v"], y["am"], y["av"]]
        compare_state(f"{name}/t{t['tid']}/b{b}", got, want, t["mode"], stats)
    log(f"{name}: mismatching elements over sampled blocks: {sum(stats.values())}")
    del lst, arr
    torch.cuda.empty_cache()
