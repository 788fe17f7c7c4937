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
from gpu_helpers import BLOCK, build_list, compare_state, descriptors, log, sample_blocks, snapshot
from precision_optimizer_step_amd import opt8
from workloads import shapes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


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
