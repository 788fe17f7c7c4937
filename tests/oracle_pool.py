"""The CPU oracle over independent runs of 2048-element blocks, in worker processes.

Test infrastructure.  Blocks are independent (a block's absmax never crosses
it, and the random bits depend on the global element index only), so a run
of consecutive blocks of a tensor, given its index_base, is stepped exactly
as inside the whole tensor.  Workers are spawned (they import numpy and the
oracle, never torch or the GPU library) and receive plain numpy arrays.
"""

import multiprocessing as mp
import os

import numpy as np

BLOCK = 2048


def _work(item):
    import oracle
    algo, mode, hp_fields, p, g, m, v, am, av, tid, base = item
    hp = oracle.Hparams(**hp_fields)
    if algo == 0:
        return oracle.step_tensor(mode, p, g, m, v, am, av, hp, tid, base)
    p2, m2, am2 = oracle.step_tensor_1state(algo, mode, p, g, m, am, hp, tid, base)
    return p2, m2, None, am2, None


class OraclePool:
    """pool.step(items) -> list of (param, m, v, absmax_m, absmax_v) per item, in order."""

    def __init__(self, workers=None):
        n = workers or min(12, os.cpu_count() or 1)
        self.pool = mp.get_context("spawn").Pool(n)

    def step(self, items, chunksize=1):
        return self.pool.map(_work, items, chunksize=chunksize)

    def close(self):
        self.pool.close()
        self.pool.join()


def hp_fields(hp):
    return dict(lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps, weight_decay=hp.weight_decay,
                step=hp.step, seed=hp.seed, param_round=hp.param_round, state_round=hp.state_round)


def runs(blocks):
    """Sorted block numbers -> list of (first, count) runs of consecutive blocks."""
    out = []
    for b in blocks:
        if out and out[-1][0] + out[-1][1] == b:
            out[-1][1] += 1
        else:
            out.append([b, 1])
    return [(a, c) for a, c in out]


def split_runs(rs, max_blocks):
    """Cut runs into pieces of at most max_blocks blocks (for load balance)."""
    out = []
    for a, c in rs:
        while c > max_blocks:
            out.append((a, max_blocks))
            a += max_blocks
            c -= max_blocks
        out.append((a, c))
    return out
