"""The worker-pool helper of the full-size GPU tests, on the CPU: runs of sampled
blocks stepped alone (with their index_base) equal the same blocks of the whole
tensor stepped at once, in every state mode."""

import numpy as np

import oracle
from oracle_pool import OraclePool, hp_fields, runs, split_runs
from workloads import gen


def test_runs_and_split():
    assert runs([0, 1, 2, 5, 7, 8]) == [(0, 3), (5, 1), (7, 2)]
    assert split_runs([(0, 5), (9, 2)], 2) == [(0, 2), (2, 2), (4, 1), (9, 2)]


def test_pool_steps_runs_of_blocks_like_the_whole_tensor():
    n = 7 * 2048 + 301
    rng = np.random.default_rng(4)
    p = gen.to_bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    g = gen.to_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
    hp = oracle.Hparams(lr=1e-3, weight_decay=0.1, step=3, seed=9)
    picked = [0, 2, 3, 4, 7]                      # with the partial last block
    pool = OraclePool(2)
    try:
        for mode in (oracle.MODE_8BIT, oracle.MODE_BF16_SR, oracle.MODE_FP32):
            if mode == oracle.MODE_8BIT:
                m, v, am, av = gen.random_state_8bit(1, 0, n)
            elif mode == oracle.MODE_BF16_SR:
                (m, v), am, av = gen.random_state_bf16(1, 0, n), None, None
            else:
                (m, v), am, av = gen.random_state_f32(1, 0, n), None, None
            whole = oracle.step_tensor(mode, p, g, m, v, am, av, hp, 5)
            items, spans = [], []
            for a, c in split_runs(runs(picked), 2):
                e0, e1 = a * 2048, min(n, (a + c) * 2048)
                items.append((0, mode, hp_fields(hp), p[e0:e1], g[e0:e1], m[e0:e1], v[e0:e1],
                              None if am is None else am[a:a + c], None if av is None else av[a:a + c],
                              5, e0))
                spans.append((a, c, e0, e1))
            for (a, c, e0, e1), r in zip(spans, pool.step(items)):
                for k, x in enumerate(r):
                    if x is None:
                        continue
                    ref = whole[k][a:a + c] if k >= 3 else whole[k][e0:e1]
                    assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(ref).view(np.uint8)), (mode, a, k)
    finally:
        pool.close()
