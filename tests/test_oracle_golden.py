"""The oracle still produces its frozen fixtures (tests/golden, written by make_golden.py).

A failure here means the oracle's arithmetic changed; the commit that rewrites
the fixtures must name the passage or reading that justifies the change.
"""
import json
import os

import numpy as np

from oracle import codebook

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = os.path.join(HERE, "golden")


def test_codebooks_match_fixture():
    s, ms, u, mu = codebook.tables()
    rows = [ln.split() for ln in open(os.path.join(GOLD, "codebooks.txt")) if not ln.startswith("#")]
    assert len(rows) == 256
    for k, (idx, sh, smh, uh, umh) in enumerate(rows):
        assert int(idx) == k
        assert int(sh, 16) == int(s[k:k + 1].view(np.uint32)[0])
        assert int(uh, 16) == int(u[k:k + 1].view(np.uint32)[0])
        if k < 255:
            assert int(smh, 16) == int(ms[k:k + 1].view(np.uint32)[0])
            assert int(umh, 16) == int(mu[k:k + 1].view(np.uint32)[0])


def test_small_step_digests_match_fixture():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(GOLD, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    want = json.load(open(os.path.join(GOLD, "oracle_step_digests.json")))
    assert mod.small_steps() == want
