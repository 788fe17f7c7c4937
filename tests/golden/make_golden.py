"""Writes the oracle's golden fixtures in this folder.  Calls only oracle/ and workloads/.

The pages print no numeric worked example for this optimizer step, so the
fixtures here freeze the oracle's own tables and a few small steps: a later
change to the oracle's arithmetic shows up as a diff of these files, and the
commit that regenerates them must name the passage or reading that justifies it.

Run:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import codebook  # noqa: E402
from oracle.adamw import Hparams, step_tensor, MODE_8BIT, MODE_BF16_SR, MODE_FP32  # noqa: E402
from workloads import gen  # noqa: E402


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def small_steps():
    rng = np.random.default_rng(2024)
    n = 2048 * 2 + 37
    p = gen.to_bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    g = gen.to_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
    out = {}
    for mode, name in ((MODE_8BIT, "8bit"), (MODE_BF16_SR, "bf16"), (MODE_FP32, "fp32")):
        if mode == MODE_8BIT:
            m, v, am, av = gen.random_state_8bit(5, 1, n)
        elif mode == MODE_BF16_SR:
            (m, v), am, av = gen.random_state_bf16(5, 1, n), None, None
        else:
            (m, v), am, av = gen.random_state_f32(5, 1, n), None, None
        for rnd in (0, 1):
            hp = Hparams(lr=1e-3, weight_decay=0.01, step=3, seed=0xDEADBEEF12345678, param_round=rnd)
            res = step_tensor(mode, p, g, m, v, am, av, hp, tensor_id=17, index_base=4096)
            out[f"{name}_round{rnd}"] = digest(*[r for r in res if r is not None])
    return out


def main():
    s, ms, u, mu = codebook.tables()
    with open(os.path.join(HERE, "codebooks.txt"), "w") as f:
        f.write("# Dynamic-tree codebooks (oracle reading), fp32 bit patterns in hex.\n")
        f.write("# columns: index signed signed_mid unsigned unsigned_mid (mid of index 255 is '-')\n")
        for k in range(256):
            sm = "%08x" % int(ms[k:k + 1].view(np.uint32)[0]) if k < 255 else "-"
            um = "%08x" % int(mu[k:k + 1].view(np.uint32)[0]) if k < 255 else "-"
            f.write("%3d %08x %s %08x %s\n" % (k, int(s[k:k + 1].view(np.uint32)[0]), sm,
                                               int(u[k:k + 1].view(np.uint32)[0]), um))
    with open(os.path.join(HERE, "oracle_step_digests.json"), "w") as f:
        json.dump(small_steps(), f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
