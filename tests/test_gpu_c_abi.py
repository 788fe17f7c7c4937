"""The boundary from plain C: one step through include/opt8.h and libopt8.so alone.

tests/c_abi/step_file.c (built with gcc by __graft_entry__.build(); no Python,
no torch) reads a tensor's inputs from files, allocates device memory with
hipMalloc, calls opt8_adamw_step or opt8_adamw_step_noalloc on the null stream
and writes the outputs back; they must match the oracle on the same inputs,
in all three state modes.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle
from gpu_helpers import compare_state, log
from workloads import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "step_file")

pytestmark = pytest.mark.gpu

DT = {oracle.MODE_8BIT: np.uint8, oracle.MODE_BF16_SR: np.uint16, oracle.MODE_FP32: np.float32}


def _inputs(mode, n, seed):
    rng = np.random.default_rng(seed)
    p = gen.to_bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    g = gen.to_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
    if mode == oracle.MODE_8BIT:
        m, v, am, av = gen.random_state_8bit(seed, 0, n)
    elif mode == oracle.MODE_BF16_SR:
        (m, v), am, av = gen.random_state_bf16(seed, 0, n), None, None
    else:
        (m, v), am, av = gen.random_state_f32(seed, 0, n), None, None
    return p, g, m, v, am, av


@pytest.mark.parametrize("noalloc", [0, 1])
@pytest.mark.parametrize("mode", [oracle.MODE_8BIT, oracle.MODE_BF16_SR, oracle.MODE_FP32])
def test_step_through_the_c_abi_alone(tmp_path, mode, noalloc):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built (run __graft_entry__.build())")
    n = 5 * 2048 + 333 if mode != oracle.MODE_FP32 else 3000
    p, g, m, v, am, av = _inputs(mode, n, seed=17 + mode)
    for name, a in (("param", p), ("grad", g), ("m", m), ("v", v), ("absmax_m", am), ("absmax_v", av)):
        if a is not None:
            np.ascontiguousarray(a).tofile(str(tmp_path / f"in_{name}.bin"))
    hp = oracle.Hparams(lr=1e-3, weight_decay=0.01, step=4, seed=2024)
    cmd = [EXE, str(tmp_path), str(n), str(mode), "9", str(hp.step), str(hp.seed), repr(hp.lr),
           repr(hp.weight_decay), str(noalloc)]
    log("running " + " ".join(cmd[1:]))
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    got = [np.fromfile(str(tmp_path / "out_param.bin"), dtype=np.uint16),
           np.fromfile(str(tmp_path / "out_m.bin"), dtype=DT[mode]),
           np.fromfile(str(tmp_path / "out_v.bin"), dtype=DT[mode]), None, None]
    if mode == oracle.MODE_8BIT:
        got[3] = np.fromfile(str(tmp_path / "out_absmax_m.bin"), dtype=np.float32)
        got[4] = np.fromfile(str(tmp_path / "out_absmax_v.bin"), dtype=np.float32)
    want = oracle.step_tensor(mode, p, g, m, v, am, av, hp, tensor_id=9)
    stats = {}
    compare_state(f"c-abi/mode{mode}/noalloc{noalloc}", got, want, mode, stats)
    assert sum(stats.values()) == 0
