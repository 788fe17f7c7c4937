"""bench.py's host-side contract, on the CPU: the one-GPU guard, the algorithmic byte counts
the roofline divides by, and how committed profiles are matched to a kernel build."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    out = json.loads(res.stdout.strip().splitlines()[-1])
    assert out["n_gpus"] == n and "one GPU" in out["error"]


def test_algorithmic_bytes_per_mode():
    """8-bit: grad 2 + param 2 + codes 1 + 1 read, param 2 + codes 1 + 1 written per element,
    and both absmax values read and written once per 2048-element block (a partial last block
    counts as a block); bf16 state 14 B, fp32 state 22 B per element; the one-state rules drop
    v and its absmax."""
    B = bench.BLOCK
    assert bench.algorithmic_bytes(0, B) == 10 * B + 16
    assert bench.algorithmic_bytes(0, B + 1) == 10 * (B + 1) + 32
    assert bench.algorithmic_bytes(0, 1) == 10 + 16
    assert bench.algorithmic_bytes(1, 1000) == 14 * 1000
    assert bench.algorithmic_bytes(2, 1000) == 22 * 1000
    assert bench.algorithmic_bytes(0, 3 * B, one_state=True) == 8 * 3 * B + 3 * 8
    assert bench.algorithmic_bytes(1, 1000, one_state=True) == 10 * 1000
    assert bench.algorithmic_bytes(2, 1000, one_state=True) == 14 * 1000


def test_the_headline_list_moves_66_6_gb_per_step():
    from workloads import shapes
    w = shapes.get("gptneo-6.7b")
    total = sum(bench.algorithmic_bytes(0, t.numel) for t in w.tensors)
    assert sum(t.numel for t in w.tensors) == 6_658_404_352
    assert total == 66_636_062_304


def test_profiled_traffic_only_for_the_matching_build(tmp_path, monkeypatch):
    """A summary is used only when kernel, workload and kernel-build fingerprint all match."""
    from precision_optimizer_step_amd.build import kernel_fingerprint
    prof = tmp_path / "profiles"
    prof.mkdir()
    fp = kernel_fingerprint()

    def summary(name, fingerprint, kernel="step_kernel<8bit>", workload="w1"):
        (prof / name).write_text("text\n```\nbench-traffic\n"
                                 f"kernel: {kernel}\nworkload: {workload}\nfingerprint: {fingerprint}\n"
                                 "traffic_bytes: 123\nvalu_issue_frac: 0.5\n```\n")
    summary("a.md", "0" * 64)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("step_kernel<8bit>", "w1") is None      # another build
    summary("b.md", fp)
    assert bench.profiled_traffic("step_kernel<8bit>", "w1") == 123.0
    assert bench.profiled_traffic("step_kernel<8bit>", "w1", "valu_issue_frac") == 0.5
    assert bench.profiled_traffic("step_kernel<8bit>", "w2") is None      # another workload
    assert bench.profiled_traffic("step_kernel<bf16>", "w1") is None      # another kernel
