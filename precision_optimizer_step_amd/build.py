"""Builds libopt8.so (host C++ + gfx950 HIP kernels) in this package directory.

    python -m precision_optimizer_step_amd.build
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libopt8.so")
SOURCES = [os.path.join(HERE, "csrc", "opt8_host.cpp"), os.path.join(HERE, "csrc", "opt8_tables.cpp"),
           os.path.join(HERE, "csrc", "opt8_kernels.hip"), os.path.join(HERE, "csrc", "opt8_map.hip")]
# bandwidth probe used by bench.py for the attainable-bandwidth context figure
PROBE_LIB = os.path.join(HERE, "libopt8_probe.so")
PROBE_SOURCES = [os.path.join(HERE, "csrc", "bw_probe.hip")]

# fp32 arithmetic must round once per operation exactly as written: no
# contraction into fused multiply-adds, IEEE sqrt/divide (hipcc's default),
# denormals kept (hipcc's default), no fast-math.  Packed fp32 instructions
# are switched off.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def kernel_fingerprint() -> str:
    """sha256 over the step kernels' sources, the table builder and the device compile flags
    (names the build of the kernels the profiles measure; the block-map fill in opt8_map.hip,
    a copy-sized kernel run when a list is uploaded, is not one of them)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("opt8_kernels.hip", "opt8_internal.h", "opt8_exact.h", "opt8_codes.h", "opt8_launch.h", "opt8_tables.cpp"):
        with open(os.path.join(HERE, "csrc", name), "rb") as f:
            h.update(f.read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libopt8.so")


def _compile(target: str, sources, verbose: bool) -> str:
    tmp = target + ".tmp"
    cmd = [hipcc(), *FLAGS, "-o", tmp, *sources]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(tmp, target)
    return target


def build(verbose: bool = False) -> str:
    """Compile libopt8.so and the bandwidth probe (always recompiles); returns libopt8's path."""
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return _compile(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
