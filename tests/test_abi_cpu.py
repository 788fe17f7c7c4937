"""The C ABI without a GPU: symbols, struct layout, host-side tables and validation.

No compute call reaches a device here: every call either fails validation
before any HIP call or stops at the device query.
"""

import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from oracle import codebook
from precision_optimizer_step_amd import opt8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "opt8.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(opt8.LIB_PATH):
        pytest.fail("libopt8.so is not built (run __graft_entry__.build())")
    return opt8.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(opt8_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert names == ["opt8_adamw_step", "opt8_adamw_step_noalloc", "opt8_default_mode", "opt8_init_codebooks",
                     "opt8_last_error", "opt8_lion_step", "opt8_momentum_step"]
    out = subprocess.run(["nm", "-D", "--defined-only", opt8.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (opt8_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_struct_layout_matches_header(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "probe.c"
    fields_t = [f for f, _ in opt8.opt8_tensor._fields_]
    fields_h = [f for f, _ in opt8.opt8_hparams._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    lines.append('printf("%zu %zu\\n", sizeof(opt8_tensor), sizeof(opt8_hparams));')
    for f in fields_t:
        lines.append(f'printf("t {f} %zu\\n", offsetof(opt8_tensor, {f}));')
    for f in fields_h:
        lines.append(f'printf("h {f} %zu\\n", offsetof(opt8_hparams, {f}));')
    lines.append("return 0;}")
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    st, sh = (int(x) for x in out[0].split())
    assert st == ctypes.sizeof(opt8.opt8_tensor) == 72
    assert sh == ctypes.sizeof(opt8.opt8_hparams) == 64
    for line in out[1:]:
        if not line:
            continue
        kind, name, off = line.split()
        cls = opt8.opt8_tensor if kind == "t" else opt8.opt8_hparams
        assert getattr(cls, name).offset == int(off), name


def test_constants_match_header(tmp_path):
    """Every enum constant and macro of the header has the binding's value."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    text = open(HEADER).read()
    names = sorted(set(re.findall(r"\b(OPT8_[A-Z0-9_]+)\s*=", text)) |
                   set(re.findall(r"#define\s+(OPT8_[A-Z0-9_]+)\s+\d", text)))
    assert "OPT8_E_CAPTURE" in names and "OPT8_BLOCK" in names
    src = tmp_path / "consts.c"
    lines = ['#include <stdio.h>', f'#include "{HEADER}"', "int main(void){"]
    lines += [f'printf("{n} %ld\\n", (long){n});' for n in names]
    lines.append("return 0;}")
    src.write_text("\n".join(lines))
    exe = tmp_path / "consts"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    got = dict(zip(out[0::2], (int(x) for x in out[1::2])))
    assert len(got) == len(names)
    for n, val in got.items():
        assert getattr(opt8, n) == val, n
    for val in (v for n, v in got.items() if n.startswith("OPT8_E_")):
        assert val in opt8.STATUS_NAMES


def test_default_mode_threshold(L):
    assert opt8.opt8_default_mode(1) == opt8.OPT8_STATE_FP32
    assert opt8.opt8_default_mode(4095) == opt8.OPT8_STATE_FP32
    assert opt8.opt8_default_mode(4096) == opt8.OPT8_STATE_8BIT
    assert opt8.opt8_default_mode(10 ** 10) == opt8.OPT8_STATE_8BIT


def test_host_codebooks_equal_the_oracle_bit_for_bit(L):
    s = np.zeros(256, np.float32)
    u = np.zeros(256, np.float32)
    rc = opt8.opt8_init_codebooks(s, u, check=False)
    assert rc in (opt8.OPT8_OK, opt8.OPT8_E_HIP)
    os_, _, ou, _ = codebook.tables()
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(u.view(np.uint32), ou.view(np.uint32))


# ----------------------------------------------------------------------------- validation
BASE = 0x7F0000000000


def fake_tensor(i, numel=4096 + 100, mode=opt8.OPT8_STATE_8BIT, tid=None, **over):
    """Descriptor with distinct, aligned, never-dereferenced addresses."""
    base = BASE + i * (1 << 32)
    d = dict(param=base, grad=base + (1 << 28), m=base + (2 << 28), v=base + (3 << 28),
             absmax_m=base + (4 << 28), absmax_v=base + (5 << 28), numel=numel,
             index_base=0, tensor_id=i if tid is None else tid, mode=mode)
    d.update(over)
    return opt8.opt8_tensor(**d)


def step(descs, hp=None, n=None):
    hp = hp or opt8.make_hparams(1e-3, weight_decay=0.01, step=1, seed=1)
    arr = opt8.tensor_array(descs)
    return opt8.opt8_adamw_step(arr, hp, stream=0, n=n, check=False)


def expect(rc, status, fragment=""):
    assert rc == status, (rc, opt8.opt8_last_error())
    msg = opt8.opt8_last_error()
    assert msg, "an error must leave a message"
    assert fragment in msg, msg


def test_null_and_size_errors(L):
    hp = opt8.make_hparams(1e-3)
    assert L.opt8_adamw_step(None, 0, ctypes.byref(hp), None) == opt8.OPT8_OK
    expect(L.opt8_adamw_step(None, 1, ctypes.byref(hp), None), opt8.OPT8_E_NULL, "list")
    expect(L.opt8_adamw_step(None, 0, None, None), opt8.OPT8_E_NULL, "hparams")
    expect(step([fake_tensor(0)], n=-1), opt8.OPT8_E_SIZE)
    expect(step([fake_tensor(0, param=None)]), opt8.OPT8_E_NULL, "tensor 0")
    expect(step([fake_tensor(0), fake_tensor(1, absmax_v=None)]), opt8.OPT8_E_NULL, "tensor 1")
    expect(step([fake_tensor(0, numel=0)]), opt8.OPT8_E_SIZE)
    expect(step([fake_tensor(0, numel=-5)]), opt8.OPT8_E_SIZE)
    expect(step([fake_tensor(0, numel=(1 << 42) + 1)]), opt8.OPT8_E_SIZE, "2^42")
    # at the bound the size check passes and validation goes on (to the missing device / init)
    rc = step([fake_tensor(0, numel=1 << 42, param=1 << 50, grad=2 << 50, m=3 << 50, v=4 << 50,
                           absmax_m=5 << 50, absmax_v=6 << 50)])
    assert rc in (opt8.OPT8_E_HIP, opt8.OPT8_E_NOT_INIT), opt8.opt8_last_error()
    expect(step([fake_tensor(0, index_base=1024)]), opt8.OPT8_E_SIZE, "index_base")
    expect(step([fake_tensor(0, index_base=-2048)]), opt8.OPT8_E_SIZE)


def test_non_8bit_modes_do_not_need_absmax(L):
    rc = step([fake_tensor(0, mode=opt8.OPT8_STATE_FP32, absmax_m=None, absmax_v=None),
               fake_tensor(1, mode=opt8.OPT8_STATE_BF16_SR, absmax_m=None, absmax_v=None)])
    assert rc in (opt8.OPT8_E_HIP, opt8.OPT8_E_NOT_INIT), opt8.opt8_last_error()


def test_alignment_errors(L):
    expect(step([fake_tensor(0, param=BASE + 8)]), opt8.OPT8_E_ALIGN)
    expect(step([fake_tensor(0, grad=BASE + (1 << 28) + 2)]), opt8.OPT8_E_ALIGN)
    expect(step([fake_tensor(0, m=BASE + (2 << 28) + 1)]), opt8.OPT8_E_ALIGN)
    expect(step([fake_tensor(0, absmax_m=BASE + (4 << 28) + 2)]), opt8.OPT8_E_ALIGN)


def test_mode_errors(L):
    expect(step([fake_tensor(0, mode=3)]), opt8.OPT8_E_MODE)
    expect(step([fake_tensor(0, mode=-1)]), opt8.OPT8_E_MODE)
    expect(step([fake_tensor(0)], hp=opt8.make_hparams(1e-3, param_round=2)), opt8.OPT8_E_MODE)


@pytest.mark.parametrize("bad", [dict(lr=-1e-3), dict(lr=float("nan")), dict(beta1=1.0),
                                 dict(beta2=-0.1), dict(eps=0.0), dict(eps=float("inf")),
                                 dict(weight_decay=-0.1), dict(step=0)])
def test_hparam_errors(L, bad):
    kw = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)
    kw.update(bad)
    expect(step([fake_tensor(0)], hp=opt8.make_hparams(**kw)), opt8.OPT8_E_HPARAM)
    hp = opt8.make_hparams(1e-3, state_round=2)
    expect(step([fake_tensor(0)], hp=hp), opt8.OPT8_E_MODE, "state_round")


def test_alias_and_duplicate_id_errors(L):
    a = fake_tensor(0)
    # second tensor's m starts inside the first tensor's param range
    b = fake_tensor(1, m=BASE + 4096)
    expect(step([a, b]), opt8.OPT8_E_ALIAS, "overlap")
    # m and v of one tensor overlap
    expect(step([fake_tensor(0, v=BASE + (2 << 28) + 16)]), opt8.OPT8_E_ALIAS)
    # fp32 state needs 4 bytes per element: an m that fits as u8 overlaps as f32
    c = fake_tensor(0, mode=opt8.OPT8_STATE_FP32, v=BASE + (2 << 28) + 4 * 4196 - 16)
    expect(step([c]), opt8.OPT8_E_ALIAS)
    expect(step([fake_tensor(0, tid=7), fake_tensor(1, tid=7)]), opt8.OPT8_E_DUPID, "7")


def test_valid_call_without_a_device_stops_before_any_work(L):
    rc = step([fake_tensor(0), fake_tensor(1, mode=opt8.OPT8_STATE_FP32, numel=100)])
    assert rc in (opt8.OPT8_E_HIP, opt8.OPT8_E_NOT_INIT)
    assert opt8.opt8_last_error()


def test_binding_raises_on_error(L):
    with pytest.raises(opt8.Opt8Error) as e:
        opt8.opt8_adamw_step([fake_tensor(0, numel=0)], opt8.make_hparams(1e-3), stream=0)
    assert e.value.status == opt8.OPT8_E_SIZE


ONE_STATE = [("opt8_lion_step", opt8.opt8_lion_step), ("opt8_momentum_step", opt8.opt8_momentum_step)]


@pytest.mark.parametrize("name,fn", ONE_STATE)
def test_one_state_rules_ignore_v_and_eps(L, name, fn):
    """Lion and momentum accept NULL v / absmax_v, overlapping garbage in v, and eps = 0;
    everything else is validated as for AdamW."""
    def run(descs, hp=None, n=None):
        hp = hp or opt8.make_hparams(1e-4, weight_decay=0.1, step=1, seed=1)
        return fn(opt8.tensor_array(descs), hp, stream=0, n=n, check=False)
    ok = (opt8.OPT8_E_HIP, opt8.OPT8_E_NOT_INIT)
    rc = run([fake_tensor(0, v=None, absmax_v=None), fake_tensor(1, mode=opt8.OPT8_STATE_FP32, numel=100,
                                                               v=None, absmax_v=None)])
    assert rc in ok, opt8.opt8_last_error()
    # v is not read: an address overlapping m is not an alias
    assert run([fake_tensor(0, v=BASE + (2 << 28))]) in ok, opt8.opt8_last_error()
    assert run([fake_tensor(0)], hp=opt8.make_hparams(1e-4, eps=0.0)) in ok, opt8.opt8_last_error()
    expect(run([fake_tensor(0, m=None)]), opt8.OPT8_E_NULL, "tensor 0")
    expect(run([fake_tensor(0, absmax_m=None)]), opt8.OPT8_E_NULL, "absmax_m")
    expect(run([fake_tensor(0, m=BASE + (2 << 28) + 1)]), opt8.OPT8_E_ALIGN)
    expect(run([fake_tensor(0, m=BASE + 4096)]), opt8.OPT8_E_ALIAS)
    expect(run([fake_tensor(0, tid=3), fake_tensor(1, tid=3)]), opt8.OPT8_E_DUPID)
    expect(run([fake_tensor(0)], hp=opt8.make_hparams(-1.0)), opt8.OPT8_E_HPARAM)
    expect(run([fake_tensor(0)], hp=opt8.make_hparams(1e-4, beta1=1.0)), opt8.OPT8_E_HPARAM)
    expect(run([fake_tensor(0)], hp=opt8.make_hparams(1e-4, step=0)), opt8.OPT8_E_HPARAM)
    expect(run([fake_tensor(0, mode=7)]), opt8.OPT8_E_MODE)
    assert run([], n=0) == opt8.OPT8_OK


# ----------------------------------------------------------------------------- binding checks
def _bufs(n=5000, mode=opt8.OPT8_STATE_8BIT, one_state=False):
    import torch
    nb = (n + 2047) // 2048
    sd = {opt8.OPT8_STATE_8BIT: torch.uint8, opt8.OPT8_STATE_BF16_SR: torch.bfloat16,
          opt8.OPT8_STATE_FP32: torch.float32}[mode]
    b = dict(param=torch.zeros(n, dtype=torch.bfloat16), grad=torch.zeros(n, dtype=torch.bfloat16),
             m=torch.zeros(n, dtype=sd), v=None if one_state else torch.zeros(n, dtype=sd),
             absmax_m=None, absmax_v=None)
    if mode == opt8.OPT8_STATE_8BIT:
        b["absmax_m"] = torch.zeros(nb, dtype=torch.float32)
        if not one_state:
            b["absmax_v"] = torch.zeros(nb, dtype=torch.float32)
    return b


def _refused(match, mode=opt8.OPT8_STATE_8BIT, **over):
    b = _bufs(mode=mode, one_state=over.pop("one_state", False))
    b.update(over)
    numel = b.pop("numel", None)
    with pytest.raises(ValueError, match=match):
        opt8.make_tensor(mode=mode, numel=numel, **b)


def test_make_tensor_refuses_mismatched_buffers():
    """Every check make_tensor runs on torch buffers before building a descriptor: the
    kernels trust the sizes, so a wrong dtype, length, layout or device must stop here."""
    import torch
    n = 5000
    M8, BF, F32 = opt8.OPT8_STATE_8BIT, opt8.OPT8_STATE_BF16_SR, opt8.OPT8_STATE_FP32
    # dtype per mode
    _refused("param: dtype", param=torch.zeros(n, dtype=torch.float32))
    _refused("grad: dtype", grad=torch.zeros(n, dtype=torch.float16))
    _refused("m: dtype", m=torch.zeros(n, dtype=torch.float32))               # fp32 state in 8-bit mode
    _refused("v: dtype", mode=BF, v=torch.zeros(n, dtype=torch.uint8))        # codes in bf16 mode
    _refused("m: dtype", mode=F32, m=torch.zeros(n, dtype=torch.uint8))       # the 4x overrun case
    _refused("absmax_m: dtype", absmax_m=torch.zeros(3, dtype=torch.float64))
    # sizes
    _refused("grad: holds 4999", grad=torch.zeros(n - 1, dtype=torch.bfloat16))
    _refused("v: holds 100", v=torch.zeros(100, dtype=torch.uint8))
    _refused("absmax_v: holds 2", absmax_v=torch.zeros(2, dtype=torch.float32))
    _refused("param: holds 5000", numel=n + 1)
    # layout
    _refused("m: must be contiguous", m=torch.zeros(2 * n, dtype=torch.uint8)[::2])
    # missing absmax in 8-bit mode
    _refused("absmax_m: required", absmax_m=None)
    _refused("absmax_v: required", absmax_v=None)
    # device: CPU buffers are refused last, so every check above ran on them
    _refused("runs on a GPU")
    _refused("runs on a GPU", mode=BF)
    _refused("runs on a GPU", mode=F32)
    _refused("runs on a GPU", one_state=True)
    with pytest.raises(ValueError, match="unknown state mode"):
        opt8.make_tensor(**_bufs(), mode=7)
    # int16 views of bf16 data and uint16 patterns pass the dtype checks
    b = _bufs(mode=BF)
    b["param"] = b["param"].view(torch.int16)
    b["m"] = b["m"].view(torch.int16)
    with pytest.raises(ValueError, match="runs on a GPU"):
        opt8.make_tensor(mode=BF, **b)
    # raw addresses are passed through unchecked
    d = opt8.make_tensor(1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40, 6 << 40, numel=n)
    assert d.numel == n and d.param == 1 << 40


def test_c_driver_links_against_the_library_and_checks_its_arguments():
    """The plain-C boundary driver (tests/c_abi/step_file.c) builds against include/opt8.h and
    libopt8.so, and refuses bad arguments before any HIP call (no GPU needed)."""
    exe = os.path.join(ROOT, "tests", "c_abi", "step_file")
    if not os.path.exists(exe):
        pytest.fail(f"{exe} is not built (run __graft_entry__.build())")
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 2 and "usage" in out.stderr
    out = subprocess.run([exe, "/nonexistent", "100", "9", "0", "1", "0", "1e-3", "0", "0"],
                         capture_output=True, text=True, timeout=60)
    assert out.returncode == 2
    deps = subprocess.run(["ldd", exe], capture_output=True, text=True).stdout
    assert "libopt8.so" in deps and "not found" not in deps.split("libopt8.so", 1)[1].splitlines()[0]
