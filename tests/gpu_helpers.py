"""Helpers of the GPU parity tests: host <-> device transfer through the C ABI binding,
and the comparison bar (bit-exact, with the stated allowance for fp32 ties)."""

import sys

import numpy as np
import torch

import oracle
from precision_optimizer_step_amd import opt8

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None

# Tolerance of the comparison: codes and bf16 values bit-exact except at most
# 1e-5 of the elements, which may differ by one code / one bf16 step (fp32 ties
# at a codebook midpoint or an SR threshold); block absmax within 1e-6 relative.
MAX_MISMATCH_FRACTION = 1e-5
ABSMAX_RTOL = 1e-6


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a).copy()).to(DEV)


def to_host(t: torch.Tensor, like: np.ndarray) -> np.ndarray:
    h = t.detach().cpu().numpy()
    return h.view(like.dtype) if h.dtype != like.dtype else h


class DevTensorSet:
    """One tensor's param/grad/state on the device, mirroring host numpy arrays."""

    def __init__(self, mode, param, grad, m, v, am=None, av=None, tensor_id=0, index_base=0):
        self.mode = mode
        self.tensor_id = tensor_id
        self.index_base = index_base
        self.host = [param, grad, m, v, am, av]
        self.P, self.G, self.M, self.V = (to_dev(x) for x in (param, grad, m, v))
        self.AM = to_dev(am) if am is not None else None
        self.AV = to_dev(av) if av is not None else None

    def set_grad(self, grad):
        self.G.copy_(to_dev(grad))
        self.host[1] = grad

    def desc(self):
        return opt8.make_tensor(self.P, self.G, self.M, self.V, self.AM, self.AV,
                                tensor_id=self.tensor_id, mode=self.mode, index_base=self.index_base)

    def read(self):
        p, g, m, v, am, av = self.host
        out = [to_host(self.P, p), to_host(self.M, m), to_host(self.V, v)]
        out.append(to_host(self.AM, am) if self.AM is not None else None)
        out.append(to_host(self.AV, av) if self.AV is not None else None)
        return out


def gpu_step(sets, hp: "oracle.Hparams"):
    descs = [s.desc() for s in sets]
    opt8.opt8_adamw_step(descs, opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                                                  hp.step, hp.seed, hp.param_round))
    torch.cuda.synchronize()


def oracle_step(s: DevTensorSet, state, hp):
    """state = (param, m, v, am, av) on the host; returns the oracle's next state."""
    p, m, v, am, av = state
    return list(oracle.step_tensor(s.mode, p, s.host[1], m, v, am, av, hp, s.tensor_id, s.index_base))


def _ulp_steps_16(a, b):
    """Distance in representable steps between bf16 patterns of the same sign."""
    sa = (a >> 15) & 1
    sb = (b >> 15) & 1
    mag = np.abs((a & 0x7FFF).astype(np.int64) - (b & 0x7FFF).astype(np.int64))
    return np.where(sa == sb, mag, (a & 0x7FFF).astype(np.int64) + (b & 0x7FFF).astype(np.int64))


def _ulp_steps_32(a, b):
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def compare(name, got, want, kind, stats=None):
    """Assert the bar; returns the mismatch count.  kind: bf16 | code | f32 | absmax."""
    assert got.shape == want.shape, (name, got.shape, want.shape)
    n = got.size
    if kind == "absmax":
        g = got.astype(np.float64)
        w = want.astype(np.float64)
        bad = np.abs(g - w) > ABSMAX_RTOL * np.abs(w)
        assert not bad.any(), f"{name}: {int(bad.sum())} absmax beyond 1e-6 relative, e.g. " \
            f"{g[bad][:3]} vs {w[bad][:3]}"
        diff = int(np.sum(got.view(np.uint32) != want.view(np.uint32)))
    else:
        if kind == "bf16":
            steps = _ulp_steps_16(got.astype(np.uint16), want.astype(np.uint16))
        elif kind == "code":
            steps = np.abs(got.astype(np.int64) - want.astype(np.int64))
        else:
            steps = _ulp_steps_32(got.astype(np.float32), want.astype(np.float32))
        diff = int(np.count_nonzero(steps))
        allowed = int(np.floor(MAX_MISMATCH_FRACTION * n))
        assert diff <= allowed, f"{name}: {diff} of {n} elements differ (allowed {allowed}); " \
            f"first at {np.flatnonzero(steps)[:5]}"
        assert int(steps.max(initial=0)) <= 1, f"{name}: a difference larger than one step"
    if stats is not None:
        stats[name] = stats.get(name, 0) + diff
    return diff


def compare_state(label, got, want, mode, stats=None):
    compare(f"{label}.param", got[0], want[0], "bf16", stats)
    if mode == oracle.MODE_8BIT:
        compare(f"{label}.m", got[1], want[1], "code", stats)
        compare(f"{label}.v", got[2], want[2], "code", stats)
        compare(f"{label}.absmax_m", got[3], want[3], "absmax", stats)
        compare(f"{label}.absmax_v", got[4], want[4], "absmax", stats)
    elif mode == oracle.MODE_BF16_SR:
        compare(f"{label}.m", got[1], want[1], "bf16", stats)
        compare(f"{label}.v", got[2], want[2], "bf16", stats)
    else:
        compare(f"{label}.m", got[1], want[1], "f32", stats)
        compare(f"{label}.v", got[2], want[2], "f32", stats)
