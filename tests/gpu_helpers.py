"""Helpers of the GPU parity tests: host <-> device transfer through the C ABI binding,
and the comparison bar (bit-exact, with the stated allowance for fp32 ties)."""

import sys

import numpy as np
import torch

import oracle
from precision_optimizer_step_amd import opt8
from workloads import gen

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
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a).copy()).to(DEV)


def to_host(t: torch.Tensor, like: np.ndarray) -> np.ndarray:
    if t is None:
        return None
    h = t.detach().cpu().numpy()
    return h.view(like.dtype) if h.dtype != like.dtype else h


class DevTensorSet:
    """One tensor's param/grad/state on the device, mirroring host numpy arrays
    (v and av are None for the one-state rules)."""

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


ALGO_ADAMW = 0
STEP_FN = {ALGO_ADAMW: "opt8_adamw_step", oracle.ALGO_LION: "opt8_lion_step",
           oracle.ALGO_MOMENTUM: "opt8_momentum_step"}


def gpu_step(sets, hp: "oracle.Hparams", algo=ALGO_ADAMW):
    descs = [s.desc() for s in sets]
    getattr(opt8, STEP_FN[algo])(descs, opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps,
                                                          hp.weight_decay, hp.step, hp.seed,
                                                          hp.param_round, hp.state_round))
    torch.cuda.synchronize()


def oracle_step(s: DevTensorSet, state, hp, algo=ALGO_ADAMW):
    """state = (param, m, v, am, av) on the host; returns the oracle's next state
    (v and av None for the one-state rules)."""
    p, m, v, am, av = state
    if algo == ALGO_ADAMW:
        return list(oracle.step_tensor(s.mode, p, s.host[1], m, v, am, av, hp, s.tensor_id, s.index_base))
    p2, m2, am2 = oracle.step_tensor_1state(algo, s.mode, p, s.host[1], m, am, hp, s.tensor_id,
                                            s.index_base)
    return [p2, m2, None, am2, None]


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
        # NaN on exactly the same blocks first (a comparison with NaN is always False)
        nan_g, nan_w = np.isnan(g), np.isnan(w)
        assert np.array_equal(nan_g, nan_w), f"{name}: NaN absmax at blocks " \
            f"{np.flatnonzero(nan_g != nan_w)[:5]} on one side only"
        g, w = g[~nan_w], w[~nan_w]
        bad = np.abs(g - w) > ABSMAX_RTOL * np.abs(w)
        bad |= np.isinf(g) != np.isinf(w)
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
    two = want[2] is not None     # the one-state rules have no v
    if mode == oracle.MODE_8BIT:
        compare(f"{label}.m", got[1], want[1], "code", stats)
        compare(f"{label}.absmax_m", got[3], want[3], "absmax", stats)
        if two:
            compare(f"{label}.v", got[2], want[2], "code", stats)
            compare(f"{label}.absmax_v", got[4], want[4], "absmax", stats)
    else:
        kind = "bf16" if mode == oracle.MODE_BF16_SR else "f32"
        compare(f"{label}.m", got[1], want[1], kind, stats)
        if two:
            compare(f"{label}.v", got[2], want[2], kind, stats)


# ----------------------------------------------------------------------------- full-size lists
# The whole list lives on the device; sampled blocks are copied to the host
# before and after one step and checked block by block against the oracle.
BLOCK = 2048


def _mode_of(w, spec):
    if w.state_mode == "bf16":
        return oracle.MODE_BF16_SR
    return opt8.opt8_default_mode(spec.numel)


def build_list(w, step=1, state_seed=7, one_state=False):
    """Device tensors of workload w: params, step-`step` grads and a random non-zero state
    (m only when one_state)."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    out = []
    for tid, spec in enumerate(w.tensors):
        n = spec.numel
        mode = _mode_of(w, spec)
        P = torch.empty(n, dtype=torch.bfloat16, device=dev)
        G = torch.empty(n, dtype=torch.bfloat16, device=dev)
        gen.param_init_device(spec, w, tid, P)
        gen.grad_init_device(spec, w, step, tid, G)
        g.manual_seed(gen.derived_seed(state_seed, 0, tid, gen.P_STATE_M))
        AM = AV = None
        if mode == oracle.MODE_8BIT:
            M = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev, generator=g)
            V = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev, generator=g)
            nb = (n + BLOCK - 1) // BLOCK
            AM = torch.empty(nb, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=g).abs_()
            AV = torch.empty(nb, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=g).square_()
        elif mode == oracle.MODE_BF16_SR:
            M = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_(0, 1e-3, generator=g)
            V = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_(0, 1e-3, generator=g).square_()
        else:
            M = torch.empty(n, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=g)
            V = torch.empty(n, dtype=torch.float32, device=dev).normal_(0, 1e-3, generator=g).square_()
        if one_state:
            V = AV = None
        out.append(dict(tid=tid, mode=mode, n=n, P=P, G=G, M=M, V=V, AM=AM, AV=AV))
    return out


def descriptors(lst):
    return opt8.tensor_array(opt8.make_tensor(t["P"], t["G"], t["M"], t["V"], t["AM"], t["AV"],
                                              tensor_id=t["tid"], mode=t["mode"]) for t in lst)


def sample_blocks(lst, per_tensor, rng):
    pick = []
    for i, t in enumerate(lst):
        nb = (t["n"] + BLOCK - 1) // BLOCK
        cand = {0, nb - 1}
        if nb > 2:
            cand |= set(int(x) for x in rng.integers(1, nb - 1, min(per_tensor, nb - 2)))
        pick += [(i, b) for b in sorted(cand)]
    return pick


def _np(t, dtype):
    h = t.detach().cpu()
    if h.dtype == torch.bfloat16:
        h = h.view(torch.int16)
    return h.numpy().view(dtype).copy()


def snapshot(lst, blocks):
    snap = []
    for i, b in blocks:
        t = lst[i]
        lo, hi = b * BLOCK, min(t["n"], (b + 1) * BLOCK)
        sd = np.uint8 if t["mode"] == oracle.MODE_8BIT else np.uint16 if t["mode"] == oracle.MODE_BF16_SR \
            else np.float32
        item = dict(p=_np(t["P"][lo:hi], np.uint16), g=_np(t["G"][lo:hi], np.uint16),
                    m=_np(t["M"][lo:hi], sd), v=None, am=None, av=None)
        if t["V"] is not None:
            item["v"] = _np(t["V"][lo:hi], sd)
        if t["AM"] is not None:
            item["am"] = _np(t["AM"][b:b + 1], np.float32)
        if t["AV"] is not None:
            item["av"] = _np(t["AV"][b:b + 1], np.float32)
        snap.append(item)
    return snap
