"""Seeded synthetic inputs (parameters, gradients, optimizer state).

Shared by the tests, the benchmark and the smoke check.  Holds none of the
optimizer's arithmetic: values are drawn in float32 and handed to torch for
the float32 -> bfloat16 conversion.

Host generator (exact, reproducible anywhere): numpy PCG64 seeded by
SeedSequence(seed, spawn_key=(step, tensor_id, purpose)).  Device generator
(for the multi-GB lists): torch's CUDA generator seeded from the same
SeedSequence; it draws the same distributions but different values.

Recipes (sigma is the standard deviation of N(0, sigma)):
  params      weights and embeddings N(0, 0.02), biases 0, LayerNorm weight 1,
              LayerNorm bias 0; the single 1M tensor N(0, 0.02).
  "single"    N(0, 1e-3), round(0.1% * n) elements (distinct, uniform) x100.
  "fan_in"    N(0, 1e-3 / sqrt(fan_in)) per tensor (fan_in: input width of a
              weight, d for embeddings, 1 for 1-D tensors).
  "nonuniform" embedding (wte) rows: round(5% * V) rows N(0, 1e-2), the
              others 0, rows redrawn per step; LayerNorm N(0, 1e-4); every
              other tensor N(0, 1e-3) with round(0.01% * n) elements x1000.
  "plain"     N(0, 1e-3).
  "outliers100" N(0, 1e-3) with round(0.01% * n) elements x100.
Outlier positions and sparse rows are redrawn per step and tensor.
"""

import math

import numpy as np
import torch

from .shapes import TensorSpec, Workload

P_PARAM, P_GRAD, P_OUTLIER, P_ROWS, P_STATE_M, P_STATE_V, P_ABSMAX = range(7)


def _rng(seed: int, step: int, tensor_id: int, purpose: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(step, tensor_id, purpose))
    return np.random.Generator(np.random.PCG64(ss))


def derived_seed(seed: int, step: int, tensor_id: int, purpose: int) -> int:
    ss = np.random.SeedSequence(seed, spawn_key=(step, tensor_id, purpose))
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), converted by torch."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _normal(rng, n, sigma):
    return rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)


# ----------------------------------------------------------------------------- host
def param_init(w: Workload, tid: int) -> np.ndarray:
    spec = w.tensors[tid]
    n = spec.numel
    if spec.kind in ("bias", "ln_bias"):
        return np.zeros(n, dtype=np.uint16)
    if spec.kind == "ln_weight":
        return np.full(n, 0x3F80, dtype=np.uint16)  # bf16 1.0
    return to_bf16_bits(_normal(_rng(w.seed, 0, tid, P_PARAM), n, 0.02))


def _outliers(x, rng, frac, scale):
    k = int(round(frac * x.size))
    if k:
        idx = rng.choice(x.size, size=k, replace=False)
        x[idx] *= np.float32(scale)
    return x


def grad_values(w: Workload, step: int, tid: int) -> np.ndarray:
    """float32 gradient values of tensor tid at 1-based step."""
    spec = w.tensors[tid]
    n = spec.numel
    rng = _rng(w.seed, step, tid, P_GRAD)
    r = w.grad_recipe
    if r == "single":
        return _outliers(_normal(rng, n, 1e-3), _rng(w.seed, step, tid, P_OUTLIER), 1e-3, 100.0)
    if r == "fan_in":
        return _normal(rng, n, 1e-3 / math.sqrt(spec.fan_in))
    if r == "plain":
        return _normal(rng, n, 1e-3)
    if r == "outliers100":
        return _outliers(_normal(rng, n, 1e-3), _rng(w.seed, step, tid, P_OUTLIER), 1e-4, 100.0)
    if r == "nonuniform":
        if spec.name == "wte":
            rows, width = spec.shape
            g = np.zeros((rows, width), dtype=np.float32)
            k = int(round(0.05 * rows))
            pick = _rng(w.seed, step, tid, P_ROWS).choice(rows, size=k, replace=False)
            g[pick] = _normal(rng, k * width, 1e-2).reshape(k, width)
            return g.reshape(-1)
        if spec.kind in ("ln_weight", "ln_bias"):
            return _normal(rng, n, 1e-4)
        return _outliers(_normal(rng, n, 1e-3), _rng(w.seed, step, tid, P_OUTLIER), 1e-4, 1000.0)
    raise ValueError(r)


def grad_init(w: Workload, step: int, tid: int) -> np.ndarray:
    return to_bf16_bits(grad_values(w, step, tid))


def random_state_8bit(seed: int, tid: int, n: int, scale: float = 1e-3):
    """Non-trivial 8-bit state: uniform codes, absmax ~ |N(0, scale)| per block."""
    nb = (n + 2047) // 2048
    qm = _rng(seed, 0, tid, P_STATE_M).integers(0, 256, n, dtype=np.uint8)
    qv = _rng(seed, 0, tid, P_STATE_V).integers(0, 256, n, dtype=np.uint8)
    ab = np.abs(_normal(_rng(seed, 0, tid, P_ABSMAX), 2 * nb, scale))
    am = ab[:nb].copy()
    av = (ab[nb:] * ab[nb:]).astype(np.float32)
    return qm, qv, am, av


def random_state_f32(seed: int, tid: int, n: int, scale: float = 1e-3):
    m = _normal(_rng(seed, 0, tid, P_STATE_M), n, scale)
    v = _normal(_rng(seed, 0, tid, P_STATE_V), n, scale)
    v = (v * v).astype(np.float32)
    return m, v


def random_state_bf16(seed: int, tid: int, n: int, scale: float = 1e-3):
    m, v = random_state_f32(seed, tid, n, scale)
    return to_bf16_bits(m), to_bf16_bits(v)


# ----------------------------------------------------------------------------- device
def _dev_gen(seed, step, tid, purpose, device):
    g = torch.Generator(device=device)
    g.manual_seed(derived_seed(seed, step, tid, purpose))
    return g


def param_init_device(spec: TensorSpec, w: Workload, tid: int, out: torch.Tensor) -> None:
    """Fill a bf16 device tensor with the parameter recipe."""
    if spec.kind in ("bias", "ln_bias"):
        out.zero_()
    elif spec.kind == "ln_weight":
        out.fill_(1.0)
    else:
        out.normal_(0.0, 0.02, generator=_dev_gen(w.seed, 0, tid, P_PARAM, out.device))


def grad_init_device(spec: TensorSpec, w: Workload, step: int, tid: int, out: torch.Tensor) -> None:
    """Fill a bf16 device tensor with the gradient recipe (same distributions as the host)."""
    dev = out.device
    g = _dev_gen(w.seed, step, tid, P_GRAD, dev)
    go = _dev_gen(w.seed, step, tid, P_OUTLIER, dev)
    n = out.numel()
    flat = out.view(-1)
    r = w.grad_recipe

    def outl(frac, scale):
        k = int(round(frac * n))
        if k:
            idx = torch.randperm(n, generator=go, device=dev)[:k] if n <= (1 << 24) else \
                torch.randint(0, n, (k,), generator=go, device=dev)
            flat[idx] = flat[idx] * scale

    if r == "single":
        flat.normal_(0.0, 1e-3, generator=g)
        outl(1e-3, 100.0)
    elif r == "fan_in":
        flat.normal_(0.0, 1e-3 / math.sqrt(spec.fan_in), generator=g)
    elif r == "plain":
        flat.normal_(0.0, 1e-3, generator=g)
    elif r == "outliers100":
        flat.normal_(0.0, 1e-3, generator=g)
        outl(1e-4, 100.0)
    elif r == "nonuniform":
        if spec.name == "wte":
            rows, width = spec.shape
            out.view(rows, width).zero_()
            k = int(round(0.05 * rows))
            pick = torch.randperm(rows, generator=_dev_gen(w.seed, step, tid, P_ROWS, dev),
                                  device=dev)[:k]
            vals = torch.empty((k, width), dtype=out.dtype, device=dev).normal_(0.0, 1e-2, generator=g)
            out.view(rows, width)[pick] = vals
        elif spec.kind in ("ln_weight", "ln_bias"):
            flat.normal_(0.0, 1e-4, generator=g)
        else:
            flat.normal_(0.0, 1e-3, generator=g)
            outl(1e-4, 1000.0)
    else:
        raise ValueError(r)
