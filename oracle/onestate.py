"""One-state optimizers on the same 8-bit machinery: Lion and SGD with momentum (oracle).

TEST INFRASTRUCTURE ONLY (see the package header).

The pages name both and define neither: "8-bit Optimizers via Block-wise
Quantization" (motivation: optimizer states of algorithms such as Adam and
Momentum) and "Stochastic rounding support for 8-bit optimizers" (motivation:
even more memory saved with 8-bit Lion).  Readings, stated here and used by
the library alike:

Lion (Chen et al., "Symbolic Discovery of Optimization Algorithms", 2023):
    c  = beta1*m1 + (1-beta1)*g          direction from the OLD moment
    m2 = beta2*m1 + (1-beta2)*g          moment update
    p' = (p - lrwd*p) - lr*sign(c)       decoupled weight decay, sign(+-0) = +0
SGD with momentum (the torch.optim.SGD form with dampening 0):
    m2 = beta1*m1 + g
    p' = (p - lrwd*p) - lr*m2            weight decay decoupled, as for AdamW
Everything else is as for the AdamW oracle: fp32 with one rounding per
operation, host scalars in double rounded once (lr, lrwd, beta, 1-beta), the
state in one of three modes (8-bit block-wise with the SIGNED dynamic-tree
codebook, rounded to the nearest entry or, as state_round asks, stochastically
between neighbouring entries; bf16 written with stochastic rounding on stream
1; or fp32), the parameter written with stochastic rounding on stream 0 (or
nearest-even).

Parity: Lion is pinned by its step-1 closed form (p(1 - lr wd) - lr sign(g)),
by the sign invariant |p' - (p - lrwd p)| == lr exactly and by a float64
trajectory; momentum by torch.optim.SGD on CPU fp32 (a library routine, test
side only) and a float64 trajectory.
"""

from dataclasses import dataclass

import numpy as np

from . import codebook
from .adamw import (BLOCK, Hparams, MODE_8BIT, MODE_BF16_SR, MODE_FP32, ROUND_NEAREST,
                    dequantize_blockwise, quantize_blockwise, _f32)
from .philox import sr_bits, STREAM_PARAM, STREAM_M
from .rounding import bf16_to_f32, f32_to_bf16_rne, f32_to_bf16_sr

ALGO_LION = 1
ALGO_MOMENTUM = 2


@dataclass
class Scalars1:
    beta1: np.float32
    w1: np.float32        # 1 - beta1
    beta2: np.float32
    w2: np.float32        # 1 - beta2
    lr: np.float32
    lrwd: np.float32


def host_scalars_1state(hp: Hparams) -> Scalars1:
    f = np.float32
    return Scalars1(beta1=f(hp.beta1), w1=f(1.0 - hp.beta1), beta2=f(hp.beta2), w2=f(1.0 - hp.beta2),
                    lr=f(hp.lr), lrwd=f(hp.lr * hp.weight_decay))


def lion_update(p, g, m1, s: Scalars1):
    """(m2, p') of one Lion step in fp32."""
    c = _f32(_f32(s.beta1 * m1) + _f32(s.w1 * g))
    m2 = _f32(_f32(s.beta2 * m1) + _f32(s.w2 * g))
    sgn = _f32(np.sign(c))                       # +-1, +0 for +-0, NaN for NaN
    pn = _f32(_f32(p - _f32(s.lrwd * p)) - _f32(s.lr * sgn))
    return m2, pn


def momentum_update(p, g, m1, s: Scalars1):
    """(m2, p') of one momentum step in fp32."""
    m2 = _f32(_f32(s.beta1 * m1) + g)
    pn = _f32(_f32(p - _f32(s.lrwd * p)) - _f32(s.lr * m2))
    return m2, pn


def step_tensor_1state(algo: int, mode: int, param, grad, m, absmax_m, hp: Hparams, tensor_id: int,
                       index_base: int = 0):
    """One Lion or momentum step on one tensor.  Inputs are not modified.

    m: uint8 codes (8-bit), uint16 bf16 (bf16 state) or float32; absmax_m float32[nblocks] in
    8-bit mode.  Returns (param, m, absmax_m or None).
    """
    if index_base % BLOCK:
        raise ValueError("index_base must be a multiple of 2048")
    s = host_scalars_1state(hp)
    param = np.asarray(param, dtype=np.uint16).reshape(-1)
    grad = np.asarray(grad, dtype=np.uint16).reshape(-1)
    n = param.size
    index = np.arange(index_base, index_base + n, dtype=np.uint64)
    p = bf16_to_f32(param)
    g = bf16_to_f32(grad)
    cs, mid_s, _, _ = codebook.tables()
    if mode == MODE_8BIT:
        m1 = dequantize_blockwise(m, absmax_m, cs)
    elif mode == MODE_BF16_SR:
        m1 = bf16_to_f32(m)
    elif mode == MODE_FP32:
        m1 = _f32(np.asarray(m, dtype=np.float32).reshape(-1))
    else:
        raise ValueError(f"unknown mode {mode}")
    if algo == ALGO_LION:
        m2, pn = lion_update(p, g, m1, s)
    elif algo == ALGO_MOMENTUM:
        m2, pn = momentum_update(p, g, m1, s)
    else:
        raise ValueError(f"unknown algorithm {algo}")
    if hp.param_round == ROUND_NEAREST:
        p_out = f32_to_bf16_rne(pn)
    else:
        p_out = f32_to_bf16_sr(pn, sr_bits(hp.seed, hp.step, tensor_id, index, STREAM_PARAM))
    if mode == MODE_8BIT:
        if hp.state_round:
            from .state_sr import quantize_blockwise_sr
            qm, am = quantize_blockwise_sr(m2, cs, codebook.SIGNED_ZERO_CODE,
                                           sr_bits(hp.seed, hp.step, tensor_id, index, STREAM_M))
            return p_out, qm, am
        qm, am = quantize_blockwise(m2, mid_s, codebook.SIGNED_ZERO_CODE)
        return p_out, qm, am
    if mode == MODE_BF16_SR:
        return p_out, f32_to_bf16_sr(m2, sr_bits(hp.seed, hp.step, tensor_id, index, STREAM_M)), None
    return p_out, m2.copy(), None
