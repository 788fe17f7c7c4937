"""One AdamW step per tensor with 8-bit, bf16 or fp32 optimizer state (oracle).

TEST INFRASTRUCTURE ONLY (see the package header).

Passages followed (page title, part of the page):
  * "8-bit Optimizers via Block-wise Quantization", method bullets: state
    tensors are cut into blocks of 2048 elements; each block's maximum
    absolute value is its normalisation constant; normalised values become
    8-bit indices by a binary search over a non-linear code; decoding is a
    table lookup times the block maximum; the state is dequantised to 32-bit,
    updated and requantised.
  * "Stochastic rounding support for 8-bit optimizers", feature request and
    the scoping comment: full-precision update, bf16 parameters rounded up or
    down at random with a probability set by the rounding error, 8-bit state
    kept, no fp32 master copy, an fp32-state fallback for small tensors, and a
    weight-decay baseline to pick.
  * "[Feat]: Stochastic rounding of AdamW momentums", the use case and the
    comment thread: Adam arithmetic in float32 with the gradient cast to fp32
    first; the parameter update p + value * exp_avg / denom with
    value = -step_size, the add and the divide in fp32; bf16 momenta cast back
    each step with stochastic rounding; weight decay that must survive bf16
    with stochastic rounding.
  * "Stochastic Rounding for LLM Training: Theory and Practice", TL;DR and
    abstract: BF16-AdamW-SR (bf16 parameters and states, stochastic rounding).

Readings where the pages are silent (each repeated where it is used):
  * Bias correction is the standard Adam one with a 1-based step t;
    step_size = lr / (1 - beta1^t) and the second-moment correction
    rbc2 = 1 / sqrt(1 - beta2^t) are host scalars.
  * eps is added outside the square root, after bias correction:
    den = sqrt(v) * rbc2 + eps.
  * Weight decay is decoupled (AdamW): lr * wd * p is taken off the OLD
    parameter in fp32 in the same expression as the Adam step, then the sum is
    rounded once: p' = (p - lrwd * p) - step_size * (m / den).
  * Host scalars are computed in double (beta^t by repeated multiplication,
    no pow) and each is rounded once to fp32.
  * The parameter update uses the fp32 moments before requantisation.
  * A block whose new absmax is below the smallest normal fp32 (2^-126,
    including an all-zero block) stores the zero code everywhere; the stored
    absmax is still the true maximum.  The last block of a tensor may be
    partial; its absmax covers the valid elements only.  Blocks start at
    element 0 of each row-major flattened tensor (index_base shifts the
    global index of a shard, in whole blocks).
  * The fp32-state fallback is a per-tensor mode; the default policy gives it
    to tensors with fewer than 4096 elements.  The bf16-state mode keeps every
    tensor in bf16 and always rounds the moments stochastically (streams 1 and
    2); the round flag chooses only how the parameter is written.
  * The 8-bit state is rounded to the nearest codebook entry unless
    state_round asks for stochastic rounding between the two neighbouring
    entries (state_sr.py; streams 1 and 2, as for bf16 momenta).

Parity: pinned by tests against closed forms at step 1, torch.optim.AdamW
on fp32 (test side only), a float64 trajectory, invariants (zero lr and wd
leave parameters untouched), brute-force block max and nearest-entry search.
"""

import math
from dataclasses import dataclass

import numpy as np

from . import codebook
from .philox import sr_bits, STREAM_PARAM, STREAM_M, STREAM_V
from .rounding import bf16_to_f32, f32_to_bf16_rne, f32_to_bf16_sr

BLOCK = 2048
FP32_STATE_THRESHOLD = 4096
MIN_NORMAL_F32 = np.float32(2.0 ** -126)

MODE_8BIT = 0
MODE_BF16_SR = 1
MODE_FP32 = 2

ROUND_STOCHASTIC = 0
ROUND_NEAREST = 1


def default_mode(numel: int) -> int:
    """fp32 state for tensors under 4096 elements, 8-bit block-wise state otherwise."""
    return MODE_FP32 if numel < FP32_STATE_THRESHOLD else MODE_8BIT


@dataclass
class Hparams:
    lr: float
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    step: int = 1          # 1-based
    seed: int = 0          # 64-bit
    param_round: int = ROUND_STOCHASTIC
    state_round: int = 0   # 8-bit state: 0 nearest entry, 1 stochastic between neighbours


@dataclass
class Scalars:
    beta1: np.float32
    beta2: np.float32
    w1: np.float32         # 1 - beta1
    w2: np.float32         # 1 - beta2
    eps: np.float32
    step_size: np.float32  # lr / (1 - beta1^t)
    rbc2: np.float32       # 1 / sqrt(1 - beta2^t)
    lrwd: np.float32       # lr * weight_decay


def host_scalars(hp: Hparams) -> Scalars:
    """Derived step scalars: double arithmetic, each rounded once to fp32."""
    b1t = 1.0
    b2t = 1.0
    for _ in range(hp.step):
        b1t *= hp.beta1
        b2t *= hp.beta2
    bc1 = 1.0 - b1t
    bc2 = 1.0 - b2t
    f = np.float32
    return Scalars(
        beta1=f(hp.beta1),
        beta2=f(hp.beta2),
        w1=f(1.0 - hp.beta1),
        w2=f(1.0 - hp.beta2),
        eps=f(hp.eps),
        step_size=f(hp.lr / bc1),
        rbc2=f(1.0 / math.sqrt(bc2)),
        lrwd=f(hp.lr * hp.weight_decay),
    )


def _f32(a):
    assert a.dtype == np.float32, a.dtype
    return a


def nblocks(numel: int) -> int:
    return (numel + BLOCK - 1) // BLOCK


def _blocked(x: np.ndarray) -> np.ndarray:
    """View a flat array as [nblocks, 2048] rows, zero-padding the last row."""
    nb = nblocks(x.size)
    pad = np.zeros(nb * BLOCK, dtype=x.dtype)
    pad[: x.size] = x
    return pad.reshape(nb, BLOCK)


def dequantize_blockwise(codes: np.ndarray, absmax: np.ndarray, table: np.ndarray) -> np.ndarray:
    """x_i = table[code_i] * absmax[i // 2048] in fp32."""
    codes = np.asarray(codes, dtype=np.uint8)
    per_elem = np.repeat(np.asarray(absmax, dtype=np.float32), BLOCK)[: codes.size]
    return _f32(table[codes] * per_elem)


def quantize_blockwise(x: np.ndarray, mid: np.ndarray, zero_code: int):
    """Block absmax, normalise by fp32(1/absmax), code = #midpoints below the value.

    Returns (codes uint8[n], absmax float32[nblocks]).
    """
    x = _f32(np.asarray(x, dtype=np.float32))
    rows = _blocked(x)                        # zero padding never raises a max of |x|
    absmax = _f32(np.max(np.abs(rows), axis=1))
    codes = np.full(rows.shape, zero_code, dtype=np.uint8)
    live = absmax >= MIN_NORMAL_F32
    if live.any():
        inv = _f32(np.float32(1.0) / absmax[live])          # one IEEE divide per block
        normed = _f32(rows[live] * inv[:, None])            # one multiply per element
        codes[live] = np.searchsorted(mid, normed, side="left").astype(np.uint8)
    return codes.reshape(-1)[: x.size], absmax


def adamw_param_update(p: np.ndarray, g: np.ndarray, m1: np.ndarray, v1: np.ndarray, s: Scalars):
    """fp32 moments and the new fp32 parameter before it is rounded to bf16."""
    m2 = _f32(_f32(s.beta1 * m1) + _f32(s.w1 * g))
    v2 = _f32(_f32(s.beta2 * v1) + _f32(s.w2 * _f32(g * g)))
    den = _f32(_f32(np.sqrt(v2) * s.rbc2) + s.eps)
    u = _f32(m2 / den)
    pn = _f32(_f32(p - _f32(s.lrwd * p)) - _f32(s.step_size * u))
    return m2, v2, pn


def _round_param(pn, hp: Hparams, tensor_id: int, index):
    if hp.param_round == ROUND_NEAREST:
        return f32_to_bf16_rne(pn)
    return f32_to_bf16_sr(pn, sr_bits(hp.seed, hp.step, tensor_id, index, STREAM_PARAM))


def step_tensor(mode: int, param, grad, m, v, absmax_m, absmax_v, hp: Hparams,
                tensor_id: int, index_base: int = 0):
    """One optimizer step on one tensor.  Inputs are not modified.

    param, grad: uint16 bf16 patterns [n].
    m, v: uint8 codes (8-bit), uint16 bf16 patterns (bf16 state) or float32 (fp32 state).
    absmax_m, absmax_v: float32[ceil(n / 2048)] in 8-bit mode, else ignored.
    Returns (param, m, v, absmax_m, absmax_v) with the same dtypes
    (absmax entries are None outside 8-bit mode).
    """
    if index_base % BLOCK:
        raise ValueError("index_base must be a multiple of 2048")
    s = host_scalars(hp)
    param = np.asarray(param, dtype=np.uint16).reshape(-1)
    grad = np.asarray(grad, dtype=np.uint16).reshape(-1)
    n = param.size
    index = np.arange(index_base, index_base + n, dtype=np.uint64)
    p = bf16_to_f32(param)
    g = bf16_to_f32(grad)

    if mode == MODE_8BIT:
        cs, mid_s, cu, mid_u = codebook.tables()
        m1 = dequantize_blockwise(m, absmax_m, cs)
        v1 = dequantize_blockwise(v, absmax_v, cu)
    elif mode == MODE_BF16_SR:
        m1 = bf16_to_f32(m)
        v1 = bf16_to_f32(v)
    elif mode == MODE_FP32:
        m1 = _f32(np.asarray(m, dtype=np.float32).reshape(-1))
        v1 = _f32(np.asarray(v, dtype=np.float32).reshape(-1))
    else:
        raise ValueError(f"unknown mode {mode}")

    m2, v2, pn = adamw_param_update(p, g, m1, v1, s)
    p_out = _round_param(pn, hp, tensor_id, index)

    if mode == MODE_8BIT:
        if hp.state_round:
            from .state_sr import quantize_blockwise_sr
            qm, am = quantize_blockwise_sr(m2, cs, codebook.SIGNED_ZERO_CODE,
                                           sr_bits(hp.seed, hp.step, tensor_id, index, STREAM_M))
            qv, av = quantize_blockwise_sr(v2, cu, codebook.UNSIGNED_ZERO_CODE,
                                           sr_bits(hp.seed, hp.step, tensor_id, index, STREAM_V))
            return p_out, qm, qv, am, av
        qm, am = quantize_blockwise(m2, mid_s, codebook.SIGNED_ZERO_CODE)
        qv, av = quantize_blockwise(v2, mid_u, codebook.UNSIGNED_ZERO_CODE)
        return p_out, qm, qv, am, av
    if mode == MODE_BF16_SR:
        m_out = f32_to_bf16_sr(m2, sr_bits(hp.seed, hp.step, tensor_id, index, STREAM_M))
        v_out = f32_to_bf16_sr(v2, sr_bits(hp.seed, hp.step, tensor_id, index, STREAM_V))
        return p_out, m_out, v_out, None, None
    return p_out, m2.copy(), v2.copy(), None, None
